// probe_slot_rmw.hip -- a measurement probe, not part of the library's API:
// the decode's state stream (in-place read-modify-write of whole 2 MB slots
// of an f32 pool, a random subset of the slots per call) with a trivial
// per-element update and none of the decode's other work.  Its rate is the
// ceiling of that access pattern on the device; bench.py --rmw-probe times it
// under several workgroup-to-region mappings.  Built into libgdn_probe.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Workgroup g streams region g % regions of the slot slots[g / regions]:
// `rows` slots of slot_floats f32 each, regions of slot_floats / regions,
// walked in batches of THREADS * LOADS 16-byte vectors (consecutive threads on
// consecutive vectors), the next batch loaded before the current one is
// updated and stored.  The host checks that a region is a whole number of
// batches.
template <int THREADS, int LOADS, bool NT>
__global__ __launch_bounds__(THREADS) void slot_rmw_kernel(float* pool, const int32_t* slots, int64_t slot_floats,
                                                            int regions) {
  const int64_t region_floats = slot_floats / regions;
  const int b = blockIdx.x / regions, rg = blockIdx.x % regions;
  float* base = pool + (int64_t)slots[b] * slot_floats + rg * region_floats;
  constexpr int BATCH = THREADS * LOADS * 4;
  const int iters = (int)(region_floats / BATCH);
  const int t = threadIdx.x;
  auto addr = [&](int it, int u) { return base + (int64_t)it * BATCH + ((int64_t)u * THREADS + t) * 4; };
  v4u raw[LOADS], nxt[LOADS];
#pragma unroll
  for (int u = 0; u < LOADS; ++u) raw[u] = *reinterpret_cast<const v4u*>(addr(0, u));
  for (int it = 0; it < iters; ++it) {
    if (it + 1 < iters) {
#pragma unroll
      for (int u = 0; u < LOADS; ++u) nxt[u] = *reinterpret_cast<const v4u*>(addr(it + 1, u));
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      float4 f = *reinterpret_cast<float4*>(&raw[u]);
      f.x = f.x * 0.999f + 1e-7f;
      f.y = f.y * 0.999f + 1e-7f;
      f.z = f.z * 0.999f + 1e-7f;
      f.w = f.w * 0.999f + 1e-7f;
      const v4u o = *reinterpret_cast<v4u*>(&f);
      if (NT) __builtin_nontemporal_store(o, reinterpret_cast<v4u*>(addr(it, u)));
      else *reinterpret_cast<v4u*>(addr(it, u)) = o;
    }
#pragma unroll
    for (int u = 0; u < LOADS; ++u) raw[u] = nxt[u];
  }
}

}  // namespace

// mode 0: 256 threads per workgroup over regions of slot_floats/regions, 8
//         loads per lane, nontemporal stores (the decode's shape at regions = 16)
// mode 1: the same with ordinary stores
// mode 2: 1024 threads per workgroup, one whole slot each (regions must be 1)
// Returns 0, or -1 when a region is not a whole number of batches, or the HIP
// error of the launch.  pool holds num_slots * slot_floats f32; slots holds
// `rows` indices in [0, num_slots), which the caller guarantees.
extern "C" int gdn_probe_slot_rmw(float* pool, const int32_t* slots, int32_t rows, int64_t slot_floats,
                                  int32_t regions, int32_t mode, void* stream) {
  if (rows <= 0 || regions <= 0 || slot_floats % regions != 0) return -1;
  const int64_t region = slot_floats / regions;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const unsigned grid = (unsigned)rows * (unsigned)regions;
  if (mode == 0 || mode == 1) {
    if (region % (256 * 8 * 4) != 0) return -1;
    if (mode == 0) slot_rmw_kernel<256, 8, true><<<grid, 256, 0, s>>>(pool, slots, slot_floats, regions);
    else slot_rmw_kernel<256, 8, false><<<grid, 256, 0, s>>>(pool, slots, slot_floats, regions);
  } else if (mode == 2) {
    if (regions != 1 || region % (1024 * 8 * 4) != 0) return -1;
    slot_rmw_kernel<1024, 8, true><<<grid, 1024, 0, s>>>(pool, slots, slot_floats, regions);
  } else {
    return -1;
  }
  return (int)hipGetLastError();
}
