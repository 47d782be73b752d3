// gdn_epilogue.hip -- the layer's output epilogue on gfx950: gated RMS norm
// of each (token, value head) row of Dv outputs,
//   out = x / sqrt(mean(x^2) + eps) * weight * act(z),  act = silu or logistic
// (vllm.cpp cpu_ops.cpp, RmsNormGatedKernel, norm before gate with one group
// per row; ferrum-kernels cpu.rs, gated_rms_norm_f32).
//
// Each lane owns 8 consecutive values of a row, so a row is Dv/8 aligned
// lanes and its sum of squares a cross-lane sum within them; a wave covers
// four groups of 64/(Dv/8) rows, issuing all their loads before it computes,
// and touches each byte of x, z and out once.  The gate is
// read through a row stride so that it can be the z columns of a packed
// [q | k | v | z] projection row.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kNormWaves = 4;
constexpr int kPerLane = 8;
constexpr int kGroups = 4;   // row groups per wave, loaded together

template <typename T, int D>
__global__ __launch_bounds__(kNormWaves * 64) void gated_rmsnorm_kernel(GatedNormParams p) {
  constexpr int LPR = D / kPerLane;  // lanes per row
  constexpr int RPW = 64 / LPR;      // rows per wave per group
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t rows = (int64_t)p.T * p.H;
  const int c = (lane % LPR) * kPerLane;
  float w[kPerLane];
  load_n<T, kPerLane>(static_cast<const T*>(p.w) + c, w);
  // kGroups groups of RPW rows per wave, all loads issued before any use;
  // lanes past the last row work on the last row (all lanes of a row agree)
  // and store nothing, so every lane joins the cross-lane sum
  const int64_t base = ((int64_t)blockIdx.x * kNormWaves + wave) * RPW * kGroups + lane / LPR;
  float x[kGroups][kPerLane], z[kGroups][kPerLane];
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int64_t row_raw = base + (int64_t)gi * RPW;
    const int64_t row = row_raw < rows ? row_raw : rows - 1;
    const int64_t t = row / p.H;
    const int h = (int)(row % p.H);
    load_n<T, kPerLane>(static_cast<const T*>(p.x) + row * D + c, x[gi]);
    load_n<T, kPerLane>(static_cast<const T*>(p.z) + t * p.z_stride + (int64_t)h * D + c, z[gi]);
  }
#pragma unroll
  for (int gi = 0; gi < kGroups; ++gi) {
    const int64_t row_raw = base + (int64_t)gi * RPW;
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) ss += x[gi][i] * x[gi][i];
    ss = group_sum<LPR>(ss);
    const float inv = 1.0f / sqrtf(ss / (float)D + p.eps);
    float y[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
      const float act = p.sig ? sigmoid_f(z[gi][i]) : silu_f(z[gi][i]);
      y[i] = x[gi][i] * inv * w[i] * act;
    }
    if (row_raw < rows) store_n<T, kPerLane>(static_cast<T*>(p.out) + row_raw * D + c, y);
  }
}

template <typename T>
hipError_t launch_t(const GatedNormParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.T * p.H;
  const int64_t rows_per_block = (int64_t)kNormWaves * kGroups * (64 / (p.D / kPerLane));
  const unsigned grid = (unsigned)((rows + rows_per_block - 1) / rows_per_block);
  switch (p.D) {
    case 16: gated_rmsnorm_kernel<T, 16><<<grid, kNormWaves * 64, 0, stream>>>(p); break;
    case 32: gated_rmsnorm_kernel<T, 32><<<grid, kNormWaves * 64, 0, stream>>>(p); break;
    case 64: gated_rmsnorm_kernel<T, 64><<<grid, kNormWaves * 64, 0, stream>>>(p); break;
    case 128: gated_rmsnorm_kernel<T, 128><<<grid, kNormWaves * 64, 0, stream>>>(p); break;
    default: gated_rmsnorm_kernel<T, 256><<<grid, kNormWaves * 64, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rmsnorm(const GatedNormParams& p, hipStream_t stream) {
  return p.io == GDN_F32 ? launch_t<float>(p, stream) : launch_t<bf16>(p, stream);
}

}  // namespace gdn
