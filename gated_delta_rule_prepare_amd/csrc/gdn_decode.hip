// gdn_decode.hip -- fused single-token GDN step against slot-indexed pools.
//
// One workgroup (4 waves) per (batch row, key head kh).  It owns the
// r = Hv/Hk value heads kh*r .. kh*r+r-1 that share q and k, i.e. R = r*Dv
// state rows of Dk elements, which sit contiguously in the slot's pool entry.
//
// Phase A (prepare, vllm.cpp cpu_ops.cpp CausalConv1dUpdateKernel and
// GdnPackedDecodeKernel): the 2*Dk + R channels of this key head are
// convolved against the slot's conv history, which is shifted left and
// appended with the raw input in place; SiLU; q and k are L2-normalised;
// g and beta per value head.  The first batch of state rows is already in
// flight while this runs, since the state loads do not depend on it.
//
// Phase B (the recurrence, vllm.cpp cpu_ops.cpp GdnHeadTokenStep): state rows
// stream through registers.  A lane holds 16 bytes of a row (Dk/lanes-per-row
// columns); a wave load covers 1 KiB of consecutive rows; a lane has eight
// such loads per batch and two batches in flight.  Per row the two
// dot products S.k and S.q are formed in one pass and summed across the
// lanes of the row; then, with d = exp(g):
//   u = d (S.k);  delta = beta (v - u);  o = d (S.q) + delta (k.q);
//   S' = d S + delta k
// which is the token step written so that the row is read once and written
// once.  Value rows are independent, so rows need no synchronisation.
//
// The outputs of a row's R value rows are kept in LDS and written out in
// one coalesced pass after the stream (rather than as scattered 2-byte
// stores during it).  With the output epilogue (gdn_decode_gated) they are
// kept rounded as they would be stored, and each wave applies the gated RMS
// norm to one value head: the workgroup owns all Dv outputs of its heads.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// The state is read and written once per call.  Ordinary loads and
// nontemporal stores measured fastest for this slot-scattered stream on
// MI355X (nontemporal loads gained nothing here).
__device__ __forceinline__ uint4 load_stream(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void store_stream(void* p, const uint4& u) {
  const v4u v = {u.x, u.y, u.z, u.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p));
}

constexpr int kDecWaves = 4;
constexpr int kDecThreads = kDecWaves * 64;
constexpr int kLoads = 8;  // 16-byte state loads per lane per batch (two batches in flight)

// value as stored in ActT and read back
template <typename ActT>
__device__ __forceinline__ float round_act(float v) {
  if constexpr (std::is_same<ActT, float>::value) return v;
  else return bf16_to_f32(f32_to_bf16(v));
}

template <typename ActT, typename StT, int DK, bool GATED>
__global__ __launch_bounds__(kDecThreads) void decode_kernel(DecodeParams p) {
  constexpr int SV = Elem<StT>::kVec;       // state elements per lane load
  constexpr int LPR = DK / SV;              // lanes per state row
  static_assert(LPR >= 1 && LPR <= 64, "lanes per row");
  constexpr int RPL = 64 / LPR;             // rows per wave load
  constexpr int ROWS_PER_ITER = kDecWaves * kLoads * RPL;

  extern __shared__ float smem[];
  const int kh = blockIdx.x;
  const int b = blockIdx.y;
  const int r = p.Hv / p.Hk;
  const int Dv = p.Dv;
  const int R = r * Dv;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  ActT* __restrict__ out = static_cast<ActT*>(p.out) + ((int64_t)b * p.Hv + (int64_t)kh * r) * Dv;
  const int slot = p.slots[b];
  if (slot < 0 || slot >= p.num_slots) {  // inert row: zero output, pools untouched
    for (int i = tid; i < R; i += kDecThreads) Elem<ActT>::store(out + i, 0.0f);
    return;
  }
  StT* __restrict__ S = static_cast<StT*>(p.ssm_pool) + ((int64_t)slot * p.Hv + (int64_t)kh * r) * Dv * DK;

  const int sub = lane / LPR;          // row within this wave's load
  const int col = (lane % LPR) * SV;   // first state column of this lane
  // Workgroups start their stream at different batches of their rows (a
  // rotation by block index; every batch is still visited once), so the
  // workgroups in flight do not all open the same offsets of their regions
  // at the same moment.
  const int iters = (R + ROWS_PER_ITER - 1) / ROWS_PER_ITER;
  const int rot = (int)((blockIdx.x * 5u + blockIdx.y * 3u) % (unsigned)iters);
  auto row_of = [&](int it, int u) {
    return ((it + rot) % iters) * ROWS_PER_ITER + (u * kDecWaves + wave) * RPL + sub;
  };

  // issue the first batch of state loads before the prepare work
  uint4 raw[kLoads];
#pragma unroll
  for (int u = 0; u < kLoads; ++u) {
    const int row = row_of(0, u);
    raw[u] = load_stream(S + (int64_t)min(row, R - 1) * DK + col);
  }

  // ---- phase A: conv update + SiLU for the 2*DK + R channels of this key head
  float* s_y = smem;                      // [2*DK + R]
  float* s_decay = smem + 2 * DK + R;     // [r]
  float* s_beta = s_decay + r;            // [r]
  float* s_red = s_beta + r;              // [4]: 1/|q|, 1/|k|, k.q
  float* s_o = s_red + 4;                 // [R] outputs, written out coalesced after the stream
  float* s_z = s_o + R;                   // [R] with the epilogue: the gate of this row's heads
  float* s_w = s_z + R;                   // [Dv] with the epilogue: the norm weight
  const int K = p.K;
  const ActT* __restrict__ x = static_cast<const ActT*>(p.x) + (int64_t)b * p.x_stride;
  const ActT* __restrict__ w = static_cast<const ActT*>(p.w);
  ActT* __restrict__ hist = static_cast<ActT*>(p.conv_pool);
  const int key_dim = p.Hk * DK;
  for (int ch = tid; ch < 2 * DK + R; ch += kDecThreads) {
    const int cg = ch < DK ? kh * DK + ch
                 : ch < 2 * DK ? key_dim + kh * DK + (ch - DK)
                               : 2 * key_dim + kh * R + (ch - 2 * DK);
    const float xv = Elem<ActT>::load(x + cg);
    float acc = Elem<ActT>::load(w + (int64_t)cg * K + (K - 1)) * xv;
    if (K > 1) {
      ActT* h = hist + ((int64_t)slot * p.Cc + cg) * p.W;  // leading K-1 of W taps
      float old[3];
#pragma unroll
      for (int j = 0; j < 3; ++j)
        if (j < K - 1) {
          old[j] = Elem<ActT>::load(h + j);
          acc += Elem<ActT>::load(w + (int64_t)cg * K + j) * old[j];
        }
#pragma unroll
      for (int j = 0; j < 2; ++j)
        if (j < K - 2) Elem<ActT>::store(h + j, old[j + 1]);
      Elem<ActT>::store(h + (K - 2), xv);
    }
    s_y[ch] = silu_f(acc);
  }
  if constexpr (GATED) {
    // the epilogue's operands, read now so that their latency hides behind the stream
    const ActT* zr = static_cast<const ActT*>(p.gz) + (int64_t)b * p.gz_stride + (int64_t)kh * R;
    for (int i = tid; i < R; i += kDecThreads) s_z[i] = Elem<ActT>::load(zr + i);
    for (int j = tid; j < Dv; j += kDecThreads) s_w[j] = Elem<ActT>::load(static_cast<const ActT*>(p.gw) + j);
  }
  __syncthreads();
  if (wave < 3) {
    // wave 0: |q|^2, wave 1: |k|^2, wave 2: k.q (raw values)
    float acc = 0.0f;
    for (int d = lane; d < DK; d += 64) {
      const float qd = s_y[d], kd = s_y[DK + d];
      acc += wave == 0 ? qd * qd : (wave == 1 ? kd * kd : kd * qd);
    }
    acc = group_sum<64>(acc);
    if (lane == 0) s_red[wave] = acc;
  } else {
    for (int j = lane; j < r; j += 64) {
      const int h = kh * r + j;
      const float a = Elem<ActT>::load(static_cast<const ActT*>(p.a) + (int64_t)b * p.a_stride + h);
      const float bb = Elem<ActT>::load(static_cast<const ActT*>(p.b) + (int64_t)b * p.b_stride + h);
      s_decay[j] = expf(-expf(p.A_log[h]) * softplus_f(a + p.dt_bias[h]));
      s_beta[j] = sigmoid_f(bb);
    }
  }
  __syncthreads();
  const float q_inv = 1.0f / sqrtf(s_red[0] + 1e-6f);
  const float k_inv = 1.0f / sqrtf(s_red[1] + 1e-6f);
  const float kq = s_red[2] * q_inv * k_inv * p.scale;  // k_hat . (scale q_hat)
  float kv[SV], qv[SV];
#pragma unroll
  for (int i = 0; i < SV; ++i) {
    kv[i] = s_y[DK + col + i] * k_inv;
    qv[i] = s_y[col + i] * q_inv * p.scale;
  }

  // ---- phase B: stream the R state rows, the next batch of loads in flight
  // while the current one computes (rows past R re-read row R-1, unused)
  auto load_batch = [&](uint4* buf, int it) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) buf[u] = load_stream(S + (int64_t)min(row_of(it, u), R - 1) * DK + col);
  };
  auto compute_batch = [&](const uint4* buf, int it) {
#pragma unroll
    for (int u = 0; u < kLoads; ++u) {
      const int row = row_of(it, u);
      if (row >= R) continue;  // uniform across the row's lanes
      float st[SV];
      Elem<StT>::unpack(buf[u], st);
      float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
      for (int i = 0; i < SV; ++i) {
        p1 += st[i] * kv[i];
        p2 += st[i] * qv[i];
      }
      p1 = group_sum<LPR>(p1);
      p2 = group_sum<LPR>(p2);
      const int hl = row / Dv;
      const float d = s_decay[hl];
      const float delta = s_beta[hl] * (s_y[2 * DK + row] - d * p1);
      const float o = d * p2 + delta * kq;
#pragma unroll
      for (int i = 0; i < SV; ++i) st[i] = d * st[i] + delta * kv[i];
      store_stream(S + (int64_t)row * DK + col, Elem<StT>::pack(st));
      if ((lane % LPR) == 0) {
        s_o[row] = GATED ? round_act<ActT>(o) : o;
      }
    }
  };
  uint4 raw2[kLoads];
  for (int it = 0; it < iters; it += 2) {
    if (it + 1 < iters) load_batch(raw2, it + 1);  // workgroup-uniform branches: no batch is loaded twice
    compute_batch(raw, it);
    if (it + 2 < iters) load_batch(raw, it + 2);
    if (it + 1 < iters) compute_batch(raw2, it + 1);
  }

  if constexpr (!GATED) {
    // the R outputs of this workgroup are contiguous: one coalesced pass
    __syncthreads();
    for (int i = tid; i < R; i += kDecThreads) Elem<ActT>::store(out + i, s_o[i]);
  }

  // ---- epilogue: gated RMS norm of each value head over its Dv outputs
  // (vllm.cpp cpu_ops.cpp RmsNormGatedKernel; ferrum-kernels cpu.rs
  // gated_rms_norm_f32), one wave per value head
  if constexpr (GATED) {
    __syncthreads();
    for (int hl = wave; hl < r; hl += kDecWaves) {
      const float* ov = s_o + hl * Dv;
      const float* zv = s_z + hl * Dv;
      float ss = 0.0f;
      for (int j = lane; j < Dv; j += 64) ss += ov[j] * ov[j];
      ss = group_sum<64>(ss);
      const float inv = 1.0f / sqrtf(ss / (float)Dv + p.geps);
      for (int j = lane; j < Dv; j += 64) {
        const float act = p.gsig ? sigmoid_f(zv[j]) : silu_f(zv[j]);
        Elem<ActT>::store(out + hl * Dv + j, ov[j] * inv * s_w[j] * act);
      }
    }
  }
}

template <typename ActT, typename StT, bool GATED>
hipError_t launch_dk(const DecodeParams& p, hipStream_t stream) {
  const int r = p.Hv / p.Hk;
  const size_t smem = (size_t)(2 * p.Dk + 2 * r * p.Dv + 2 * r + 4 + (GATED ? r * p.Dv + p.Dv : 0)) * sizeof(float);
  dim3 grid(p.Hk, p.B);
  switch (p.Dk) {
    case 16: decode_kernel<ActT, StT, 16, GATED><<<grid, kDecThreads, smem, stream>>>(p); break;
    case 32: decode_kernel<ActT, StT, 32, GATED><<<grid, kDecThreads, smem, stream>>>(p); break;
    case 64: decode_kernel<ActT, StT, 64, GATED><<<grid, kDecThreads, smem, stream>>>(p); break;
    case 128: decode_kernel<ActT, StT, 128, GATED><<<grid, kDecThreads, smem, stream>>>(p); break;
    default: decode_kernel<ActT, StT, 256, GATED><<<grid, kDecThreads, smem, stream>>>(p); break;
  }
  return hipGetLastError();
}

template <typename ActT, bool GATED>
hipError_t launch_state(const DecodeParams& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_dk<ActT, float, GATED>(p, stream);
    case GDN_BF16: return launch_dk<ActT, bf16, GATED>(p, stream);
    default: return launch_dk<ActT, f16, GATED>(p, stream);
  }
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.gated) return p.act == GDN_F32 ? launch_state<float, true>(p, stream) : launch_state<bf16, true>(p, stream);
  return p.act == GDN_F32 ? launch_state<float, false>(p, stream) : launch_state<bf16, false>(p, stream);
}

}  // namespace gdn
