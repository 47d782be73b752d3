// gdn_spec.hip -- speculative multi-token GDN decode against slot-indexed
// pools: each request brings up to C tokens (its last accepted token and
// the drafts after it) and a row of C state slots; the state after every
// token is kept, so that the next step can resume after whichever token was
// accepted last (vllm.cpp cpu_ops.cpp, CausalConv1dSpecUpdateKernel and
// GdnSpecDecodeKernel).
//
// One workgroup (4 waves) per (request, key head kh), owning the r = Hv/Hk
// value heads that share q and k: R = r*Dv state rows of Dk elements.
//
// Phase A: for the 2*Dk + R channels of this key head, the conv over the
// request's L tokens reads the K-1 taps of the widened conv row starting at
// tap num_accepted-1, then the L raw inputs; the row is then rewritten in
// place as its taps from num_accepted onwards followed by the L inputs.
// SiLU; per token the L2 norms of q and k, k.q and the gates.  All of it is
// kept in LDS, token-major.
//
// Phase B: the R state rows of the initial slot stream through registers
// once.  A row is advanced token by token with the single-token step
//   u = d (S.k);  delta = beta (v - u);  o = d (S.q) + delta (k.q);
//   S' = d S + delta k          (d = exp(g))
// and after token t it is stored into the slot of column t, so the state is
// read once and written L times: the kernel is bound by those writes.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef unsigned int v4u __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_state(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void store_state(void* p, const uint4& u) {
  const v4u v = {u.x, u.y, u.z, u.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p));
}

constexpr int kSpecWaves = 4;
constexpr int kSpecThreads = kSpecWaves * 64;
constexpr int kSpecLoads = 4;     // 16-byte state loads per lane per batch (two batches in flight)
constexpr int kSpecMaxCols = 8;
// 16-byte state loads per row per lane: with two, a row of 128 f32 columns
// spans 16 lanes, and its sums reduce within a 16-lane row of the wave
constexpr int kSpecVecsPerRow = 2;
constexpr int kSpecMaxKeep = 16;  // conv-row taps kept in registers across the shift

// LDS floats: per token the 2*Dk + R conv outputs, R outputs, r decays, r betas
// and 4 reductions; plus the C slot columns.
__host__ __device__ inline int spec_lds_floats(int Dk, int R, int r, int cols) {
  return cols * (2 * Dk + 2 * R + 2 * r + 4) + cols;
}

template <typename ActT, typename StT, int DK>
__global__ __launch_bounds__(kSpecThreads) void spec_decode_kernel(SpecDecodeParams p) {
  constexpr int SV = Elem<StT>::kVec;       // state elements per 16-byte load
  constexpr int NV = kSpecVecsPerRow < DK / SV ? kSpecVecsPerRow : DK / SV;  // 16-byte loads per row per lane
  constexpr int LPR = DK / (SV * NV);       // lanes per state row
  static_assert(LPR >= 1 && LPR <= 64, "lanes per row");
  static_assert(kSpecLoads % NV == 0, "whole rows per batch");
  constexpr int RPL = 64 / LPR;             // rows per wave load
  constexpr int RPB = kSpecLoads / NV;      // rows per lane per batch
  constexpr int ROWS_PER_ITER = kSpecWaves * RPB * RPL;

  extern __shared__ float smem[];
  const int kh = blockIdx.x;
  const int req = blockIdx.y;
  const int r = p.Hv / p.Hk;
  const int Dv = p.Dv;
  const int R = r * Dv;
  const int nch = 2 * DK + R;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t out_tok = (int64_t)p.Hv * Dv;  // output elements per token

  const int lo = p.cu[req];
  const int L = p.cu[req + 1] - lo;
  ActT* __restrict__ out = static_cast<ActT*>(p.out) + (int64_t)lo * out_tok + (int64_t)kh * R;
  if (L <= 0) return;
  const int32_t* __restrict__ srow = p.state_idx + (int64_t)req * p.cols;
  const int nat = p.num_accepted[req];
  const int init = (nat >= 1 && nat <= p.cols) ? srow[nat - 1] : -1;
  const int cslot = srow[0];
  if (init < 0 || init >= p.num_slots || cslot < 0 || cslot >= p.num_slots || L > p.cols) {
    // padding request: zero output, pools untouched
    for (int t = 0; t < L; ++t)
      for (int i = tid; i < R; i += kSpecThreads) Elem<ActT>::store(out + t * out_tok + i, 0.0f);
    return;
  }
  const StT* __restrict__ S0 = static_cast<const StT*>(p.ssm_pool) + ((int64_t)init * p.Hv + (int64_t)kh * r) * Dv * DK;

  // a lane holds NV groups of SV columns of a row, LPR*SV columns apart, so
  // that each load instruction of a wave reads whole 256-byte row segments
  const int sub = lane / LPR;          // row within this wave's load
  const int col = (lane % LPR) * SV;   // first column of the lane's first group
  auto row_of = [&](int it, int u) { return it * ROWS_PER_ITER + (u * kSpecWaves + wave) * RPL + sub; };
  auto load_batch = [&](uint4* buf, int it) {
#pragma unroll
    for (int u = 0; u < RPB; ++u)
#pragma unroll
      for (int v = 0; v < NV; ++v)
        buf[u * NV + v] = load_state(S0 + (int64_t)min(row_of(it, u), R - 1) * DK + v * LPR * SV + col);
  };

  // the first batch of state loads goes out before the prepare work
  uint4 raw[kSpecLoads];
  load_batch(raw, 0);

  float* s_y = smem;                          // [L][nch] conv outputs; q, k normalised in place
  float* s_o = s_y + p.cols * nch;            // [L][R] outputs
  float* s_decay = s_o + p.cols * R;          // [L][r]
  float* s_beta = s_decay + p.cols * r;       // [L][r]
  float* s_red = s_beta + p.cols * r;         // [L][4]: |q|^2, |k|^2, k.q, then k_hat.(scale q_hat)
  int* s_snap = reinterpret_cast<int*>(s_red + p.cols * 4);  // [C] snapshot slot per column, -1 = none

  // ---- phase A: widened-window conv + SiLU for the channels of this key head
  {
    const int K = p.K;
    const int W = p.W;
    const int off = nat - 1;
    const int keep = W - L;  // >= K-2 >= 0 since W >= (K-1) + (C-1) and L <= C
    const ActT* __restrict__ x = static_cast<const ActT*>(p.x) + (int64_t)lo * p.x_stride;
    const ActT* __restrict__ w = static_cast<const ActT*>(p.w);
    ActT* __restrict__ crow = static_cast<ActT*>(p.conv_pool) + (int64_t)cslot * p.Cc * W;
    const int key_dim = p.Hk * DK;
    for (int ch = tid; ch < nch; ch += kSpecThreads) {
      const int cg = ch < DK ? kh * DK + ch
                   : ch < 2 * DK ? key_dim + kh * DK + (ch - DK)
                                 : 2 * key_dim + kh * R + (ch - 2 * DK);
      ActT* row = crow + (int64_t)cg * W;
      // register arrays are indexed with compile-time indices only (selects
      // on K), so that they stay in registers
      float wk[3], win[3], xs[kSpecMaxCols];
      const float wcur = Elem<ActT>::load(w + (int64_t)cg * K + (K - 1));  // tap of the current token
#pragma unroll
      for (int j = 0; j < 3; ++j) wk[j] = j < K - 1 ? Elem<ActT>::load(w + (int64_t)cg * K + j) : 0.0f;
#pragma unroll
      for (int j = 0; j < 3; ++j) win[j] = (j < K - 1 && off + j < W) ? Elem<ActT>::load(row + off + j) : 0.0f;
#pragma unroll
      for (int t = 0; t < kSpecMaxCols; ++t) xs[t] = t < L ? Elem<ActT>::load(x + (int64_t)t * p.x_stride + cg) : 0.0f;
      // win[j] is the stream value K-1-j positions before the current token
#pragma unroll
      for (int t = 0; t < kSpecMaxCols; ++t) {
        if (t < L) {
          float acc = wcur * xs[t];
#pragma unroll
          for (int j = 0; j < 3; ++j)
            if (j < K - 1) acc += wk[j] * win[j];
          s_y[t * nch + ch] = silu_f(acc);
#pragma unroll
          for (int j = 0; j < 3; ++j) win[j] = j < K - 2 ? win[(j + 1) % 3] : (j == K - 2 ? xs[t] : win[j]);
        }
      }
      // the row becomes taps off+1 .. off+W-L, then the L inputs.  The kept
      // taps are all read before the first write; for rows wider than the
      // register buffer, reading ahead of the write position keeps the
      // in-place shift safe
      if (keep <= kSpecMaxKeep) {
        float kept[kSpecMaxKeep];
#pragma unroll
        for (int j = 0; j < kSpecMaxKeep; ++j)
          kept[j] = (j < keep && off + 1 + j < W) ? Elem<ActT>::load(row + off + 1 + j) : 0.0f;
#pragma unroll
        for (int j = 0; j < kSpecMaxKeep; ++j)
          if (j < keep) Elem<ActT>::store(row + j, kept[j]);
      } else {
        for (int j = 0; j < keep; ++j) {
          const int src = off + 1 + j;
          Elem<ActT>::store(row + j, src < W ? Elem<ActT>::load(row + src) : 0.0f);
        }
      }
#pragma unroll
      for (int t = 0; t < kSpecMaxCols; ++t)
        if (t < L) Elem<ActT>::store(row + keep + t, xs[t]);
    }
  }
  if (tid < p.cols) {
    const int s = tid < L ? srow[tid] : -1;
    s_snap[tid] = (s >= 0 && s < p.num_slots) ? s : -1;
  }
  __syncthreads();
  if (wave < 3) {
    // wave 0: |q|^2, wave 1: |k|^2, wave 2: k.q (raw values), per token
    for (int t = 0; t < L; ++t) {
      const float* y = s_y + t * nch;
      float acc = 0.0f;
      for (int d = lane; d < DK; d += 64) {
        const float qd = y[d], kd = y[DK + d];
        acc += wave == 0 ? qd * qd : (wave == 1 ? kd * kd : kd * qd);
      }
      acc = group_sum<64>(acc);
      if (lane == 0) s_red[t * 4 + wave] = acc;
    }
  } else {
    for (int e = lane; e < L * r; e += 64) {
      const int t = e / r, j = e % r;
      const int h = kh * r + j;
      const float a = Elem<ActT>::load(static_cast<const ActT*>(p.a) + (int64_t)(lo + t) * p.a_stride + h);
      const float bb = Elem<ActT>::load(static_cast<const ActT*>(p.b) + (int64_t)(lo + t) * p.b_stride + h);
      s_decay[e] = expf(-expf(p.A_log[h]) * softplus_f(a + p.dt_bias[h]));
      s_beta[e] = sigmoid_f(bb);
    }
  }
  __syncthreads();
  // normalise q (with the scale) and k in place; k_hat . (scale q_hat) per token
  for (int e = tid; e < L * 2 * DK; e += kSpecThreads) {
    const int t = e / (2 * DK), d = e % (2 * DK);
    const float* red = s_red + t * 4;
    const float f = d < DK ? p.scale / sqrtf(red[0] + 1e-6f) : 1.0f / sqrtf(red[1] + 1e-6f);
    s_y[t * nch + d] *= f;
  }
  if (tid < L) {
    const float* red = s_red + tid * 4;
    s_red[tid * 4 + 3] = red[2] * (1.0f / sqrtf(red[0] + 1e-6f)) * (1.0f / sqrtf(red[1] + 1e-6f)) * p.scale;
  }
  __syncthreads();

  // ---- phase B: stream the R rows of the initial state; per row, L token
  // steps with a snapshot store after each
  StT* __restrict__ pool = static_cast<StT*>(p.ssm_pool);
  const int64_t head_off = (int64_t)kh * r * Dv * DK;
  const int iters = (R + ROWS_PER_ITER - 1) / ROWS_PER_ITER;
  // token-outer, row-inner: the kSpecLoads rows of a lane advance together,
  // so their reductions overlap and one token's q and k are read from LDS
  // once for all of them
  auto compute_batch = [&](const uint4* buf, int it) {
    float st[RPB][NV * SV];
#pragma unroll
    for (int u = 0; u < RPB; ++u)
#pragma unroll
      for (int v = 0; v < NV; ++v) Elem<StT>::unpack(buf[u * NV + v], st[u] + v * SV);
    for (int t = 0; t < L; ++t) {
      const float* y = s_y + t * nch;
      float kv[NV * SV], qv[NV * SV];
#pragma unroll
      for (int v = 0; v < NV; ++v)
#pragma unroll
        for (int i = 0; i < SV; ++i) {
          kv[v * SV + i] = y[DK + v * LPR * SV + col + i];
          qv[v * SV + i] = y[v * LPR * SV + col + i];
        }
      const float kq = s_red[t * 4 + 3];
      const int slot = s_snap[t];
      StT* __restrict__ snap = pool + (int64_t)max(slot, 0) * p.Hv * Dv * DK + head_off;
#pragma unroll
      for (int u = 0; u < RPB; ++u) {
        const int row = row_of(it, u);
        if (row >= R) continue;  // uniform across the row's lanes
        float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
        for (int i = 0; i < NV * SV; ++i) {
          p1 += st[u][i] * kv[i];
          p2 += st[u][i] * qv[i];
        }
        p1 = group_sum<LPR>(p1);
        p2 = group_sum<LPR>(p2);
        const int hl = row / Dv;
        const float d = s_decay[t * r + hl];
        const float delta = s_beta[t * r + hl] * (y[2 * DK + row] - d * p1);
        const float o = d * p2 + delta * kq;
#pragma unroll
        for (int i = 0; i < NV * SV; ++i) st[u][i] = d * st[u][i] + delta * kv[i];
        if (slot >= 0)
#pragma unroll
          for (int v = 0; v < NV; ++v)
            store_state(snap + (int64_t)row * DK + v * LPR * SV + col, Elem<StT>::pack(st[u] + v * SV));
        if ((lane % LPR) == 0) s_o[t * R + row] = o;
      }
    }
  };
  uint4 raw2[kSpecLoads];
  for (int it = 0; it < iters; it += 2) {
    load_batch(raw2, min(it + 1, iters - 1));
    compute_batch(raw, it);
    load_batch(raw, min(it + 2, iters - 1));
    if (it + 1 < iters) compute_batch(raw2, it + 1);
  }

  // the R outputs of each token are contiguous: one coalesced pass per token
  __syncthreads();
  for (int t = 0; t < L; ++t)
    for (int i = tid; i < R; i += kSpecThreads) Elem<ActT>::store(out + t * out_tok + i, s_o[t * R + i]);
}

template <typename ActT, typename StT>
hipError_t launch_dk(const SpecDecodeParams& p, hipStream_t stream) {
  const int r = p.Hv / p.Hk;
  const size_t smem = (size_t)spec_lds_floats(p.Dk, r * p.Dv, r, p.cols) * sizeof(float);
  dim3 grid(p.Hk, p.N);
  switch (p.Dk) {
    case 16: spec_decode_kernel<ActT, StT, 16><<<grid, kSpecThreads, smem, stream>>>(p); break;
    case 32: spec_decode_kernel<ActT, StT, 32><<<grid, kSpecThreads, smem, stream>>>(p); break;
    case 64: spec_decode_kernel<ActT, StT, 64><<<grid, kSpecThreads, smem, stream>>>(p); break;
    case 128: spec_decode_kernel<ActT, StT, 128><<<grid, kSpecThreads, smem, stream>>>(p); break;
    default: spec_decode_kernel<ActT, StT, 256><<<grid, kSpecThreads, smem, stream>>>(p); break;
  }
  return hipGetLastError();
}

template <typename ActT>
hipError_t launch_state(const SpecDecodeParams& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_dk<ActT, float>(p, stream);
    case GDN_BF16: return launch_dk<ActT, bf16>(p, stream);
    default: return launch_dk<ActT, f16>(p, stream);
  }
}

}  // namespace

size_t decode_spec_lds_bytes(int Hk, int Hv, int Dk, int Dv, int cols) {
  const int r = Hv / Hk;
  return (size_t)spec_lds_floats(Dk, r * Dv, r, cols) * sizeof(float);
}

hipError_t launch_decode_spec(const SpecDecodeParams& p, hipStream_t stream) {
  return p.act == GDN_F32 ? launch_state<float>(p, stream) : launch_state<bf16>(p, stream);
}

}  // namespace gdn
