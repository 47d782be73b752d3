// gdn_prefill.hip -- varlen prefill of the gated delta rule on gfx950.
//
// Token-sequential kernel: one wave per (sequence, value head, block of RB
// value rows).  Value rows of the state are independent under the delta
// rule (row e only meets v[e] and the shared k, q, g, beta), so a block of
// rows can run the whole sequence on its own with its rows in registers:
// per token, S.k and S.q are formed in one pass over the registers and
// summed across the lanes of a row, then
//   u = d (S.k);  delta = beta (v - u);  o = d (S.q) + delta (k.q);
//   S <- d S + delta k,      d = exp(g)
// (vllm.cpp cpu_ops.cpp, GdnHeadTokenStep and GdnPrefillKernel).  The state
// is read from its slot at the storage dtype once and written back rounded
// once at the end of the sequence.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kSeqRows = 16;  // value rows per wave

template <typename QkvT, typename StT, int DK>
__global__ __launch_bounds__(64) void prefill_sequential_kernel(PrefillParams p) {
  constexpr int LPR = DK / 4;           // lanes per row; a lane holds 4 columns
  constexpr int RPL = 64 / LPR >= 1 ? 64 / LPR : 1;
  constexpr int NS = kSeqRows / RPL > 0 ? kSeqRows / RPL : 1;  // rows held per lane
  const int blk = blockIdx.x;
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x;
  const int r = p.Hv / p.Hk;
  const int kh = h / r;
  const int Dv = p.Dv;
  const int sub = lane / LPR;
  const int col = (lane % LPR) * 4;
  const int64_t start = p.cu[s], end = p.cu[s + 1];
  const int slot = p.slots ? p.slots[s] : s;
  const bool has = p.has_init == nullptr || p.has_init[s] != 0;

  StT* __restrict__ Sg = static_cast<StT*>(p.ssm_pool) + ((int64_t)slot * p.Hv + h) * Dv * DK;
  float st[NS][4];
  int rows[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    rows[j] = blk * kSeqRows + j * RPL + sub;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      st[j][i] = (has && rows[j] < Dv) ? Elem<StT>::load(Sg + (int64_t)rows[j] * DK + col + i) : 0.0f;
  }

  const QkvT* __restrict__ qp = static_cast<const QkvT*>(p.q);
  const QkvT* __restrict__ kp = static_cast<const QkvT*>(p.k);
  const QkvT* __restrict__ vp = static_cast<const QkvT*>(p.v);
  QkvT* __restrict__ op = static_cast<QkvT*>(p.out);

  for (int64_t t = start; t < end; ++t) {
    float kv[4], qv[4];
    const int64_t qk_off = (t * p.Hk + kh) * DK + col;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kv[i] = Elem<QkvT>::load(kp + qk_off + i);
      qv[i] = Elem<QkvT>::load(qp + qk_off + i);
    }
    if (p.l2norm) {
      float kk = 0.0f, qq = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kk += kv[i] * kv[i];
        qq += qv[i] * qv[i];
      }
      kk = group_sum<LPR>(kk);
      qq = group_sum<LPR>(qq);
      const float ki = 1.0f / sqrtf(kk + 1e-6f), qi = 1.0f / sqrtf(qq + 1e-6f);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kv[i] *= ki;
        qv[i] *= qi;
      }
    }
    float kq = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] *= p.scale;
      kq += kv[i] * qv[i];
    }
    kq = group_sum<LPR>(kq);
    const float d = expf(p.g[t * p.Hv + h]);
    const float bt = p.beta[t * p.Hv + h];
    const int64_t v_off = (t * p.Hv + h) * Dv;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (rows[j] >= Dv) continue;  // uniform per row group
      float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p1 += st[j][i] * kv[i];
        p2 += st[j][i] * qv[i];
      }
      p1 = group_sum<LPR>(p1);
      p2 = group_sum<LPR>(p2);
      const float delta = bt * (Elem<QkvT>::load(vp + v_off + rows[j]) - d * p1);
      const float o = d * p2 + delta * kq;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[j][i] = d * st[j][i] + delta * kv[i];
      if ((lane % LPR) == 0) Elem<QkvT>::store(op + v_off + rows[j], o);
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (rows[j] < Dv)
#pragma unroll
      for (int i = 0; i < 4; ++i) Elem<StT>::store(Sg + (int64_t)rows[j] * DK + col + i, st[j][i]);
}

template <typename QkvT, typename StT>
hipError_t launch_seq(const PrefillParams& p, hipStream_t stream) {
  dim3 grid((p.Dv + kSeqRows - 1) / kSeqRows, p.Hv, p.N);
  switch (p.Dk) {
    case 16: prefill_sequential_kernel<QkvT, StT, 16><<<grid, 64, 0, stream>>>(p); break;
    case 32: prefill_sequential_kernel<QkvT, StT, 32><<<grid, 64, 0, stream>>>(p); break;
    case 64: prefill_sequential_kernel<QkvT, StT, 64><<<grid, 64, 0, stream>>>(p); break;
    case 128: prefill_sequential_kernel<QkvT, StT, 128><<<grid, 64, 0, stream>>>(p); break;
    default: prefill_sequential_kernel<QkvT, StT, 256><<<grid, 64, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

template <typename QkvT>
hipError_t launch_state(const PrefillParams& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_seq<QkvT, float>(p, stream);
    case GDN_BF16: return launch_seq<QkvT, bf16>(p, stream);
    default: return launch_seq<QkvT, f16>(p, stream);
  }
}

}  // namespace

size_t prefill_workspace_bytes(int, int, int, int, int, int64_t, int) { return 0; }

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  return p.qkv == GDN_F32 ? launch_state<float>(p, stream) : launch_state<bf16>(p, stream);
}

}  // namespace gdn
