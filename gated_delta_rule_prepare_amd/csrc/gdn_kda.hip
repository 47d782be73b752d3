// gdn_kda.hip -- KDA: the gated delta rule with one log-decay per key
// channel (vllm.cpp cpu_ops.cpp, KdaHeadTokenStep / KdaGatedDeltaRuleKernel,
// and the gate of KdaChunkPrefillKernel).  Per token, for value head h with
// key head h / (Hv/Hk) and the [Dv, Dk] state S:
//   S[:, d] <- exp(g[t,h,d]) S[:, d];  u = S k;  delta = beta (v - u);
//   S <- S + delta k^T;  o = S (scale q)
// With the gate, g[t,h,d] = -exp(A_log[h]) softplus(g_raw[t,h,d] + dt_bias[h,d]).
//
// Token-sequential kernel: one wave per (sequence, value head, 16 value
// rows), four waves to a workgroup, the rows in registers for the whole
// sequence.  A lane holds four consecutive columns of a row.  With
// d_i = exp(g_i) for the lane's columns, the decay folds into the two dot
// products:
//   u = sum_i st_i d_i k_i,   o = sum_i st_i d_i q_i + delta (k . q),
//   st_i <- d_i st_i + delta k_i
// so each row is read once and updated once per token.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kKdaRows = 16;  // value rows per wave
constexpr int kKdaWaves = 4;  // waves per workgroup

// the lane's four log-decays of token t (gate applied when A_log is given)
__device__ __forceinline__ void kda_log_decay(const KdaParams& p, int64_t t, int h, int DK, int col, float* gv) {
  const float4 raw = *reinterpret_cast<const float4*>(p.g + (t * p.Hv + h) * DK + col);
  gv[0] = raw.x;
  gv[1] = raw.y;
  gv[2] = raw.z;
  gv[3] = raw.w;
  if (p.A_log) {
    const float a = -expf(p.A_log[h]);
    float bias[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (p.dt_bias) {
      const float4 bv = *reinterpret_cast<const float4*>(p.dt_bias + (int64_t)h * DK + col);
      bias[0] = bv.x;
      bias[1] = bv.y;
      bias[2] = bv.z;
      bias[3] = bv.w;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) gv[i] = a * softplus_f(gv[i] + bias[i]);
  }
}

template <typename QkvT, typename StT, int DK>
__global__ __launch_bounds__(64 * kKdaWaves) void kda_recurrent_kernel(KdaParams p) {
  constexpr int LPR = DK / 4;           // lanes per row; a lane holds 4 columns
  constexpr int RPL = 64 / LPR >= 1 ? 64 / LPR : 1;
  constexpr int NS = kKdaRows / RPL > 0 ? kKdaRows / RPL : 1;  // rows held per lane
  const int blk = blockIdx.x * kKdaWaves + (threadIdx.x >> 6);
  const int h = blockIdx.y;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
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
    rows[j] = blk * kKdaRows + j * RPL + sub;
    if (has && rows[j] < Dv) load_n<StT, 4>(Sg + (int64_t)rows[j] * DK + col, st[j]);
    else
#pragma unroll
      for (int i = 0; i < 4; ++i) st[j][i] = 0.0f;
  }

  const QkvT* __restrict__ qp = static_cast<const QkvT*>(p.q);
  const QkvT* __restrict__ kp = static_cast<const QkvT*>(p.k);
  const QkvT* __restrict__ vp = static_cast<const QkvT*>(p.v);
  QkvT* __restrict__ op = static_cast<QkvT*>(p.out);

  for (int64_t t = start; t < end; ++t) {
    float kv[4], qv[4], gv[4];
    const int64_t qk_off = (t * p.Hk + kh) * DK + col;
    load_n<QkvT, 4>(kp + qk_off, kv);
    load_n<QkvT, 4>(qp + qk_off, qv);
    kda_log_decay(p, t, h, DK, col, gv);
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
    float kq = 0.0f, dk[4], dq[4], dd[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qv[i] *= p.scale;
      kq += kv[i] * qv[i];
      dd[i] = expf(gv[i]);
      dk[i] = dd[i] * kv[i];
      dq[i] = dd[i] * qv[i];
    }
    kq = group_sum<LPR>(kq);
    const float bt = p.beta[t * p.Hv + h];
    const int64_t v_off = (t * p.Hv + h) * Dv;
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      if (rows[j] >= Dv) continue;  // uniform per row group
      float p1 = 0.0f, p2 = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p1 += st[j][i] * dk[i];
        p2 += st[j][i] * dq[i];
      }
      p1 = group_sum<LPR>(p1);
      p2 = group_sum<LPR>(p2);
      const float delta = bt * (Elem<QkvT>::load(vp + v_off + rows[j]) - p1);
      const float o = p2 + delta * kq;
#pragma unroll
      for (int i = 0; i < 4; ++i) st[j][i] = dd[i] * st[j][i] + delta * kv[i];
      if ((lane % LPR) == 0) Elem<QkvT>::store(op + v_off + rows[j], o);
    }
  }
  // the final state (an empty sequence writes back its initial state)
#pragma unroll
  for (int j = 0; j < NS; ++j)
    if (rows[j] < Dv) {
      // f32 rows are written once and not read again here: nontemporal stores
      if constexpr (std::is_same<StT, float>::value) {
        typedef float v4f __attribute__((ext_vector_type(4)));
        const v4f x = {st[j][0], st[j][1], st[j][2], st[j][3]};
        __builtin_nontemporal_store(x, reinterpret_cast<v4f*>(Sg + (int64_t)rows[j] * DK + col));
      } else {
        store_n<StT, 4>(Sg + (int64_t)rows[j] * DK + col, st[j]);
      }
    }
}

template <typename QkvT, typename StT>
hipError_t launch_rec(const KdaParams& p, hipStream_t stream) {
  const int blocks = (p.Dv + kKdaRows - 1) / kKdaRows;  // 16-row blocks per head
  dim3 grid((blocks + kKdaWaves - 1) / kKdaWaves, p.Hv, p.N);
  constexpr int threads = 64 * kKdaWaves;
  switch (p.Dk) {
    case 16: kda_recurrent_kernel<QkvT, StT, 16><<<grid, threads, 0, stream>>>(p); break;
    case 32: kda_recurrent_kernel<QkvT, StT, 32><<<grid, threads, 0, stream>>>(p); break;
    case 64: kda_recurrent_kernel<QkvT, StT, 64><<<grid, threads, 0, stream>>>(p); break;
    case 128: kda_recurrent_kernel<QkvT, StT, 128><<<grid, threads, 0, stream>>>(p); break;
    default: kda_recurrent_kernel<QkvT, StT, 256><<<grid, threads, 0, stream>>>(p); break;
  }
  return hipGetLastError();
}

template <typename QkvT>
hipError_t launch_rec_state(const KdaParams& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_rec<QkvT, float>(p, stream);
    case GDN_BF16: return launch_rec<QkvT, bf16>(p, stream);
    default: return launch_rec<QkvT, f16>(p, stream);
  }
}

}  // namespace

hipError_t launch_kda_recurrent(const KdaParams& p, hipStream_t stream) {
  return p.qkv == GDN_F32 ? launch_rec_state<float>(p, stream) : launch_rec_state<bf16>(p, stream);
}

}  // namespace gdn
