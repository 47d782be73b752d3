// gdn_prepare.hip -- varlen prepare step of the GDN layer on gfx950.
//
// Kernel 1 (conv): one wave owns a block of 64*V consecutive channels
// (V = 16 bytes of input per lane) and a strip of tokens.  It walks its
// tokens in order keeping the last K-1 raw inputs of each channel in
// registers (a sliding window), so every input element is read from HBM once
// (plus K-1 halo rows per strip).  Per token it forms the causal depthwise
// conv + SiLU, L2-normalises q and k heads with a cross-lane sum over the
// lanes of one head (a head of Dk channels is Dk/V aligned lanes), and
// stores q/k/v.  Strips may cross sequence boundaries: the window is
// reloaded from the slot's conv history (or zeros) where a sequence starts.
// Conv semantics: vllm.cpp cpu_ops.cpp, CausalConv1dFwdKernel; split and
// norm: GdnPostConvKernel, L2NormKernel.
//
// The workgroups of a strip also form the per-(token, value head) gates g and
// beta of its tokens (vllm.cpp cpu_ops.cpp, GdnGBetaKernel), after their
// stream.
//
// The new conv history row of a sequence (its last K-1 raw inputs) is
// written by the workgroup whose strip holds the sequence's first token,
// after that workgroup has read the old row, when the first K-1 tokens of
// every sequence lie in the strip of its first token (the host checks the
// offsets): then no other workgroup reads that old row.  Otherwise kernel 2
// (finish) writes every history row after kernel 1 on the same stream.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kConvWaves = 4;   // waves per workgroup (one channel block each)
constexpr int kStrip = 32;      // tokens per wave
constexpr int kAhead = 4;       // token rows loaded before they are used

// Largest s in [0, N) with cu[s] <= t, found by the whole wave (t is
// wave-uniform and cu[0] = 0 <= t).  Each round splits the candidate range
// into 64 pieces and keeps the one the ballot points at.
__device__ int find_sequence(const int32_t* cu, int N, int64_t t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = N;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const bool le = idx < hi && cu[idx] <= t;
    const int cnt = __popcll(__ballot(le));
    lo += (cnt - 1) * step;
    hi = min(hi, lo + step);
  }
  return lo;
}

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
// Inputs are read once and outputs written once: nontemporal accesses.
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void store_stream(void* p, const uint4& u) {
  const v4u v = {u.x, u.y, u.z, u.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p));
}

// g and beta of one (token, value head) item i = t * Hv + h: its inputs,
// then the two outputs
struct GateIn {
  float a, b, A_log, dt_bias;
};
template <typename ActT>
__device__ __forceinline__ GateIn gate_load(const PrepareParams& p, int64_t i) {
  const int64_t t = i / p.Hv;
  const int h = (int)(i % p.Hv);
  return {Elem<ActT>::load(static_cast<const ActT*>(p.a) + t * p.a_stride + h),
          Elem<ActT>::load(static_cast<const ActT*>(p.b) + t * p.b_stride + h), p.A_log[h], p.dt_bias[h]};
}
__device__ __forceinline__ void gate_store(const PrepareParams& p, int64_t i, const GateIn& in) {
  p.g[i] = -expf(in.A_log) * softplus_f(in.a + in.dt_bias);
  p.beta[i] = sigmoid_f(in.b);
}
template <typename ActT>
__device__ __forceinline__ void gate_item(const PrepareParams& p, int64_t i) {
  gate_store(p, i, gate_load<ActT>(p, i));
}

template <typename ActT, typename QkvT, int K, bool HIST>
__global__ __launch_bounds__(kConvWaves * 64) void prepare_conv_kernel(PrepareParams p) {
  // the gates of this strip's tokens, spread over the strip's workgroups
  // (one item per thread at the usual shapes)
  const int64_t g_end = min(p.T, (int64_t)(blockIdx.y + 1) * kStrip) * p.Hv;
  const int64_t g_first = (int64_t)blockIdx.y * kStrip * p.Hv + (int64_t)blockIdx.x * (kConvWaves * 64) + threadIdx.x;
  const int64_t g_step = (int64_t)gridDim.x * (kConvWaves * 64);
  constexpr int V = Elem<ActT>::kVec;
  constexpr int H = K > 1 ? K - 1 : 1;  // history length (storage for K = 1 unused)
  constexpr int OW = (int)sizeof(QkvT) * V / 16;  // 16-byte words per lane of output
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c0 = (blockIdx.x * kConvWaves + wave) * 64 * V;
  if (c0 >= p.Cc) {  // wave-uniform; the kernel uses no block barrier
    for (int64_t i = g_first; i < g_end; i += g_step) gate_item<ActT>(p, i);
    return;
  }
  const int c = c0 + lane * V;
  const bool active = c < p.Cc;  // Cc is a multiple of 16, so lanes are all-in or all-out
  const int cl = active ? c : 0;  // in-bounds column for lanes past the end
  const int64_t t0 = (int64_t)blockIdx.y * kStrip;
  const int64_t t1 = min(p.T, t0 + kStrip);

  const ActT* __restrict__ x = static_cast<const ActT*>(p.x);
  // the inputs of this thread's first gate item, loaded before the stream
  // so that the gates after it wait on no load
  const bool g_has = g_first < g_end;
  GateIn gin{};
  if (g_has) gin = gate_load<ActT>(p, g_first);
  const ActT* __restrict__ w = static_cast<const ActT*>(p.w);
  const ActT* __restrict__ hist = static_cast<const ActT*>(p.conv_pool);
  const int key_dim = p.Hk * p.Dk;
  const int region = c < key_dim ? 0 : (c < 2 * key_dim ? 1 : 2);
  const int head_lanes = p.Dk / V;  // lanes sharing one q or k head

  // block of kAhead token rows in flight; rows past t1 re-read row t1-1
  uint4 bufA[kAhead], bufB[kAhead];
  auto load_block = [&](uint4* buf, int64_t tb) {
#pragma unroll
    for (int u = 0; u < kAhead; ++u) buf[u] = load_stream(x + min(tb + u, t1 - 1) * p.x_stride + cl);
  };
  load_block(bufA, t0);

  // taps: wt[j][i] multiplies the input K-1-j tokens back, channel c+i.
  // A lane's V channels hold V*K consecutive weights: K 16-byte words.
  float wt[K][V];
  {
    float wf[K * V];
    if (active) {
      const uint4* wp = reinterpret_cast<const uint4*>(w + (int64_t)c * K);
#pragma unroll
      for (int j = 0; j < K; ++j) Elem<ActT>::unpack(wp[j], wf + j * V);
    } else {
#pragma unroll
      for (int e = 0; e < K * V; ++e) wf[e] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < V; ++i)
#pragma unroll
      for (int j = 0; j < K; ++j) wt[j][i] = wf[i * K + j];
  }

  // win[j][i]: raw input j+1 tokens back
  float win[H][V];
  int s = find_sequence(p.cu, p.N, t0);
  const int s_first = s;
  int64_t seq_start = p.cu[s];
  int64_t seq_end = p.cu[s + 1];

  // the history of sequence seq for this lane's channels: hw[d-1][i] is the
  // input d tokens before the sequence start (1 <= d <= K-1), zero without
  // an initial state.  In rows of exactly K-1 taps a lane's V channels hold
  // (K-1)*V consecutive history values: K-1 16-byte words.  Widened rows
  // (W > K-1 taps) are read tap by tap.
  auto hist_window = [&](int seq, float (&hw)[H][V]) {
    float hf[H * V];
    const bool has = active && (p.has_init == nullptr || p.has_init[seq] != 0);
    if (has && p.W == K - 1) {
      const int slot = p.slots ? p.slots[seq] : seq;
      const uint4* hp = reinterpret_cast<const uint4*>(hist + ((int64_t)slot * p.Cc + c) * (K - 1));
#pragma unroll
      for (int j = 0; j < K - 1; ++j) Elem<ActT>::unpack(hp[j], hf + j * V);
    } else if (has) {
      // widened rows (speculative decoding): the leading K-1 of W taps per channel
      const int slot = p.slots ? p.slots[seq] : seq;
      const ActT* hp = hist + ((int64_t)slot * p.Cc + c) * p.W;
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int j = 0; j < K - 1; ++j) hf[i * (K - 1) + j] = Elem<ActT>::load(hp + (int64_t)i * p.W + j);
    } else {
#pragma unroll
      for (int e = 0; e < H * V; ++e) hf[e] = 0.0f;
    }
    // channel c+i's history column m holds the input K-1-m tokens back
#pragma unroll
    for (int d = 1; d <= K - 1; ++d)
#pragma unroll
      for (int i = 0; i < V; ++i) hw[d - 1][i] = hf[i * (K - 1) + (K - 1 - d)];
  };
  if constexpr (K > 1) {
    float hw[H][V];
    if (t0 - (K - 1) < seq_start) hist_window(s, hw);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t tp = t0 - 1 - j;
      if (tp >= seq_start) {
        if (active) load_vec<ActT>(x + tp * p.x_stride + c, win[j]);
        else
#pragma unroll
          for (int i = 0; i < V; ++i) win[j][i] = 0.0f;
      } else {
        const int d = (int)(seq_start - tp);  // 1 <= d <= K-1
#pragma unroll
        for (int dd = 1; dd <= K - 1; ++dd)
          if (dd == d)
#pragma unroll
            for (int i = 0; i < V; ++i) win[j][i] = hw[dd - 1][i];
      }
    }
  }

  QkvT* __restrict__ out_base;
  int64_t out_row;
  int out_col;
  if (region == 0) {
    out_base = static_cast<QkvT*>(p.q); out_row = key_dim; out_col = c;
  } else if (region == 1) {
    out_base = static_cast<QkvT*>(p.k); out_row = key_dim; out_col = c - key_dim;
  } else {
    out_base = static_cast<QkvT*>(p.v); out_row = (int64_t)p.Hv * p.Dv; out_col = c - 2 * key_dim;
  }

  // sum over the lanes of one q/k head (head_lanes a power of two <= 32):
  // a fixed butterfly whose steps wider than the head add nothing.  With 16
  // lanes per head (the usual Dk = 128) the steps run as row rotations of
  // the data-parallel primitives (DPP): after the step of distance 8 every
  // partial sum is the same for lanes i and i ^ 8, so a rotation by 4 within
  // the 16-lane row reads the same value as lane i ^ 4, and so on down to 1;
  // the sums are bit for bit those of the butterfly.
  auto head_sum = [&](float v) {
    if (head_lanes == 16) {
      auto ror_add = [](float x, auto ctrl) {
        return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xf, 0xf, false));
      };
      v = ror_add(v, std::integral_constant<int, 0x128>{});  // row_ror:8
      v = ror_add(v, std::integral_constant<int, 0x124>{});  // row_ror:4
      v = ror_add(v, std::integral_constant<int, 0x122>{});  // row_ror:2
      v = ror_add(v, std::integral_constant<int, 0x121>{});  // row_ror:1
      return v;
    }
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) {
      const float o = __shfl_xor(v, off, 64);
      v += off < head_lanes ? o : 0.0f;
    }
    return v;
  };
  auto store_row = [&](int64_t t, const float* y) {
    if (!active) return;
    QkvT* dst = out_base + t * out_row + out_col;
    if constexpr (OW >= 1) {
#pragma unroll
      for (int o = 0; o < OW; ++o) {
        const float* yo = y + o * Elem<QkvT>::kVec;
        if constexpr (std::is_same<QkvT, bf16>::value) store_stream(dst + o * Elem<QkvT>::kVec, pack_bf16x8_hw(yo));
        else store_stream(dst + o * Elem<QkvT>::kVec, Elem<QkvT>::pack(yo));
      }
    } else {
      store_n<QkvT, V>(dst, y);
    }
  };
  // conv + SiLU of one token from its input xv and the K-1 inputs before it
  // (prev(j) = the input j+1 tokens back), then the q/k L2 norm; stores.
  auto finish_token = [&](int64_t t, const float* xv, auto prev) {
    float y[V];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      float acc = wt[K - 1][i] * xv[i];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) acc += wt[K - 2 - j][i] * prev(j, i);
      y[i] = silu_f(acc);
      ss += y[i] * y[i];
    }
    if (p.l2norm && region < 2) {
      const float inv = __builtin_amdgcn_rsqf(head_sum(ss) + 1e-6f);
#pragma unroll
      for (int i = 0; i < V; ++i) y[i] *= inv;
    }
    store_row(t, y);
  };
  auto process = [&](const uint4* buf, int64_t tb) {
    if (tb + kAhead <= t1 && tb + kAhead <= seq_end) {
      // the whole block lies in the current sequence: every earlier input
      // comes from this block's rows or the window, at fixed positions
      float xs[kAhead][V];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) Elem<ActT>::unpack(buf[u], xs[u]);
#pragma unroll
      for (int u = 0; u < kAhead; ++u)
        finish_token(tb + u, xs[u], [&](int j, int i) { return u - 1 - j >= 0 ? xs[u - 1 - j][i] : win[j - u][i]; });
      if constexpr (K > 1) {
        // new window: input j+1 tokens before the next block
        float nw[H][V];
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
          for (int i = 0; i < V; ++i) nw[j][i] = kAhead - 1 - j >= 0 ? xs[kAhead - 1 - j][i] : win[j - kAhead][i];
#pragma unroll
        for (int j = 0; j < K - 1; ++j)
#pragma unroll
          for (int i = 0; i < V; ++i) win[j][i] = nw[j][i];
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int64_t t = tb + u;
      if (t >= t1) break;  // wave-uniform
      if (t == seq_end) {  // a new sequence starts here: reload its history
        ++s;
        seq_start = t;
        seq_end = p.cu[s + 1];
        if constexpr (K > 1) hist_window(s, win);
      }
      float xv[V];
      Elem<ActT>::unpack(buf[u], xv);
      finish_token(t, xv, [&](int j, int i) { return win[j][i]; });
      if constexpr (K > 1) {
#pragma unroll
        for (int j = K - 2; j > 0; --j)
#pragma unroll
          for (int i = 0; i < V; ++i) win[j][i] = win[j - 1][i];
#pragma unroll
        for (int i = 0; i < V; ++i) win[0][i] = xv[i];
      }
    }
  };

  // two blocks per trip, each loaded one block ahead of its use
  for (int64_t tb = t0; tb < t1; tb += 2 * kAhead) {
    load_block(bufB, tb + kAhead);
    process(bufA, tb);
    load_block(bufA, tb + 2 * kAhead);
    process(bufB, tb + kAhead);
  }
  if (g_has) gate_store(p, g_first, gin);
  for (int64_t i = g_first + g_step; i < g_end; i += g_step) gate_item<ActT>(p, i);

  if constexpr (HIST && K > 1) {
    // new history rows of the sequences that start in this strip, after this
    // lane's reads of their old rows (above, in program order): column j
    // holds the input K-1-j tokens before the sequence end, or for a
    // sequence shorter than K-1 an entry of the old row (zero without one)
    if (!active) return;
    ActT* __restrict__ hw = static_cast<ActT*>(p.conv_pool);
    for (int sq = (p.cu[s_first] == t0 ? s_first : s_first + 1); sq < p.N && p.cu[sq] < t1; ++sq) {
      const int64_t start = p.cu[sq];
      const int64_t len = p.cu[sq + 1] - start;
      const int slot = p.slots ? p.slots[sq] : sq;
      const bool has = p.has_init == nullptr || p.has_init[sq] != 0;
      ActT* row = hw + ((int64_t)slot * p.Cc + c) * p.W;
      float nv[K - 1][V];
#pragma unroll
      for (int j = 0; j < K - 1; ++j) {
        const int64_t tp = len - (K - 1) + j;  // position of the input column j holds
        if (tp >= 0) {
          load_vec<ActT>(x + (start + tp) * p.x_stride + c, nv[j]);
        } else {
#pragma unroll
          for (int i = 0; i < V; ++i)
            nv[j][i] = has ? Elem<ActT>::load(row + (int64_t)i * p.W + (K - 1) + tp) : 0.0f;
        }
      }
#pragma unroll
      for (int i = 0; i < V; ++i)
#pragma unroll
        for (int j = 0; j < K - 1; ++j) Elem<ActT>::store(row + (int64_t)i * p.W + j, nv[j][i]);
    }
  }
}

template <typename ActT, int K>
__global__ __launch_bounds__(256) void prepare_finish_kernel(PrepareParams p) {
  if constexpr (K > 1) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (int64_t)p.N * p.Cc) return;
    const int s = (int)(i / p.Cc);
    const int c = (int)(i % p.Cc);
    const int64_t start = p.cu[s];
    const int64_t len = p.cu[s + 1] - start;
    const int slot = p.slots ? p.slots[s] : s;
    const bool has = p.has_init == nullptr || p.has_init[s] != 0;
    ActT* row = static_cast<ActT*>(p.conv_pool) + ((int64_t)slot * p.Cc + c) * p.W;
    const ActT* x = static_cast<const ActT*>(p.x);
    float old[K - 1];
#pragma unroll
    for (int j = 0; j < K - 1; ++j) old[j] = Elem<ActT>::load(row + j);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) {
      const int64_t tp = len - (K - 1) + j;  // position of the input history column j holds
      const float val = tp >= 0 ? Elem<ActT>::load(x + (start + tp) * p.x_stride + c)
                                : (has ? old[(K - 1) + tp] : 0.0f);
      Elem<ActT>::store(row + j, val);
    }
  }
}

// True when the first K-1 tokens of every sequence lie in the strip of its
// first token, so that the strip's workgroups are the only readers of the
// sequence's old history row.
bool history_in_conv(const PrepareParams& p) {
  if (p.K <= 1 || p.cu_host == nullptr) return false;
  for (int s = 0; s < p.N; ++s)
    if (p.cu_host[s] % kStrip > kStrip - (p.K - 1)) return false;
  return true;
}

template <typename ActT, typename QkvT, int K>
hipError_t launch_typed(const PrepareParams& p, hipStream_t stream) {
  constexpr int V = Elem<ActT>::kVec;
  const int chans_per_block = kConvWaves * 64 * V;
  dim3 grid((p.Cc + chans_per_block - 1) / chans_per_block, (unsigned)((p.T + kStrip - 1) / kStrip));
  if (history_in_conv(p)) {
    prepare_conv_kernel<ActT, QkvT, K, true><<<grid, kConvWaves * 64, 0, stream>>>(p);
    return hipGetLastError();
  }
  prepare_conv_kernel<ActT, QkvT, K, false><<<grid, kConvWaves * 64, 0, stream>>>(p);
  if (K > 1) {
    const int hist_blocks = (int)(((int64_t)p.N * p.Cc + 255) / 256);
    prepare_finish_kernel<ActT, K><<<hist_blocks, 256, 0, stream>>>(p);
  }
  return hipGetLastError();
}

template <typename ActT, typename QkvT>
hipError_t launch_k(const PrepareParams& p, hipStream_t stream) {
  switch (p.K) {
    case 1: return launch_typed<ActT, QkvT, 1>(p, stream);
    case 2: return launch_typed<ActT, QkvT, 2>(p, stream);
    case 3: return launch_typed<ActT, QkvT, 3>(p, stream);
    default: return launch_typed<ActT, QkvT, 4>(p, stream);
  }
}

}  // namespace

hipError_t launch_prepare(const PrepareParams& p, hipStream_t stream) {
  if (p.act == GDN_F32)
    return p.qkv == GDN_F32 ? launch_k<float, float>(p, stream) : launch_k<float, bf16>(p, stream);
  return p.qkv == GDN_F32 ? launch_k<bf16, float>(p, stream) : launch_k<bf16, bf16>(p, stream);
}

}  // namespace gdn
