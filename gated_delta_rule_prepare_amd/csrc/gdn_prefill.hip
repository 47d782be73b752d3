// gdn_prefill.hip -- varlen prefill of the gated delta rule on gfx950.
//
// The recurrence (vllm.cpp cpu_ops.cpp, GdnHeadTokenStep / GdnPrefillKernel;
// ferrum-kernels cpu.rs, recurrent_gated_delta_rule_varlen_f32) is computed
// in chunks of 64 tokens in the WY / UT-transform form.  Within one chunk of
// one (sequence, value head), with G_i the running sum of g from the chunk
// start, gamma_i = exp(G_i) and S0 the entering [Dv, Dk] state:
//   A[i][j] = beta_i exp(G_i - G_j) (k_i . k_j)   for j < i
//   T       = (I + A)^-1
//   W       = T diag(beta gamma) K,   U = T diag(beta) V
//   Delta   = U - W S0^T                               (row i = delta of token i)
//   O       = diag(scale gamma) Q S0^T + P Delta,
//             P[i][j] = scale exp(G_i - G_j) (q_i . k_j)  for j <= i
//   S_C     = gamma_C S0 + Delta^T diag(exp(G_C - G_j)) K
// which follows from unrolling S_i = exp(g_i) S_{i-1} + delta_i k_i^T.
//
// Kernels (all on the caller's stream):
//  1. chunk_table_kernel: chunk ids -> (sequence, first token); chunks never
//     cross sequences and a sequence's last chunk may be short.
//  2. chunk_prep_kernel, one workgroup per (chunk, value head), no state
//     dependence: K K^T and Q K^T on MFMA, the unit-triangular inverse T in
//     LDS (16x16 diagonal blocks by substitution, then block products), W and
//     U on MFMA.  Writes W, U, P, gamma and exp(G_C - G_j) to the workspace.
//     The running sums G are formed in double precision and every decay
//     factor is exp of a difference taken in double, so long chunks of
//     strong decay keep full f32 accuracy.
//  3. chunk_scan_kernel, one workgroup (4 waves) per (sequence, value head,
//     block of 16 value rows): walks the sequence's chunks in order with the
//     16 x Dk state block held in registers in the MFMA B-operand layout,
//     and forms Delta, O and the next state on MFMA (f32 16x16x4).  Value rows
//     of the state are independent, so row blocks never communicate.
//
// A token-sequential kernel (one wave per sequence, value head and 16 value
// rows, state rows in registers) serves head dims above 128.
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma16x16x4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

constexpr int kChunk = 64;

// ---------------------------------------------------------------------------
// Workspace layout.
// ---------------------------------------------------------------------------
__host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

struct ChunkWs {
  int32_t* seq_chunk_off;  // [N+1] first chunk id of each sequence
  int32_t* chunk_seq;      // [NC]
  int32_t* chunk_start;    // [NC] first token (global index)
  float* blocks;           // [NC, Hv, block_floats]
  int64_t block_floats;    // 64*Dk (W) + 64*Dv (U) + 64*64 (P) + 64 (gamma) + 64 (exp(G_C - G_j))
};

__host__ __device__ inline int64_t block_floats(int Dk, int Dv) {
  return (int64_t)kChunk * (Dk + Dv + kChunk) + 2 * kChunk;
}

inline int64_t max_chunks(int N, int64_t T) { return T / kChunk + N; }

ChunkWs carve(void* base, int Dk, int Dv, int N, int64_t T) {
  char* p = static_cast<char*>(base);
  ChunkWs w;
  const int64_t nc = max_chunks(N, T);
  w.seq_chunk_off = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)(N + 1) * 4);
  w.chunk_seq = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nc * 4);
  w.chunk_start = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nc * 4);
  w.blocks = reinterpret_cast<float*>(p);
  w.block_floats = block_floats(Dk, Dv);
  return w;
}

bool chunked_dims(int Dk, int Dv) { return Dk == Dv && Dk >= 16 && Dk <= 128; }

// ---------------------------------------------------------------------------
// 1. chunk table
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void chunk_table_kernel(const int32_t* cu, int N, ChunkWs ws) {
  __shared__ int32_t part[1024];
  const int tid = threadIdx.x;
  const int per = (N + 1023) / 1024;
  const int s0 = min(N, tid * per), s1 = min(N, s0 + per);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (cu[s + 1] - cu[s] + kChunk - 1) / kChunk;
  part[tid] = local;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive scan
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int c = part[tid] - local;
  for (int s = s0; s < s1; ++s) {
    ws.seq_chunk_off[s] = c;
    for (int t = cu[s]; t < cu[s + 1]; t += kChunk) {
      ws.chunk_seq[c] = s;
      ws.chunk_start[c] = t;
      ++c;
    }
  }
  if (tid == 1023) ws.seq_chunk_off[N] = part[1023];
}

// Copy rows [0, n) of a [*, D] slice (row stride `gstride` elements) into LDS
// as f32 with row stride `ls`; rows n..63 become zero.
template <typename T, int D>
__device__ __forceinline__ void stage_rows(float* lds, int ls, const T* __restrict__ src, int64_t gstride, int n) {
  constexpr int V = Elem<T>::kVec < D ? Elem<T>::kVec : D;
  constexpr int PER_ROW = D / V;
  for (int idx = threadIdx.x; idx < kChunk * PER_ROW; idx += blockDim.x) {
    const int r = idx / PER_ROW, c = (idx % PER_ROW) * V;
    float v[V];
    if (r < n) {
      load_n<T, V>(src + (int64_t)r * gstride + c, v);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < V; ++i) lds[r * ls + c + i] = v[i];
  }
}

// L2-normalise `rows` rows of an LDS matrix (eps 1e-6 inside the root), one
// wave per row at a time.
template <int D>
__device__ __forceinline__ void l2norm_rows(float* lds, int ls, int rows) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int r = wave; r < rows; r += nw) {
    float ss = 0.0f;
    for (int c = lane; c < D; c += 64) ss += lds[r * ls + c] * lds[r * ls + c];
    ss = group_sum<64>(ss);
    const float inv = 1.0f / sqrtf(ss + 1e-6f);
    for (int c = lane; c < D; c += 64) lds[r * ls + c] *= inv;
  }
}

// ---------------------------------------------------------------------------
// 2. per-chunk work
// ---------------------------------------------------------------------------
template <typename QkvT, int D>
__global__ __launch_bounds__(256) void chunk_prep_kernel(PrefillParams p, ChunkWs ws) {
  constexpr int LS = D + 4;        // LDS row stride of K / Q / V
  constexpr int TS = kChunk + 4;   // LDS row stride of A / T
  __shared__ float Ks[kChunk * LS];
  __shared__ float Xs[kChunk * LS];  // Q, later V
  __shared__ float As[kChunk * TS];
  __shared__ float Ts[kChunk * TS];
  __shared__ float Tmp[3 * 256];
  __shared__ double Gs[kChunk];
  __shared__ float bs[kChunk], gs[kChunk];

  const int cid = blockIdx.x, h = blockIdx.y;
  const int r_heads = p.Hv / p.Hk, kh = h / r_heads;
  const int seq = ws.chunk_seq[cid];
  const int64_t t0 = ws.chunk_start[cid];
  const int n = (int)min((int64_t)kChunk, (int64_t)p.cu[seq + 1] - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  float* blk = ws.blocks + ((int64_t)cid * p.Hv + h) * ws.block_floats;
  float* Wg = blk;
  float* Ug = blk + kChunk * D;
  float* Pg = blk + 2 * kChunk * D;
  float* gam_g = Pg + kChunk * kChunk;
  float* dc_g = gam_g + kChunk;

  const QkvT* kp = static_cast<const QkvT*>(p.k) + (t0 * p.Hk + kh) * D;
  const QkvT* qp = static_cast<const QkvT*>(p.q) + (t0 * p.Hk + kh) * D;
  stage_rows<QkvT, D>(Ks, LS, kp, (int64_t)p.Hk * D, n);
  stage_rows<QkvT, D>(Xs, LS, qp, (int64_t)p.Hk * D, n);
  for (int i = tid; i < kChunk * TS; i += 256) As[i] = 0.0f;
  float gval = 0.0f;
  if (tid < kChunk) {
    // a decay factor exp(g) below e^-200 is exactly zero in f32; the clamp
    // keeps the running sums finite when g = -inf
    gval = tid < n ? fmaxf(p.g[(t0 + tid) * p.Hv + h], -200.0f) : 0.0f;
    bs[tid] = tid < n ? p.beta[(t0 + tid) * p.Hv + h] : 0.0f;
  }
  __syncthreads();
  if (p.l2norm) {
    l2norm_rows<D>(Ks, LS, kChunk);
    l2norm_rows<D>(Xs, LS, kChunk);
  }
  if (wave == 0) {
    double G = (double)gval;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(G, off, 64);
      if (lane >= off) G += o;
    }
    Gs[lane] = G;
    const double Glast = __shfl(G, 63, 64);
    const float gam = expf((float)G);
    gs[lane] = gam;
    gam_g[lane] = gam;
    dc_g[lane] = expf((float)(Glast - G));
  }
  __syncthreads();

  // K K^T (masked into A) and Q K^T (masked into P): lower-triangular 16x16 tiles
  for (int idx = wave; idx < 20; idx += 4) {
    const bool qk = idx >= 10;
    const int t = qk ? idx - 10 : idx;
    const int I = t < 1 ? 0 : t < 3 ? 1 : t < 6 ? 2 : 3;
    const int J = t - I * (I + 1) / 2;
    const float* Arow = (qk ? Xs : Ks) + (16 * I + li) * LS + lg;
    const float* Brow = Ks + (16 * J + li) * LS + lg;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < D / 4; ++s) acc = mfma16x16x4(Arow[4 * s], Brow[4 * s], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * I + 4 * lg + r, j = 16 * J + li;
      const float dec = j <= i ? expf((float)(Gs[i] - Gs[j])) : 0.0f;
      if (!qk) {
        As[i * TS + j] = j < i ? bs[i] * dec * acc[r] : 0.0f;
      } else {
        Pg[i * kChunk + j] = j <= i ? p.scale * dec * acc[r] : 0.0f;
      }
    }
  }
  __syncthreads();
  // Q is no longer needed: bring in this value head's V
  const QkvT* vp = static_cast<const QkvT*>(p.v) + (t0 * p.Hv + h) * D;
  stage_rows<QkvT, D>(Xs, LS, vp, (int64_t)p.Hv * D, n);

  // T = (I + A)^-1, diagonal 16x16 blocks by forward substitution (column per lane)
  if (wave == 0) {
    const int B = lg, j = li;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m)
        if (m >= j) acc += As[(16 * B + i) * TS + 16 * B + m] * tc[m];
      tc[i] = i < j ? 0.0f : (i == j ? 1.0f : -acc);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ts[(16 * B + i) * TS + 16 * B + j] = tc[i];
  }
  __syncthreads();
  // off-diagonal blocks: T_IJ = -T_II sum_{K=J}^{I-1} A_IK T_KJ, by distance I-J
  for (int dist = 1; dist < 4; ++dist) {
    const int npairs = 4 - dist;
    for (int e = tid; e < npairs * 256; e += 256) {
      const int J = e >> 8, I = J + dist, a = (e >> 4) & 15, b = e & 15;
      float acc = 0.0f;
      for (int K = J; K < I; ++K)
#pragma unroll
        for (int c = 0; c < 16; ++c) acc += As[(16 * I + a) * TS + 16 * K + c] * Ts[(16 * K + c) * TS + 16 * J + b];
      Tmp[e] = acc;
    }
    __syncthreads();
    for (int e = tid; e < npairs * 256; e += 256) {
      const int J = e >> 8, I = J + dist, a = (e >> 4) & 15, b = e & 15;
      float acc = 0.0f;
#pragma unroll
      for (int c = 0; c < 16; ++c) acc += Ts[(16 * I + a) * TS + 16 * I + c] * Tmp[(J << 8) + c * 16 + b];
      Ts[(16 * I + a) * TS + 16 * J + b] = -acc;
    }
    __syncthreads();
  }

  // W = T diag(beta gamma) K and U = T diag(beta) V; column tiles spread over waves
  for (int ct = wave; ct < 2 * (D / 16); ct += 4) {
    const bool isK = ct < D / 16;
    const int col0 = 16 * (isK ? ct : ct - D / 16);
    const float* X = isK ? Ks : Xs;
    float* out = isK ? Wg : Ug;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int J = 0; J <= I; ++J)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int k = 16 * J + 4 * s + lg;
          const float sc = isK ? bs[k] * gs[k] : bs[k];
          acc = mfma16x16x4(Ts[(16 * I + li) * TS + k], sc * X[k * LS + col0 + li], acc);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) out[(16 * I + 4 * lg + r) * D + col0 + li] = acc[r];
    }
  }
}

// ---------------------------------------------------------------------------
// 3. sequential pass over chunks
// ---------------------------------------------------------------------------
// State fragment: lane (li = lane%16, lg = lane/16) holds S[e0 + li][col(lg, j)]
// for j < D/4 with col(lg, j) = 16*(j/4) + 4*lg + j%4, which is at once the
// B operand of the W S0^T and Q S0^T products (k index = col) and the output
// layout of the S^T update tiles.
__device__ __forceinline__ int frag_col(int lg, int j) { return 16 * (j >> 2) + 4 * lg + (j & 3); }

template <typename QkvT, typename StT, int D>
__global__ __launch_bounds__(256) void chunk_scan_kernel(PrefillParams p, ChunkWs ws) {
  constexpr int NJ = D / 4;
  constexpr int LS = D + 4;
  constexpr int NCT = D / 16;  // 16-column tiles of the state
  __shared__ float Ks[kChunk * LS];
  __shared__ float Qs[kChunk * LS];
  __shared__ float Ds[kChunk * 17];
  __shared__ float Ss[16 * LS];
  __shared__ float gam_s[kChunk], dc_s[kChunk];

  const int e0 = 16 * blockIdx.x, h = blockIdx.y, s = blockIdx.z;
  const int r_heads = p.Hv / p.Hk, kh = h / r_heads;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int slot = p.slots ? p.slots[s] : s;
  const bool has = p.has_init == nullptr || p.has_init[s] != 0;
  const int64_t seq_end = p.cu[s + 1];
  StT* Sg = static_cast<StT*>(p.ssm_pool) + (((int64_t)slot * p.Hv + h) * D + e0 + li) * D;

  float Sf[NJ];
#pragma unroll
  for (int q = 0; q < NCT; ++q) {
    float v[4];
    if (has) {
      load_n<StT, 4>(Sg + 16 * q + 4 * lg, v);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) Sf[4 * q + i] = v[i];
  }

  const QkvT* kbase = static_cast<const QkvT*>(p.k) + (int64_t)kh * D;
  const QkvT* qbase = static_cast<const QkvT*>(p.q) + (int64_t)kh * D;
  QkvT* obase = static_cast<QkvT*>(p.out) + (int64_t)h * D + e0 + li;
  const int c_begin = ws.seq_chunk_off[s], c_end = ws.seq_chunk_off[s + 1];
  for (int cid = c_begin; cid < c_end; ++cid) {
    const int64_t t0 = ws.chunk_start[cid];
    const int n = (int)min((int64_t)kChunk, seq_end - t0);
    const float* blk = ws.blocks + ((int64_t)cid * p.Hv + h) * ws.block_floats;
    const float* Wg = blk;
    const float* Ug = blk + kChunk * D;
    const float* Pg = blk + 2 * kChunk * D;
    const float* gam_g = Pg + kChunk * kChunk;
    const float* dc_g = gam_g + kChunk;

    stage_rows<QkvT, D>(Ks, LS, kbase + t0 * p.Hk * D, (int64_t)p.Hk * D, n);
    stage_rows<QkvT, D>(Qs, LS, qbase + t0 * p.Hk * D, (int64_t)p.Hk * D, n);
    if (tid < kChunk) {
      gam_s[tid] = gam_g[tid];
      dc_s[tid] = dc_g[tid];
    }
    // this wave's operands from the workspace
    const int row = 16 * wave + li;
    float Wf[NJ];
#pragma unroll
    for (int q = 0; q < NCT; ++q) {
      const float4 w4 = *reinterpret_cast<const float4*>(Wg + row * D + 16 * q + 4 * lg);
      Wf[4 * q] = w4.x; Wf[4 * q + 1] = w4.y; Wf[4 * q + 2] = w4.z; Wf[4 * q + 3] = w4.w;
    }
    float Uv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) Uv[r] = Ug[(16 * wave + 4 * lg + r) * D + e0 + li];
    __syncthreads();
    if (p.l2norm) {
      l2norm_rows<D>(Ks, LS, kChunk);
      l2norm_rows<D>(Qs, LS, kChunk);
      __syncthreads();
    }

    // Delta rows of this wave's 16 tokens: U - W S0^T
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc = mfma16x16x4(Wf[j], Sf[j], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) Ds[(16 * wave + 4 * lg + r) * 17 + li] = Uv[r] - acc[r];
    // scale gamma_i Q S0^T
    f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
    const float* qrow = Qs + row * LS;
#pragma unroll
    for (int j = 0; j < NJ; ++j) o = mfma16x16x4(qrow[frag_col(lg, j)], Sf[j], o);
#pragma unroll
    for (int r = 0; r < 4; ++r) o[r] *= p.scale * gam_s[16 * wave + 4 * lg + r];
    __syncthreads();

    // + P Delta over the token blocks up to this one
    for (int J = 0; J <= wave; ++J) {
      const float4 p4 = *reinterpret_cast<const float4*>(Pg + row * kChunk + 16 * J + 4 * lg);
      const float pv[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
      for (int s2 = 0; s2 < 4; ++s2) o = mfma16x16x4(pv[s2], Ds[(16 * J + 4 * lg + s2) * 17 + li], o);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 16 * wave + 4 * lg + r;
      if (i < n) Elem<QkvT>::store(obase + (t0 + i) * (int64_t)p.Hv * D, o[r]);
    }

    // S^T tiles owned by this wave: S_new = gamma_C S0 + Delta^T diag(exp(G_C - G_j)) K
    const float gC = gam_s[kChunk - 1];
    for (int ct = wave; ct < NCT; ct += 4) {
      f32x4 a2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s2 = 0; s2 < kChunk / 4; ++s2) {
        const int k = 4 * s2 + lg;
        a2 = mfma16x16x4(dc_s[k] * Ks[k * LS + 16 * ct + li], Ds[k * 17 + li], a2);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) Ss[li * LS + 16 * ct + 4 * lg + r] = gC * Sf[4 * ct + r] + a2[r];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NJ; ++j) Sf[j] = Ss[li * LS + frag_col(lg, j)];
  }
  if (wave == 0) {
#pragma unroll
    for (int q = 0; q < NCT; ++q) store_n<StT, 4>(Sg + 16 * q + 4 * lg, Sf + 4 * q);
  }
}

// ---------------------------------------------------------------------------
// Token-sequential kernel (head dims above 128).
// ---------------------------------------------------------------------------
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

template <typename QkvT, typename StT, int D>
hipError_t launch_chunked_d(const PrefillParams& p, const ChunkWs& ws, hipStream_t stream) {
  chunk_prep_kernel<QkvT, D><<<dim3((unsigned)p.num_chunks, p.Hv), 256, 0, stream>>>(p, ws);
  chunk_scan_kernel<QkvT, StT, D><<<dim3(D / 16, p.Hv, p.N), 256, 0, stream>>>(p, ws);
  return hipGetLastError();
}

template <typename QkvT, typename StT>
hipError_t launch_typed(const PrefillParams& p, hipStream_t stream) {
  if (!chunked_dims(p.Dk, p.Dv)) return launch_seq<QkvT, StT>(p, stream);
  const ChunkWs ws = carve(p.workspace, p.Dk, p.Dv, p.N, p.T);
  chunk_table_kernel<<<1, 1024, 0, stream>>>(p.cu, p.N, ws);
  switch (p.Dk) {
    case 16: return launch_chunked_d<QkvT, StT, 16>(p, ws, stream);
    case 32: return launch_chunked_d<QkvT, StT, 32>(p, ws, stream);
    case 64: return launch_chunked_d<QkvT, StT, 64>(p, ws, stream);
    default: return launch_chunked_d<QkvT, StT, 128>(p, ws, stream);
  }
}

template <typename QkvT>
hipError_t launch_state(const PrefillParams& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_typed<QkvT, float>(p, stream);
    case GDN_BF16: return launch_typed<QkvT, bf16>(p, stream);
    default: return launch_typed<QkvT, f16>(p, stream);
  }
}

}  // namespace

size_t prefill_workspace_bytes(int Hk, int Hv, int Dk, int Dv, int N, int64_t T, int chunk) {
  (void)Hk;
  (void)chunk;
  if (N <= 0 || T <= 0 || !chunked_dims(Dk, Dv)) return 0;
  const int64_t nc = max_chunks(N, T);
  return align256((size_t)(N + 1) * 4) + 2 * align256((size_t)nc * 4) +
         (size_t)nc * Hv * block_floats(Dk, Dv) * sizeof(float);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  return p.qkv == GDN_F32 ? launch_state<float>(p, stream) : launch_state<bf16>(p, stream);
}

}  // namespace gdn
