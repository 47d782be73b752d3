// gdn_mamba2.hip -- Mamba2 / SSD (vllm.cpp cpu_ops.cpp, Mamba2ChunkScanKernel
// and Mamba2StateUpdateKernel).  Not the gated delta rule: per head h with
// group g = h / (H/G), step dt (softplus of dt + dt_bias, clamped) and the
// [P, N] state S,
//   S <- exp(A[h] dt) S + dt x B^T,   y = S C + D x,   y *= silu(z)
//
// Decode (mamba2_update_kernel): one workgroup per (row, head) streams the
// P state rows once, like the GDN decode kernel: per row
//   s' = da s + (dt x_p) B,   y_p = s' . C
//
// Prefill, in chunks of 64 tokens (the dual form; within a chunk, with
// L_i = sum_{j<=i} A dt_j):
//   Y_intra = (M * C B^T) X,  M[i][j] = exp(L_i - L_j) dt_j  (j <= i)
//   Y_inter[i] = exp(L_i) S0 C_i
//   S_C = exp(L_C) S0 + sum_j exp(L_C - L_j) dt_j x_j B_j^T
// ssd_chunk_kernel (one workgroup per chunk and head) forms Y_intra and the
// chunk's state contribution on the f16 hi/lo MFMA; ssd_scan_kernel (one wave
// per sequence, head and 16 state rows) carries S through the chunks in
// registers, adds Y_inter (MFMA), D x and the gate, and writes the final state.
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

constexpr int kSsdChunk = 64;
constexpr int kTS = kSsdChunk + 8;  // row stride (halves) of transposed [column][token] tiles

// the processed step of token t, head h
__device__ __forceinline__ float ssd_dt(const Mamba2Params& p, float raw, int h) {
  float d = raw + (p.dt_bias ? p.dt_bias[h] : 0.0f);
  if (p.dt_softplus) d = d <= 20.0f ? log1pf(expf(d)) : d;
  return fminf(fmaxf(d, p.dt_min), p.dt_max);
}

// ---------------------------------------------------------------------------
// Decode
// ---------------------------------------------------------------------------
constexpr int kUpdWaves = 4;
constexpr int kUpdThreads = kUpdWaves * 64;
constexpr int kUpdLoads = 4;

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16_nt(void* p, const uint4& u) {
  const v4u v = {u.x, u.y, u.z, u.w};
  __builtin_nontemporal_store(v, reinterpret_cast<v4u*>(p));
}

template <typename ActT, typename StT, int N>
__global__ __launch_bounds__(kUpdThreads) void mamba2_update_kernel(Mamba2Params p) {
  constexpr int SV = Elem<StT>::kVec;
  constexpr int LPR = N / SV;                    // lanes per state row
  static_assert(LPR >= 1 && LPR <= 64, "lanes per row");
  constexpr int RPL = 64 / LPR;
  constexpr int ROWS_PER_ITER = kUpdWaves * kUpdLoads * RPL;
  __shared__ float s_x[1024], s_y[1024];
  const int h = blockIdx.x, b = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int P = p.P;
  ActT* __restrict__ out = static_cast<ActT*>(p.out) + ((int64_t)b * p.H + h) * P;
  const int slot = p.slots[b];
  if (slot < 0 || slot >= p.num_slots) {  // inert row: zero output, pool untouched
    for (int i = tid; i < P; i += kUpdThreads) Elem<ActT>::store(out + i, 0.0f);
    return;
  }
  StT* __restrict__ S = static_cast<StT*>(p.ssm_pool) + ((int64_t)slot * p.H + h) * P * N;
  const int sub = lane / LPR, col = (lane % LPR) * SV;
  auto row_of = [&](int it, int u) { return it * ROWS_PER_ITER + (u * kUpdWaves + wave) * RPL + sub; };
  uint4 raw[kUpdLoads], raw2[kUpdLoads];
  auto load_batch = [&](uint4* buf, int it) {
#pragma unroll
    for (int u = 0; u < kUpdLoads; ++u) buf[u] = ld16(S + (int64_t)min(row_of(it, u), P - 1) * N + col);
  };
  load_batch(raw, 0);

  const int g = h / (p.H / p.G);
  const ActT* __restrict__ xr = static_cast<const ActT*>(p.x) + ((int64_t)b * p.H + h) * P;
  for (int i = tid; i < P; i += kUpdThreads) s_x[i] = Elem<ActT>::load(xr + i);
  const float dt = ssd_dt(p, Elem<ActT>::load(static_cast<const ActT*>(p.dt) + (int64_t)b * p.H + h), h);
  const float da = expf(p.A[h] * dt);
  float bv[SV], cv[SV];
  {
    const ActT* Br = static_cast<const ActT*>(p.B) + ((int64_t)b * p.G + g) * N + col;
    const ActT* Cr = static_cast<const ActT*>(p.C) + ((int64_t)b * p.G + g) * N + col;
#pragma unroll
    for (int i = 0; i < SV; ++i) {
      bv[i] = Elem<ActT>::load(Br + i) * dt;
      cv[i] = Elem<ActT>::load(Cr + i);
    }
  }
  __syncthreads();

  const int iters = (P + ROWS_PER_ITER - 1) / ROWS_PER_ITER;
  auto compute_batch = [&](const uint4* buf, int it) {
#pragma unroll
    for (int u = 0; u < kUpdLoads; ++u) {
      const int row = row_of(it, u);
      if (row >= P) continue;  // uniform across the row's lanes
      float st[SV];
      Elem<StT>::unpack(buf[u], st);
      const float xv = s_x[row];
      float y = 0.0f;
#pragma unroll
      for (int i = 0; i < SV; ++i) {
        st[i] = da * st[i] + xv * bv[i];
        y += st[i] * cv[i];
      }
      y = group_sum<LPR>(y);
      st16_nt(S + (int64_t)row * N + col, Elem<StT>::pack(st));
      if ((lane % LPR) == 0) s_y[row] = y;
    }
  };
  for (int it = 0; it < iters; it += 2) {
    load_batch(raw2, min(it + 1, iters - 1));
    compute_batch(raw, it);
    load_batch(raw, min(it + 2, iters - 1));
    if (it + 1 < iters) compute_batch(raw2, it + 1);
  }
  __syncthreads();
  const ActT* zr = p.z ? static_cast<const ActT*>(p.z) + ((int64_t)b * p.H + h) * P : nullptr;
  for (int i = tid; i < P; i += kUpdThreads) {
    float y = s_y[i];
    if (p.D) y += (p.D_per_p ? p.D[h * P + i] : p.D[h]) * s_x[i];
    if (zr) y *= silu_f(Elem<ActT>::load(zr + i));
    Elem<ActT>::store(out + i, y);
  }
}

// ---------------------------------------------------------------------------
// Prefill: workspace
// ---------------------------------------------------------------------------
// Per (chunk, head) block: Y_intra [P/16][4][64 lanes][4] f32 (the scan's
// accumulator order), the chunk's state contribution [P][N] f32, and
// exp(L_i) [64] then exp(L_C).
__host__ __device__ constexpr int64_t ssd_blk_y(int, int) { return 0; }
__host__ __device__ constexpr int64_t ssd_blk_st(int P, int) { return (int64_t)kSsdChunk * P * 4; }
__host__ __device__ constexpr int64_t ssd_blk_vec(int P, int N) { return ssd_blk_st(P, N) + (int64_t)P * N * 4; }
__host__ __device__ constexpr int64_t ssd_blk_bytes(int P, int N) {
  return (ssd_blk_vec(P, N) + (kSsdChunk + 4) * 4 + 255) / 256 * 256;
}

struct SsdWs {
  int32_t* seq_chunk_off;  // [Nseq+1]
  int32_t* chunk_seq;      // [NC]
  int32_t* chunk_start;    // [NC]
  char* blocks;            // [NC, H] blocks
};

__host__ __device__ inline size_t ssd_align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline int64_t ssd_max_chunks(int Ns, int64_t T) { return T / kSsdChunk + Ns; }

SsdWs ssd_carve(void* base, int Ns, int64_t T) {
  char* q = static_cast<char*>(base);
  SsdWs w;
  const int64_t nc = ssd_max_chunks(Ns, T);
  w.seq_chunk_off = reinterpret_cast<int32_t*>(q);
  q += ssd_align256((size_t)(Ns + 1) * 4);
  w.chunk_seq = reinterpret_cast<int32_t*>(q);
  q += ssd_align256((size_t)nc * 4);
  w.chunk_start = reinterpret_cast<int32_t*>(q);
  q += ssd_align256((size_t)nc * 4);
  w.blocks = q;
  return w;
}

__global__ __launch_bounds__(64) void ssd_table_kernel(const int32_t* cu, int Ns, SsdWs ws) {
  const int lane = threadIdx.x;
  const int per = (Ns + 63) / 64;
  const int s0 = min(Ns, lane * per), s1 = min(Ns, s0 + per);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (cu[s + 1] - cu[s] + kSsdChunk - 1) / kSsdChunk;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  int c = incl - local;
  for (int s = s0; s < s1; ++s) {
    ws.seq_chunk_off[s] = c;
    const int a = cu[s], e = cu[s + 1];
    for (int t = a; t < e; t += kSsdChunk) {
      ws.chunk_seq[c] = s;
      ws.chunk_start[c] = t;
      ++c;
    }
  }
  if (lane == 63) ws.seq_chunk_off[Ns] = incl;
}

// [64 tokens][W] rows of an activation, transposed into LDS as f16 [W][kTS]
// (hi, and lo for f32), rows past n zero.  Each thread moves 8 columns of
// one token.
template <typename ActT, int W>
__device__ __forceinline__ void stage_transposed(const ActT* src, int64_t stride, int n, _Float16* hi,
                                                 _Float16* lo) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  for (int v = threadIdx.x; v < kSsdChunk * (W / 8); v += blockDim.x) {
    const int t = v % kSsdChunk, c0 = 8 * (v / kSsdChunk);
    float x[8];
    if (t < n) load_n<ActT, 8>(src + (int64_t)t * stride + c0, x);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const _Float16 h = (_Float16)x[i];
      hi[(c0 + i) * kTS + t] = h;
      if constexpr (SPLIT) lo[(c0 + i) * kTS + t] = (_Float16)(x[i] - (float)h);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill: per (chunk, head)
// ---------------------------------------------------------------------------
template <typename ActT, int P, int N>
__global__ __launch_bounds__(256) void ssd_chunk_kernel(Mamba2Params p, SsdWs ws) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  constexpr int MS = kSsdChunk + 4;   // f32 row stride of M
  __shared__ __attribute__((aligned(16))) _Float16 CTh[N * kTS], BTh[N * kTS], XTh[P * kTS];
  __shared__ __attribute__((aligned(16))) _Float16 CTl[SPLIT ? N * kTS : 8], BTl[SPLIT ? N * kTS : 8],
      XTl[SPLIT ? P * kTS : 8];
  __shared__ __attribute__((aligned(16))) float Ms[kSsdChunk * MS];
  __shared__ double Ls[kSsdChunk];
  __shared__ float dts[kSsdChunk], ws_[kSsdChunk];

  const int cid = blockIdx.x, h = blockIdx.y;
  const int g = h / (p.H / p.G);
  const int seq = ws.chunk_seq[cid];
  const int64_t t0 = ws.chunk_start[cid];
  const int n = (int)min((int64_t)kSsdChunk, (int64_t)p.cu[seq + 1] - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  char* blk = ws.blocks + ((int64_t)cid * p.H + h) * ssd_blk_bytes(P, N);
  float* Yg = reinterpret_cast<float*>(blk + ssd_blk_y(P, N));
  float* Stg = reinterpret_cast<float*>(blk + ssd_blk_st(P, N));
  float* Vg = reinterpret_cast<float*>(blk + ssd_blk_vec(P, N));

  const ActT* Cp = static_cast<const ActT*>(p.C) + (t0 * p.G + g) * N;
  const ActT* Bp = static_cast<const ActT*>(p.B) + (t0 * p.G + g) * N;
  const ActT* Xp = static_cast<const ActT*>(p.x) + (t0 * p.H + h) * P;
  stage_transposed<ActT, N>(Cp, (int64_t)p.G * N, n, CTh, CTl);
  stage_transposed<ActT, N>(Bp, (int64_t)p.G * N, n, BTh, BTl);
  stage_transposed<ActT, P>(Xp, (int64_t)p.H * P, n, XTh, XTl);
  if (wave == 0) {
    const bool valid = lane < n;
    const float d = valid ? ssd_dt(p, Elem<ActT>::load(static_cast<const ActT*>(p.dt) + (t0 + lane) * p.H + h), h)
                          : 0.0f;
    double L = (double)p.A[h] * (double)d;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(L, off, 64);
      if (lane >= off) L += o;
    }
    const double Lc = __shfl(L, 63, 64);
    Ls[lane] = L;
    dts[lane] = d;
    ws_[lane] = d * (float)exp(Lc - L);      // weight of token j in the chunk's state
    Vg[lane] = (float)exp(L);                // exp(L_i) for the scan's inter-chunk term
    if (lane == 0) Vg[kSsdChunk] = (float)exp(Lc);
  }
  __syncthreads();

  // C B^T, row block I = wave: lane holds rows i = 16I + 4lg + r, column j = 16J + li
  {
    constexpr int NK = N / 32;
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
      if (J <= wave) {
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          // A operand: C rows 16 wave + li over n = 32 s + 8 lg .. ; B operand: B rows 16 J + li
          h8 ch, bh;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            ch[e] = CTh[(32 * s + 8 * lg + e) * kTS + 16 * wave + li];
            bh[e] = BTh[(32 * s + 8 * lg + e) * kTS + 16 * J + li];
          }
          acc = mfma_f16(ch, bh, acc);
          if constexpr (SPLIT) {
            h8 cl, bl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              cl[e] = CTl[(32 * s + 8 * lg + e) * kTS + 16 * wave + li];
              bl[e] = BTl[(32 * s + 8 * lg + e) * kTS + 16 * J + li];
            }
            acc = mfma_f16(ch, bl, acc);
            acc = mfma_f16(cl, bh, acc);
          }
        }
      }
      // D[4lg + r][li] = C_i . B_j with i = 16 wave + 4lg + r, j = 16J + li
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * wave + 4 * lg + r, j = 16 * J + li;
        Ms[i * MS + j] = (j <= i && J <= wave) ? acc[r] * expf((float)(Ls[i] - Ls[j])) * dts[j] : 0.0f;
      }
    }
  }
  __syncthreads();

  // Y_intra = M X: row tile I = wave; column tiles pt over P
#pragma unroll
  for (int pt = 0; pt < P / 16; ++pt) {
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if (32 * s > 16 * wave + 15) break;
      float m[8];
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const float4 v = *reinterpret_cast<const float4*>(Ms + (16 * wave + li) * MS + 32 * s + 8 * lg + 4 * e4);
        m[4 * e4] = v.x; m[4 * e4 + 1] = v.y; m[4 * e4 + 2] = v.z; m[4 * e4 + 3] = v.w;
      }
      h8 mh, ml;
      split8(m, mh, ml);
      const h8 xh = ld_h8(XTh + (16 * pt + li) * kTS + 32 * s + 8 * lg);
      acc = mfma_f16(mh, xh, acc);
      acc = mfma_f16(ml, xh, acc);
      if constexpr (SPLIT) acc = mfma_f16(mh, ld_h8(XTl + (16 * pt + li) * kTS + 32 * s + 8 * lg), acc);
    }
    // D[4lg + r][li] = Y[i = 16 wave + 4lg + r][p = 16 pt + li]: the scan's order
    *reinterpret_cast<float4*>(Yg + (((int64_t)pt * 4 + wave) * 64 + lane) * 4) =
        make_float4(acc[0], acc[1], acc[2], acc[3]);
  }

  // the chunk's state contribution St[p][n] = sum_j x_j[p] w_j B_j[n]:
  // row tiles of P over the waves, column tiles of N
  for (int pt = wave; pt < P / 16; pt += 4) {
#pragma unroll
    for (int nt = 0; nt < N / 16; ++nt) {
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        // A operand: x rows p = 16 pt + li over tokens j = 32 s + 8 lg .. scaled by w_j
        float a[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int j = 32 * s + 8 * lg + e;
          float xv = (float)XTh[(16 * pt + li) * kTS + j];
          if constexpr (SPLIT) xv += (float)XTl[(16 * pt + li) * kTS + j];
          a[e] = xv * ws_[j];
        }
        h8 ah, al;
        split8(a, ah, al);
        const h8 bh = ld_h8(BTh + (16 * nt + li) * kTS + 32 * s + 8 * lg);
        acc = mfma_f16(ah, bh, acc);
        acc = mfma_f16(al, bh, acc);
        if constexpr (SPLIT) acc = mfma_f16(ah, ld_h8(BTl + (16 * nt + li) * kTS + 32 * s + 8 * lg), acc);
      }
      // D[4lg + r][li] = St[p = 16 pt + 4lg + r][n = 16 nt + li]
#pragma unroll
      for (int r = 0; r < 4; ++r) Stg[(int64_t)(16 * pt + 4 * lg + r) * N + 16 * nt + li] = acc[r];
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill: the sequential pass, one wave per (sequence, head, 16 state rows)
// ---------------------------------------------------------------------------
// The wave holds rows p = 16 pb + li of S as the B operand of S^T: lane
// (li, lg) holds S[p][32 s + 8 lg + e] for s < N/32, e < 8.
template <typename ActT, typename StT, int P, int N>
__global__ __launch_bounds__(64) void ssd_scan_kernel(Mamba2Params p, SsdWs ws) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  constexpr int NK = N / 32;
  const int pb = blockIdx.x, h = blockIdx.y, s_idx = blockIdx.z;
  const int lane = threadIdx.x, li = lane & 15, lg = lane >> 4;
  const int g = h / (p.H / p.G);
  const int slot = p.slots ? p.slots[s_idx] : s_idx;
  const bool has = p.has_init == nullptr || p.has_init[s_idx] != 0;
  const int prow = 16 * pb + li;
  StT* Sg = static_cast<StT*>(p.ssm_pool) + (((int64_t)slot * p.H + h) * P + prow) * N;
  float Sf[NK][8];
#pragma unroll
  for (int s = 0; s < NK; ++s) {
    if (has) load_n<StT, 8>(Sg + 32 * s + 8 * lg, Sf[s]);
    else
#pragma unroll
      for (int e = 0; e < 8; ++e) Sf[s][e] = 0.0f;
  }
  const int c_begin = ws.seq_chunk_off[s_idx], c_end = ws.seq_chunk_off[s_idx + 1];
  const int64_t seq_start = p.cu[s_idx], seq_end = p.cu[s_idx + 1];
  const ActT* xg = static_cast<const ActT*>(p.x);
  const ActT* zg = static_cast<const ActT*>(p.z);
  ActT* og = static_cast<ActT*>(p.out);
  const float dcoef = p.D ? (p.D_per_p ? p.D[h * P + prow] : p.D[h]) : 0.0f;
  for (int cid = c_begin; cid < c_end; ++cid) {
    const char* blk = ws.blocks + ((int64_t)cid * p.H + h) * ssd_blk_bytes(P, N);
    const float* Yg = reinterpret_cast<const float*>(blk + ssd_blk_y(P, N));
    const float* Stg = reinterpret_cast<const float*>(blk + ssd_blk_st(P, N));
    const float* Vg = reinterpret_cast<const float*>(blk + ssd_blk_vec(P, N));
    const int64_t t0 = seq_start + (int64_t)kSsdChunk * (cid - c_begin);
    const int n = (int)min((int64_t)kSsdChunk, seq_end - t0);
    // S split into f16 halves as the B operand
    h8 Sh[NK], Sl[NK];
#pragma unroll
    for (int s = 0; s < NK; ++s) split8(Sf[s], Sh[s], Sl[s]);
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      if (16 * it >= n) break;
      // A operand: C rows t0 + 16 it + li over n = 32 s + 8 lg ..
      const int crow = min(16 * it + li, n - 1);
      const ActT* cr = static_cast<const ActT*>(p.C) + ((t0 + crow) * p.G + g) * N;
      f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        float c8[8];
        load_n<ActT, 8>(cr + 32 * s + 8 * lg, c8);
        h8 chh, cl;
        split8(c8, chh, cl);
        acc = mfma_f16(chh, Sh[s], acc);
        acc = mfma_f16(chh, Sl[s], acc);
        if constexpr (SPLIT) acc = mfma_f16(cl, Sh[s], acc);
      }
      // D[4lg + r][li] = (C S^T)[i = 16 it + 4lg + r][p = 16 pb + li]
      const float4 yv = *reinterpret_cast<const float4*>(Yg + (((int64_t)pb * 4 + it) * 64 + lane) * 4);
      const float4 ev = *reinterpret_cast<const float4*>(Vg + 16 * it + 4 * lg);
      const float ya[4] = {yv.x, yv.y, yv.z, yv.w}, ea[4] = {ev.x, ev.y, ev.z, ev.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * it + 4 * lg + r;
        if (i < n) {
          const int64_t off = ((t0 + i) * p.H + h) * P + prow;
          float y = ea[r] * acc[r] + ya[r];
          if (p.D) y += dcoef * Elem<ActT>::load(xg + off);
          if (p.z) y *= silu_f(Elem<ActT>::load(zg + off));
          Elem<ActT>::store(og + off, y);
        }
      }
    }
    // S <- exp(L_C) S + St
    const float eL = Vg[kSsdChunk];
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const float4 a = *reinterpret_cast<const float4*>(Stg + (int64_t)prow * N + 32 * s + 8 * lg);
      const float4 b = *reinterpret_cast<const float4*>(Stg + (int64_t)prow * N + 32 * s + 8 * lg + 4);
      const float add[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) Sf[s][e] = eL * Sf[s][e] + add[e];
    }
  }
#pragma unroll
  for (int s = 0; s < NK; ++s) store_n<StT, 8>(Sg + 32 * s + 8 * lg, Sf[s]);
}

template <typename ActT, typename StT, int N>
hipError_t launch_update_n(const Mamba2Params& p, hipStream_t stream) {
  mamba2_update_kernel<ActT, StT, N><<<dim3(p.H, p.Nseq), kUpdThreads, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename ActT, typename StT>
hipError_t launch_update(const Mamba2Params& p, hipStream_t stream) {
  switch (p.N) {
    case 16: return launch_update_n<ActT, StT, 16>(p, stream);
    case 32: return launch_update_n<ActT, StT, 32>(p, stream);
    case 64: return launch_update_n<ActT, StT, 64>(p, stream);
    case 128: return launch_update_n<ActT, StT, 128>(p, stream);
    default: return launch_update_n<ActT, StT, 256>(p, stream);
  }
}

template <typename ActT, typename StT, int P, int N>
hipError_t launch_chunked_pn(const Mamba2Params& p, const SsdWs& ws, hipStream_t stream) {
  if (p.num_chunks > 0) ssd_chunk_kernel<ActT, P, N><<<dim3((unsigned)p.num_chunks, p.H), 256, 0, stream>>>(p, ws);
  ssd_scan_kernel<ActT, StT, P, N><<<dim3(P / 16, p.H, p.Nseq), 64, 0, stream>>>(p, ws);
  return hipGetLastError();
}

template <typename ActT, typename StT, int P>
hipError_t launch_chunked_p(const Mamba2Params& p, const SsdWs& ws, hipStream_t stream) {
  switch (p.N) {
    case 32: return launch_chunked_pn<ActT, StT, P, 32>(p, ws, stream);
    case 64: return launch_chunked_pn<ActT, StT, P, 64>(p, ws, stream);
    default: return launch_chunked_pn<ActT, StT, P, 128>(p, ws, stream);
  }
}

template <typename ActT, typename StT>
hipError_t launch_chunked(const Mamba2Params& p, hipStream_t stream) {
  const SsdWs ws = ssd_carve(p.workspace, p.Nseq, p.T);
  ssd_table_kernel<<<1, 64, 0, stream>>>(p.cu, p.Nseq, ws);
  switch (p.P) {
    case 32: return launch_chunked_p<ActT, StT, 32>(p, ws, stream);
    case 64: return launch_chunked_p<ActT, StT, 64>(p, ws, stream);
    default: return launch_chunked_p<ActT, StT, 128>(p, ws, stream);
  }
}

template <typename ActT>
hipError_t dispatch_state(const Mamba2Params& p, bool chunked, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return chunked ? launch_chunked<ActT, float>(p, stream) : launch_update<ActT, float>(p, stream);
    case GDN_BF16: return chunked ? launch_chunked<ActT, bf16>(p, stream) : launch_update<ActT, bf16>(p, stream);
    default: return chunked ? launch_chunked<ActT, f16>(p, stream) : launch_update<ActT, f16>(p, stream);
  }
}

}  // namespace

size_t mamba2_workspace_bytes(int H, int P, int N, int Ns, int64_t T) {
  if (Ns <= 0) return 0;
  const int64_t nc = ssd_max_chunks(Ns, T);
  return ssd_align256((size_t)(Ns + 1) * 4) + 2 * ssd_align256((size_t)nc * 4) + (size_t)nc * H * ssd_blk_bytes(P, N);
}

hipError_t launch_mamba2_update(const Mamba2Params& p, hipStream_t stream) {
  return p.act == GDN_F32 ? dispatch_state<float>(p, false, stream) : dispatch_state<bf16>(p, false, stream);
}

hipError_t launch_mamba2_chunk_scan(const Mamba2Params& p, hipStream_t stream) {
  return p.act == GDN_F32 ? dispatch_state<float>(p, true, stream) : dispatch_state<bf16>(p, true, stream);
}

}  // namespace gdn
