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
// L_i = sum_{j<=i} A dt_j and S0 the state entering it):
//   Y_intra = (M * C B^T) X,  M[i][j] = exp(L_i - L_j) dt_j  (j <= i)
//   Y_inter[i] = exp(L_i) S0 C_i
//   S_C = exp(L_C) S0 + sum_j exp(L_C - L_j) dt_j x_j B_j^T
// in three passes, each parallel over the whole chip: ssd_state_kernel (per
// pair of consecutive chunks and head) forms both chunks' state contributions
// on the f16 hi/lo MFMA and the pair's; ssd_pass_kernel (element-wise over
// the state) carries S across the pairs and leaves each pair's S0 in the
// workspace; ssd_out_kernel (per chunk and head) forms the second chunk's S0
// of a pair from the first's, forms both output terms on the MFMA and applies
// D x and the gate.  Carrying the state per pair halves the state traffic of
// the pass; the second chunk's S0 costs one more [P, N] read.
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
// Per (chunk, head) block: a [P][N] f32 state, then the chunk's decay
// vector (exp(L_C), for a pair's first chunk exp(L_C + L_C') of the pair,
// then per token dt_j, exp(L_j) f32 and L_j f64; 1280 bytes), then a [P][N]
// f16 state.  A pair's first block holds the pair's contribution St_pair in
// f32; the state pass overwrites it with the state entering the pair in f32
// with f32 activations (the output kernel splits it into f16 hi/lo), else
// writes the f16 copy, which the output kernel's product C S0^T takes as is
// (its outputs round to 16 bits).  A pair's second block holds the first
// chunk's St: in f32 with f32 activations, else in the f16 slot.
__host__ __device__ constexpr int64_t ssd_blk_vec(int P, int N) { return (int64_t)P * N * 4; }
__host__ __device__ constexpr int64_t ssd_blk_s0h(int P, int N) { return ssd_blk_vec(P, N) + 1280; }
// offsets within the decay vector
constexpr int kVecDt = 16, kVecEL = 16 + 4 * 64, kVecL = 16 + 8 * 64;
__host__ __device__ constexpr int64_t ssd_blk_bytes(int P, int N) { return ssd_blk_s0h(P, N) + (int64_t)P * N * 2; }

struct SsdWs {
  int32_t* seq_chunk_off;  // [Nseq+1]
  int32_t* chunk_seq;      // [NC]
  int32_t* chunk_start;    // [NC]
  char* blocks;            // [NC, H] blocks
  int single;              // one sequence: chunk c starts at token 64 c, and no table is built
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
  w.single = Ns == 1;
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
// (hi, and lo for f32), rows past n zero.  Each of the 256 threads moves 8
// columns of one token per item; all its loads are issued before the stores.
template <typename ActT, int W>
__device__ __forceinline__ void stage_transposed(const ActT* src, int64_t stride, int n, _Float16* hi,
                                                 _Float16* lo) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  constexpr int ITEMS = kSsdChunk * (W / 8) / 256;
  static_assert(ITEMS >= 1 && kSsdChunk * (W / 8) % 256 == 0, "staging items");
  float x[ITEMS][8];
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const int v = threadIdx.x + 256 * u;
    const int t = v % kSsdChunk, c0 = 8 * (v / kSsdChunk);
    if (t < n) load_n<ActT, 8>(src + (int64_t)t * stride + c0, x[u]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const int v = threadIdx.x + 256 * u;
    const int t = v % kSsdChunk, c0 = 8 * (v / kSsdChunk);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const _Float16 h = (_Float16)x[u][i];
      hi[(c0 + i) * kTS + t] = h;
      if constexpr (SPLIT) lo[(c0 + i) * kTS + t] = (_Float16)(x[u][i] - (float)h);
    }
  }
}

// [64 tokens][W] rows of an activation into LDS as f16 [64][W + 8] (hi, and
// lo for f32), rows past n zero; loads first, as above.
template <typename ActT, int W>
__device__ __forceinline__ void stage_rows(const ActT* src, int64_t stride, int n, _Float16* hi, _Float16* lo) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  constexpr int RS = W + 8;
  constexpr int ITEMS = kSsdChunk * (W / 8) / 256;
  static_assert(ITEMS >= 1 && kSsdChunk * (W / 8) % 256 == 0, "staging items");
  float x[ITEMS][8];
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const int v = threadIdx.x + 256 * u;
    const int t = v / (W / 8), c0 = 8 * (v % (W / 8));
    if (t < n) load_n<ActT, 8>(src + (int64_t)t * stride + c0, x[u]);
    else
#pragma unroll
      for (int i = 0; i < 8; ++i) x[u][i] = 0.0f;
  }
#pragma unroll
  for (int u = 0; u < ITEMS; ++u) {
    const int v = threadIdx.x + 256 * u;
    const int t = v / (W / 8), c0 = 8 * (v % (W / 8));
    h8 xh, xl;
    split8(x[u], xh, xl);
    *reinterpret_cast<h8*>(hi + t * RS + c0) = xh;
    if constexpr (SPLIT) *reinterpret_cast<h8*>(lo + t * RS + c0) = xl;
  }
}

// The same two stagings split in two: load() issues the loads (16-byte
// vectors kept in their storage form, rows past n zero), store() converts
// and writes LDS, so that a kernel can issue every load it needs before it
// waits on the first.  tx is the thread's index among the 256 that share the
// tile.
template <typename ActT, int W, bool ROWS>
struct Staged {
  static constexpr bool kSplit = std::is_same<ActT, float>::value;
  static constexpr int kItems = kSsdChunk * (W / 8) / 256;
  static constexpr int kVecs = 8 / Elem<ActT>::kVec;  // 16-byte vectors per item
  static_assert(kItems >= 1 && kSsdChunk * (W / 8) % 256 == 0, "staging items");
  uint4 r[kItems][kVecs];
  __device__ __forceinline__ static void item(int tx, int u, int& t, int& c0) {
    const int v = tx + 256 * u;
    if (ROWS) {
      t = v / (W / 8);
      c0 = 8 * (v % (W / 8));
    } else {
      t = v % kSsdChunk;
      c0 = 8 * (v / kSsdChunk);
    }
  }
  __device__ __forceinline__ void load(const ActT* src, int64_t stride, int n, int tx) {
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      int t, c0;
      item(tx, u, t, c0);
#pragma unroll
      for (int w = 0; w < kVecs; ++w)
        r[u][w] = t < n ? *reinterpret_cast<const uint4*>(src + (int64_t)t * stride + c0 + w * Elem<ActT>::kVec)
                        : make_uint4(0u, 0u, 0u, 0u);
    }
  }
  __device__ __forceinline__ void store(_Float16* hi, _Float16* lo, int tx) const {
#pragma unroll
    for (int u = 0; u < kItems; ++u) {
      int t, c0;
      item(tx, u, t, c0);
      float x[8];
#pragma unroll
      for (int w = 0; w < kVecs; ++w) Elem<ActT>::unpack(r[u][w], x + w * Elem<ActT>::kVec);
      if (ROWS) {
        h8 xh, xl;
        split8(x, xh, xl);
        *reinterpret_cast<h8*>(hi + t * (W + 8) + c0) = xh;
        if constexpr (kSplit) *reinterpret_cast<h8*>(lo + t * (W + 8) + c0) = xl;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const _Float16 h = (_Float16)x[i];
          hi[(c0 + i) * kTS + t] = h;
          if constexpr (kSplit) lo[(c0 + i) * kTS + t] = (_Float16)(x[i] - (float)h);
        }
      }
    }
  }
};

// One wave: the chunk's steps dt_j and cumulative log-decays L_i =
// sum_{j<=i} A dt_j (f64 scan; tokens past n have dt = 0).  Returns L_i and
// dt_i of lane i and L_C through lc.
template <typename ActT>
__device__ __forceinline__ double chunk_log_decay(const Mamba2Params& p, int64_t t0, int n, int h, int lane, float& d,
                                                  double& lc) {
  d = lane < n ? ssd_dt(p, Elem<ActT>::load(static_cast<const ActT*>(p.dt) + (t0 + lane) * p.H + h), h) : 0.0f;
  double L = (double)p.A[h] * (double)d;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double o = __shfl_up(L, off, 64);
    if (lane >= off) L += o;
  }
  lc = __shfl(L, 63, 64);
  return L;
}

// ---------------------------------------------------------------------------
// Prefill pass 1, per (pair of consecutive chunks of a sequence, head): the
// contribution of each chunk to the state after it,
//   St[p][n] = sum_j exp(L_C - L_j) dt_j x_j[p] B_j[n],
// computed as St^T = B^T (w X) on the MFMA, and the pair's
//   St_pair = exp(L_C') St + St'   (' marks the second chunk).
// The state pass then steps from pair to pair, and the output kernel of a
// pair's second chunk forms the state entering it, exp(L_C) S0 + St, from
// the pair's entering state S0 and the first chunk's St, which this kernel
// leaves in the second chunk's block.  Pairs start at even chunk offsets
// within a sequence; the last chunk of a sequence with an odd chunk count
// is a pair of one.  Each half of the workgroup loads one chunk; the first
// is staged (B and x rows, row-major), its tiles formed, then the second
// staged over it.  With one sequence the grid holds one workgroup per pair;
// otherwise one per chunk, and the workgroup of a pair's second chunk has
// nothing to do.  The grid is one dimensional, head fastest: workgroups are dealt to the XCDs in turn, so
// with the chunk fastest every busy workgroup would land on every other XCD.
// With H a multiple of 8 the heads are permuted so that one XCD takes whole
// groups of heads, which share B.
// ---------------------------------------------------------------------------
// Three workgroups of eight waves per CU where 80 registers suffice (16-bit
// activations up to P * N = 64 * 128); the other shapes take what they need.
template <typename ActT, int P, int N>
constexpr int kSsdStateWaves = (!std::is_same<ActT, float>::value && P * N <= 64 * 128) ? 6 : 1;

template <typename ActT, int P, int N>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(kSsdStateWaves<ActT, P, N>))) void ssd_state_kernel(Mamba2Params p, SsdWs ws) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  constexpr int PT = P / 16, NT = N / 16, TILES = PT * NT, TPW = (TILES + 7) / 8;
  // B and x rows, row-major: the products take their columns through
  // transposing LDS reads
  constexpr int BS = N + 8, XS = P + 8;  // halves per row
  __shared__ __attribute__((aligned(16))) _Float16 Brh[kSsdChunk * BS], Xrh[kSsdChunk * XS];
  __shared__ __attribute__((aligned(16))) _Float16 Brl[SPLIT ? kSsdChunk * BS : 8], Xrl[SPLIT ? kSsdChunk * XS : 8];
  __shared__ __attribute__((aligned(16))) float ws_[2][kSsdChunk];
  __shared__ double lc_s[2];
  __shared__ float elc_s[2];

  const int hx = (int)(blockIdx.x % (unsigned)p.H), bx = (int)(blockIdx.x / (unsigned)p.H);
  const int cid = ws.single ? 2 * bx : bx;
  const int h = p.H % 8 == 0 ? (hx % 8) * (p.H / 8) + hx / 8 : hx;
  const int seq = ws.single ? 0 : ws.chunk_seq[cid];
  const int c_first = ws.single ? 0 : ws.seq_chunk_off[seq];
  if ((cid - c_first) & 1) return;
  const int c_end = ws.single ? (int)p.num_chunks : ws.seq_chunk_off[seq + 1];
  const bool two = cid + 1 < c_end;
  const int g = h / (p.H / p.G);
  const int64_t t0 = ws.single ? (int64_t)kSsdChunk * cid : ws.chunk_start[cid];
  const int tid = threadIdx.x, half = tid >> 8, ht = tid & 255, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  // half k loads chunk cid + k (nothing for the second half of a pair of one)
  const int64_t tk = t0 + (int64_t)kSsdChunk * half;
  const int nk = (half == 0 || two) ? (int)min((int64_t)kSsdChunk, (int64_t)p.cu[seq + 1] - tk) : 0;
  const int64_t bb = ssd_blk_bytes(P, N);
  char* blk = ws.blocks + ((int64_t)cid * p.H + h) * bb;
  char* blk2 = blk + (int64_t)p.H * bb;  // the second chunk's block (same head)

  // both chunks' loads first; the second chunk is staged once the first is
  // done with
  Staged<ActT, N, true> bt;
  Staged<ActT, P, true> xt;
  bt.load(static_cast<const ActT*>(p.B) + (tk * p.G + g) * N, (int64_t)p.G * N, nk, ht);
  xt.load(static_cast<const ActT*>(p.x) + (tk * p.H + h) * P, (int64_t)p.H * P, nk, ht);
  if ((wave & 3) == 0 && nk > 0) {  // the first wave of each half with a chunk
    float dec_dt;
    double dec_lc;
    const double dec_L = chunk_log_decay<ActT>(p, tk, nk, h, lane, dec_dt, dec_lc);
    // exponentials in f32 of the f64 log-decays and their differences
    ws_[half][lane] = dec_dt * expf((float)(dec_lc - dec_L));
    const float elc = expf((float)dec_lc);
    if (lane == 0) {
      lc_s[half] = dec_lc;
      elc_s[half] = elc;
    }
    // each chunk's decay vector, which the output kernel reads instead of
    // forming it again (the first chunk's also holds the pair's
    // exp(L_C + L_C'), written below)
    char* vec = (half ? blk2 : blk) + ssd_blk_vec(P, N);
    if (lane == 0) reinterpret_cast<float*>(vec)[0] = elc;
    reinterpret_cast<float*>(vec + kVecDt)[lane] = dec_dt;
    reinterpret_cast<float*>(vec + kVecEL)[lane] = expf((float)dec_L);
    reinterpret_cast<double*>(vec + kVecL)[lane] = dec_L;
  }
  if (half == 0) {
    bt.store(Brh, Brl, ht);
    xt.store(Xrh, Xrl, ht);
  }
  __syncthreads();

  if (tid == 0)
    reinterpret_cast<float*>(blk + ssd_blk_vec(P, N))[1] = expf((float)(lc_s[0] + (two ? lc_s[1] : 0.0)));
  // tiles in pt-major order, TPW consecutive tiles to a wave
  const float e2 = two ? elc_s[1] : 1.0f;  // exp(L_C') scales the first chunk's St
  float* Stg = reinterpret_cast<float*>(blk);
  h8 bh[2], bl[2];
  // column c0 + li of rows 32 s + 8 lg .. +7 of a row-major tile: in each
  // 16-lane group a transposing read hands lane 4a + c element c of the
  // 8-byte reads of lanes a, a+4, a+8, a+12, so lane li reads row
  // 32 s + 8 lg + 4 e + li / 4 at columns c0 + 4 (li % 4) .. +3
  auto column8 = [&](const _Float16* rows, int stride, int s, int c0) {
    const int r0 = 32 * s + 8 * lg + (li >> 2), c = c0 + 4 * (li & 3);
    const uint2 a0 = lds_read_tr16(rows + r0 * stride + c), a1 = lds_read_tr16(rows + (r0 + 4) * stride + c);
    return __builtin_bit_cast(h8, u32x4{a0.x, a0.y, a1.x, a1.y});
  };
  // B operand (w X)[j][p] of chunk k: column p = 16 pt + li, rows j = 32 s + 8 lg ..
  auto operand = [&](int k, int pt) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int j0 = 32 * s + 8 * lg;
      const h8 xh = column8(Xrh, XS, s, 16 * pt);
      h8 xl;
      if constexpr (SPLIT) xl = column8(Xrl, XS, s, 16 * pt);
      const float4 w0 = *reinterpret_cast<const float4*>(&ws_[k][j0]);
      const float4 w1 = *reinterpret_cast<const float4*>(&ws_[k][j0 + 4]);
      const float w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float xv = (float)xh[e];
        if constexpr (SPLIT) xv += (float)xl[e];
        v[e] = xv * w[e];
      }
      split8(v, bh[s], bl[s]);
    }
  };
  // D[4lg + r][li] = St^T[n = 16 nt + 4lg + r][p = 16 pt + li]
  auto product = [&](int nt, f32x4 acc) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      // A operand B^T[n][j]: row n = 16 nt + li, a column of the B rows
      const h8 ah = column8(Brh, BS, s, 16 * nt);
      acc = mfma_f16(ah, bh[s], acc);
      acc = mfma_f16(ah, bl[s], acc);
      if constexpr (SPLIT) acc = mfma_f16(column8(Brl, BS, s, 16 * nt), bh[s], acc);
    }
    return acc;
  };
  auto offset = [&](int pt, int nt) { return (int64_t)(16 * pt + li) * N + 16 * nt + 4 * lg; };

  // the first chunk's St: the pair's St_pair for a pair of one, else kept
  // (scaled by exp(L_C')) for the second chunk's products and stored for
  // the second chunk's entering state (f32 with f32 activations, else f16
  // in the entering-state slot)
  f32x4 acc1[TPW];
  int cur_pt = -1;
#pragma unroll
  for (int q = 0; q < TPW; ++q) {
    const int tile = wave * TPW + q;
    if (tile >= TILES) break;  // wave-uniform
    const int pt = tile / NT, nt = tile % NT;
    if (pt != cur_pt) {
      cur_pt = pt;
      operand(0, pt);
    }
    f32x4 acc = product(nt, f32x4{0.0f, 0.0f, 0.0f, 0.0f});
    const int64_t o = offset(pt, nt);
    if (!two) {
      *reinterpret_cast<float4*>(Stg + o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
      continue;
    }
    if constexpr (SPLIT) {
      *reinterpret_cast<float4*>(reinterpret_cast<float*>(blk2) + o) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(blk2 + ssd_blk_s0h(P, N)) + o) =
          make_uint2((uint32_t)f32_to_f16(acc[0]) | ((uint32_t)f32_to_f16(acc[1]) << 16),
                     (uint32_t)f32_to_f16(acc[2]) | ((uint32_t)f32_to_f16(acc[3]) << 16));
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) acc1[q][r] = acc[r] * e2;
  }
  if (two) {
    __syncthreads();  // the first chunk's tiles are done with
    if (half == 1) {
      bt.store(Brh, Brl, ht);
      xt.store(Xrh, Xrl, ht);
    }
    __syncthreads();
    cur_pt = -1;
#pragma unroll
    for (int q = 0; q < TPW; ++q) {
      const int tile = wave * TPW + q;
      if (tile >= TILES) break;
      const int pt = tile / NT, nt = tile % NT;
      if (pt != cur_pt) {
        cur_pt = pt;
        operand(1, pt);
      }
      const f32x4 acc = product(nt, acc1[q]);
      *reinterpret_cast<float4*>(Stg + offset(pt, nt)) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill pass 2, element-wise over (sequence, head, 4 state entries): carry
// S through the sequence's chunk pairs, S <- exp(L_C + L_C') S + St_pair,
// leaving in each pair's first block the state that enters the pair (f32 in
// place with f32 activations, else the f16 copy); the final S goes to the
// pool.
// ---------------------------------------------------------------------------
constexpr int kPassAhead = 4;

template <typename StT>
__global__ __launch_bounds__(256) void ssd_pass_kernel(Mamba2Params p, SsdWs ws) {
  const int h = blockIdx.y, s_idx = blockIdx.z;
  const int64_t PN = (int64_t)p.P * p.N;
  const int64_t e0 = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= PN) return;
  const int slot = p.slots ? p.slots[s_idx] : s_idx;
  const bool has = p.has_init == nullptr || p.has_init[s_idx] != 0;
  StT* Sg = static_cast<StT*>(p.ssm_pool) + ((int64_t)slot * p.H + h) * PN + e0;
  float S[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (has) load_n<StT, 4>(Sg, S);
  const int c_begin = ws.single ? 0 : ws.seq_chunk_off[s_idx];
  const int c_end = ws.single ? (int)((p.T + kSsdChunk - 1) / kSsdChunk) : ws.seq_chunk_off[s_idx + 1];
  const int64_t bb = ssd_blk_bytes(p.P, p.N), vo = ssd_blk_vec(p.P, p.N), ho = ssd_blk_s0h(p.P, p.N);
  const bool f16_s0 = p.act != GDN_F32;
  for (int c = c_begin; c < c_end; c += 2 * kPassAhead) {
    float4 v[kPassAhead];
    float eL[kPassAhead];
#pragma unroll
    for (int u = 0; u < kPassAhead; ++u) {
      if (c + 2 * u < c_end) {
        const char* blk = ws.blocks + ((int64_t)(c + 2 * u) * p.H + h) * bb;
        v[u] = *reinterpret_cast<const float4*>(blk + e0 * 4);
        eL[u] = reinterpret_cast<const float*>(blk + vo)[1];
      }
    }
#pragma unroll
    for (int u = 0; u < kPassAhead; ++u) {
      if (c + 2 * u < c_end) {
        char* blk = ws.blocks + ((int64_t)(c + 2 * u) * p.H + h) * bb;
        if (f16_s0) {
          const uint2 w = make_uint2((uint32_t)f32_to_f16(S[0]) | ((uint32_t)f32_to_f16(S[1]) << 16),
                                     (uint32_t)f32_to_f16(S[2]) | ((uint32_t)f32_to_f16(S[3]) << 16));
          *reinterpret_cast<uint2*>(blk + ho + e0 * 2) = w;
        } else {
          *reinterpret_cast<float4*>(blk + e0 * 4) = make_float4(S[0], S[1], S[2], S[3]);
        }
        S[0] = eL[u] * S[0] + v[u].x;
        S[1] = eL[u] * S[1] + v[u].y;
        S[2] = eL[u] * S[2] + v[u].z;
        S[3] = eL[u] * S[3] + v[u].w;
      }
    }
  }
  store_n<StT, 4>(Sg, S);
}

// ---------------------------------------------------------------------------
// Prefill pass 3, per (chunk, group of heads that share B and C): outputs
//   Y = (M * C B^T) X + diag(exp(L)) C S0^T,  y = (Y + D x) silu(z)
// with S0 the state entering the chunk: the pair's entering state for the
// first chunk of a pair, exp(L_C) S0 + St of the first chunk for the second.
// C B^T does not depend on the head: the workgroup stages C and B once,
// keeps C B^T in registers and C in LDS, and walks the group's heads; each
// head's loads are issued while the head before it is formed.  C, B and X
// are staged row-major (the k index of C B^T and C S0^T is n); M X takes X's
// columns as its B operand through transposing LDS reads.
// ---------------------------------------------------------------------------
template <int P, int N, bool SPLIT>
struct SsdOutLds {
  static constexpr int RS = N + 8;            // halves per C/B row
  static constexpr int MS = kSsdChunk + 4;    // floats per M row
  static constexpr int YS = P + 4;            // floats per Y row
  static constexpr int XS = P + 8;            // halves per X row
  static constexpr int kRowHalves = kSsdChunk * RS;
  static constexpr int kXHalves = kSsdChunk * XS;
  static constexpr int kParts = SPLIT ? 2 : 1;
  static constexpr int kRowsBytes = kRowHalves * kParts * 2;
  static constexpr int kMBytes = kSsdChunk * MS * 4;
  static constexpr int kYBytes = kSsdChunk * YS * 4;
  // C (hi, lo) at 0 for the whole workgroup; then B (hi, lo), which M goes
  // over once C B^T is in registers, and each head's Y over its M
  static constexpr int kU = kRowsBytes;
  static constexpr int kUBytes = kRowsBytes > kMBytes ? (kRowsBytes > kYBytes ? kRowsBytes : kYBytes)
                                                      : (kMBytes > kYBytes ? kMBytes : kYBytes);
  static constexpr int kX = kU + kUBytes;                    // X rows (hi, lo) of the current head
  static constexpr int kL = kX + kXHalves * kParts * 2;      // double L[64]
  static constexpr int kDt = kL + kSsdChunk * 8;
  static constexpr int kE = kDt + kSsdChunk * 4;
  static constexpr int kD = kE + kSsdChunk * 4;              // the head's D per column
  static constexpr int kBytes = kD + P * 4;
};

// Two workgroups per CU (one per (chunk, group) fills the chip twice at the
// usual shapes) where 256 registers hold two heads' loads (16-bit
// activations with P <= 64); the other shapes hold one head's loads and take
// the registers they need.
template <typename ActT, int P, int N>
constexpr int kSsdOutWaves = (!std::is_same<ActT, float>::value && P <= 64) ? 2 : 1;

template <typename ActT, int P, int N>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kSsdOutWaves<ActT, P, N>))) void ssd_out_kernel(Mamba2Params p, SsdWs ws) {
  constexpr bool SPLIT = std::is_same<ActT, float>::value;
  using Lay = SsdOutLds<P, N, SPLIT>;
  constexpr int RS = Lay::RS, MS = Lay::MS, YS = Lay::YS, XS = Lay::XS;
  constexpr int NK = N / 32;
  constexpr int NPT = P / 64 > 0 ? P / 64 : 1;  // column tiles of 16 per wave
  __shared__ __attribute__((aligned(16))) char smem[Lay::kBytes];
  _Float16* Ch = reinterpret_cast<_Float16*>(smem);
  _Float16* Cl = Ch + Lay::kRowHalves;   // f32 activations only
  _Float16* Bh = reinterpret_cast<_Float16*>(smem + Lay::kU);
  _Float16* Bl = Bh + Lay::kRowHalves;
  float* Ms = reinterpret_cast<float*>(smem + Lay::kU);  // over B
  float* Ys = reinterpret_cast<float*>(smem + Lay::kU);  // over M
  _Float16* Xh = reinterpret_cast<_Float16*>(smem + Lay::kX);
  _Float16* Xl = Xh + Lay::kXHalves;
  double* Ls = reinterpret_cast<double*>(smem + Lay::kL);
  float* dts = reinterpret_cast<float*>(smem + Lay::kDt);
  float* eLs = reinterpret_cast<float*>(smem + Lay::kE);
  float* Ds = reinterpret_cast<float*>(smem + Lay::kD);

  const int cid = blockIdx.x, g = blockIdx.y;
  const int hpg = p.H / p.G;  // heads per group
  const int seq = ws.single ? 0 : ws.chunk_seq[cid];
  const int64_t t0 = ws.single ? (int64_t)kSsdChunk * cid : ws.chunk_start[cid];
  const int n = (int)min((int64_t)kSsdChunk, (int64_t)p.cu[seq + 1] - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int64_t bb = ssd_blk_bytes(P, N);
  // the second chunk of a pair takes the pair's entering state from the
  // first chunk's block and the first chunk's St from its own
  const int c_first = ws.single ? 0 : ws.seq_chunk_off[seq];
  const bool second = ((cid - c_first) & 1) != 0;
  auto block = [&](int h) { return ws.blocks + ((int64_t)cid * p.H + h) * bb; };
  const bool has_cols = 16 * wave < P;  // the wave's column tiles pt = wave + 4 q (P = 32: waves 2, 3 have none)

  // per head, loaded while the head before it is formed (two register sets,
  // used in turn): the wave's S0 rows as the B operand S0^T[n][p] (f32
  // activations: f32, with a pair's second chunk's exp(L_C) S0 + St formed
  // as they arrive, split where used; else the f16 copy, and for a pair's
  // second chunk the first chunk's St); the chunk's x and z (8 consecutive
  // p of one token per item, kept packed; x is staged as rows and feeds the
  // epilogue's D x); the decay vector the state kernel wrote (wave 0), the
  // head's D (thread p holds column p's) and for a second chunk the first
  // chunk's exp(L_C)
  constexpr int EPI = kSsdChunk * (P / 8) / 256;
  static_assert(EPI >= 1 && kSsdChunk * (P / 8) % 256 == 0, "x items");
  constexpr int NV = 8 / Elem<ActT>::kVec;  // 16-byte vectors per item
  struct HeadRegs {
    float sv[SPLIT ? NPT : 1][SPLIT ? NK : 1][8];
    h8 svh[SPLIT ? 1 : NPT][SPLIT ? 1 : NK], sth[SPLIT ? 1 : NPT][SPLIT ? 1 : NK];
    uint4 xr[EPI][NV], zr[EPI][NV];
    double dec_L;
    float dec_dt, dec_eL, e1, d;
  };
  const ActT* xg = static_cast<const ActT*>(p.x);
  const ActT* zg = static_cast<const ActT*>(p.z);
  // per-thread element offsets of head 0 (a head adds h * P) of the x and z
  // items; rows past n re-read row n - 1 (their X rows meet zero columns of
  // M, their outputs are not stored)
  int64_t epi_off[EPI];
#pragma unroll
  for (int u = 0; u < EPI; ++u) {
    const int v = tid + 256 * u;
    const int i = v / (P / 8), p0 = 8 * (v % (P / 8));
    epi_off[u] = (t0 + min(i, n - 1)) * p.H * P + p0;
  }
  auto load_head = [&](HeadRegs& R, int h) __attribute__((always_inline)) {
    const char* blk0 = block(h);
    const char* blkS = second ? blk0 - (int64_t)p.H * bb : blk0;
    R.e1 = second ? reinterpret_cast<const float*>(blkS + ssd_blk_vec(P, N))[0] : 0.0f;
    if (has_cols) {
#pragma unroll
      for (int q = 0; q < NPT; ++q)
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          const int64_t o = (int64_t)(16 * (wave + 4 * q) + li) * N + 32 * s + 8 * lg;
          if constexpr (SPLIT) {
            const float* S0 = reinterpret_cast<const float*>(blkS);
            const float* St1 = reinterpret_cast<const float*>(blk0);
            const float4 a = *reinterpret_cast<const float4*>(S0 + o);
            const float4 b = *reinterpret_cast<const float4*>(S0 + o + 4);
            float* sv = R.sv[q][s];
            sv[0] = a.x; sv[1] = a.y; sv[2] = a.z; sv[3] = a.w;
            sv[4] = b.x; sv[5] = b.y; sv[6] = b.z; sv[7] = b.w;
            if (second) {
              const float4 c = *reinterpret_cast<const float4*>(St1 + o);
              const float4 d = *reinterpret_cast<const float4*>(St1 + o + 4);
              const float t[8] = {c.x, c.y, c.z, c.w, d.x, d.y, d.z, d.w};
#pragma unroll
              for (int e = 0; e < 8; ++e) sv[e] = R.e1 * sv[e] + t[e];
            }
          } else {
            R.svh[q][s] = ld_h8(reinterpret_cast<const _Float16*>(blkS + ssd_blk_s0h(P, N)) + o);
            if (second) R.sth[q][s] = ld_h8(reinterpret_cast<const _Float16*>(blk0 + ssd_blk_s0h(P, N)) + o);
          }
        }
    }
    if (wave == 0) {
      const char* vec = blk0 + ssd_blk_vec(P, N);
      R.dec_L = reinterpret_cast<const double*>(vec + kVecL)[lane];
      R.dec_dt = reinterpret_cast<const float*>(vec + kVecDt)[lane];
      R.dec_eL = reinterpret_cast<const float*>(vec + kVecEL)[lane];
    }
    if (p.D && tid < P) R.d = p.D_per_p ? p.D[h * P + tid] : p.D[h];
#pragma unroll
    for (int u = 0; u < EPI; ++u)
#pragma unroll
      for (int w = 0; w < NV; ++w) {
        R.xr[u][w] = ld16(xg + epi_off[u] + h * P + w * Elem<ActT>::kVec);
        if (zg) R.zr[u][w] = ld16(zg + epi_off[u] + h * P + w * Elem<ActT>::kVec);
      }
  };

  const int h_first = g * hpg;
  HeadRegs RA, RB;
  {
    Staged<ActT, N, true> crow, brow;
    crow.load(static_cast<const ActT*>(p.C) + (t0 * p.G + g) * N, (int64_t)p.G * N, n, tid);
    brow.load(static_cast<const ActT*>(p.B) + (t0 * p.G + g) * N, (int64_t)p.G * N, n, tid);
    load_head(RA, h_first);
    crow.store(Ch, Cl, tid);
    brow.store(Bh, Bl, tid);
  }
  __syncthreads();

  // C B^T, row block I = wave, column blocks J <= I, kept for every head
  f32x4 cb[4];
#pragma unroll
  for (int J = 0; J < 4; ++J) {
    cb[J] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (J > wave) continue;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      const int k0 = 32 * s + 8 * lg;
      const h8 ch = ld_h8(Ch + (16 * wave + li) * RS + k0);
      const h8 bh = ld_h8(Bh + (16 * J + li) * RS + k0);
      cb[J] = mfma_f16(ch, bh, cb[J]);
      if constexpr (SPLIT) {
        cb[J] = mfma_f16(ch, ld_h8(Bl + (16 * J + li) * RS + k0), cb[J]);
        cb[J] = mfma_f16(ld_h8(Cl + (16 * wave + li) * RS + k0), bh, cb[J]);
      }
    }
  }
  __syncthreads();  // B is done with: each head's M and Y go over it

  ActT* og = static_cast<ActT*>(p.out);
  auto process = [&](const HeadRegs& R, int h) __attribute__((always_inline)) {
    // X rows and the decay vector of head h into LDS (rows past n hold row
    // n - 1 again; M is zero there, as B is)
#pragma unroll
    for (int u = 0; u < EPI; ++u) {
      const int v = tid + 256 * u;
      const int i = v / (P / 8), p0 = 8 * (v % (P / 8));
      float xv[8];
#pragma unroll
      for (int w = 0; w < NV; ++w) Elem<ActT>::unpack(R.xr[u][w], xv + w * Elem<ActT>::kVec);
      h8 xh8, xl8;
      if constexpr (SPLIT) {
        split8(xv, xh8, xl8);
        *reinterpret_cast<h8*>(Xl + i * XS + p0) = xl8;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xh8[e] = (_Float16)xv[e];
      }
      *reinterpret_cast<h8*>(Xh + i * XS + p0) = xh8;
    }
    if (wave == 0) {
      Ls[lane] = R.dec_L;
      dts[lane] = R.dec_dt;
      eLs[lane] = R.dec_eL;
    }
    // C S0^T for the wave's column tiles (C stays staged for every head)
    float cs[NPT][4][4];
    if (has_cols) {
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        h8 sh[NK], sl[NK];
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          if constexpr (SPLIT) {
            split8(R.sv[q][s], sh[s], sl[s]);
          } else if (second) {
#pragma unroll
            for (int e = 0; e < 8; ++e) sh[s][e] = (_Float16)(R.e1 * (float)R.svh[q][s][e] + (float)R.sth[q][s][e]);
          } else {
            sh[s] = R.svh[q][s];
          }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          f32x4 acc2 = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s = 0; s < NK; ++s) {
            const int k0 = 32 * s + 8 * lg;
            const h8 ch = ld_h8(Ch + (16 * it + li) * RS + k0);
            acc2 = mfma_f16(ch, sh[s], acc2);
            if constexpr (SPLIT) {
              acc2 = mfma_f16(ch, sl[s], acc2);
              acc2 = mfma_f16(ld_h8(Cl + (16 * it + li) * RS + k0), sh[s], acc2);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) cs[q][it][r] = acc2[r];
        }
      }
    }
    __syncthreads();  // X and the vector are in; the last head's Y is read
    // the head's D, read only by the epilogue: written past the barrier that
    // every thread reaches after the last head's epilogue
    if (p.D && tid < P) Ds[tid] = R.d;

    // exp(L_i) C S0^T, which seeds the accumulators of M X below
    if (has_cols) {
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const float4 ev = *reinterpret_cast<const float4*>(eLs + 16 * it + 4 * lg);
#pragma unroll
        for (int q = 0; q < NPT; ++q) {
          cs[q][it][0] *= ev.x;
          cs[q][it][1] *= ev.y;
          cs[q][it][2] *= ev.z;
          cs[q][it][3] *= ev.w;
        }
      }
    }
    // M = (C B^T) masked and weighted by head h's decays; the blocks above
    // the diagonal are zero
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > wave) {
#pragma unroll
        for (int r = 0; r < 4; ++r) Ms[(16 * wave + 4 * lg + r) * MS + 16 * J + li] = 0.0f;
        continue;
      }
      const int j = 16 * J + li;
      const double Lj = Ls[j];
      const float dj = dts[j];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * wave + 4 * lg + r;
        const float mv = cb[J][r] * fast_exp((float)(Ls[i] - Lj)) * dj;
        Ms[i * MS + j] = (J < wave || j <= i) ? mv : 0.0f;
      }
    }
    __syncthreads();

    // Y[16 it + .., 16 pt + ..] = (M X) + exp(L_i) (C S0^T), pt = the wave's
    // tiles, accumulated over the second term.  With 16-bit activations M
    // enters as its f16 hi part alone: Y only feeds the 16-bit outputs
    if (has_cols) {
#pragma unroll
      for (int q = 0; q < NPT; ++q) {
        const int pt = wave + 4 * q;
        // X[32 s + 8 lg .. +7][16 pt + li] from the X rows: in each 16-lane
        // group a transposing read hands lane 4a + c element c of the
        // 8-byte reads of lanes a, a+4, a+8, a+12, so lane li reads token
        // 32 s + 8 lg + 4 e + li / 4 at columns 16 pt + 4 (li % 4) .. +3
        h8 xh[2], xl[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const int r0 = 32 * s + 8 * lg + (li >> 2), c = 16 * pt + 4 * (li & 3);
          const uint2 a0 = lds_read_tr16(Xh + r0 * XS + c), a1 = lds_read_tr16(Xh + (r0 + 4) * XS + c);
          xh[s] = __builtin_bit_cast(h8, u32x4{a0.x, a0.y, a1.x, a1.y});
          if constexpr (SPLIT) {
            const uint2 b0 = lds_read_tr16(Xl + r0 * XS + c), b1 = lds_read_tr16(Xl + (r0 + 4) * XS + c);
            xl[s] = __builtin_bit_cast(h8, u32x4{b0.x, b0.y, b1.x, b1.y});
          }
        }
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          f32x4 acc = {cs[q][it][0], cs[q][it][1], cs[q][it][2], cs[q][it][3]};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            if (32 * s > 16 * it + 15) break;
            float m[8];
#pragma unroll
            for (int e4 = 0; e4 < 2; ++e4) {
              const float4 v = *reinterpret_cast<const float4*>(Ms + (16 * it + li) * MS + 32 * s + 8 * lg + 4 * e4);
              m[4 * e4] = v.x; m[4 * e4 + 1] = v.y; m[4 * e4 + 2] = v.z; m[4 * e4 + 3] = v.w;
            }
            h8 mh, ml;
            if constexpr (SPLIT) {
              split8(m, mh, ml);
              acc = mfma_f16(mh, xh[s], acc);
              acc = mfma_f16(ml, xh[s], acc);
              acc = mfma_f16(mh, xl[s], acc);
            } else {
#pragma unroll
              for (int e = 0; e < 8; ++e) mh[e] = (_Float16)m[e];
              acc = mfma_f16(mh, xh[s], acc);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) cs[q][it][r] = acc[r];
        }
      }
    }
    __syncthreads();  // M and X are done with; Y goes over M
    if (has_cols) {
#pragma unroll
      for (int q = 0; q < NPT; ++q)
#pragma unroll
        for (int it = 0; it < 4; ++it)
#pragma unroll
          for (int r = 0; r < 4; ++r) Ys[(16 * it + 4 * lg + r) * YS + 16 * (wave + 4 * q) + li] = cs[q][it][r];
    }
    __syncthreads();

    // epilogue, 8 consecutive p of one token per item: + D x, * silu(z)
#pragma unroll
    for (int u = 0; u < EPI; ++u) {
      const int v = tid + 256 * u;
      const int i = v / (P / 8), p0 = 8 * (v % (P / 8));
      if (v >= kSsdChunk * (P / 8) || i >= n) continue;
      const int64_t off = ((t0 + i) * p.H + h) * P + p0;
      const float4 y0 = *reinterpret_cast<const float4*>(Ys + i * YS + p0);
      const float4 y1 = *reinterpret_cast<const float4*>(Ys + i * YS + p0 + 4);
      float y[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
      if (p.D) {
        float xv[8];
#pragma unroll
        for (int w = 0; w < NV; ++w) Elem<ActT>::unpack(R.xr[u][w], xv + w * Elem<ActT>::kVec);
        const float4 d0 = *reinterpret_cast<const float4*>(Ds + p0);
        const float4 d1 = *reinterpret_cast<const float4*>(Ds + p0 + 4);
        const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] += dv[e] * xv[e];
      }
      if (zg) {
        float zv[8];
#pragma unroll
        for (int w = 0; w < NV; ++w) Elem<ActT>::unpack(R.zr[u][w], zv + w * Elem<ActT>::kVec);
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] *= silu_f(zv[e]);
      }
      store_n<ActT, 8>(og + off, y);
    }
  };

  if constexpr (kSsdOutWaves<ActT, P, N> > 1) {
    // the heads in turn, two per trip, each trip's second head loaded while
    // its first is formed and the next trip's first while its second is
#pragma unroll 1
    for (int k = 0; k < hpg; k += 2) {
      if (k + 1 < hpg) load_head(RB, h_first + k + 1);
      process(RA, h_first + k);
      if (k + 1 >= hpg) break;
      if (k + 2 < hpg) load_head(RA, h_first + k + 2);
      process(RB, h_first + k + 1);
    }
  } else {
    // wider shapes: one register set, each head loaded where it starts
#pragma unroll 1
    for (int k = 0; k < hpg; ++k) {
      if (k > 0) load_head(RA, h_first + k);
      process(RA, h_first + k);
    }
  }
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

template <typename ActT, int P, int N>
hipError_t launch_chunked_pn(const Mamba2Params& p, const SsdWs& ws, hipStream_t stream) {
  if (p.num_chunks > 0) {
    const dim3 grid((unsigned)p.num_chunks, p.H);
    const int64_t units = ws.single ? (p.num_chunks + 1) / 2 : p.num_chunks;
    ssd_state_kernel<ActT, P, N><<<dim3((unsigned)(units * p.H)), 512, 0, stream>>>(p, ws);
    switch (p.state) {
      case GDN_F32: ssd_pass_kernel<float><<<dim3(P * N / 1024, p.H, p.Nseq), 256, 0, stream>>>(p, ws); break;
      case GDN_BF16: ssd_pass_kernel<bf16><<<dim3(P * N / 1024, p.H, p.Nseq), 256, 0, stream>>>(p, ws); break;
      default: ssd_pass_kernel<f16><<<dim3(P * N / 1024, p.H, p.Nseq), 256, 0, stream>>>(p, ws); break;
    }
    ssd_out_kernel<ActT, P, N><<<dim3((unsigned)p.num_chunks, p.G), 256, 0, stream>>>(p, ws);
  }
  return hipGetLastError();
}

template <typename ActT, int P>
hipError_t launch_chunked_p(const Mamba2Params& p, const SsdWs& ws, hipStream_t stream) {
  switch (p.N) {
    case 32: return launch_chunked_pn<ActT, P, 32>(p, ws, stream);
    case 64: return launch_chunked_pn<ActT, P, 64>(p, ws, stream);
    default: return launch_chunked_pn<ActT, P, 128>(p, ws, stream);
  }
}

template <typename ActT>
hipError_t launch_chunked(const Mamba2Params& p, hipStream_t stream) {
  const SsdWs ws = ssd_carve(p.workspace, p.Nseq, p.T);
  if (!ws.single) ssd_table_kernel<<<1, 64, 0, stream>>>(p.cu, p.Nseq, ws);
  switch (p.P) {
    case 32: return launch_chunked_p<ActT, 32>(p, ws, stream);
    case 64: return launch_chunked_p<ActT, 64>(p, ws, stream);
    default: return launch_chunked_p<ActT, 128>(p, ws, stream);
  }
}

template <typename ActT>
hipError_t dispatch_update(const Mamba2Params& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_update<ActT, float>(p, stream);
    case GDN_BF16: return launch_update<ActT, bf16>(p, stream);
    default: return launch_update<ActT, f16>(p, stream);
  }
}

}  // namespace

size_t mamba2_workspace_bytes(int H, int P, int N, int Ns, int64_t T) {
  if (Ns <= 0) return 0;
  const int64_t nc = ssd_max_chunks(Ns, T);
  return ssd_align256((size_t)(Ns + 1) * 4) + 2 * ssd_align256((size_t)nc * 4) + (size_t)nc * H * ssd_blk_bytes(P, N);
}

hipError_t launch_mamba2_update(const Mamba2Params& p, hipStream_t stream) {
  return p.act == GDN_F32 ? dispatch_update<float>(p, stream) : dispatch_update<bf16>(p, stream);
}

hipError_t launch_mamba2_chunk_scan(const Mamba2Params& p, hipStream_t stream) {
  return p.act == GDN_F32 ? launch_chunked<float>(p, stream) : launch_chunked<bf16>(p, stream);
}

}  // namespace gdn
