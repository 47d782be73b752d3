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
// Matrix products run on the f16 16x16x32 MFMA.  An f32 operand x enters as
// two f16 halves hi = f16(x), lo = f16(x - hi), and a product of two such
// operands as hi*hi + hi*lo + lo*hi (f32 accumulation): about 22 significant
// bits, where bf16 q/k/v need no split at all (every bf16 value of the
// normalised q/k range is exact in f16).  Products that feed only a bf16
// output (Q S^T and P Delta with bf16 q/k/v) use the f16 hi parts alone: one
// f16 rounding (2^-11) of an operand, several times below the bf16 rounding
// (2^-9) of the output itself; everything that feeds the state keeps the split.  The small inverse T uses the f32
// 16x16x4 MFMA.  The running sums G are formed in double precision and every
// decay factor is exp of a difference taken in double.
//
// Kernels (all on the caller's stream):
//  1. chunk_table_kernel: chunk ids -> (sequence, first token); chunks never
//     cross sequences and a sequence's last chunk may be short.  A single
//     sequence needs no table (chunk c starts at token 64 c).
//  2. chunk_prep_kernel, one workgroup per (chunk, value head), no state
//     dependence: K K^T and Q K^T with operands read straight from memory,
//     T = (I + A)^-1 (16x16 diagonal blocks by substitution in registers,
//     off-diagonal blocks T_IJ = -T_II sum_K A_IK T_KJ on MFMA).  Writes P
//     (f16), gamma, exp(G_C - G_j) and the q/k row scales to the workspace,
//     and then
//       - with bf16 q/k/v (the "T form"): T diag(beta) (f16 hi/lo, MFMA
//         fragment order) and, once per key head, the K rows in the scan's
//         contraction order and the q rows as MFMA fragments (unscaled);
//       - with f32 q/k/v (the "W form"): the row-scaled K^T (f16 hi/lo), W
//         (f16 hi/lo) and U^T (f32), formed against K^T / V^T staged in LDS.
//  3. chunk_scan_kernel, one workgroup (8 waves) per (sequence, value head,
//     block of 16 value rows), placed so that the row blocks and value heads
//     of one key head share an XCD's L2: walks the sequence's chunks in order.
//     Four waves carry the 16 x Dk state block in registers and run only the
//     serial part (Delta and the state update); four more do the bulk loads,
//     staging the chunk operands into LDS, and form the output of each chunk
//     from the state and Delta published in LDS.  One barrier per chunk (two
//     in the T form).  Value rows of the state are independent, so row blocks never
//     communicate.  Delta = U - W S0^T in the W form; in the T form
//     Delta = T diag(beta) (V - diag(gamma) K S0^T), the same quantity by
//     (I + A) Delta = diag(beta) V - diag(beta gamma) K S0^T, which moves the
//     two [c, c] x [c, D] products W and U out of the per-chunk work.
//
// Shapes the chunked kernels do not cover (Dk != Dv, or head dims 16 or
// 256) run a token-sequential kernel: one wave per sequence, value head and
// 16 value rows, with the state rows in registers.
#include <algorithm>
#include <atomic>
#include <mutex>
#include <type_traits>

#include "gdn_device.h"
#include "gdn_internal.h"
#include "gdn_mfma.h"

namespace gdn {
namespace {

// Eight consecutive input elements in their storage form (one 16-byte word
// for bf16, two for f32).
template <typename T>
struct Raw8 {
  static constexpr int kWords = (int)sizeof(T) / 2;
  uint4 w[kWords];
  __device__ __forceinline__ void load(const T* p) {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = reinterpret_cast<const uint4*>(p)[i];
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int i = 0; i < kWords; ++i) w[i] = make_uint4(0, 0, 0, 0);
  }
  __device__ __forceinline__ void get(float* o) const {
#pragma unroll
    for (int i = 0; i < kWords; ++i) Elem<T>::unpack(w[i], o + i * Elem<T>::kVec);
  }
};

constexpr int kChunk = 64;
constexpr int KTS = kChunk + 8;  // row stride (halves) of transposed [column][token] tiles

// ---------------------------------------------------------------------------
// Workspace layout.
// ---------------------------------------------------------------------------
__host__ __device__ constexpr size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Per (chunk, value head) block, byte offsets (D = head dim):
//   W hi [64][D] f16, W lo [64][D] f16, U^T [D][64] f32,
//   P hi [64 x 64] f16, P lo [64 x 64] f16 (MFMA fragment order, p_frag),
//   K^T hi [D][64] f16, K^T lo [D][64] f16 (written for f32 q/k/v only; K
//   already scaled by its row scale), gamma [64], exp(G_C - G_j) [64],
//   k row scale [64], q row scale [64] f32
// W's columns are stored in the scan's contraction order: within each group
// of 32, position 8b + 4a + c holds column 16a + 4b + c (a < 2, b < 4, c < 4).
__host__ __device__ constexpr int64_t blk_w_hi(int) { return 0; }
__host__ __device__ constexpr int64_t blk_w_lo(int D) { return (int64_t)kChunk * D * 2; }
__host__ __device__ constexpr int64_t blk_ut(int D) { return (int64_t)kChunk * D * 4; }
__host__ __device__ constexpr int64_t blk_p_hi(int D) { return (int64_t)kChunk * D * 8; }
__host__ __device__ constexpr int64_t blk_p_lo(int D) { return blk_p_hi(D) + kChunk * kChunk * 2; }
__host__ __device__ constexpr int64_t blk_kt_hi(int D) { return blk_p_hi(D) + kChunk * kChunk * 4; }
__host__ __device__ constexpr int64_t blk_kt_lo(int D) { return blk_kt_hi(D) + (int64_t)D * kChunk * 2; }
__host__ __device__ constexpr int64_t blk_vec(int D) { return blk_kt_hi(D) + (int64_t)D * kChunk * 4; }
__host__ __device__ constexpr int64_t blk_bytes(int D) { return blk_vec(D) + 4 * kChunk * 4; }

// With bf16 q/k/v the block holds T diag(beta) (f16 hi [64 x 64], then lo,
// each in MFMA fragment order) in place of W and U^T, and the scan forms
// Delta = T diag(beta) (V - diag(gamma) K S0^T) itself; the block of a key
// head's first value head also holds the key head's K rows (K^T lo slot)
// and q fragments (K^T hi slot).  The first 16 KiB of a block always lie inside
// the W / U^T region (blk_p_hi(D) = 512 D >= 16 KiB for D >= 32).
__host__ __device__ constexpr int64_t blk_tb_hi() { return 0; }
__host__ __device__ constexpr int64_t blk_tb_lo() { return (int64_t)kChunk * kChunk * 2; }

// The first value head of h's key head within the launch's head range
// [h0, h0 + hg): with bf16 q/k/v its block holds the key head's K^T and K
// rows for every value head of the key head in the launch.
__host__ __device__ inline int kv_first(const PrefillParams& p, int h) {
  const int r = p.Hv / p.Hk;
  const int f = h - h % r;
  return f > p.h0 ? f : p.h0;
}

struct ChunkWs {
  int32_t* seq_chunk_off;  // [N+1] first chunk id of each sequence
  int32_t* chunk_seq;      // [NC]
  int32_t* chunk_start;    // [NC] first token (global index)
  char* blocks;            // [NC, Hv] blocks of blk_bytes(D)
  int single;              // one sequence: chunk c starts at token 64 c, and no table is built
};

inline int64_t max_chunks(int N, int64_t T) { return T / kChunk + N; }

ChunkWs carve(void* base, int N, int64_t T) {
  char* p = static_cast<char*>(base);
  ChunkWs w;
  const int64_t nc = max_chunks(N, T);
  w.seq_chunk_off = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)(N + 1) * 4);
  w.chunk_seq = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nc * 4);
  w.chunk_start = reinterpret_cast<int32_t*>(p);
  p += align256((size_t)nc * 4);
  w.blocks = p;
  w.single = N == 1;
  return w;
}

bool chunked_dims(int Dk, int Dv) { return Dk == Dv && (Dk == 32 || Dk == 64 || Dk == 128); }

// ---------------------------------------------------------------------------
// 1. chunk table
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void chunk_table_kernel(const int32_t* cu, int N, ChunkWs ws) {
  // one wave: lane l takes sequences [l*per, (l+1)*per), an exclusive scan of
  // their chunk counts gives each lane its first chunk id
  const int lane = threadIdx.x;
  const int per = (N + 63) / 64;
  const int s0 = min(N, lane * per), s1 = min(N, s0 + per);
  int local = 0;
  for (int s = s0; s < s1; ++s) local += (cu[s + 1] - cu[s] + kChunk - 1) / kChunk;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off, 64);
    if (lane >= off) incl += o;
  }
  int c = incl - local;
  for (int s = s0; s < s1; ++s) {
    ws.seq_chunk_off[s] = c;
    const int a = cu[s], e = cu[s + 1];  // read once: the stores below may alias cu as far as the compiler knows
    for (int t = a; t < e; t += kChunk) {
      ws.chunk_seq[c] = s;
      ws.chunk_start[c] = t;
      ++c;
    }
  }
  if (lane == 63) ws.seq_chunk_off[N] = incl;
}

// four consecutive elements (one 8-byte read for bf16, 16 for f32)
__device__ __forceinline__ void load4(const float* p, float* o) {
  const float4 v = *reinterpret_cast<const float4*>(p);
  o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
}
__device__ __forceinline__ void load4(const bf16* p, float* o) {
  const uint2 v = *reinterpret_cast<const uint2*>(p);
  o[0] = __uint_as_float(v.x << 16);
  o[1] = __uint_as_float(v.x & 0xffff0000u);
  o[2] = __uint_as_float(v.y << 16);
  o[3] = __uint_as_float(v.y & 0xffff0000u);
}

// Transposed staging of a [64 tokens][D] tile into LDS as [D][KTS] f16 (hi
// and, for f32 inputs, lo).  Lane l of a wave takes tokens 2(l%32), 2(l%32)+1
// of one 8-column segment, so each 32-lane half writes 32 consecutive words.
// threadIdx.x behind an empty asm statement: a value the compiler cannot
// hoist out of a loop, so that the per-lane offsets the helpers below derive
// from it are formed where they are used instead of being held in registers
// across a persistent kernel's loop
__device__ __forceinline__ int thread_index() {
  int t = (int)threadIdx.x;
  asm volatile("" : "+v"(t));
  return t;
}

template <typename T, int D, int NW = 4>
struct TransposedTile {
  static constexpr bool kSplit = std::is_same<T, float>::value;
  static constexpr int kSegs = D / 8;
  static constexpr int kPasses = (kSegs + 2 * NW - 1) / (2 * NW);
  Raw8<T> r0[kPasses], r1[kPasses];
  // Loads are unconditional (rows past the chunk end re-read row n-1, and
  // segments past D re-read segment 0) so that no load sits under a branch;
  // store() zeroes what lies outside the tile.
  __device__ __forceinline__ void load(const T* src, int64_t stride, int n) {
    const int tix = thread_index(), lane = tix & 63, wave = tix >> 6;
    const int t = 2 * (lane & 31), seg0 = wave * 2 + (lane >> 5);
    const int ta = min(t, n - 1), tb = min(t + 1, n - 1);
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int seg = seg0 + 2 * NW * ps < kSegs ? seg0 + 2 * NW * ps : 0;
      r0[ps].load(src + (int64_t)ta * stride + seg * 8);
      r1[ps].load(src + (int64_t)tb * stride + seg * 8);
    }
  }
  // row scales (l2 norm) are per token; null means 1
  __device__ __forceinline__ void store(_Float16* hi, _Float16* lo, const float* rowscale, int n) const {
    const int t = 2 * (thread_index() & 31);
    store(hi, lo, rowscale ? rowscale[t] : 1.0f, rowscale ? rowscale[t + 1] : 1.0f, n);
  }
  // s0, s1: scales of this lane's two tokens 2(l%32), 2(l%32)+1
  __device__ __forceinline__ void store(_Float16* hi, _Float16* lo, float s0, float s1, int n) const {
    const int tix = thread_index(), lane = tix & 63, wave = tix >> 6;
    const int t = 2 * (lane & 31), seg0 = wave * 2 + (lane >> 5);
    if (t >= n) s0 = 0.0f;
    if (t + 1 >= n) s1 = 0.0f;
#pragma unroll
    for (int ps = 0; ps < kPasses; ++ps) {
      const int seg = seg0 + 2 * NW * ps;
      if (seg >= kSegs) continue;
      float x0[8], x1[8];
      r0[ps].get(x0);
      r1[ps].get(x1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float a = x0[i] * s0, b = x1[i] * s1;
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        const uint32_t wh = (uint32_t)__builtin_bit_cast(uint16_t, ha) |
                            ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
        *reinterpret_cast<uint32_t*>(hi + (seg * 8 + i) * KTS + t) = wh;
        if constexpr (kSplit) {
          const _Float16 la = (_Float16)(a - (float)ha), lb = (_Float16)(b - (float)hb);
          const uint32_t wl = (uint32_t)__builtin_bit_cast(uint16_t, la) |
                              ((uint32_t)__builtin_bit_cast(uint16_t, lb) << 16);
          *reinterpret_cast<uint32_t*>(lo + (seg * 8 + i) * KTS + t) = wl;
        }
      }
    }
  }
};

// ---------------------------------------------------------------------------
// 2. per-chunk work
// ---------------------------------------------------------------------------
// Wave w owns token block I = w: it loads the K rows of blocks 0..w and the Q
// rows of block w as MFMA fragments straight from memory, and forms the
// transposed tiles (K_J K_w^T) and (K_J Q_w^T), so that each lane ends up with
// four consecutive columns of a row of A and P.
__device__ __forceinline__ void store_h4(_Float16* p, const float* v) {
  _Float16 h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = (_Float16)v[i];
  uint2 w;
  w.x = (uint32_t)__builtin_bit_cast(uint16_t, h[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16);
  w.y = (uint32_t)__builtin_bit_cast(uint16_t, h[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}
// f16 hi/lo of four consecutive values
__device__ __forceinline__ void store_h4_split(_Float16* hi, _Float16* lo, const float* v) {
  float h[4], l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = (float)(_Float16)v[i];
    l[i] = v[i] - h[i];
  }
  store_h4(hi, h);
  store_h4(lo, l);
}

// P is stored in MFMA fragment order: for row block I and 32-column step s,
// the A-operand fragments of the 64 lanes (lane li + 16 g holds row 16I + li,
// columns 32s + 8g .. +7) are one contiguous 1 KiB run.  Offset (in halves)
// of the four columns 16J + 4q .. +3 of row 16I + li:
__device__ __forceinline__ int p_frag(int I, int li, int J, int q) {
  return ((2 * I + (J >> 1)) * 64 + li + 16 * (2 * (J & 1) + (q >> 1))) * 8 + 4 * (q & 1);
}

// T = (I + A)^-1 of the 64 x 64 strictly lower A (row stride TS) into Ts;
// Ms is 4 x 16 x 17 floats of scratch.  Diagonal block w by wave w, lane li
// solving column li by substitution; off-diagonal blocks by distance on the
// f32 MFMA: T_IJ = -T_II sum_K A_IK T_KJ.  Waves 0-3 do the work (every
// wave of the workgroup takes the barriers).  Ends with a barrier.
template <int TS>
__device__ __forceinline__ void unit_lower_inverse(const float* As, float* Ts, float* Ms) {
  const int tid = thread_index(), lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  if (wave < 4) {
    const int B0 = 16 * wave, j = li;
    float tc[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float arow[16];
#pragma unroll
      for (int m4 = 0; m4 < 4; ++m4) {
        const float4 v = *reinterpret_cast<const float4*>(As + (B0 + i) * TS + B0 + 4 * m4);
        arow[4 * m4] = v.x; arow[4 * m4 + 1] = v.y; arow[4 * m4 + 2] = v.z; arow[4 * m4 + 3] = v.w;
      }
      float acc = 0.0f;
#pragma unroll
      for (int m = 0; m < i; ++m) acc += arow[m] * tc[m];  // tc[m] = 0 for m < j
      tc[i] = i < j ? 0.0f : (i == j ? 1.0f : -acc);
    }
    if (lg == 0)
#pragma unroll
      for (int i = 0; i < 16; ++i) Ts[(B0 + i) * TS + B0 + j] = tc[i];
  }
  __syncthreads();
  // off-diagonal blocks, by distance: wave I computes T_{I, I-dist}
  for (int dist = 1; dist < 4; ++dist) {
    const int I = wave, J = wave - dist;
    const bool act = wave < 4 && J >= 0;
    if (act) {
      f32x4 M = {0.0f, 0.0f, 0.0f, 0.0f};
      for (int K = J; K < I; ++K)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          M = mfma_f32(As[(16 * I + li) * TS + 16 * K + 4 * s + lg], Ts[(16 * K + 4 * s + lg) * TS + 16 * J + li], M);
#pragma unroll
      for (int r = 0; r < 4; ++r) Ms[wave * 272 + (4 * lg + r) * 17 + li] = M[r];
    }
    __syncthreads();
    if (act) {
      f32x4 X = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < 4; ++s)
        X = mfma_f32(Ts[(16 * I + li) * TS + 16 * I + 4 * s + lg], Ms[wave * 272 + (4 * s + lg) * 17 + li], X);
#pragma unroll
      for (int r = 0; r < 4; ++r) Ts[(16 * I + 4 * lg + r) * TS + 16 * J + li] = -X[r];
    }
    __syncthreads();
  }
}

// W = T diag(bw) K and U = T diag(bu) V, computed as W^T = K^T (T diag(bw))^T
// and U^T = V^T (T diag(bu))^T so that each lane gets four consecutive
// columns of a row of W / U; column tiles over the waves.  K^T and V^T are
// [D][KTS] f16 tiles (with lo halves when K_LO / V_LO).  W is written f16 hi/lo
// in the scan's contraction order, U^T as f32 [D][64].
template <bool K_LO, bool V_LO, int TS, int D, int NW = 4>
__device__ __forceinline__ void w_u_products(const float* Ts, const float* bw, const float* bu, const _Float16* KTh,
                                             const _Float16* KTl, const _Float16* VTh, const _Float16* VTl,
                                             _Float16* Wh, _Float16* Wl, float* UTg) {
  constexpr int NCT = D / 16;
  const int tid = thread_index(), lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  constexpr int NT = (2 * NCT + NW - 1) / NW;  // tiles per wave
#pragma unroll
  for (int I = 0; I < 4; ++I) {
    const int i = 16 * I + li;
    f32x4 acc[NT];
#pragma unroll
    for (int m = 0; m < NT; ++m) acc[m] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s <= I / 2; ++s) {
      float tw[8], tu[8];
#pragma unroll
      for (int e4 = 0; e4 < 2; ++e4) {
        const float4 v = *reinterpret_cast<const float4*>(Ts + i * TS + 32 * s + 8 * lg + 4 * e4);
        tu[4 * e4] = v.x; tu[4 * e4 + 1] = v.y; tu[4 * e4 + 2] = v.z; tu[4 * e4 + 3] = v.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int tk = 32 * s + 8 * lg + e;
        const float tv = tk <= i ? tu[e] : 0.0f;
        tw[e] = tv * bw[tk];
        tu[e] = tv * bu[tk];
      }
      h8 twh, twl, tuh, tul;
      split8(tw, twh, twl);
      split8(tu, tuh, tul);
#pragma unroll
      for (int m = 0; m < NT; ++m) {
        const int ct = wave + NW * m;
        if (ct >= 2 * NCT) break;
        const bool isW = ct < NCT;
        const int col0 = 16 * (isW ? ct : ct - NCT);
        const h8 xh = ld_h8((isW ? KTh : VTh) + (col0 + li) * KTS + 32 * s + 8 * lg);
        acc[m] = mfma_f16(xh, isW ? twh : tuh, acc[m]);
        acc[m] = mfma_f16(xh, isW ? twl : tul, acc[m]);
        if constexpr (K_LO || V_LO) {
          if (isW ? K_LO : V_LO)
            acc[m] = mfma_f16(ld_h8((isW ? KTl : VTl) + (col0 + li) * KTS + 32 * s + 8 * lg), isW ? twh : tuh, acc[m]);
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NT; ++m) {
      const int ct = wave + NW * m;
      if (ct >= 2 * NCT) break;
      const float v[4] = {acc[m][0], acc[m][1], acc[m][2], acc[m][3]};
      if (ct < NCT) {
        // columns 16ct + 4lg .. +3, stored in the scan's contraction order
        const int pos = 32 * (ct >> 1) + 8 * lg + 4 * (ct & 1);
        store_h4_split(Wh + i * D + pos, Wl + i * D + pos, v);
      } else {
        const int col = 16 * (ct - NCT) + 4 * lg;
#pragma unroll
        for (int r = 0; r < 4; ++r) UTg[(col + r) * kChunk + i] = v[r];
      }
    }
  }
}

// T diag(beta) as f16 hi/lo for the scan (bf16 q/k/v), each in MFMA
// fragment order: for row block I and 32-column step s a 1 KiB run in which
// lane li + 16 g holds row 16 I + li at positions 32 s + 8 g .. +7, the
// columns of each group of 32 in the scan's contraction order (position
// 8b + 4a + c holds column 16a + 4b + c).  Entries above the diagonal are
// zero.  Thread t forms positions 16 (t % 4) .. +15 of row t / 4.
template <int TS>
__device__ __forceinline__ void store_t_beta(const float* Ts, const float* bs, _Float16* hi, _Float16* lo) {
  const int i = threadIdx.x >> 2, q = threadIdx.x & 3;
  float v[16];
  // positions 16 q + 4 g .. +3 are four consecutive columns j0 .. j0 + 3
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const int pos = 16 * q + 4 * g;
    const int j0 = (pos & ~31) + 16 * (g & 1) + 8 * (q & 1) + 4 * (g >> 1);
    const float4 t4 = *reinterpret_cast<const float4*>(Ts + i * TS + j0);
    const float4 b4 = *reinterpret_cast<const float4*>(bs + j0);
    const float tv[4] = {t4.x, t4.y, t4.z, t4.w}, bv[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) v[4 * g + e] = j0 + e <= i ? tv[e] * bv[e] : 0.0f;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    h8 vh, vl;
    split8(v + 8 * h, vh, vl);
    // positions 16 q + 8 h .. +7: step s = q / 2, lane group g = 2 (q % 2) + h
    const int f = ((2 * (i >> 4) + (q >> 1)) * 64 + (i & 15) + 16 * (2 * (q & 1) + h)) * 8;
    *reinterpret_cast<h8*>(hi + f) = vh;
    *reinterpret_cast<h8*>(lo + f) = vl;
  }
}

// With bf16 q/k/v the kernel needs 40 KB of LDS and under 128 VGPRs (the
// other blocks' K rows are read from LDS where they are used), so four
// workgroups share a CU.
// occupancy the register allocation aims at: three waves per SIMD with bf16
// q/k/v (four workgroups share a CU); f32 q/k/v keep the compiler's choice
template <typename QkvT>
constexpr int kPrepWaves = std::is_same<QkvT, float>::value ? 1 : 3;

// Value heads per prep workgroup: with bf16 q/k/v (the T form) one
// workgroup takes every value head of a key head, up to kMaxVpw of them,
// and forms K K^T and Q K^T once for all; otherwise one value head each.
// Two keep the LDS at 40 KB, four workgroups to a CU.
constexpr int kMaxVpw = 2;
__host__ __device__ inline int prep_vpw(const PrefillParams& p) {
  const int r = p.Hv / p.Hk;
  return (p.qkv != GDN_F32 && r <= kMaxVpw && p.h0 % r == 0 && p.hg % r == 0) ? r : 1;
}

template <typename QkvT, int D, int VPW>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kPrepWaves<QkvT>))) void chunk_prep_kernel(PrefillParams p, ChunkWs ws) {
  constexpr bool SPLIT = std::is_same<QkvT, float>::value;
  static_assert(VPW >= 1 && VPW <= kMaxVpw && (VPW == 1 || !SPLIT), "several value heads per workgroup only in the T form");
  constexpr int NKS = D / 32;      // 32-wide k steps over the head dim
  constexpr int NCT = D / 16;      // 16-column tiles of W (and of U)
  constexpr int TS = kChunk + 4;   // f32 row stride of A and T
  // the transposed K and V tiles feed W and U, which only f32 inputs form here
  __shared__ __attribute__((aligned(16))) _Float16 KTh[SPLIT ? D * KTS : 8];
  __shared__ __attribute__((aligned(16))) _Float16 VTh[SPLIT ? D * KTS : 8];
  __shared__ __attribute__((aligned(16))) _Float16 KTl[SPLIT ? D * KTS : 8];
  __shared__ __attribute__((aligned(16))) _Float16 VTl[SPLIT ? D * KTS : 8];
  __shared__ __attribute__((aligned(16))) float As[kChunk * TS];
  __shared__ __attribute__((aligned(16))) float Ts[kChunk * TS];
  __shared__ float Ms[4 * 16 * 17];
  __shared__ double Gs[VPW][kChunk];
  __shared__ __attribute__((aligned(16))) float bs[VPW][kChunk];
  __shared__ float bg[kChunk], kn[kChunk];

  // value heads hv0 .. hv0 + VPW - 1 of one key head (VPW > 1 only with bf16
  // q/k/v, where nothing below depends on V); a trip count fixed at compile
  // time keeps the per-head pointers out of long-lived scalar registers
  constexpr int vpw = VPW;
  const int cid = blockIdx.x, hv0 = p.h0 + (int)blockIdx.y * vpw;
  const int h = hv0;
  const int kh = h / (p.Hv / p.Hk);
  const int seq = ws.single ? 0 : ws.chunk_seq[cid];
  const int64_t t0 = ws.single ? (int64_t)kChunk * cid : ws.chunk_start[cid];
  const int n = (int)min((int64_t)kChunk, (int64_t)p.cu[seq + 1] - t0);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6), li = lane & 15, lg = lane >> 4;  // wave index in a scalar register
  // the block of value head hv0 + v
  auto block_of = [&](int v) { return ws.blocks + ((int64_t)cid * p.hg + (hv0 - p.h0 + v)) * blk_bytes(D); };
  char* blk = block_of(0);
  _Float16* Wh = reinterpret_cast<_Float16*>(blk + blk_w_hi(D));
  _Float16* Wl = reinterpret_cast<_Float16*>(blk + blk_w_lo(D));
  float* UTg = reinterpret_cast<float*>(blk + blk_ut(D));

  const int64_t qk_stride = (int64_t)p.Hk * D, v_stride = (int64_t)p.Hv * D;
  const QkvT* kp = static_cast<const QkvT*>(p.k) + (t0 * p.Hk + kh) * D;
  const QkvT* qp = static_cast<const QkvT*>(p.q) + (t0 * p.Hk + kh) * D;
  const QkvT* vp = static_cast<const QkvT*>(p.v) + (t0 * p.Hv + h) * D;

  // All loads first.  With bf16 inputs the chunk's K and Q rows are read
  // whole (contiguous 16-byte vectors) into row-major LDS tiles that borrow
  // the T and A buffers (not yet in use); the K and Q row fragments, and the
  // K rows and q fragments the scan reads, are formed from there.  With f32
  // inputs the K and V tiles are read in the transposed pattern and the
  // fragments straight from memory.  Then the gates.
  constexpr bool STAGE = !SPLIT;
  constexpr int RS = D + 8;  // row stride (elements) of the staged rows
  static_assert(!STAGE || kChunk * RS * 2 <= kChunk * TS * 4, "staged rows fit the A / T buffers");
  QkvT* Ks = reinterpret_cast<QkvT*>(Ts);
  QkvT* Qs = reinterpret_cast<QkvT*>(As);  // the Q rows, read before A is formed
  TransposedTile<QkvT, D> ktile, vtile;
  Raw8<QkvT> kf[4][NKS], qf[NKS];
  if constexpr (STAGE) {
    constexpr int VPR = D / 8, NV = kChunk * VPR / 256;
    u32x4 kr[NV], qr[NV];
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + 256 * j, r = v / VPR, c = v % VPR, rr = min(r, n - 1);
      kr[j] = *reinterpret_cast<const u32x4*>(kp + rr * qk_stride + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + 256 * j, r = v / VPR, c = v % VPR, rr = min(r, n - 1);
      qr[j] = *reinterpret_cast<const u32x4*>(qp + rr * qk_stride + 8 * c);
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + 256 * j, r = v / VPR, c = v % VPR;
      *reinterpret_cast<u32x4*>(Ks + r * RS + 8 * c) = kr[j];
    }
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + 256 * j, r = v / VPR, c = v % VPR;
      *reinterpret_cast<u32x4*>(Qs + r * RS + 8 * c) = qr[j];
    }
  } else {
    ktile.load(kp, qk_stride, n);
    vtile.load(vp, v_stride, n);
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J > wave) break;
      const int rr = min(16 * J + li, n - 1);
#pragma unroll
      for (int s = 0; s < NKS; ++s) kf[J][s].load(kp + rr * qk_stride + 32 * s + 8 * lg);
    }
  }
  if constexpr (!STAGE) {
    const int rr = min(16 * wave + li, n - 1);
#pragma unroll
    for (int s = 0; s < NKS; ++s) qf[s].load(qp + rr * qk_stride + 32 * s + 8 * lg);
  }
  const int gt = min(lane, n - 1);
  // the gates of the value head whose scan this wave runs (wave v: head
  // hv0 + v); a decay factor exp(g) below e^-200 is exactly zero in f32; the
  // clamp keeps the running sums finite when g = -inf
  const int gv = wave < vpw ? wave : 0;
  const float graw = fmaxf(p.g[(t0 + gt) * p.Hv + hv0 + gv], -200.0f);
  const float braw = p.beta[(t0 + gt) * p.Hv + hv0 + gv];
  if constexpr (STAGE) {
    __syncthreads();
    // this wave's own K rows (rows past the end hold the last row again, their
    // scale is 0); the other blocks' rows are read from LDS where they are used
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      kf[0][s].load(Ks + (16 * wave + li) * RS + 32 * s + 8 * lg);
      qf[s].load(Qs + (16 * wave + li) * RS + 32 * s + 8 * lg);
    }
  }

  // row scales of this wave's block: 1/sqrt(|row|^2 + 1e-6) with the L2 norm, else 1; zero past the end
  const int row = 16 * wave + li;
  float ksc, qsc;
  {
    float sk = 0.0f, sq = 0.0f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      float xq[8];
      qf[s].get(xq);
#pragma unroll
      for (int i = 0; i < 8; ++i) sq += xq[i] * xq[i];
    }
    // K rows of this block are kf[wave] (kf[0] with staged rows)
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J != (STAGE ? 0 : wave)) continue;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        float xk[8];
        kf[J][s].get(xk);
#pragma unroll
        for (int i = 0; i < 8; ++i) sk += xk[i] * xk[i];
      }
    }
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    const bool valid = row < n;
    ksc = valid ? (p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f) : 0.0f;
    qsc = valid ? (p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) : 0.0f;
    if (lg == 0) {
      kn[row] = ksc;
#pragma unroll
      for (int v = 0; v < vpw; ++v) {
        float* kn_g = reinterpret_cast<float*>(block_of(v) + blk_vec(D)) + 2 * kChunk;
        kn_g[row] = ksc;
        kn_g[kChunk + row] = qsc;
      }
    }
  }
  if (wave < vpw) {  // the gates of value head hv0 + wave
    const bool valid = lane < n;
    double G = valid ? (double)graw : 0.0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(G, off, 64);
      if (lane >= off) G += o;
    }
    Gs[wave][lane] = G;
    const double Glast = __shfl(G, 63, 64);
    const float gam = expf((float)G);
    const float bt = valid ? braw : 0.0f;
    bs[wave][lane] = bt;
    if (wave == 0) bg[lane] = bt * gam;  // W form only (one value head)
    float* gam_g = reinterpret_cast<float*>(block_of(wave) + blk_vec(D));
    gam_g[lane] = gam;
    gam_g[kChunk + lane] = expf((float)(Glast - G));
  }
  __syncthreads();
  if constexpr (!STAGE) {
    ktile.store(KTh, KTl, kn, n);
    vtile.store(VTh, VTl, nullptr, n);
  }

  // (K_J K_w^T) and (K_J Q_w^T): lane holds row i = 16w + li, columns j =
  // 16J + 4lg + r; they depend on the key head only and are kept for every
  // value head's A and P
  f32x4 akks[4], aqks[4];
  {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      akks[J] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      aqks[J] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      if (J > wave) continue;
      const float sj = kn[16 * J + li];  // scale of the K row this lane feeds as operand A
      f32x4 akk = {0.0f, 0.0f, 0.0f, 0.0f}, aqk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        float a[8], bk[8], bq[8];
        if constexpr (STAGE) {
          Raw8<QkvT> kj;
          kj.load(Ks + (16 * J + li) * RS + 32 * s + 8 * lg);
          kj.get(a);
          kf[0][s].get(bk);
        } else {
          kf[J][s].get(a);
#pragma unroll
          for (int J2 = 0; J2 < 4; ++J2)
            if (J2 == wave) kf[J2][s].get(bk);
        }
        qf[s].get(bq);
        if constexpr (SPLIT) {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            a[e] *= sj;
            bk[e] *= ksc;
            bq[e] *= qsc;
          }
          h8 ah, al, kh8, kl8, qh8, ql8;
          split8(a, ah, al);
          split8(bk, kh8, kl8);
          split8(bq, qh8, ql8);
          akk = mfma_f16(ah, kh8, akk);
          akk = mfma_f16(ah, kl8, akk);
          akk = mfma_f16(al, kh8, akk);
          aqk = mfma_f16(ah, qh8, aqk);
          aqk = mfma_f16(ah, ql8, aqk);
          aqk = mfma_f16(al, qh8, aqk);
        } else {
          // bf16 rows are exact in f16; the row scales go on the f32 products
          const h8 ah = to_h8(a);
          akk = mfma_f16(ah, to_h8(bk), akk);
          aqk = mfma_f16(ah, to_h8(bq), aqk);
        }
      }
      if constexpr (!SPLIT) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sk = kn[16 * J + 4 * lg + r];
          akk[r] *= ksc * sk;
          aqk[r] *= qsc * sk;
        }
      }
      akks[J] = akk;
      aqks[J] = aqk;
    }
  }
  // A and P of value head hv0 + v: A into LDS for the inverse, P to the block
  auto form_a_p = [&](int v) {
    const int i = row;
    const double Gi = Gs[v][i];
    const float bi = bs[v][i];
    char* bv = block_of(v);
    _Float16* Ph = reinterpret_cast<_Float16*>(bv + blk_p_hi(D));
    _Float16* Pl = reinterpret_cast<_Float16*>(bv + blk_p_lo(D));
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      float av[4], pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int j = 16 * J + 4 * lg + r;
        // the hardware exponential: its relative error (about 1e-7 times
        // the exponent's magnitude) is that of rounding the f64 difference
        const float dec = (J <= wave && j <= i) ? fast_exp((float)(Gi - Gs[v][j])) : 0.0f;
        av[r] = (J <= wave && j < i) ? bi * dec * akks[J][r] : 0.0f;
        pv[r] = (J <= wave && j <= i) ? p.scale * dec * aqks[J][r] : 0.0f;
      }
      if (J <= wave) *reinterpret_cast<float4*>(As + i * TS + 16 * J + 4 * lg) = make_float4(av[0], av[1], av[2], av[3]);
      if constexpr (SPLIT)
        store_h4_split(Ph + p_frag(wave, li, J, lg), Pl + p_frag(wave, li, J, lg), pv);
      else
        store_h4(Ph + p_frag(wave, li, J, lg), pv);
    }
  };
  if constexpr (SPLIT) form_a_p(0);
  __syncthreads();
  // K^T and the K rows depend on the key head only: the first value head of
  // the key head in this launch writes them, and the scan reads them from
  // that head's block
  if (STAGE && (vpw > 1 || h == kv_first(p, h))) {
    // T form: the K rows for the scan, each group of 32 columns in the
    // contraction order (position 8b + 4a + c holds column 16a + 4b + c), in
    // the K^T lo slot (unused with bf16 q/k/v).  f16 holds bf16 rows
    // exactly, so the rows stay unscaled (the scan applies the k scale, which
    // is zero past the end, to E and to K S0^T).  The scan reads the K^T
    // tiles of the state update from these rows with transposing LDS reads.
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int v = tid + 256 * j, r = v / (D / 8), c8 = v % (D / 8);
      h8 o;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int pos = 8 * c8 + e, w = pos & 31;
        const int col = (pos & ~31) + 16 * ((w >> 2) & 1) + 4 * (w >> 3) + (w & 3);
        o[e] = (_Float16)Elem<QkvT>::load(Ks + r * RS + col);
      }
      *reinterpret_cast<h8*>(blk + blk_kt_lo(D) + (r * D + 8 * c8) * 2) = o;
    }
    // the q rows as the scan's MFMA fragments (f16, exact for bf16), in the
    // K^T hi slot: for token block I and k step s a 1 KiB run in which lane
    // (li, lg) holds row 16 I + li at the contraction positions 32 s + 8 lg
    // .. +7, i.e. columns 32 s + 4 lg .. +3 and 32 s + 16 + 4 lg .. +3
    // (unscaled: the scan applies the q row scale, zero past the end)
#pragma unroll
    for (int j = 0; j < D / 32; ++j) {
      const int f = tid + 256 * j, I = f / (NKS * 64), s = (f / 64) % NKS, ln = f % 64;
      const int rq = 16 * I + (ln & 15), c0 = 32 * s + 4 * (ln >> 4);
      float a[4], b[4];
      load4(Qs + rq * RS + c0, a);
      load4(Qs + rq * RS + c0 + 16, b);
      h8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = (_Float16)a[e];
        o[4 + e] = (_Float16)b[e];
      }
      *reinterpret_cast<h8*>(blk + blk_kt_hi(D) + f * 16) = o;
    }
  }
  if constexpr (STAGE) __syncthreads();  // the staged rows live in Ts, which the inverse overwrites
  // f32 inputs: the scaled K^T tile for the scan, without the LDS row padding
#pragma unroll
  for (int j = 0; j < (STAGE ? 0 : D / 32); ++j) {
    const int v = tid + 256 * j, r = v >> 3, c8 = v & 7;
    *reinterpret_cast<uint4*>(blk + blk_kt_hi(D) + (r * kChunk + 8 * c8) * 2) =
        *reinterpret_cast<const uint4*>(KTh + r * KTS + 8 * c8);
    if constexpr (SPLIT)
      *reinterpret_cast<uint4*>(blk + blk_kt_lo(D) + (r * kChunk + 8 * c8) * 2) =
          *reinterpret_cast<const uint4*>(KTl + r * KTS + 8 * c8);
  }

  if constexpr (SPLIT) {
    unit_lower_inverse<TS>(As, Ts, Ms);
    w_u_products<SPLIT, SPLIT, TS, D>(Ts, bg, bs[0], KTh, KTl, VTh, VTl, Wh, Wl, UTg);
  } else {
    // per value head: A and P, T = (I + A)^-1, T diag(beta).  The barrier
    // after A also orders the last head's reads of T before this head's
    // inverse writes it.
#pragma unroll
    for (int v = 0; v < vpw; ++v) {
      form_a_p(v);
      __syncthreads();
      unit_lower_inverse<TS>(As, Ts, Ms);
      char* bv = block_of(v);
      store_t_beta<TS>(Ts, bs[v], reinterpret_cast<_Float16*>(bv + blk_tb_hi()), reinterpret_cast<_Float16*>(bv + blk_tb_lo()));
    }
  }
}

// ---------------------------------------------------------------------------
// 2b. per-chunk work of KDA (one log-decay per key channel)
// ---------------------------------------------------------------------------
// Within a chunk, with G_t[d] the log-decay of channel d summed from the
// chunk start through token t (vllm.cpp cpu_ops.cpp, KdaHeadTokenStep):
//   A[t][i] = beta_t sum_d k_t[d] k_i[d] exp(G_t[d] - G_i[d])   (i < t)
//   P[t][i] = scale sum_d q_t[d] k_i[d] exp(G_t[d] - G_i[d])    (i <= t)
//   W = T diag(beta) (K * exp(G)),  U = T diag(beta) V,  T = (I + A)^-1
//   O = (scale Q * exp(G)) S0^T + P Delta,  Delta = U - W S0^T
//   S_C = S0 diag(exp(G_C)) + Delta^T (K * exp(G_C - G))
// exp(G_t - G_i) is never formed as exp(G_t) exp(-G_i), which overflows once
// a channel decays strongly.  With rho_I the sum through the token before
// block I (16 tokens), for t in block I and i in an earlier block J
//   exp(G_t - G_i) = exp(G_t - rho_I) exp(rho_I - rho_{J+1}) exp(rho_{J+1} - G_i),
// three factors each at most 1, so the off-diagonal blocks are matrix
// products of scaled rows (f16 hi/lo MFMA); inside a diagonal block the
// factor is taken per pair.  The scan kernel runs unchanged on the result,
// given q * exp(G) in place of q, exp(G_C) per state column in place of the
// chunk's scalar decay, and 1 for every per-token decay it would apply.
//
// KDA block: the GDN block, then q * exp(G) rows [64][D] (f32 with f32 q/k/v,
// else f16), then exp(G_C) [D] f32.
template <typename QT>
__host__ __device__ constexpr int64_t blk_kda_q(int D) { return blk_bytes(D); }
template <typename QT>
__host__ __device__ constexpr int64_t blk_kda_gam(int D) { return blk_bytes(D) + (int64_t)kChunk * D * (int64_t)sizeof(QT); }
template <typename QT>
__host__ __device__ constexpr int64_t blk_kda_bytes(int D) { return align256(blk_kda_gam<QT>(D) + (int64_t)D * 4); }

template <typename QkvT>
using KdaQ = typename std::conditional<std::is_same<QkvT, float>::value, float, f16>::type;

constexpr double kLog2e = 1.4426950408889634;
// 2^x with the hardware exponential (about 1 ulp; 0 far below the f32 range)
__device__ __forceinline__ float exp2_f(float x) { return __builtin_amdgcn_exp2f(x); }

template <typename QkvT, int D>
__global__ __launch_bounds__(512) void kda_prep_kernel(KdaParams p, ChunkWs ws) {
  constexpr int NW = 8;                 // waves: 0-3 own token blocks, 4-7 help
  constexpr bool SPLIT = std::is_same<QkvT, float>::value;
  using QT = KdaQ<QkvT>;
  constexpr int NKS = D / 32;
  constexpr int TS = kChunk + 4;        // f32 row stride of A and T
  constexpr int GS = D + 4;             // f32 row stride of the log-decay rows
  constexpr int CPL = D / 4;            // channels per lane in the diagonal blocks
  static_assert(kChunk * GS <= 2 * kChunk * TS, "decay rows fit the A and T buffers");
  __shared__ __attribute__((aligned(16))) float GA[2 * kChunk * TS];  // Gb rows, later A then T
  __shared__ __attribute__((aligned(16))) _Float16 KTh[D * KTS];     // (k exp(G))^T hi
  __shared__ __attribute__((aligned(16))) _Float16 KTl[D * KTS];     // and lo
  __shared__ __attribute__((aligned(16))) _Float16 VTh[D * KTS];
  __shared__ __attribute__((aligned(16))) _Float16 VTl[SPLIT ? D * KTS : 8];
  __shared__ float Ms[4 * 16 * 17];
  __shared__ float Px[4 * 16 * 17];     // exact same-sub-block entries of P (those of A go to Ms)
  __shared__ __attribute__((aligned(16))) float Bk[4][D];   // block totals (rho_{J+1} - rho_J) log2(e)
  __shared__ __attribute__((aligned(16))) float Er[4][D];   // exp(rho_I)
  __shared__ __attribute__((aligned(16))) float Ec[4][D];   // exp(rho_4 - rho_{I+1})
  __shared__ __attribute__((aligned(16))) float Em[3][D];   // exp(rho_I - rho_{J+1}): (2,0), (3,1), (3,0)
  __shared__ float bs[kChunk], kn[kChunk], qn[kChunk];
  __shared__ double Bt[4][D];           // per-channel block totals of the log-decays
  // with bf16 q/k/v the chunk's K and Q rows are staged once (the diagonal
  // blocks and the element-wise tiles read them many times)
  constexpr bool STAGE = !SPLIT;
  constexpr int RS = D + 8;              // row stride (elements) of the staged rows
  __shared__ __attribute__((aligned(16))) QkvT Ks[STAGE ? kChunk * RS : 8];
  __shared__ __attribute__((aligned(16))) QkvT Qs[STAGE ? kChunk * RS : 8];
  // [64][GS]: the log-decays, then (G_t - rho_{I(t)}) log2(e): in base 2 every
  // decay factor below is one exp2
  float* Gb = GA;
  float* As = GA;
  float* Ts = GA + kChunk * TS;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int64_t qk_stride = (int64_t)p.Hk * D, v_stride = (int64_t)p.Hv * D;
  constexpr int VPR = D / 8, NV = STAGE ? (kChunk * VPR + 64 * NW - 1) / (64 * NW) : 1;
  constexpr int NG = (kChunk * (D / 4) + 64 * NW - 1) / (64 * NW);
  static_assert((64 * NW) % (D / 4) == 0, "a thread's channels are the same for each item");

  // The workgroups are persistent: each takes the items (chunk, value head)
  // blockIdx.x, + gridDim.x, ... (chunks of a head consecutive), one
  // workgroup to a CU (the LDS).  The loads that feed an item's staging are
  // issued as soon as the item before it is staged, so that they are in
  // flight during that item's work: the V tile, beta, the raw K and Q rows,
  // the raw log-decays (4 channels each) and the channels' dt bias.
  struct Item {
    int cid, h, kh, n;
    int64_t t0;
  };
  auto item_of = [&](int it) {
    Item I;
    I.cid = it % p.num_chunks;
    I.h = it / p.num_chunks;
    I.kh = I.h / (p.Hv / p.Hk);
    const int seq = ws.single ? 0 : ws.chunk_seq[I.cid];
    I.t0 = ws.single ? (int64_t)kChunk * I.cid : ws.chunk_start[I.cid];
    I.n = (int)min((int64_t)kChunk, (int64_t)p.cu[seq + 1] - I.t0);
    return I;
  };
  TransposedTile<QkvT, D, NW> vtile;
  u32x4 krow[NV], qrow[NV];
  float4 raw[NG], bias;
  float braw;
  auto issue = [&](const Item& I, int tid) {
    const QkvT* kq = static_cast<const QkvT*>(p.k) + (I.t0 * p.Hk + I.kh) * D;
    const QkvT* qq = static_cast<const QkvT*>(p.q) + (I.t0 * p.Hk + I.kh) * D;
    vtile.load(static_cast<const QkvT*>(p.v) + (I.t0 * p.Hv + I.h) * D, v_stride, I.n);
    braw = tid < kChunk ? p.beta[(I.t0 + min(tid, I.n - 1)) * p.Hv + I.h] : 0.0f;
    if constexpr (STAGE) {
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int v = min(tid + 64 * NW * j, kChunk * VPR - 1), r = v / VPR, c = v % VPR, rr = min(r, I.n - 1);
        krow[j] = *reinterpret_cast<const u32x4*>(kq + rr * qk_stride + 8 * c);
        qrow[j] = *reinterpret_cast<const u32x4*>(qq + rr * qk_stride + 8 * c);
      }
    }
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int v = min(tid + 64 * NW * j, kChunk * (D / 4) - 1), t = v / (D / 4), c = 4 * (v % (D / 4));
      raw[j] = *reinterpret_cast<const float4*>(p.g + ((I.t0 + min(t, I.n - 1)) * p.Hv + I.h) * D + c);
    }
    bias = p.dt_bias ? *reinterpret_cast<const float4*>(p.dt_bias + (int64_t)I.h * D + 4 * (tid % (D / 4)))
                     : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  };
  const int nitems = p.num_chunks * p.Hv;
  Item nxt = item_of(blockIdx.x);
  issue(nxt, tid);
  for (int item = blockIdx.x; item < nitems; item += gridDim.x) {
  // the thread index made opaque to the compiler in each pass, so that the
  // many per-lane LDS offsets below are formed where they are used rather
  // than hoisted out of the loop and held in registers through it
  int tid_pass = (int)threadIdx.x;
  asm volatile("" : "+v"(tid_pass));
  const int tid = tid_pass, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const Item cur = nxt;
  const int cid = cur.cid, h = cur.h, kh = cur.kh, n = cur.n;
  const int64_t t0 = cur.t0;
  // the next item's chunk bounds (dependent loads), read while this one is staged
  const bool more = item + (int)gridDim.x < nitems;
  if (more) nxt = item_of(item + (int)gridDim.x);
  char* blk = ws.blocks + ((int64_t)cid * p.Hv + h) * blk_kda_bytes<QT>(D);
  _Float16* Wh = reinterpret_cast<_Float16*>(blk + blk_w_hi(D));
  _Float16* Wl = reinterpret_cast<_Float16*>(blk + blk_w_lo(D));
  _Float16* Ph = reinterpret_cast<_Float16*>(blk + blk_p_hi(D));
  _Float16* Pl = reinterpret_cast<_Float16*>(blk + blk_p_lo(D));
  _Float16* KBh = reinterpret_cast<_Float16*>(blk + blk_kt_hi(D));
  _Float16* KBl = reinterpret_cast<_Float16*>(blk + blk_kt_lo(D));
  float* UTg = reinterpret_cast<float*>(blk + blk_ut(D));
  float* vec_g = reinterpret_cast<float*>(blk + blk_vec(D));
  QT* Qg = reinterpret_cast<QT*>(blk + blk_kda_q<QT>(D));
  float* gam_g = reinterpret_cast<float*>(blk + blk_kda_gam<QT>(D));

  const QkvT* kp = static_cast<const QkvT*>(p.k) + (t0 * p.Hk + kh) * D;
  const QkvT* qp = static_cast<const QkvT*>(p.q) + (t0 * p.Hk + kh) * D;

  // Waves 0-3 (row waves) each own token block I = wave: its row scales,
  // its diagonal block of A and P.  Waves 4-7 (helpers) form the element-wise
  // tiles and the six off-diagonal blocks of A and P.  The W / U products run
  // on all eight.
  const bool roww = wave < 4;
  const int ht = tid - 256;             // helper thread index
  // ---- staging (the item before this one is done with the LDS)
  if (item != (int)blockIdx.x) __syncthreads();
  if (tid < kChunk) bs[tid] = tid < n ? braw : 0.0f;
  if constexpr (STAGE) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int v = tid + 64 * NW * j, r = v / VPR, c = v % VPR;
      if (v < kChunk * VPR) {
        *reinterpret_cast<u32x4*>(Ks + r * RS + 8 * c) = krow[j];
        *reinterpret_cast<u32x4*>(Qs + r * RS + 8 * c) = qrow[j];
      }
    }
  }
  vtile.store(VTh, VTl, nullptr, n);
  // the chunk's log-decays, gate applied, all threads, 4 channels each
  {
    const float a = p.A_log ? -expf(p.A_log[h]) : 0.0f;
#pragma unroll
    for (int j = 0; j < NG; ++j) {
      const int v = tid + 64 * NW * j, t = v / (D / 4), c = 4 * (v % (D / 4));
      if (v >= kChunk * (D / 4)) break;
      float x[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
      const float bb[4] = {bias.x, bias.y, bias.z, bias.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        // gate: a softplus(x + bias), softplus(z) = ln(1 + u), u = e^z, by the
        // hardware exp2/log2 with the correction ln(1 + u) = ln(w) u / (w - 1),
        // w = 1 + u rounded, which keeps the relative accuracy for small u;
        // e^-200 and below is 0 in f32, and the clamp keeps the sums finite
        // for g = -inf
        float y = x[i];
        if (p.A_log) {
          const float z = y + bb[i];
          const float u = exp2_f(z * 1.44269504f), w = 1.0f + u;
          const float lp = w == 1.0f ? u : 0.69314718f * __builtin_amdgcn_logf(w) * (u / (w - 1.0f));
          y = a * (z > 20.0f ? z : lp);
        }
        x[i] = t < n ? fmaxf(y, -200.0f) : 0.0f;
      }
      *reinterpret_cast<float4*>(Gb + t * GS + c) = make_float4(x[0], x[1], x[2], x[3]);
    }
  }
  __syncthreads();

  // the K / Q fragments of a row wave's own block
  Raw8<QkvT> kfo[NKS], qf[NKS];
  {
    const int r = 16 * (wave & 3) + li, rr = min(r, n - 1);
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if constexpr (STAGE) {
        kfo[s].load(Ks + r * RS + 32 * s + 8 * lg);
        qf[s].load(Qs + r * RS + 32 * s + 8 * lg);
      } else {
        kfo[s].load(kp + rr * qk_stride + 32 * s + 8 * lg);
        qf[s].load(qp + rr * qk_stride + 32 * s + 8 * lg);
      }
    }
  }

  // ---- per-channel running sums (f64), one thread per (channel, token
  // block), in place: the sums within the block, then the block totals
  const int sd = tid % D, sI = tid / D;
  if (sI < 4) {
    double G = 0.0;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int t = 16 * sI + j;
      G += (double)Gb[t * GS + sd];
      Gb[t * GS + sd] = (float)(G * kLog2e);
    }
    Bt[sI][sd] = G;
  }
  __syncthreads();
  if (sI < 4) {
    double rho[5];
    rho[0] = 0.0;
#pragma unroll
    for (int I = 0; I < 4; ++I) rho[I + 1] = rho[I] + Bt[I][sd];
    Bk[sI][sd] = (float)(Bt[sI][sd] * kLog2e);
    Er[sI][sd] = (float)exp(rho[sI]);
    Ec[sI][sd] = (float)exp(rho[4] - rho[sI + 1]);
    if (sI < 3)
      Em[sI][sd] = (float)exp(sI == 0 ? rho[2] - rho[1] : sI == 1 ? rho[3] - rho[2] : rho[3] - rho[1]);
    else
      gam_g[sd] = (float)exp(rho[4]);
  }

  // ---- row scales of a row wave's block (L2 norm, else 1; zero past the end)
  const int row = 16 * (wave & 3) + li;
  float ksc = 0.0f, qsc = 0.0f;
  if (roww) {
    float sk = 0.0f, sq = 0.0f;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      float xq[8], xk[8];
      qf[s].get(xq);
      kfo[s].get(xk);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        sq += xq[i] * xq[i];
        sk += xk[i] * xk[i];
      }
    }
    sk += __shfl_xor(sk, 16, 64);
    sk += __shfl_xor(sk, 32, 64);
    sq += __shfl_xor(sq, 16, 64);
    sq += __shfl_xor(sq, 32, 64);
    const bool valid = row < n;
    ksc = valid ? (p.l2norm ? 1.0f / sqrtf(sk + 1e-6f) : 1.0f) : 0.0f;
    qsc = valid ? (p.l2norm ? 1.0f / sqrtf(sq + 1e-6f) : 1.0f) : 0.0f;
    if (lg == 0) {
      kn[row] = ksc;
      qn[row] = qsc;
      vec_g[row] = 1.0f;                 // gamma: the decays are folded into q * exp(G)
      vec_g[kChunk + row] = 1.0f;        // exp(G_C - G_j): folded into K^T
      vec_g[2 * kChunk + row] = 1.0f;    // k row scale (folded)
      vec_g[3 * kChunk + row] = valid ? 1.0f : 0.0f;  // q row scale (folded), zero past the end
    }
  }
  __syncthreads();

  // ---- element-wise tiles: (k exp(G))^T into LDS, (k exp(G_C - G))^T and
  // q exp(G) into the block.  Item (t, 8 channels), t fastest; V^T by all
  // eight waves, the rest by the helpers.
  for (int e_item = roww ? kChunk * (D / 8) : ht; e_item < kChunk * (D / 8); e_item += 256) {
    const int t = e_item & (kChunk - 1), c0 = 8 * (e_item / kChunk), I = t >> 4;
    const int rr = min(t, n - 1);
    Raw8<QkvT> kr, qr;
    if constexpr (STAGE) {
      kr.load(Ks + t * RS + c0);
      qr.load(Qs + t * RS + c0);
    } else {
      kr.load(kp + rr * qk_stride + c0);
      qr.load(qp + rr * qk_stride + c0);
    }
    float kx[8], qx[8];
    kr.get(kx);
    qr.get(qx);
    const float ks = kn[t], qs = qn[t];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int d = c0 + i;
      const float gb = Gb[t * GS + d];
      const float eg = exp2_f(gb) * Er[I][d];                    // exp(G_t)
      const float ec = exp2_f(Bk[I][d] - gb) * Ec[I][d];         // exp(G_C - G_t)
      const float kt = kx[i] * ks * eg, kb = kx[i] * ks * ec, qt = qx[i] * qs * eg;
      const _Float16 hi = (_Float16)kt, bh = (_Float16)kb;
      KTh[d * KTS + t] = hi;
      KTl[d * KTS + t] = (_Float16)(kt - (float)hi);
      KBh[d * kChunk + t] = bh;
      KBl[d * kChunk + t] = (_Float16)(kb - (float)bh);
      qx[i] = qt;
    }
    if constexpr (SPLIT) {
      *reinterpret_cast<float4*>(Qg + t * D + c0) = make_float4(qx[0], qx[1], qx[2], qx[3]);
      *reinterpret_cast<float4*>(Qg + t * D + c0 + 4) = make_float4(qx[4], qx[5], qx[6], qx[7]);
    } else {
      uint32_t w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)f32_to_f16(qx[2 * i]) | ((uint32_t)f32_to_f16(qx[2 * i + 1]) << 16);
      *reinterpret_cast<uint4*>(Qg + t * D + c0) = make_uint4(w[0], w[1], w[2], w[3]);
    }
  }

  // Rows of the chunk as MFMA fragments: lane (li, lg) of row r, k step s
  auto kfrag = [&](Raw8<QkvT>& f, int r, int s) {
    if constexpr (STAGE)
      f.load(Ks + r * RS + 32 * s + 8 * lg);
    else
      f.load(kp + min(r, n - 1) * qk_stride + 32 * s + 8 * lg);
  };
  auto qfrag = [&](Raw8<QkvT>& f, int r, int s) {
    if constexpr (STAGE)
      f.load(Qs + r * RS + 32 * s + 8 * lg);
    else
      f.load(qp + min(r, n - 1) * qk_stride + 32 * s + 8 * lg);
  };

  // ---- off-diagonal blocks (I, J), J < I, on the helpers: lane holds row
  // t = 16I + li, columns 16J + 4lg + r.  Helper 0 takes (3,2) and (1,0),
  // helper 1 (3,1) and (2,1), helper 2 (3,0), helper 3 (2,0).  A operand =
  // rows i of block J scaled by exp(rho_{J+1} - G_i) exp(rho_I - rho_{J+1}),
  // B operand = rows t scaled by exp(G_t - rho_I).
  float avh[2][4];
  int nblk = 0, bI[2] = {0, 0}, bJ[2] = {0, 0};
  if (!roww) {
    const int hw = wave - 4;
    nblk = hw < 2 ? 2 : 1;
    bI[0] = 3;
    bJ[0] = hw == 0 ? 2 : hw == 1 ? 1 : 0;
    if (hw == 3) bI[0] = 2;
    bI[1] = hw == 0 ? 1 : 2;
    bJ[1] = hw == 0 ? 0 : 1;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u >= nblk) break;
      const int I = bI[u], J = bJ[u];
      const int t = 16 * I + li;
      const float bt = bs[t], tk = kn[t], tq = qn[t];
      const int i = 16 * J + li;  // the A-operand row this lane feeds
      const float si = kn[i];
      const float* em = (I - J >= 2) ? Em[I == 2 ? 0 : (J == 1 ? 1 : 2)] : nullptr;
      f32x4 akk = {0.0f, 0.0f, 0.0f, 0.0f}, aqk = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        Raw8<QkvT> fa, fk, fq;
        kfrag(fa, i, s);
        kfrag(fk, t, s);
        qfrag(fq, t, s);
        float a[8], lk[8], lq[8];
        fa.get(a);
        fk.get(lk);
        fq.get(lq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 32 * s + 8 * lg + e;
          float f = exp2_f(Bk[J][d] - Gb[i * GS + d]);
          if (em) f *= em[d];
          a[e] *= si * f;
          const float ea = exp2_f(Gb[t * GS + d]);
          lk[e] *= tk * ea;
          lq[e] *= tq * ea;
        }
        h8 ah, al, kh8, kl8, qh8, ql8;
        split8(a, ah, al);
        split8(lk, kh8, kl8);
        split8(lq, qh8, ql8);
        akk = mfma_f16(ah, kh8, akk);
        akk = mfma_f16(ah, kl8, akk);
        akk = mfma_f16(al, kh8, akk);
        aqk = mfma_f16(ah, qh8, aqk);
        if constexpr (SPLIT) {
          aqk = mfma_f16(ah, ql8, aqk);
          aqk = mfma_f16(al, qh8, aqk);
        }
      }
      float pv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        avh[u][r] = bt * akk[r];
        pv[r] = p.scale * aqk[r];
      }
      if constexpr (SPLIT)
        store_h4_split(Ph + p_frag(I, li, J, lg), Pl + p_frag(I, li, J, lg), pv);
      else
        store_h4(Ph + p_frag(I, li, J, lg), pv);
    }
  }
  float avd[4];
  if (roww) {
    // diagonal block I = wave, in sub-blocks of 4 tokens.  With sigma_b the
    // running sum at the token before sub-block b, a pair in different
    // sub-blocks (i in b' < b, t in b) factors as
    //   exp(G_t - G_i) = exp(G_t - sigma_b) exp(sigma_b - G_i),  both <= 1,
    // so for each b one MFMA product of rows i < 4b (scaled by the second
    // factor) with the rows t of sub-block b (scaled by the first) gives those
    // entries, the other rows zeroed.  Pairs inside a sub-block are taken
    // exactly, one pair per lane.
    const float* gb_row = Gb + row * GS;
    f32x4 ck = {0.0f, 0.0f, 0.0f, 0.0f}, cq = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int b = 1; b < 4; ++b) {
      const bool rmask = li < 4 * b;        // this lane's row feeds the product as a row i
      const bool lmask = (li >> 2) == b;    // and as a row t
      const float* sig = Gb + (16 * wave + 4 * b - 1) * GS;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        float xk[8], xq[8], r8[8], l8[8], m8[8];
        kfo[s].get(xk);
        qf[s].get(xq);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 32 * s + 8 * lg + e;
          // exp2(min(x, 0)) and exp2(min(-x, 0)): one of the two is 1, the
          // other exp2(-|x|), so one exponential gives both
          const float x = gb_row[d] - sig[d];
          const float ex = exp2_f(-fabsf(x));
          const float fl = x <= 0.0f ? ex : 1.0f, fr = x >= 0.0f ? ex : 1.0f;
          r8[e] = rmask ? xk[e] * ksc * fr : 0.0f;
          l8[e] = lmask ? xk[e] * ksc * fl : 0.0f;
          m8[e] = lmask ? xq[e] * qsc * fl : 0.0f;
        }
        h8 rh, rl, lh, ll, mh, ml;
        split8(r8, rh, rl);
        split8(l8, lh, ll);
        split8(m8, mh, ml);
        ck = mfma_f16(rh, lh, ck);
        ck = mfma_f16(rh, ll, ck);
        ck = mfma_f16(rl, lh, ck);
        cq = mfma_f16(rh, mh, cq);
        if constexpr (SPLIT) {
          cq = mfma_f16(rh, ml, cq);
          cq = mfma_f16(rl, mh, cq);
        }
      }
    }
    {
      // lane (b, tt, ii) = (lg, (li >> 2), li & 3): pair t = 4b + tt, i = 4b + ii
      const int tt = li >> 2, ii = li & 3;
      const int tl = 4 * lg + tt, il = 4 * lg + ii;
      const int t = 16 * wave + tl, i = 16 * wave + il;
      float sa = 0.0f, sp = 0.0f;
      if (ii <= tt) {
        const int rt = min(t, n - 1), ri = min(i, n - 1);
        float sa4[4] = {0.0f, 0.0f, 0.0f, 0.0f}, sp4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 4
        for (int c = 0; c < D; c += 4) {
          float kt4[4], ki4[4], qt4[4];
          if constexpr (STAGE) {
            load4(Ks + t * RS + c, kt4);
            load4(Ks + i * RS + c, ki4);
            load4(Qs + t * RS + c, qt4);
          } else {
            load4(kp + rt * qk_stride + c, kt4);
            load4(kp + ri * qk_stride + c, ki4);
            load4(qp + rt * qk_stride + c, qt4);
          }
          const float4 gt = *reinterpret_cast<const float4*>(Gb + t * GS + c);
          const float4 gi = *reinterpret_cast<const float4*>(Gb + i * GS + c);
          const float ex[4] = {gt.x - gi.x, gt.y - gi.y, gt.z - gi.z, gt.w - gi.w};
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float ke = ki4[j] * exp2_f(fminf(ex[j], 0.0f));
            sa4[j] += kt4[j] * ke;
            sp4[j] += qt4[j] * ke;
          }
        }
        sa = (sa4[0] + sa4[1]) + (sa4[2] + sa4[3]);
        sp = (sp4[0] + sp4[1]) + (sp4[2] + sp4[3]);
      }
      Ms[wave * 272 + tl * 17 + il] = ii < tt ? bs[t] * kn[t] * kn[i] * sa : 0.0f;
      Px[wave * 272 + tl * 17 + il] = ii <= tt ? p.scale * qn[t] * kn[i] * sp : 0.0f;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // lane (li, lg) holds row t = 16 wave + li, columns 4 lg + r of the block
    const bool same = lg == (li >> 2);
    const float bt = bs[row];
    float pvd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      avd[r] = same ? Ms[wave * 272 + li * 17 + 4 * lg + r] : bt * ck[r];
      pvd[r] = same ? Px[wave * 272 + li * 17 + 4 * lg + r] : p.scale * cq[r];
    }
    // P fragments go straight to the block; blocks above the diagonal are zero
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J < wave) continue;
      float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      const float* v = J == wave ? pvd : z;
      if constexpr (SPLIT)
        store_h4_split(Ph + p_frag(wave, li, J, lg), Pl + p_frag(wave, li, J, lg), v);
      else
        store_h4(Ph + p_frag(wave, li, J, lg), v);
    }
  }
  __syncthreads();  // every read of the decay rows is done: A may overwrite them
  if (roww) {
#pragma unroll
    for (int J = 0; J < 4; ++J) {
      if (J < wave) continue;
      float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      const float* v = J == wave ? avd : z;
      *reinterpret_cast<float4*>(As + row * TS + 16 * J + 4 * lg) = make_float4(v[0], v[1], v[2], v[3]);
    }
  } else {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      if (u >= nblk) break;
      *reinterpret_cast<float4*>(As + (16 * bI[u] + li) * TS + 16 * bJ[u] + 4 * lg) =
          make_float4(avh[u][0], avh[u][1], avh[u][2], avh[u][3]);
    }
  }
  // the next item's loads, in flight during the inverse and the W / U
  // products (they hold no registers through the block products above)
  if (more) issue(nxt, tid);
  __syncthreads();
  unit_lower_inverse<TS>(As, Ts, Ms);
  w_u_products<true, SPLIT, TS, D, NW>(Ts, bs, bs, KTh, KTl, VTh, VTl, Wh, Wl, UTg);
  }
}

// ---------------------------------------------------------------------------
// 3. sequential pass over chunks
// ---------------------------------------------------------------------------
// Four consecutive input elements in their storage form (8 bytes for bf16,
// 16 for f32).
template <typename T>
struct Raw4 {
  static constexpr int kWords = (int)sizeof(T);  // 32-bit words holding four elements
  uint32_t w[kWords];
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (kWords == 2) {
      const uint2 v = *reinterpret_cast<const uint2*>(p);
      w[0] = v.x;
      w[1] = v.y;
    } else {
      const uint4 v = *reinterpret_cast<const uint4*>(p);
      w[0] = v.x;
      w[1] = v.y;
      w[2] = v.z;
      w[3] = v.w;
    }
  }
  __device__ __forceinline__ void get(float* o) const {
    if constexpr (kWords == 2) {
      float t[8];
      Elem<T>::unpack(make_uint4(w[0], w[1], 0u, 0u), t);
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = t[i];
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(w[i]);
    }
  }
};

// Four consecutive outputs in one store.
__device__ __forceinline__ void store4(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void store4(bf16* p, const float* v) {
  uint2 w;
  w.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
  w.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = w;
}

// One workgroup of 8 waves carries rows e0 .. e0+15 of one value head's
// state through the chunks of one sequence.
//
// Waves 0-3 (the state waves) run only the serial part.  Each holds the whole
// 16 x D block in registers as the MFMA B operand of S^T: lane (li, lg) holds
// row e0 + li at the columns
//   k(s, i) = 32 s + 16 (i / 4) + 4 lg + i % 4,   s < D/32, i < 8,
// so the contraction over k runs in this permuted order (W is stored so, Q is
// loaded so).  The order is chosen so that the state update, computed as its
// transpose S'^T = gamma_C S^T + K^T E one 16-column tile at a time, leaves
// tile ct in exactly the registers that hold columns 16 ct .. 16 ct + 15.  Per
// chunk a state wave splits the state into f16 hi/lo and publishes its share
// of the split to LDS, forms Delta = U - W S^T for its 16 tokens (three
// independent MFMA chains), writes Delta and E = diag(exp(G_C - G_j)) Delta
// to LDS, and after the barrier applies the whole update (every state wave
// the same; the matrix cores have room to spare).
//
// Waves 4-7 (the output waves) do all the loading: they stage the next
// chunk's W, U^T rows and decay factors (before the barrier) and K^T (after
// it) into LDS for the state waves, and after the barrier form O = diag(scale gamma) Q S^T + P Delta for
// 16 tokens each from the published state and Delta.  They form it
// transposed, O^T = S Q^T + Delta^T P^T (the same register fragments with the
// operand roles swapped), so each lane ends with four consecutive value rows
// of one token and stores them as one vector.  With f32 q/k/v the LDS holds
// no W; the state waves then load W themselves.
//
// One barrier per chunk.  Every LDS buffer is double-buffered by chunk parity
// and written and read in phases that a barrier separates.  Loads run one to
// two chunks ahead and are unconditional (the last chunk re-loads itself) so
// that none sits under a branch.  Sequences are never empty (the host rejects
// them), so every workgroup has a chunk.
// With KDA the block is a KDA block (kda_prep_kernel): q * exp(G) replaces q,
// exp(G_C) per state column replaces the chunk's scalar decay, and the K^T
// tile always has its lo half (it carries per-channel decays).
template <typename QkvT, typename StT, int D, bool KDA>
__global__ __launch_bounds__(512) void chunk_scan_kernel(PrefillParams p, ChunkWs ws) {
  constexpr bool SPLIT = std::is_same<QkvT, float>::value;
  constexpr bool KT_LO = SPLIT || KDA;  // K^T lo tiles
  // bf16 q/k/v (GDN): the block holds T diag(beta) rather than W and U^T
  // (T form); the state waves form Delta = T diag(beta) (V - diag(gamma) K S0^T)
  constexpr bool TF = !KT_LO;
  using QT = typename std::conditional<KDA, KdaQ<QkvT>, QkvT>::type;  // q rows as the scan reads them
  constexpr int NKS = D / 32;     // 32-wide k steps
  constexpr int NCT = D / 16;     // 16-column tiles of the state
  constexpr int WS = D + 8;       // f16 row stride of W and of the published state
  constexpr int KTV = D / 32;     // 16-byte K^T vectors per output-wave lane (per hi / lo)
  // K rows in LDS: D halves per row, the 16-byte units of row r XOR-permuted
  // by ((r & 3) << 2 | (r >> 2) & 3) (within the row's D / 8 units), which
  // keeps the row reads of K S0^T, the transposing reads of the update and
  // the staging writes free of bank conflicts without padding
  auto krow_at = [](int r, int unit) {
    return r * D + 8 * (unit ^ ((((r & 3) << 2) | ((r >> 2) & 3)) & (D / 8 - 1)));
  };
  // K^T [column][token]; the T form reads the update's K^T tiles from the K
  // rows instead, with transposing LDS reads
  __shared__ __attribute__((aligned(16))) _Float16 KTh[2][TF ? 8 : D * KTS];
  __shared__ __attribute__((aligned(16))) _Float16 KTl[2][KT_LO ? D * KTS : 8];
  __shared__ __attribute__((aligned(16))) _Float16 Krow[2][TF ? kChunk * D : 8];     // K rows, contraction order
  __shared__ __attribute__((aligned(16))) _Float16 DTh[2][16 * KTS];  // Delta^T [e][token]
  __shared__ __attribute__((aligned(16))) _Float16 DTl[2][SPLIT ? 16 * KTS : 8];
  __shared__ __attribute__((aligned(16))) _Float16 ETh[2][16 * KTS];  // (exp(G_C - G_j) Delta)^T
  __shared__ __attribute__((aligned(16))) _Float16 ETl[2][16 * KTS];
  __shared__ __attribute__((aligned(16))) _Float16 SSh[2][(SPLIT ? 2 : 1) * 16 * WS];  // state hi rows (then lo rows)
  __shared__ __attribute__((aligned(16))) float Us[2][TF ? 4 : 16 * 68];  // U^T rows e0 .. e0+15 (W form)
  __shared__ __attribute__((aligned(16))) uint16_t Vb[2][TF ? 16 * 68 : 8];  // T form: V^T rows e0 .. e0+15 (bf16)
  // T form: each state wave's Y (its 16 tokens, f16 hi then lo), per lane
  __shared__ __attribute__((aligned(16))) uint32_t Yx[TF ? 4 * 64 * 4 : 4];
  // exp(G_C - G_j), then gamma (T form: both times the k row scale, then gamma_C)
  __shared__ __attribute__((aligned(16))) float Vs[2][2 * kChunk + (TF ? 4 : 0)];
  // KDA: exp(G_C) per state column, three buffers by chunk: the output waves
  // stage chunk c+1's before the barrier of chunk c, while the state waves
  // may still read chunk c-1's in their update after the barrier of c-1
  __shared__ __attribute__((aligned(16))) float Gm[3][KDA ? D : 4];
  constexpr int QEV = 16 / (int)sizeof(QT);     // q elements per 16-byte vector
  constexpr int QVPR = D / QEV;                  // vectors per q row
  constexpr int NQV = 16 * QVPR / 64;            // vectors per lane for a wave's 16 rows
  constexpr int QS = D + QEV;                    // row stride (elements) of the staged rows
  // each output wave's 16 q rows (the T form reads q as MFMA fragments the prep wrote instead)
  __shared__ __attribute__((aligned(16))) QT Qsm[4][TF ? 8 : 16 * QS];

  // Workgroups are handed to the 8 XCDs round-robin by id.  Remap so that the
  // row blocks of one head, and the value heads of one key head, run on the
  // same XCD and share its L2 (they read the same W, P, K and Q blocks).
  const int nwg = (D / 16) * p.hg * p.N;
  const int per_xcd = (int)gridDim.x / 8;
  const int logical = ((int)blockIdx.x % 8) * per_xcd + (int)blockIdx.x / 8;
  if (logical >= nwg) return;
  const int e0 = 16 * (logical % (D / 16));
  const int hl = (logical / (D / 16)) % p.hg;  // head within this launch's group
  const int h = p.h0 + hl;
  const int s_idx = logical / ((D / 16) * p.hg);
  const int kh = h / (p.Hv / p.Hk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, lg = lane >> 4;
  const int w4 = wave & 3;
  const bool state_wave = wave < 4;
  const int slot = p.slots ? p.slots[s_idx] : s_idx;
  const bool has = p.has_init == nullptr || p.has_init[s_idx] != 0;
  const int64_t seq_start = p.cu[s_idx], seq_end = p.cu[s_idx + 1];
  const int64_t qk_stride = (int64_t)p.Hk * D;
  StT* Sg = static_cast<StT*>(p.ssm_pool) + (((int64_t)slot * p.Hv + h) * D + e0 + li) * D;
  const QkvT* qbase = static_cast<const QkvT*>(p.q) + (int64_t)kh * D;
  QkvT* obase = static_cast<QkvT*>(p.out) + (int64_t)h * D + e0;
  const int c_begin = ws.single ? 0 : ws.seq_chunk_off[s_idx];
  const int c_end = ws.single ? (int)((p.T + kChunk - 1) / kChunk) : ws.seq_chunk_off[s_idx + 1];
  constexpr int64_t kBlk = KDA ? blk_kda_bytes<QT>(D) : blk_bytes(D);
  auto blk_of = [&](int cid) { return ws.blocks + ((int64_t)cid * p.hg + hl) * kBlk; };
  // T form: the key head's K^T and K rows sit in the block of its first value head
  const int hk_blk = TF ? kv_first(p, h) - p.h0 : hl;
  auto kblk_of = [&](int cid) { return ws.blocks + ((int64_t)cid * p.hg + hk_blk) * kBlk; };
  if (c_begin == c_end) {
    // an empty sequence (KDA allows them): its final state is its initial
    // state, zero without one
    if (!has) {
      StT* S0 = static_cast<StT*>(p.ssm_pool) + (((int64_t)slot * p.Hv + h) * D + e0) * D;
      for (int e = tid; e < 16 * D; e += 512) Elem<StT>::store(S0 + e, 0.0f);
    }
    return;
  }
  auto tok0 = [&](int cid) { return seq_start + (int64_t)kChunk * (cid - c_begin); };
  auto ntok = [&](int cid) { return (int)min((int64_t)kChunk, seq_end - tok0(cid)); };

  // ---- state-wave operands
  float Sf[8 * NKS];
  // T form: this wave's T diag(beta) fragments (row block w4; hi then lo of
  // k steps 0 and 1), loaded a chunk ahead straight from the block
  u32x4 Tf[TF ? 4 : 1];
  auto load_tf = [&](int cid) {
    if constexpr (TF) {
      const auto rb = buf_rsrc(blk_of(cid), (uint32_t)kBlk);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t o = (uint32_t)(((2 * w4 + s2) * 64 + lane) * 16);
        Tf[2 * s2] = buf_ld16(rb, (uint32_t)blk_tb_hi() + o);
        Tf[2 * s2 + 1] = buf_ld16(rb, (uint32_t)blk_tb_lo() + o);
      }
    }
  };
  h8 Wgh[TF ? 1 : NKS], Wgl[TF ? 1 : NKS];  // W fragments (W form), straight from memory
  auto load_wg = [&](int cid) {
    if constexpr (!TF) {
      const char* b = blk_of(cid);
      const int row = 16 * w4 + li;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        Wgh[s] = ld_h8(reinterpret_cast<const _Float16*>(b + blk_w_hi(D)) + row * D + 32 * s + 8 * lg);
        Wgl[s] = ld_h8(reinterpret_cast<const _Float16*>(b + blk_w_lo(D)) + row * D + 32 * s + 8 * lg);
      }
    }
  };

  // ---- output-wave operands
  u32x4 Qraw[TF ? 1 : NQV];      // q rows 16 w4 .. 16 w4 + 15 of a chunk ahead, as stored
  h8 Qf[TF ? NKS : 1];           // T form: this chunk's q fragments (contraction order, f16)
  h8 Pfh[2], Pfl[SPLIT ? 2 : 1];
  float qsv, gmv;                // q row scale and gamma at token 16 w4 + li
  u32x4 KTr[KTV], KTrl[KT_LO ? KTV : 1];
  u32x4 Kr[TF ? KTV : 1];
  const int ot = tid - 256;      // output-wave thread index
  // a wave's q rows move whole 16-byte vectors (contiguous per row) and are
  // read back in the contraction order from its own LDS slice
  auto load_q = [&](int cid) {
    const int n = ntok(cid);
    const auto r16 = KDA ? buf_rsrc(blk_of(cid) + blk_kda_q<QT>(D), kChunk * D * (int)sizeof(QT))
                         : buf_rsrc(qbase + tok0(cid) * qk_stride, (uint32_t)(n * qk_stride * (int64_t)sizeof(QkvT)));
#pragma unroll
    for (int j = 0; j < NQV; ++j) {
      const int v = lane + 64 * j, r = v / QVPR, c = v % QVPR;
      const int rr = min(16 * w4 + r, n - 1);  // rows past the end re-read the last row; their scale is 0
      const int64_t el = KDA ? (int64_t)rr * D + c * QEV : rr * qk_stride + c * QEV;
      Qraw[j] = buf_ld16(r16, (uint32_t)(el * (int64_t)sizeof(QT)));
    }
  };
  // T form: the q fragments the prep wrote in the key head's block (K^T hi slot)
  auto load_qf = [&](int cid) {
    if constexpr (TF) {
      const auto rk = buf_rsrc(kblk_of(cid), (uint32_t)kBlk);
#pragma unroll
      for (int s = 0; s < NKS; ++s)
        Qf[s] = __builtin_bit_cast(h8, buf_ld16(rk, (uint32_t)(blk_kt_hi(D) + ((w4 * NKS + s) * 64 + lane) * 16)));
    }
  };
  auto stage_q = [&]() {
#pragma unroll
    for (int j = 0; j < NQV; ++j) {
      const int v = lane + 64 * j, r = v / QVPR, c = v % QVPR;
      *reinterpret_cast<u32x4*>(Qsm[w4] + r * QS + c * QEV) = Qraw[j];
    }
  };
  auto load_pv = [&](int cid) {
    const auto rb = buf_rsrc(blk_of(cid), (uint32_t)kBlk);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t o = (uint32_t)(((2 * w4 + s) * 64 + lane) * 16);
      Pfh[s] = __builtin_bit_cast(h8, buf_ld16(rb, (uint32_t)blk_p_hi(D) + o));
      if constexpr (SPLIT) Pfl[s] = __builtin_bit_cast(h8, buf_ld16(rb, (uint32_t)blk_p_lo(D) + o));
    }
    gmv = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(blk_vec(D) + 4 * (16 * w4 + li)), 0, 0));
    qsv = __uint_as_float(
        __builtin_amdgcn_raw_buffer_load_b32(rb, (uint32_t)(blk_vec(D) + 4 * (3 * kChunk + 16 * w4 + li)), 0, 0));
  };
  auto load_kt = [&](int cid) {
    const auto rk = buf_rsrc(kblk_of(cid), (uint32_t)kBlk);
#pragma unroll
    for (int j = 0; j < KTV; ++j) {
      const uint32_t o = (uint32_t)((ot + 256 * j) * 16);
      KTr[j] = buf_ld16(rk, (uint32_t)blk_kt_hi(D) + o);
      if constexpr (KT_LO) KTrl[j] = buf_ld16(rk, (uint32_t)blk_kt_lo(D) + o);
    }
  };
  auto stage_kt = [&](int bb) {
#pragma unroll
    for (int j = 0; j < KTV; ++j) {
      const int v = ot + 256 * j, r = v >> 3, c8 = v & 7;
      *reinterpret_cast<u32x4*>(KTh[bb] + r * KTS + 8 * c8) = KTr[j];
      if constexpr (KT_LO) *reinterpret_cast<u32x4*>(KTl[bb] + r * KTS + 8 * c8) = KTrl[j];
    }
  };
  // T form: the K rows in the contraction order
  auto load_kr = [&](int cid) {
    if constexpr (TF) {
      const auto rk = buf_rsrc(kblk_of(cid), (uint32_t)kBlk);
#pragma unroll
      for (int j = 0; j < KTV; ++j) Kr[j] = buf_ld16(rk, (uint32_t)(blk_kt_lo(D) + (ot + 256 * j) * 16));
    }
  };
  // U^T rows e0 .. e0+15 (one float4 per lane), exp(G_C - G_j) and gamma
  // (and with KDA exp(G_C) per column)
  float4 Ur, Vr, Gr, Kv;
  uint2 Vt;  // T form: four bf16 values of V, token ot / 4, rows e0 + 4 (ot % 4) .. +3
  auto load_uv = [&](int cid) {
    const auto rb = buf_rsrc(blk_of(cid), (uint32_t)kBlk);
    if constexpr (TF) {
      const int n = ntok(cid);
      const int tk = min(ot >> 2, n - 1);  // rows past the end re-read the last row (beta = 0 there)
      const int64_t vrow = (int64_t)p.Hv * D;
      const auto rv = buf_rsrc(static_cast<const QkvT*>(p.v) + tok0(cid) * vrow + (int64_t)h * D + e0,
                               (uint32_t)(((n - 1) * vrow + 16) * (int64_t)sizeof(QkvT)));
      Vt = buf_ld8(rv, (uint32_t)((tk * vrow + 4 * (ot & 3)) * (int64_t)sizeof(QkvT)));
    } else {
      Ur = __builtin_bit_cast(float4, buf_ld16(rb, (uint32_t)(blk_ut(D) + 4 * ((e0 + (ot >> 4)) * kChunk + 4 * (ot & 15)))));
    }
    Vr = __builtin_bit_cast(float4, buf_ld16(rb, (uint32_t)(blk_vec(D) + 4 * (ot < 16 ? kChunk + 4 * ot : 4 * (ot & 15)))));
    if constexpr (TF) Kv = __builtin_bit_cast(float4, buf_ld16(rb, (uint32_t)(blk_vec(D) + 4 * (2 * kChunk + 4 * (ot & 15)))));
    if constexpr (KDA)
      Gr = __builtin_bit_cast(float4, buf_ld16(rb, (uint32_t)(blk_kda_gam<QT>(D) + 4 * (4 * (ot % (D / 4))))));
  };
  auto stage_uv = [&](int bb, int b3) {
    if constexpr (TF) {
      const int tk = ot >> 2, e = 4 * (ot & 3);
      Vb[bb][e * 68 + tk] = (uint16_t)(Vt.x & 0xffffu);
      Vb[bb][(e + 1) * 68 + tk] = (uint16_t)(Vt.x >> 16);
      Vb[bb][(e + 2) * 68 + tk] = (uint16_t)(Vt.y & 0xffffu);
      Vb[bb][(e + 3) * 68 + tk] = (uint16_t)(Vt.y >> 16);
    } else {
      *reinterpret_cast<float4*>(Us[bb] + (ot >> 4) * 68 + 4 * (ot & 15)) = Ur;
    }
    if constexpr (TF) {
      // K^T and the K rows are unscaled in the T form: the k row scale goes
      // on E (with exp(G_C - G_j)) and on K S0^T (with gamma)
      if (ot < 32)
        *reinterpret_cast<float4*>(Vs[bb] + 4 * ot) = make_float4(Vr.x * Kv.x, Vr.y * Kv.y, Vr.z * Kv.z, Vr.w * Kv.w);
      if (ot == 31) Vs[bb][2 * kChunk] = Vr.w;  // gamma_C
    } else {
      if (ot < 32) *reinterpret_cast<float4*>(Vs[bb] + 4 * ot) = Vr;
    }
    if constexpr (KDA)
      if (ot < D / 4) *reinterpret_cast<float4*>(Gm[b3] + 4 * ot) = Gr;
  };
  auto stage_kr = [&](int bb) {
    if constexpr (TF) {
#pragma unroll
      for (int j = 0; j < KTV; ++j) {
        const int v = ot + 256 * j, r = v / (D / 8), c8 = v % (D / 8);
        *reinterpret_cast<u32x4*>(Krow[bb] + krow_at(r, c8)) = Kr[j];
      }
    }
  };

  // k step w4 of the split state, published for the output waves' Q S0^T
  auto publish_split = [&](const h8* Sh, const h8* Sl, int bb) {
#pragma unroll
    for (int s = 0; s < NKS; ++s)
      if (s == w4) {
        *reinterpret_cast<h8*>(SSh[bb] + li * WS + 32 * s + 8 * lg) = Sh[s];
        if constexpr (SPLIT) *reinterpret_cast<h8*>(SSh[bb] + (16 + li) * WS + 32 * s + 8 * lg) = Sl[s];
      }
  };
  // T form: Y_J = V_J - diag(gamma) K_J S0^T for this wave's token block J =
  // w4, published (f16 hi/lo) for every state wave; then Delta = T diag(beta)
  // Y over the lower-triangular row block.  Lane (li, lg) holds tokens
  // 16 J + 4 lg + r of row li, and in the contraction order of T diag(beta)'s
  // columns the B operand of step s2 is the Y of blocks 2 s2 and 2 s2 + 1 at
  // this same lane.  Blocks past w4 meet zero columns of T diag(beta).
  // K S0^T, k step s (K rows from buffer bb against the state hi and lo)
  auto ks_step = [&](const h8& sh, const h8& sl, int bb, int s, f32x4& xh, f32x4& xl) {
    const h8 kf = ld_h8(Krow[bb] + krow_at(16 * w4 + li, 4 * s + lg));
    xh = mfma_f16(kf, sh, xh);
    xl = mfma_f16(kf, sl, xl);
  };
  // Y from K S0^T and V, gamma of buffer bb, split and published
  auto finish_y = [&](const f32x4& xh, const f32x4& xl, int bb) {
    const uint2 vv = *reinterpret_cast<const uint2*>(Vb[bb] + li * 68 + 16 * w4 + 4 * lg);
    const float vt[4] = {__uint_as_float(vv.x << 16), __uint_as_float(vv.x & 0xffff0000u),
                         __uint_as_float(vv.y << 16), __uint_as_float(vv.y & 0xffff0000u)};
    const float4 gm = *reinterpret_cast<const float4*>(Vs[bb] + kChunk + 16 * w4 + 4 * lg);
    const float g4[4] = {gm.x, gm.y, gm.z, gm.w};
    uint32_t hw[2], lw[2];
#pragma unroll
    for (int r2 = 0; r2 < 2; ++r2) {
      const float y0 = vt[2 * r2] - g4[2 * r2] * (xh[2 * r2] + xl[2 * r2]);
      const float y1 = vt[2 * r2 + 1] - g4[2 * r2 + 1] * (xh[2 * r2 + 1] + xl[2 * r2 + 1]);
      split2(y0, y1, hw[r2], lw[r2]);
    }
    *reinterpret_cast<u32x4*>(Yx + (w4 * 64 + lane) * 4) = u32x4{hw[0], hw[1], lw[0], lw[1]};
  };

  // ---- prologue
  if (state_wave) {
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      if (has) {
        load_n<StT, 4>(Sg + 32 * s + 4 * lg, Sf + 8 * s);
        load_n<StT, 4>(Sg + 32 * s + 16 + 4 * lg, Sf + 8 * s + 4);
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) Sf[8 * s + i] = 0.0f;
      }
    }
    load_wg(c_begin);
    load_tf(c_begin);
  } else {
    load_kr(c_begin);
    load_uv(c_begin);
    if constexpr (!TF) load_kt(c_begin);
    if constexpr (!TF) load_q(c_begin);
    stage_kr(0);
    stage_uv(0, 0);
    if constexpr (!TF) stage_kt(0);
    if constexpr (!TF) stage_q();
    // the loads in flight at the loop's head, issued in the order one pass of
    // the loop issues them, so that the waits the compiler places at the
    // head (which must hold for both ways in) wait for no more than the
    // loop's own order needs
    const int n1 = min(c_begin + 1, c_end - 1);
    load_uv(n1);
    load_kr(n1);
    load_pv(c_begin);
    if constexpr (TF)
      load_qf(c_begin);
    else
      load_q(n1);
    if constexpr (!TF) load_kt(n1);
  }
  __syncthreads();
  if (TF && state_wave) {
    // the first chunk's Y and split state
    h8 Sh[NKS], Sl[NKS];
    f32x4 xh = {0.0f, 0.0f, 0.0f, 0.0f}, xl = xh;
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      split8(Sf + 8 * s, Sh[s], Sl[s]);
      ks_step(Sh[s], Sl[s], 0, s, xh, xl);
    }
    publish_split(Sh, Sl, 0);
    finish_y(xh, xl, 0);
  }

  for (int cid = c_begin; cid < c_end; ++cid) {
    const int b = (cid - c_begin) & 1;
    const int cn = min(cid + 1, c_end - 1);
    if (state_wave) {
      h8 Sh[NKS], Sl[NKS];
      if constexpr (!TF) {
#pragma unroll
        for (int s = 0; s < NKS; ++s) split8(Sf + 8 * s, Sh[s], Sl[s]);
        publish_split(Sh, Sl, b);
      }
      // Delta rows of this wave's 16 tokens
      float dl[4];
      if constexpr (TF) {
        // Y of this chunk, and its split state for the output waves, were
        // published at the end of the previous chunk (or in the prologue)
        __syncthreads();  // every state wave's Y is published
        f32x4 dhh = {0.0f, 0.0f, 0.0f, 0.0f}, dhl = dhh, dlh = dhh;
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          if (2 * s2 > w4) break;
          const u32x4 y0 = *reinterpret_cast<const u32x4*>(Yx + ((2 * s2) * 64 + lane) * 4);
          const u32x4 y1 = *reinterpret_cast<const u32x4*>(Yx + ((2 * s2 + 1) * 64 + lane) * 4);
          const h8 yh = __builtin_bit_cast(h8, u32x4{y0.x, y0.y, y1.x, y1.y});
          const h8 yl = __builtin_bit_cast(h8, u32x4{y0.z, y0.w, y1.z, y1.w});
          const h8 th = __builtin_bit_cast(h8, Tf[2 * s2]);
          const h8 tl = __builtin_bit_cast(h8, Tf[2 * s2 + 1]);
          dhh = mfma_f16(th, yh, dhh);
          dhl = mfma_f16(th, yl, dhl);
          dlh = mfma_f16(tl, yh, dlh);
        }
        const f32x4 dd = dhh + (dhl + dlh);
        load_tf(cn);  // the next chunk's fragments; this chunk's are consumed
#pragma unroll
        for (int r = 0; r < 4; ++r) dl[r] = dd[r];
      } else {
        // U - W S0^T, three independent chains
        f32x4 ahh = {0.0f, 0.0f, 0.0f, 0.0f}, ahl = ahh, alh = ahh;
#pragma unroll
        for (int s = 0; s < NKS; ++s) {
          ahh = mfma_f16(Wgh[s], Sh[s], ahh);
          ahl = mfma_f16(Wgh[s], Sl[s], ahl);
          alh = mfma_f16(Wgl[s], Sh[s], alh);
        }
        const f32x4 acc = ahh + (ahl + alh);
        const float4 utv = *reinterpret_cast<const float4*>(Us[b] + li * 68 + 16 * w4 + 4 * lg);
        const float us[4] = {utv.x, utv.y, utv.z, utv.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) dl[r] = us[r] - acc[r];
      }
      const float4 dcv = *reinterpret_cast<const float4*>(Vs[b] + 16 * w4 + 4 * lg);
      const float gc = Vs[b][TF ? 2 * kChunk : 2 * kChunk - 1];
      const float dcs[4] = {dcv.x, dcv.y, dcv.z, dcv.w};
      load_wg(cn);
      {
        // Delta^T and E^T (f16 hi/lo), 4 consecutive tokens per lane
        uint32_t w[4][2];
#pragma unroll
        for (int r2 = 0; r2 < 2; ++r2) {
          const float d0 = dl[2 * r2], d1 = dl[2 * r2 + 1];
          if constexpr (SPLIT) {
            split2(d0, d1, w[0][r2], w[1][r2]);
          } else {
            w[0][r2] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)d0) |
                       ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)d1) << 16);
          }
          split2(d0 * dcs[2 * r2], d1 * dcs[2 * r2 + 1], w[2][r2], w[3][r2]);
        }
        const int off = li * KTS + 16 * w4 + 4 * lg;
        *reinterpret_cast<uint2*>(DTh[b] + off) = make_uint2(w[0][0], w[0][1]);
        if constexpr (SPLIT) *reinterpret_cast<uint2*>(DTl[b] + off) = make_uint2(w[1][0], w[1][1]);
        *reinterpret_cast<uint2*>(ETh[b] + off) = make_uint2(w[2][0], w[2][1]);
        *reinterpret_cast<uint2*>(ETl[b] + off) = make_uint2(w[3][0], w[3][1]);
      }
      __syncthreads();
      // S'^T = gamma_C S0^T + K^T E, tile ct = columns 16ct .. 16ct+15
      h8 eh[2], el[2];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        eh[s] = ld_h8(ETh[b] + li * KTS + 32 * s + 8 * lg);
        el[s] = ld_h8(ETl[b] + li * KTS + 32 * s + 8 * lg);
      }
      // T form: the next chunk's Y follows the update k step by k step: k
      // step s of the state is tiles 2s and 2s+1, split and multiplied into
      // K S^T as soon as both are updated, so the two chains overlap
      const bool next_y = TF && cid + 1 < c_end;
      f32x4 xh = {0.0f, 0.0f, 0.0f, 0.0f}, xl = xh;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        float* sc = Sf + 8 * (ct >> 1) + 4 * (ct & 1);
        f32x4 a2;
        if constexpr (KDA) {
          // this lane's four columns 16 ct + 4 lg .. +3 decay by exp(G_C) of each
          const float4 gv = *reinterpret_cast<const float4*>(Gm[(cid - c_begin) % 3] + 16 * ct + 4 * lg);
          a2 = f32x4{gv.x * sc[0], gv.y * sc[1], gv.z * sc[2], gv.w * sc[3]};
        } else {
          a2 = f32x4{gc * sc[0], gc * sc[1], gc * sc[2], gc * sc[3]};
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          h8 kk;
          if constexpr (TF) {
            // K^T rows 16 ct .. 16 ct + 15 at tokens 32 s + 8 lg .. +7 from
            // the K rows: in each 16-lane group a transposing read hands
            // lane 4a + c element c of the 8-byte reads of lanes a, a+4, a+8,
            // a+12, so lane li reads token 32 s + 8 lg + 4 h + li / 4 at the
            // four columns 16 ct + 4 (li % 4) .. +3, which sit together in
            // the contraction order
            const int kr = 32 * s + 8 * lg + (li >> 2), ku = 4 * (ct >> 1) + (li & 3);
            const uint2 k0 = lds_read_tr16(Krow[b] + krow_at(kr, ku) + 4 * (ct & 1));
            const uint2 k1 = lds_read_tr16(Krow[b] + krow_at(kr + 4, ku) + 4 * (ct & 1));
            kk = __builtin_bit_cast(h8, u32x4{k0.x, k0.y, k1.x, k1.y});
          } else {
            kk = ld_h8(KTh[b] + (16 * ct + li) * KTS + 32 * s + 8 * lg);
          }
          a2 = mfma_f16(kk, eh[s], a2);
          a2 = mfma_f16(kk, el[s], a2);
          if constexpr (KT_LO) a2 = mfma_f16(ld_h8(KTl[b] + (16 * ct + li) * KTS + 32 * s + 8 * lg), eh[s], a2);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = a2[r];
        if (next_y && (ct & 1)) {
          const int s = ct >> 1;
          split8(Sf + 8 * s, Sh[s], Sl[s]);
          ks_step(Sh[s], Sl[s], b ^ 1, s, xh, xl);
        }
      }
      if (next_y) {
        publish_split(Sh, Sl, b ^ 1);
        finish_y(xh, xl, b ^ 1);
      }
    } else {
      // next chunk's V^T (W form: U^T) and decay factors into the other
      // buffer, then start loading the one after
      stage_uv(b ^ 1, (cid - c_begin + 1) % 3);
      load_uv(min(cid + 2, c_end - 1));
      // T form: this is the barrier behind which the state waves publish Y
      // (and, before it, this chunk's split state), so Q S0^T runs while
      // they form Delta; a second barrier below publishes Delta.  Other
      // forms: the one barrier of the chunk.
      __syncthreads();
      // T form: the next chunk's K rows.  The state waves read the other
      // buffer's rows until their update of the previous chunk, which ends
      // before the barrier above; they read these after the next one.
      stage_kr(b ^ 1);
      load_kr(min(cid + 2, c_end - 1));
      // O of this chunk: diag(scale gamma) Q S0^T with Q's row scale, + P Delta
      f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f}, o2 = o;
#pragma unroll
      for (int s = 0; s < NKS; ++s) {
        const h8 sh = ld_h8(SSh[b] + li * WS + 32 * s + 8 * lg);
        if constexpr (TF) {
          o = mfma_f16(sh, Qf[s], o);
          continue;
        }
        Raw4<QT> qa, qb;
        qa.load(Qsm[w4] + li * QS + 32 * s + 4 * lg);
        qb.load(Qsm[w4] + li * QS + 32 * s + 16 + 4 * lg);
        float qx[8];
        qa.get(qx);
        qb.get(qx + 4);
        if constexpr (SPLIT) {
          const h8 sl = ld_h8(SSh[b] + (16 + li) * WS + 32 * s + 8 * lg);
          h8 qh, ql;
          split8(qx, qh, ql);
          o = mfma_f16(sh, qh, o);
          o2 = mfma_f16(sl, qh, o2);
          o2 = mfma_f16(sh, ql, o2);
        } else {
          o = mfma_f16(sh, to_h8(qx), o);
        }
      }
      o += o2;
      const float osc = qsv * p.scale * gmv;
#pragma unroll
      for (int r = 0; r < 4; ++r) o[r] *= osc;
      if constexpr (TF) __syncthreads();  // Delta is published
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s > (w4 >> 1)) break;
        const h8 dh = ld_h8(DTh[b] + li * KTS + 32 * s + 8 * lg);
        o = mfma_f16(dh, Pfh[s], o);
        if constexpr (SPLIT) {
          o = mfma_f16(ld_h8(DTl[b] + li * KTS + 32 * s + 8 * lg), Pfh[s], o);
          o = mfma_f16(dh, Pfl[s], o);
        }
      }
      // lane holds O[token 16 w4 + li][e0 + 4 lg + r], r = 0..3
      const int i = 16 * w4 + li;
      if (i < ntok(cid)) {
        const float vals[4] = {o[0], o[1], o[2], o[3]};
        store4(obase + (tok0(cid) + i) * (int64_t)p.Hv * D + 4 * lg, vals);
      }
      // next chunk's K^T and q rows; operands of the chunks ahead
      if constexpr (!TF) stage_kt(b ^ 1);
      if constexpr (!TF) stage_q();
      load_pv(cn);
      if constexpr (TF)
        load_qf(cn);
      else
        load_q(min(cid + 2, c_end - 1));
      if constexpr (!TF) load_kt(min(cid + 2, c_end - 1));
    }
  }
  if (wave == 0)
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      store_n<StT, 4>(Sg + 32 * s + 4 * lg, Sf + 8 * s);
      store_n<StT, 4>(Sg + 32 * s + 16 + 4 * lg, Sf + 8 * s + 4);
    }
}

// ---------------------------------------------------------------------------
// Token-sequential kernel (shapes the chunked kernels do not cover).
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
  if (!std::is_same<QkvT, float>::value && prep_vpw(p) == 2)
    chunk_prep_kernel<QkvT, D, std::is_same<QkvT, float>::value ? 1 : 2><<<dim3((unsigned)p.num_chunks, p.hg / 2), 256, 0, stream>>>(p, ws);
  else
    chunk_prep_kernel<QkvT, D, 1><<<dim3((unsigned)p.num_chunks, p.hg), 256, 0, stream>>>(p, ws);
  const int nwg = (D / 16) * p.hg * p.N;
  chunk_scan_kernel<QkvT, StT, D, false><<<(unsigned)((nwg + 7) / 8 * 8), 512, 0, stream>>>(p, ws);
  return hipGetLastError();
}

template <typename QkvT, typename StT>
hipError_t launch_typed(const PrefillParams& p, hipStream_t stream, bool build_table = true) {
  if (!chunked_dims(p.Dk, p.Dv)) return launch_seq<QkvT, StT>(p, stream);
  const ChunkWs ws = carve(p.workspace, p.N, p.T);
  if (!ws.single && build_table) chunk_table_kernel<<<1, 64, 0, stream>>>(p.cu, p.N, ws);
  switch (p.Dk) {
    case 32: return launch_chunked_d<QkvT, StT, 32>(p, ws, stream);
    case 64: return launch_chunked_d<QkvT, StT, 64>(p, ws, stream);
    default: return launch_chunked_d<QkvT, StT, 128>(p, ws, stream);
  }
}

template <typename QkvT>
hipError_t launch_state(const PrefillParams& p, hipStream_t stream, bool build_table = true) {
  switch (p.state) {
    case GDN_F32: return launch_typed<QkvT, float>(p, stream, build_table);
    case GDN_BF16: return launch_typed<QkvT, bf16>(p, stream, build_table);
    default: return launch_typed<QkvT, f16>(p, stream, build_table);
  }
}

// compute units of the current device, queried once per device (the size of
// a persistent grid)
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

// ---- KDA
template <typename QkvT, typename StT, int D>
hipError_t launch_kda_chunked_d(const KdaParams& p, const ChunkWs& ws, hipStream_t stream) {
  // persistent prep workgroups, one per CU (each holds 146 KB of LDS)
  const int64_t items = (int64_t)p.num_chunks * p.Hv;
  if (items > 0)
    kda_prep_kernel<QkvT, D><<<(unsigned)std::min<int64_t>(items, device_cus()), 512, 0, stream>>>(p, ws);
  // the scan reads what it needs of the layer through the GDN parameter block
  PrefillParams pp{};
  pp.Hk = p.Hk; pp.Hv = p.Hv; pp.Dk = p.Dk; pp.Dv = p.Dv; pp.N = p.N; pp.T = p.T; pp.cu = p.cu;
  pp.q = p.q; pp.k = p.k; pp.v = p.v; pp.beta = p.beta; pp.ssm_pool = p.ssm_pool; pp.num_slots = p.num_slots;
  pp.slots = p.slots; pp.has_init = p.has_init; pp.scale = p.scale; pp.l2norm = p.l2norm; pp.chunk = kChunk;
  pp.out = p.out; pp.workspace = p.workspace; pp.workspace_bytes = p.workspace_bytes; pp.num_chunks = p.num_chunks;
  pp.max_chunks_per_seq = p.max_chunks_per_seq; pp.qkv = p.qkv; pp.state = p.state;
  pp.h0 = 0; pp.hg = p.Hv;
  const int nwg = (D / 16) * p.Hv * p.N;
  chunk_scan_kernel<QkvT, StT, D, true><<<(unsigned)((nwg + 7) / 8 * 8), 512, 0, stream>>>(pp, ws);
  return hipGetLastError();
}

template <typename QkvT, typename StT>
hipError_t launch_kda_typed(const KdaParams& p, hipStream_t stream) {
  const ChunkWs ws = carve(p.workspace, p.N, p.T);
  if (!ws.single) chunk_table_kernel<<<1, 64, 0, stream>>>(p.cu, p.N, ws);
  switch (p.Dk) {
    case 32: return launch_kda_chunked_d<QkvT, StT, 32>(p, ws, stream);
    case 64: return launch_kda_chunked_d<QkvT, StT, 64>(p, ws, stream);
    default: return launch_kda_chunked_d<QkvT, StT, 128>(p, ws, stream);
  }
}

template <typename QkvT>
hipError_t launch_kda_state(const KdaParams& p, hipStream_t stream) {
  switch (p.state) {
    case GDN_F32: return launch_kda_typed<QkvT, float>(p, stream);
    case GDN_BF16: return launch_kda_typed<QkvT, bf16>(p, stream);
    default: return launch_kda_typed<QkvT, f16>(p, stream);
  }
}

}  // namespace

size_t kda_prefill_workspace_bytes(int Hv, int Dk, int Dv, int N, int64_t T, gdn_dtype qkv) {
  if (N <= 0 || !chunked_dims(Dk, Dv)) return 0;
  const int64_t nc = max_chunks(N, T);
  const int64_t blk = qkv == GDN_F32 ? blk_kda_bytes<float>(Dk) : blk_kda_bytes<f16>(Dk);
  return align256((size_t)(N + 1) * 4) + 2 * align256((size_t)nc * 4) + (size_t)nc * Hv * blk;
}

bool kda_chunked_dims(int Dk, int Dv) { return chunked_dims(Dk, Dv); }

hipError_t launch_kda_prefill(const KdaParams& p, hipStream_t stream) {
  if (!chunked_dims(p.Dk, p.Dv)) return launch_kda_recurrent(p, stream);
  return p.qkv == GDN_F32 ? launch_kda_state<float>(p, stream) : launch_kda_state<bf16>(p, stream);
}

size_t prefill_workspace_bytes(int Hk, int Hv, int Dk, int Dv, int N, int64_t T, int chunk) {
  (void)Hk;
  (void)chunk;
  if (N <= 0 || T <= 0 || !chunked_dims(Dk, Dv)) return 0;
  const int64_t nc = max_chunks(N, T);
  return align256((size_t)(N + 1) * 4) + 2 * align256((size_t)nc * 4) + (size_t)nc * Hv * blk_bytes(Dk);
}

size_t prefill_workspace_bytes_per_head(int Dk, int Dv, int N, int64_t T) {
  return prefill_workspace_bytes(0, 1, Dk, Dv, N, T, kChunk);
}

hipError_t launch_prefill(const PrefillParams& p, hipStream_t stream) {
  PrefillParams q = p;
  q.h0 = 0;
  q.hg = p.Hv;
  return q.qkv == GDN_F32 ? launch_state<float>(q, stream) : launch_state<bf16>(q, stream);
}

// ---------------------------------------------------------------------------
// The prefill without allocation: a static scratch array in device memory.
// Its name is a host-side stand-in in host code; the device address comes
// from hipGetSymbolAddress, once per device, and only that address reaches
// the kernels.  Every call on a device shares the array (calls that overlap
// on one device race); the prefill needs no part of it cleared.
// ---------------------------------------------------------------------------
}  // namespace gdn

static __device__ __align__(256) char scratch[gdn::kNoAllocScratchBytes];

namespace gdn {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch address (resolved on its first use there).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_prefill_noalloc(const PrefillParams& p, hipStream_t stream) {
  void* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return e;
  PrefillParams q = p;
  q.workspace = base;
  q.workspace_bytes = kNoAllocScratchBytes;
  const size_t one = prefill_workspace_bytes_per_head(p.Dk, p.Dv, p.N, p.T);
  if (one == 0) {  // the token-sequential kernel: no scratch at all
    q.h0 = 0;
    q.hg = p.Hv;
    return q.qkv == GDN_F32 ? launch_state<float>(q, stream) : launch_state<bf16>(q, stream);
  }
  // value heads per launch: as many as the scratch holds, whole key-head
  // groups where more than one fits (they share the L2 of one XCD)
  const size_t table = one - (size_t)max_chunks(p.N, p.T) * blk_bytes(p.Dk);
  const size_t per_head = one - table;
  int hg = (int)std::min<size_t>((size_t)p.Hv, (kNoAllocScratchBytes - table) / per_head);
  const int r = p.Hv / p.Hk;
  if (hg >= r) hg -= hg % r;
  for (int h0 = 0; h0 < p.Hv; h0 += hg) {
    q.h0 = h0;
    q.hg = std::min(hg, p.Hv - h0);
    // the chunk table depends on the offsets only: built by the first launch
    e = q.qkv == GDN_F32 ? launch_state<float>(q, stream, h0 == 0) : launch_state<bf16>(q, stream, h0 == 0);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace gdn
