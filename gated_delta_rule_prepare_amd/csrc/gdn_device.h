// gdn_device.h -- device-side helpers shared by the GDN kernels (gfx950,
// wave64): storage dtypes, 16-byte vector loads and stores, cross-lane sums.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

// Storage tags for the 16-bit formats; values are always handled as f32.
struct bf16 {
  uint16_t bits;
};
struct f16 {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// f32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint16_t b) {
  _Float16 h = __builtin_bit_cast(_Float16, b);
  return (float)h;
}

// f32 -> f16 with the hardware conversion (round to nearest even).
__device__ __forceinline__ uint16_t f32_to_f16(float f) {
  _Float16 h = (_Float16)f;
  return __builtin_bit_cast(uint16_t, h);
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
  static constexpr int kVec = 4;  // elements per 16 bytes
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float v) { *p = v; }
  __device__ __forceinline__ static void unpack(const uint4& r, float* o) {
    o[0] = __uint_as_float(r.x);
    o[1] = __uint_as_float(r.y);
    o[2] = __uint_as_float(r.z);
    o[3] = __uint_as_float(r.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* v) {
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
  }
};

template <typename Conv>
struct Elem16 {
  static constexpr int kVec = 8;
  __device__ __forceinline__ static void unpack(const uint4& r, float* o) {
    const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = Conv::to_f32((uint16_t)(w[i] & 0xffffu));
      o[2 * i + 1] = Conv::to_f32((uint16_t)(w[i] >> 16));
    }
  }
  __device__ __forceinline__ static uint4 pack(const float* v) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = (uint32_t)Conv::from_f32(v[2 * i]) | ((uint32_t)Conv::from_f32(v[2 * i + 1]) << 16);
    return make_uint4(w[0], w[1], w[2], w[3]);
  }
};

// Eight f32 -> bf16 with the gfx950 conversion instruction (two values per
// instruction, round to nearest even): finite values round exactly as
// f32_to_bf16 does; a NaN stays a NaN (its payload may differ).
__device__ __forceinline__ uint4 pack_bf16x8_hw(const float* v) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f32x2_t a = {v[2 * i], v[2 * i + 1]};
    w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_t));
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

struct BF16Conv {
  __device__ __forceinline__ static float to_f32(uint16_t b) { return bf16_to_f32(b); }
  __device__ __forceinline__ static uint16_t from_f32(float f) { return f32_to_bf16(f); }
};
struct F16Conv {
  __device__ __forceinline__ static float to_f32(uint16_t b) { return f16_to_f32(b); }
  __device__ __forceinline__ static uint16_t from_f32(float f) { return f32_to_f16(f); }
};

template <>
struct Elem<bf16> : Elem16<BF16Conv> {
  __device__ __forceinline__ static float load(const bf16* p) { return bf16_to_f32(p->bits); }
  __device__ __forceinline__ static void store(bf16* p, float v) { p->bits = f32_to_bf16(v); }
};

template <>
struct Elem<f16> : Elem16<F16Conv> {
  __device__ __forceinline__ static float load(const f16* p) { return f16_to_f32(p->bits); }
  __device__ __forceinline__ static void store(f16* p, float v) { p->bits = f32_to_f16(v); }
};

// Load / store kVec consecutive elements (16 bytes; p must be 16-byte aligned).
template <typename T>
__device__ __forceinline__ void load_vec(const T* p, float* o) {
  Elem<T>::unpack(*reinterpret_cast<const uint4*>(p), o);
}
template <typename T>
__device__ __forceinline__ void store_vec(T* p, const float* v) {
  *reinterpret_cast<uint4*>(p) = Elem<T>::pack(v);
}

// Load / store n (a multiple of 4 for f32, of 8 for 16-bit) consecutive elements.
template <typename T, int N>
__device__ __forceinline__ void load_n(const T* p, float* o) {
  constexpr int V = Elem<T>::kVec;
  static_assert(N % V == 0 || N < V, "width");
  if constexpr (N < V) {
#pragma unroll
    for (int i = 0; i < N; ++i) o[i] = Elem<T>::load(p + i);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += V) load_vec<T>(p + i, o + i);
  }
}
template <typename T, int N>
__device__ __forceinline__ void store_n(T* p, const float* v) {
  constexpr int V = Elem<T>::kVec;
  if constexpr (N < V) {
#pragma unroll
    for (int i = 0; i < N; ++i) Elem<T>::store(p + i, v[i]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += V) store_vec<T>(p + i, v + i);
  }
}

// Sum over aligned groups of W consecutive lanes (W a power of two <= 64).
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = W / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// e^x through the hardware base-2 exponential: relative error about 1e-7 * |x|
// (from rounding x*log2(e)), far inside the f32 tolerances used here.
__device__ __forceinline__ float fast_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.4426950408889634f); }
// 1/x with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float silu_f(float x) { return x * fast_rcp(1.0f + fast_exp(-x)); }
__device__ __forceinline__ float sigmoid_f(float x) { return fast_rcp(1.0f + fast_exp(-x)); }
// ln(1 + e^x); above 20 the identity is closer than f32 can tell.
__device__ __forceinline__ float softplus_f(float x) { return x > 20.0f ? x : log1pf(expf(x)); }

}  // namespace gdn
