// gdn_mfma.h -- f16 MFMA helpers shared by the chunked kernels (gfx950).
//
// 16x16x32 f16 layout (64 lanes, lane l = 16 g + i): A operand lane l holds
// A[i][8g .. 8g+7], B operand B[8g .. 8g+7][i], accumulator D[4g + r][i].
// An f32 value x enters as two f16 halves hi = f16(x), lo = f16(x - hi); a
// product of two such operands as hi*hi + hi*lo + lo*hi (f32 accumulation)
// carries about 22 significant bits.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(const h8& a, const h8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 to_h8(const float* x) {
  h8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)x[i];
  return r;
}
// x ~= hi + lo, both f16
__device__ __forceinline__ void split8(const float* x, h8& hi, h8& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const _Float16 h = (_Float16)x[i];
    hi[i] = h;
    lo[i] = (_Float16)(x[i] - (float)h);
  }
}
__device__ __forceinline__ h8 ld_h8(const _Float16* p) { return *reinterpret_cast<const h8*>(p); }
__device__ __forceinline__ h8 zero_h8() {
  h8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (_Float16)0.0f;
  return r;
}

}  // namespace
}  // namespace gdn
