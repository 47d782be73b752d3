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
// Two values into packed f16 halves: hi = f16(x) (round to nearest even) and
// lo = f16(x - hi), x0 in the low 16 bits of each word.  x - hi is exact in
// f32, so lo is the same as the plain-C form; the mixed-precision FMA forms
// it straight from the packed hi without converting hi back to f32 (three
// instructions per pair instead of about eight).
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
  const float m1 = -1.0f;
  asm("v_cvt_pk_f16_f32 %0, %2, %3\n\t"
      "v_fma_mixlo_f16 %1, %0, %4, %2 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mixhi_f16 %1, %0, %4, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "=&v"(hi), "=&v"(lo)
      : "v"(x0), "v"(x1), "v"(m1));
}
// x ~= hi + lo, both f16
__device__ __forceinline__ void split8(const float* x, h8& hi, h8& lo) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) split2(x[2 * i], x[2 * i + 1], hw[i], lw[i]);
  hi = __builtin_bit_cast(h8, u32x4{hw[0], hw[1], hw[2], hw[3]});
  lo = __builtin_bit_cast(h8, u32x4{lw[0], lw[1], lw[2], lw[3]});
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4a + c receives
// element c (a 16-bit value) of the 8-byte reads of lanes a, a + 4, a + 8 and
// a + 12 of its group, in that order.
typedef __fp16 fp16x4_lds __attribute__((__vector_size__(4 * sizeof(__fp16))));
__device__ __forceinline__ uint2 lds_read_tr16(const _Float16* p) {
  const fp16x4_lds v = __builtin_amdgcn_ds_read_tr16_b64_v4f16((__attribute__((address_space(3))) fp16x4_lds*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Buffer-resource loads: the base address sits in scalar registers and the
// per-lane byte offset in one 32-bit register, so a loop that moves only the
// base (chunk by chunk) keeps its offsets in registers.  Accesses at or past
// `bytes` from the base return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint2 buf_ld8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v[0], v[1]);
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
