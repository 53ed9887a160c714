// h3q_device.hpp -- device-side building blocks shared by the gfx950 kernels of libh3q.
//
// NVFP4 decode (FL2VA Turbo, "Implementation": the packed 4-bit base): an E2M1 element times its
// E4M3 block scale is exactly representable in bf16 (at most 2 x 4 significant bits, exponent well
// inside bf16's range), so the kernels decode into bf16 tiles without rounding; the fp32 tensor
// scale is applied to the fp32 accumulator in the epilogue instead, where it costs one multiply.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace h3q {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------------------------
// Scalar conversions
// ---------------------------------------------------------------------------------------------

// fp32 -> bf16 bits, round to nearest even (NaN stays a quiet NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// E4M3 ("FN": bias 7, no inf, NaN = 0x7F) scale in byte SEL of w -> fp32. gfx950's
// v_cvt_f32_fp8 decodes the OCP E4M3FN variant (checked over all 256 codes against the format table).
template <int SEL>
__device__ __forceinline__ float e4m3_byte_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(w), SEL);
}

// Two bf16 (low half = a) from two fp32 whose low 16 bits are zero (exact bf16 values).
__device__ __forceinline__ uint32_t pack_exact_bf16x2(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}

// Eight E2M1 codes (one dword: element i in nibble i, low nibble first) times the block scale s ->
// eight bf16 in element order, two per dword. v_cvt_scalef32_pk_f32_fp4 with scale 1.0 yields the
// exact E2M1 values (its scale operand contributes only a power of two, so the E4M3 mantissa must
// be applied separately); the fp32 product with s is exact and its high half is the exact bf16.
__device__ __forceinline__ u32x4 nvfp4_dword_to_bf16x8(uint32_t cw, float s) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 0);
  const f32x2 v1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 1);
  const f32x2 v2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 2);
  const f32x2 v3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw, 1.0f, 3);
  u32x4 out;
  out.x = pack_exact_bf16x2(v0.x * s, v0.y * s);
  out.y = pack_exact_bf16x2(v1.x * s, v1.y * s);
  out.z = pack_exact_bf16x2(v2.x * s, v2.y * s);
  out.w = pack_exact_bf16x2(v3.x * s, v3.y * s);
  return out;
}

// ---------------------------------------------------------------------------------------------
// LDS tile geometry shared by the GEMM-shaped kernels: a tile is R rows of 64 bf16 (128 bytes);
// each row holds eight 16-byte chunks whose positions are XOR-swizzled by (row / 2) % 8 so that
// the 32 rows read by one 32x32x16 MFMA operand load spread over all LDS banks.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t lds_chunk_offset(uint32_t row, uint32_t chunk) {
  return row * 128u + ((chunk ^ ((row >> 1) & 7u)) << 4);
}

}  // namespace h3q
