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

// E4M3 ("FN", bias 7) scale code -> fp32, for the non-negative finite codes 0x00..0x7E that
// packing and quantization produce. Exponent 0 is subnormal: m * 2^-9.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : static_cast<float>(m) * 0x1p-9f;
}

// Magnitude of an E2M1 code (its low 3 bits) as fp32 bits: exponent field e (bias 1), mantissa m.
__device__ __forceinline__ uint32_t e2m1_mag_f32_bits(uint32_t c) {
  const uint32_t e = (c >> 1) & 3u, m = c & 1u;
  return e ? (((e + 126u) << 23) | (m << 22)) : (m ? 0x3f000000u : 0u);
}

// One element: bf16 bits of E2M1(c) * s for a non-negative scale s. The fp32 product is exact and
// its low 16 bits are zero, so taking the high half is the exact bf16; the sign comes from the code
// (IEEE product sign, so negative zero codes and zero scales give -0).
__device__ __forceinline__ uint32_t nvfp4_elem_bf16(uint32_t c, float s) {
  const float v = __uint_as_float(e2m1_mag_f32_bits(c)) * s;
  return (__float_as_uint(v) >> 16) | ((c & 8u) << 12);
}

// Eight E2M1 codes (one 32-bit word, element 2i in the low nibble of byte i) times scale s ->
// eight bf16 packed two per word, element order preserved.
__device__ __forceinline__ u32x4 nvfp4_word_to_bf16x8(uint32_t w, float s) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t byte = (w >> (8 * i)) & 0xffu;
    out[i] = nvfp4_elem_bf16(byte & 0xfu, s) | (nvfp4_elem_bf16(byte >> 4, s) << 16);
  }
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
