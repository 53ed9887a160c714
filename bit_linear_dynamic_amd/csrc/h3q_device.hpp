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

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// fp32 -> bf16 bits by the hardware conversion (v_cvt_pk_bf16_f32: round to nearest even).
__device__ __forceinline__ uint32_t f32_to_bf16_hw(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two fp32 values as a bf16 pair (low half: lo), one hardware conversion (round to nearest even).
__device__ __forceinline__ uint32_t bf16x2_hw(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

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
// ... in a 32-deep tile (64-byte rows): rows are paired into 128-byte lines, then as above.
__device__ __forceinline__ uint32_t lds_chunk_offset32(uint32_t row, uint32_t chunk) {
  return lds_chunk_offset(row >> 1, ((row & 1u) << 2) | chunk);
}

// ---------------------------------------------------------------------------------------------
// Buffer memory operations written as inline asm, so that the kernels count their vector-memory
// operations themselves (the compiler neither sees nor waits on them): global->LDS copies
// (buffer_load_dwordx4 ... lds, 16 bytes per lane to LDS address M0 + 16 * lane) and 16-byte
// buffer stores. M0 is saved and restored around each copy. A raw buffer descriptor returns zero
// for reads past its size and drops writes past it. Each block opens with s_nop 4: a vector-memory
// instruction must not read an SGPR for 5 wait states after a VALU instruction wrote it (v_readlane
// after a spill, v_readfirstlane), and the compiler does not look inside the block to insert them.
// A store closes with s_nop 1: a store of more than 64 bits reads its data VGPRs after issue, and
// they may not be overwritten by a VALU instruction for one wait state.
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ u32x4 buf_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return u32x4{static_cast<uint32_t>(a), static_cast<uint32_t>(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Copy 16 bytes per lane from buffer offset voff + soff to LDS byte address lds + 16 * lane.
__device__ __forceinline__ void dma16(u32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
  uint32_t msv;
  asm volatile(
      "s_nop 4\n\ts_mov_b32 %[msv], m0\n\ts_mov_b32 m0, %[m]\n\ts_nop 0\n\t"
      "buffer_load_dwordx4 %[v], %[r], %[s] offen lds\n\ts_mov_b32 m0, %[msv]"
      : [msv] "=&s"(msv)
      : [m] "s"(lds), [v] "v"(voff), [r] "s"(r), [s] "s"(soff)
      : "memory");
}

// The same on lanes 0..LANES-1 only.
template <int LANES>
__device__ __forceinline__ void dma16_lanes(u32x4 r, uint32_t lds, uint32_t voff, uint32_t soff) {
  static_assert(LANES > 0 && LANES <= 32, "lane count");
  uint32_t msv;
  uint64_t ex;
  asm volatile(
      "s_nop 4\n\ts_mov_b32 %[msv], m0\n\ts_mov_b64 %[ex], exec\n\ts_mov_b32 exec_lo, %[lm]\n\ts_mov_b32 exec_hi, 0\n\t"
      "s_mov_b32 m0, %[m]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[v], %[r], %[s] offen lds\n\t"
      "s_mov_b64 exec, %[ex]\n\ts_mov_b32 m0, %[msv]"
      : [msv] "=&s"(msv), [ex] "=&s"(ex)
      : [lm] "i"((LANES == 32) ? 0xffffffffu : ((1u << LANES) - 1u)), [m] "s"(lds), [v] "v"(voff), [r] "s"(r),
        [s] "s"(soff)
      : "memory");
}

// Store 16 bytes per lane at buffer offset voff + soff.
__device__ __forceinline__ void buf_store16(u32x4 data, u32x4 r, uint32_t voff, uint32_t soff) {
  asm volatile("s_nop 4\n\tbuffer_store_dwordx4 %[d], %[v], %[r], %[s] offen\n\ts_nop 1"
               :
               : [d] "v"(data), [v] "v"(voff), [r] "s"(r), [s] "s"(soff)
               : "memory");
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Stage handover: this wave's vector-memory operations except the newest N have completed, its LDS
// reads have returned, then all waves of the workgroup meet. Written as asm so the compiler adds no
// fence (a fence would wait for every copy, including tiles still in flight).
template <int N>
__device__ __forceinline__ void stage_barrier() {
  wait_vmcnt<N>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace h3q
