// act_quant.hip -- dynamic NVFP4 quantization of the activation for the W4A4 variant (gfx950).
//
// MiniMax-H3 Ultra Fast, "Kernel path", item 1: activations are quantized to NVFP4 on every call
// for the FP4 x FP4 base GEMM. The pages give no scale rules beyond the format's name; this library
// reads them as (the same reading the CPU reference implements independently):
//   v     = f32(x) * pqs[k]                           one fp32 rounding
//   ts    = f32( amax|v| / 2688 )                     2688 = 6 * 448; 1 if v is all zero
//   s_b   = E4M3_rne_satfinite( amax_b|v| / (6 ts) )  per 16 consecutive k
//   code  = E2M1_rne_sat( v / (E4M3(s_b) * ts) )      0 when s_b = 0
// with every quotient the exact quotient rounded once:
//   * ts: the fp64 quotient is correctly rounded and rounding that to fp32 is again correct;
//   * s_b: the fp64 quotient lies on the same side of every E4M3 midpoint as the exact one (24-bit
//     numerator, 26-bit divisor), and fp64 -> E4M3 is done by rint() of the exact scaled mantissa;
//   * code: no division at all -- |v| is compared in fp64 with the seven E2M1 decision points
//     (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5) * d, d = E4M3(s_b) * ts, all exact products; on a tie
//     the comparison direction picks the neighbour with the even mantissa bit.
// The same quantizer serves the merged-weight route on an fp32 input (ActQuantParams::xf: v = the
// input itself). Two passes: a grid-wide amax (blocks of 8 rows over workgroups, 16-byte chunk
// columns over threads; atomic max on the fp32 bit pattern, exact and order-free), then one thread per 16-element block;
// without pqs, v = x * 1 = x in both. The second pass can also write the decoded activation
// E2M1 * E4M3 (exact bf16, tensor scale left to the GEMM epilogue) as the GEMM's operand.
#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

__global__ void zero_word_kernel(uint32_t* p) { *p = 0u; }

// Rows in blocks of kAmaxRows (grid-strided over workgroups); thread t owns the 16-byte chunk
// columns t, t + 256, ... of a block and loads that column of all the block's rows before reducing
// them, so it keeps kAmaxRows independent loads in flight and reads its pqs values once per column.
// (One load per thread at a time, a row at a time, streamed x at ~2 TB/s.)
constexpr int kAmaxRows = 8;
// Grid cap of both passes (their loops stride over the grid, so any size gives the same result).
constexpr int64_t kMaxGrid = int64_t{1} << 20;

__global__ __launch_bounds__(256) void amax_kernel(ActQuantParams p) {
  float m = 0.0f;
  const int64_t nblk = (p.S + kAmaxRows - 1) / kAmaxRows;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t r0 = blk * kAmaxRows;
    const int64_t nr = p.S - r0 < kAmaxRows ? p.S - r0 : kAmaxRows;  // rows of this block
    if (p.xf) {  // fp32 input: 4 values per chunk (K % 16 == 0)
      const int64_t chunks = p.K / 4;
      for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
        f32x4 v[kAmaxRows];
#pragma unroll
        for (int i = 0; i < kAmaxRows; ++i)
          v[i] = i < nr ? *reinterpret_cast<const f32x4*>(p.xf + (r0 + i) * p.K + c * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kAmaxRows; ++i)
          m = fmaxf(m, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
      }
    } else {  // bf16 input times pqs: 8 values per chunk
      const int64_t chunks = p.K / 8;
      for (int64_t c = threadIdx.x; c < chunks; c += blockDim.x) {
        u32x4 v[kAmaxRows];
#pragma unroll
        for (int i = 0; i < kAmaxRows; ++i)
          v[i] = i < nr ? *reinterpret_cast<const u32x4*>(p.x + (r0 + i) * p.K + c * 8) : u32x4{0u, 0u, 0u, 0u};
        float pq[8];
        if (p.pqs) {
          const f32x4 q0 = *reinterpret_cast<const f32x4*>(p.pqs + c * 8);
          const f32x4 q1 = *reinterpret_cast<const f32x4*>(p.pqs + c * 8 + 4);
          pq[0] = q0.x; pq[1] = q0.y; pq[2] = q0.z; pq[3] = q0.w;
          pq[4] = q1.x; pq[5] = q1.y; pq[6] = q1.z; pq[7] = q1.w;
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pq[e] = 1.0f;
        }
#pragma unroll
        for (int i = 0; i < kAmaxRows; ++i) {
          const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            m = fmaxf(m, fabsf(bf16_bits_to_f32(w[e] & 0xffffu) * pq[2 * e]));
            m = fmaxf(m, fabsf(__uint_as_float(w[e] & 0xffff0000u) * pq[2 * e + 1]));
          }
        }
      }
    }
  }
  // wave64 reduction, the four waves through LDS, then one atomic per workgroup (|v| >= 0: fp32 bit
  // patterns order as unsigned)
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  __shared__ float wave_max[4];
  if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(p.amax_bits, __float_as_uint(fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]))));
}

__device__ __forceinline__ float tensor_scale(uint32_t amax_bits) {
  const float amax = __uint_as_float(amax_bits);
  return amax == 0.0f ? 1.0f : static_cast<float>(static_cast<double>(amax) / 2688.0);
}

// E4M3 code (0..0x7E) nearest to q >= 0, ties to even mantissa, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne_satfinite(double q) {
  if (!(q > 0.0)) return 0u;
  if (q >= 448.0) return 0x7Eu;
  if (q < 0x1p-6) return static_cast<uint32_t>(rint(q * 512.0));  // subnormal step 2^-9; 8 -> 0x08
  int e;
  const double fr = frexp(q, &e);                 // q = fr * 2^e, fr in [0.5, 1)
  double m = rint((2.0 * fr - 1.0) * 8.0);        // exact scaled mantissa, rounded half-even
  int E = e - 1;
  if (m == 8.0) { m = 0.0; E += 1; }
  return static_cast<uint32_t>(((E + 7) << 3) | static_cast<int>(m));
}

__device__ __forceinline__ uint32_t e2m1_code(float v, double d) {
  if (d == 0.0) return 0u;
  const double a = fabs(static_cast<double>(v));
  const uint32_t mag = (a > 0.25 * d) + (a >= 0.75 * d) + (a > 1.25 * d) + (a >= 1.75 * d) +
                       (a > 2.5 * d) + (a >= 3.5 * d) + (a > 5.0 * d);
  return mag == 0u ? 0u : (mag | (v < 0.0f ? 8u : 0u));
}

__global__ __launch_bounds__(256) void quantize_kernel(ActQuantParams p) {
  const int64_t blocks_per_row = p.K / 16;
  const int64_t total = p.S * blocks_per_row;
  const float ts = tensor_scale(*p.amax_bits);
  const double six_ts = 6.0 * static_cast<double>(ts);
  if (blockIdx.x == 0 && threadIdx.x == 0 && p.ts_out) *p.ts_out = ts;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = idx / blocks_per_row;
    const int64_t k0 = (idx - row * blocks_per_row) * 16;
    float v[16];
    if (p.xf) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4 f = *reinterpret_cast<const f32x4*>(p.xf + row * p.K + k0 + 4 * q);
        v[4 * q] = f.x;
        v[4 * q + 1] = f.y;
        v[4 * q + 2] = f.z;
        v[4 * q + 3] = f.w;
      }
    } else {
      const u32x4 x0 = *reinterpret_cast<const u32x4*>(p.x + row * p.K + k0);
      const u32x4 x1 = *reinterpret_cast<const u32x4*>(p.x + row * p.K + k0 + 8);
      const uint32_t xw[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
      float pq[16];
      if (p.pqs) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x4 f = *reinterpret_cast<const f32x4*>(p.pqs + k0 + 4 * q);
          pq[4 * q] = f.x;
          pq[4 * q + 1] = f.y;
          pq[4 * q + 2] = f.z;
          pq[4 * q + 3] = f.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) pq[i] = 1.0f;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = bf16_bits_to_f32(xw[i] & 0xffffu) * pq[2 * i];
        v[2 * i + 1] = bf16_bits_to_f32(xw[i] >> 16) * pq[2 * i + 1];
      }
    }
    float amax_b = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax_b = fmaxf(amax_b, fabsf(v[i]));
    const uint32_t sc = e4m3_rne_satfinite(static_cast<double>(amax_b) / six_ts);
    const float s = e4m3_byte_to_f32<0>(sc);
    const double d = static_cast<double>(s) * static_cast<double>(ts);  // exact
    uint32_t cw[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) cw[i >> 3] |= e2m1_code(v[i], d) << (4 * (i & 7));
    if (p.codes) *reinterpret_cast<u32x2*>(p.codes + row * (p.K / 2) + k0 / 2) = u32x2{cw[0], cw[1]};
    if (p.scales) p.scales[row * blocks_per_row + k0 / 16] = static_cast<uint8_t>(sc);
    if (p.xq_out) {
      uint16_t* dst = p.xq_out + row * p.xq_ld + k0;
      *reinterpret_cast<u32x4*>(dst) = nvfp4_dword_to_bf16x8(cw[0], s);
      *reinterpret_cast<u32x4*>(dst + 8) = nvfp4_dword_to_bf16x8(cw[1], s);
    }
  }
  // zero the K padding of the decoded operand, if any
  if (p.xq_out && p.xq_ld > p.K) {
    const int64_t pad = p.xq_ld - p.K;
    const int64_t ptotal = p.S * pad;
    for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < ptotal;
         idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
      const int64_t row = idx / pad;
      p.xq_out[row * p.xq_ld + p.K + (idx - row * pad)] = 0;
    }
  }
}

}  // namespace

hipError_t launch_act_quant(const ActQuantParams& p, hipStream_t stream) {
  hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, stream, p.amax_bits);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.S > 0) {
    // one row block per workgroup: a grid-stride loop over fewer workgroups left its last round
    // partly empty (2.3 rounds of 2048 workgroups at S = 37726: 3.6 TB/s)
    const int64_t blocks = (p.S + kAmaxRows - 1) / kAmaxRows;
    const int64_t grid = blocks < kMaxGrid ? blocks : kMaxGrid;
    hipLaunchKernelGGL(amax_kernel, dim3(grid), dim3(256), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  int64_t grid = (p.S * (p.K / 16) + 255) / 256;  // one 16-block per thread where the grid allows
  if (grid < 1) grid = 1;
  if (grid > kMaxGrid) grid = kMaxGrid;
  hipLaunchKernelGGL(quantize_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3q
