// misc.hip -- diagnostic kernels: the packed weight decoded back to the caller's [N][K] order with
// the decode routine the GEMM uses (E2M1 * E4M3, exact in bf16, without the tensor scale), and a pure
// matrix-core loop that measures the MFMA throughput the board sustains.
#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

template <int SEL>
__device__ __forceinline__ void decode_block(const DequantParams& p, int64_t tile, int64_t c, uint32_t sc,
                                             uint16_t* dst, int64_t k0) {
  const float s = e4m3_byte_to_f32<SEL>(sc);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kc = 2 * SEL + h;
    if (k0 + kc * 8 >= p.K) return;
    const uint32_t cw = p.wcodes_dw[(tile * kCodeChunksPerTile + kc) * kGemmBN + c];
    *reinterpret_cast<u32x4*>(dst + kc * 8) = nvfp4_dword_to_bf16x8(cw, s);
  }
}

// one thread per (packed row, K-tile): 8 code dwords + 1 scale dword -> 64 bf16
__global__ __launch_bounds__(256) void debug_dequant_kernel(DequantParams p) {
  const int64_t rows = static_cast<int64_t>(p.n_tiles) * kGemmBN;
  const int64_t total = rows * p.k_tiles;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t prow = idx / p.k_tiles;
    const int64_t kt = idx - prow * p.k_tiles;
    const int64_t nt = prow / kGemmBN, c = prow % kGemmBN;
    const int64_t n = packed_row_source(nt, c, p.gate_up, p.N);
    if (n < 0) continue;
    const int64_t tile = nt * p.k_tiles + kt;
    const uint32_t sc = p.wscales_dw[tile * kGemmBN + c];
    const int64_t k0 = kt * kGemmBK;
    uint16_t* dst = p.out + n * p.K + k0;
    decode_block<0>(p, tile, c, sc, dst, k0);
    decode_block<1>(p, tile, c, sc, dst, k0);
    decode_block<2>(p, tile, c, sc, dst, k0);
    decode_block<3>(p, tile, c, sc, dst, k0);
  }
}

// Matrix-core ceiling under the board's power limit: every wave keeps 8 accumulator chains of
// v_mfma_f32_32x32x16_bf16 busy with 8 operand pairs that rotate every step (so consecutive MFMAs see
// different data, as in a GEMM), two waves per SIMD as the main GEMM runs, no memory traffic in the
// loop. The accumulators are summed into `sink` so that nothing is optimized away.
__global__ __launch_bounds__(256, 2) void mfma_loop_kernel(const u32x4* ops_a, const u32x4* ops_b, int32_t iters,
                                                          float* sink) {
  const int tid = threadIdx.x;
  bf16x8 a[8], b[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = __builtin_bit_cast(bf16x8, ops_a[j * 256 + tid]);
    b[j] = __builtin_bit_cast(bf16x8, ops_b[j * 256 + tid]);
  }
  f32x16 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + s) & 7], acc[j], 0, 0, 0);
  }
  float t = 0.0f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) t += acc[j][e];
  sink[static_cast<int64_t>(blockIdx.x) * 256 + tid] = t;
}

}  // namespace

hipError_t launch_mfma_loop(const uint16_t* ops_a, const uint16_t* ops_b, int32_t iters, int32_t workgroups,
                            float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, stream, reinterpret_cast<const u32x4*>(ops_a),
                     reinterpret_cast<const u32x4*>(ops_b), iters, sink);
  return hipGetLastError();
}

hipError_t launch_debug_dequant(const DequantParams& p, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.n_tiles) * kGemmBN * p.k_tiles;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  hipLaunchKernelGGL(debug_dequant_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3q
