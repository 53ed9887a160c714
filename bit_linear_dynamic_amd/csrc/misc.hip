// misc.hip -- diagnostic kernel: the packed weight decoded back to the caller's [N][K] order with
// the same decode routine the GEMM uses (E2M1 * E4M3, exact in bf16, without the tensor scale).
#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

// one thread per (packed row, K-tile): 32 code bytes + 4 scales -> 64 bf16
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
    const uint8_t* cp = p.wcodes + (tile * kGemmBN + c) * kCodeBytesPerRowTile;
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(p.wscales + (tile * kGemmBN + c) * kScaleBytesPerRowTile);
    for (int ch = 0; ch < 8; ++ch) {
      const int64_t k = kt * kGemmBK + ch * 8;
      if (k >= p.K) break;
      const uint32_t w = *reinterpret_cast<const uint32_t*>(cp + ch * 4);
      const u32x4 v = nvfp4_word_to_bf16x8(w, e4m3_to_f32((sc >> (8 * (ch >> 1))) & 0xffu));
      *reinterpret_cast<u32x4*>(p.out + n * p.K + k) = v;
    }
  }
}

}  // namespace

hipError_t launch_debug_dequant(const DequantParams& p, hipStream_t stream) {
  const int64_t total = static_cast<int64_t>(p.n_tiles) * kGemmBN * p.k_tiles;
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  hipLaunchKernelGGL(debug_dequant_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3q
