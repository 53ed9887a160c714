// merge.hip -- the merged route, kept beside the dynamic path to measure what not merging costs and
// buys: the adapter update folded into the weight before quantizing (MiniMax-H3 Turbo CMF card,
// "What the conversion did", backbone item; "Which file"), which the dynamic path of FL2VA Turbo,
// "Implementation", never does. The base weight multiplies x * pqs, so the merged weight carries the
// adapter term divided by pqs per input column:
//   m[n][k] = f32( Wq[n][k] * ts + (c * sum_{j < r_pad} B[n][j] * A[j][k]) / pqs[k] ),
//   c = strength * alpha / rank,
// in fp64 with j ascending and one rounding to fp32 at the end. Wq = E2M1 * E4M3 comes from the
// dequant kernel (exact in bf16, so Wq * ts is exact in fp64); every product B * A of two bf16 values
// is exact in fp64, so a fused and a separate multiply-add give the same sum, and the zero padding
// columns j >= rank add exact zeros. The NVFP4 quantizer (act_quant.hip, fp32 input) then runs on m.
//
// Geometry: 64 packed weight rows x 64 k per workgroup of 256 threads, 4 x 4 outputs per thread
// (rows ty + 16 i, columns tx + 16 q), 32 adapter columns per LDS step. A one-off conversion, not
// the per-call path.
#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int kMT = 64;
constexpr int kKT = 64;
constexpr int kJT = kLoraBK;  // one 32-column rank tile of the packed B per step

__global__ __launch_bounds__(256) void lora_merge_kernel(MergeParams p) {
  __shared__ double bs[kMT][kJT + 1];
  __shared__ double as[kJT][kKT];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t prow0 = static_cast<int64_t>(blockIdx.y) * kMT;  // first packed row of this tile
  const int64_t k0 = static_cast<int64_t>(blockIdx.x) * kKT;
  const int64_t nt = prow0 / kGemmBN;
  const int64_t c0 = prow0 % kGemmBN;
  const int r_tiles = p.r_pad / kJT;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.0;
  for (int jt = 0; jt < r_tiles; ++jt) {
    const uint16_t* btile = p.B + ((nt * r_tiles + jt) * kGemmBN + c0) * kJT;  // 64 rows x 32, contiguous
    for (int e = threadIdx.x; e < kMT * kJT; e += 256)
      bs[e / kJT][e % kJT] = static_cast<double>(bf16_bits_to_f32(btile[e]));
    for (int e = threadIdx.x; e < kJT * kKT; e += 256) {
      const int j = e / kKT, kk = e % kKT;
      as[j][kk] = static_cast<double>(bf16_bits_to_f32(p.A[static_cast<int64_t>(jt * kJT + j) * p.K_pad + k0 + kk]));
    }
    __syncthreads();
    for (int j = 0; j < kJT; ++j) {
      double b[4], a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) b[i] = bs[ty + 16 * i][j];
#pragma unroll
      for (int q = 0; q < 4; ++q) a[q] = as[j][tx + 16 * q];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[i][q] = fma(b[i], a[q], acc[i][q]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t n = packed_row_source(nt, c0 + ty + 16 * i, p.gate_up, p.N);
    if (n < 0) continue;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t k = k0 + tx + 16 * q;
      if (k >= p.K) continue;
      const double wd = static_cast<double>(bf16_bits_to_f32(p.wq[n * p.K + k])) * p.ts;
      const double t = p.c * acc[i][q];
      const double u = p.pqs ? t / static_cast<double>(p.pqs[k]) : t;
      p.m[n * p.K + k] = static_cast<float>(wd + u);
    }
  }
}

}  // namespace

hipError_t launch_lora_merge(const MergeParams& p, hipStream_t stream) {
  const int64_t gx = p.K_pad / kKT, gy = static_cast<int64_t>(p.n_tiles) * (kGemmBN / kMT);
  if (gx == 0 || gy == 0) return hipSuccess;
  hipLaunchKernelGGL(lora_merge_kernel, dim3(static_cast<uint32_t>(gx), static_cast<uint32_t>(gy)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace h3q
