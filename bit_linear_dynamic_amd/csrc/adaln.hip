// adaln.hip -- the AdaLN modulation curve with the adapter folded in (MiniMax-H3 Turbo CMF card, "What
// the conversion did"; MiniMax-H3 Ultra Fast, "Why the pruned transformer matters"). Per block b:
//   adaln_b(t) = W_p,b u(t) + bias_b + c B_b (A_b silu(e(t)))  =  [W_p,b | B_b] v_b(t) + bias_b,
//   v_b(t)     = [u(t) ; c A_b silu(e(t))],   c = strength * alpha / rank,
// the same K-concatenation that folds the LoRA-up into the main GEMM. u (rb values, shared by the
// blocks) and e (E values) are sampled at S points t_i = i / (S - 1); v_b is tabulated there and
// interpolated linearly.
//
// adaln_table_kernel: one wave per pair of samples of one block; lanes split the E-wide dot products
//   A_b[j] . silu(e_i) (fp32, silu(z) = z / (1 + exp(-z))), then a butterfly reduction. A one-off per
//   adapter and strength: 2 * blocks * S * rl * E flops (2.2 GFLOP for 50 blocks of rank 16).
// adaln_apply_kernel: a stream over [W_p | B] (bf16 [rows][R] per block, R = rb + rl): one row per
//   thread, R / 8 16-byte loads, T outputs per row from the T interpolated v's kept in LDS. Bytes per
//   call: blocks * rows * (2 R + 4 [bias] + 4 T [out]) -- HBM-bound.
#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int kMaxRl = 32;

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

__global__ __launch_bounds__(256) void adaln_table_kernel(AdalnTableParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  const int i0 = (blockIdx.x * 4 + wave) * 2;
  if (i0 >= p.S) return;
  const bool two = i0 + 1 < p.S;
  const int R = p.rb + p.rl;
  float acc[2][kMaxRl];
#pragma unroll
  for (int j = 0; j < kMaxRl; ++j) acc[0][j] = acc[1][j] = 0.0f;
  const float* e0 = p.emb + static_cast<int64_t>(i0) * p.E;
  const float* e1 = two ? e0 + p.E : e0;
  const uint16_t* Ab = p.A + static_cast<int64_t>(b) * p.rl * p.E;
  for (int k = lane; k < p.E; k += 64) {
    const float s0 = silu_f32(e0[k]), s1 = silu_f32(e1[k]);
    const uint16_t* ap = Ab + k;  // walks down column k of A_b
#pragma unroll
    for (int j = 0; j < kMaxRl; ++j) {
      if (j < p.rl) {
        const float a = bf16_bits_to_f32(*ap);
        ap += p.E;
        acc[0][j] = fmaf(a, s0, acc[0][j]);
        acc[1][j] = fmaf(a, s1, acc[1][j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxRl; ++j) {
    if (j < p.rl) {
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) {
        acc[0][j] += __shfl_xor(acc[0][j], off);
        acc[1][j] += __shfl_xor(acc[1][j], off);
      }
    }
  }
  for (int s = 0; s < (two ? 2 : 1); ++s) {
    float* row = p.table + (static_cast<int64_t>(b) * p.S + i0 + s) * R;
    if (lane < p.rb) row[lane] = p.u[static_cast<int64_t>(i0 + s) * p.rb + lane];
#pragma unroll
    for (int j = 0; j < kMaxRl; ++j)
      if (j < p.rl && lane == j) row[p.rb + j] = p.c * acc[s][j];
  }
}

constexpr int kApplyThreads = 256;
constexpr int kMaxT = 8;
constexpr int kMaxR = 64;

__global__ __launch_bounds__(kApplyThreads) void adaln_apply_kernel(AdalnApplyParams p) {
  __shared__ float v[kMaxT][kMaxR];
  const int b = blockIdx.y;
  for (int e = threadIdx.x; e < p.T * p.R; e += kApplyThreads) {
    const int tau = e / p.R, q = e % p.R;
    const float tt = fminf(fmaxf(p.t[tau], 0.0f), 1.0f);
    const float pos = tt * static_cast<float>(p.S - 1);
    const int i0 = min(static_cast<int>(floorf(pos)), p.S - 2);
    const float th = pos - static_cast<float>(i0);
    const float* t0 = p.table + (static_cast<int64_t>(b) * p.S + i0) * p.R;
    v[tau][q] = (1.0f - th) * t0[q] + th * t0[p.R + q];
  }
  __syncthreads();
  const int64_t r = static_cast<int64_t>(blockIdx.x) * kApplyThreads + threadIdx.x;
  if (r >= p.rows) return;
  const int64_t row = static_cast<int64_t>(b) * p.rows + r;
  const u32x4* src = reinterpret_cast<const u32x4*>(p.M + row * p.R);
  float acc[kMaxT];
  const float bias = p.bias ? p.bias[row] : 0.0f;
#pragma unroll
  for (int tau = 0; tau < kMaxT; ++tau) acc[tau] = bias;
  for (int c8 = 0; c8 < p.R / 8; ++c8) {
    const u32x4 w = src[c8];
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const float m0 = bf16_bits_to_f32(ws[h] & 0xffffu), m1 = bf16_bits_to_f32(ws[h] >> 16);
      const int q = c8 * 8 + 2 * h;
#pragma unroll
      for (int tau = 0; tau < kMaxT; ++tau)
        if (tau < p.T) acc[tau] = fmaf(m1, v[tau][q + 1], fmaf(m0, v[tau][q], acc[tau]));
    }
  }
#pragma unroll
  for (int tau = 0; tau < kMaxT; ++tau)
    if (tau < p.T) p.out[(static_cast<int64_t>(tau) * p.blocks + b) * p.rows + r] = acc[tau];
}

}  // namespace

hipError_t launch_adaln_table(const AdalnTableParams& p, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((p.S + 7) / 8), static_cast<uint32_t>(p.blocks));
  hipLaunchKernelGGL(adaln_table_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_adaln_apply(const AdalnApplyParams& p, hipStream_t stream) {
  if (p.rows == 0) return hipSuccess;
  const dim3 grid(static_cast<uint32_t>((p.rows + kApplyThreads - 1) / kApplyThreads), static_cast<uint32_t>(p.blocks));
  hipLaunchKernelGGL(adaln_apply_kernel, grid, dim3(kApplyThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3q
