// adaln.hip -- the AdaLN modulation curve with the adapter folded in (MiniMax-H3 Turbo CMF card, "What
// the conversion did"; MiniMax-H3 Ultra Fast, "Why the pruned transformer matters"). Per block b:
//   adaln_b(t) = W_p,b u(t) + bias_b + c B_b (A_b silu(e(t)))  =  [W_p,b | B_b] v_b(t) + bias_b,
//   v_b(t)     = [u(t) ; c A_b silu(e(t))],   c = strength * alpha / rank,
// the same K-concatenation that folds the LoRA-up into the main GEMM. u (rb values, shared by the
// blocks) and e (E values) are sampled at S points t_i = i / (S - 1); v_b is tabulated there and
// interpolated linearly.
//
// adaln_table_kernel: one wave per 4 samples of one block; lanes split the E-wide dot products
//   A_b[j] . silu(e_i) (fp32, silu(z) = z / (1 + exp(-z))) in 8-column chunks, then a butterfly
//   reduction. The block is the fast grid index, so the workgroups of one group of 16 samples run
//   together and read those embedding rows from L2 instead of streaming e once per block. A
//   one-off per adapter and strength: 2 * blocks * S * rl * E flops (4.4 GFLOP for 50 blocks of
//   rank 16).
// adaln_apply_kernel: a stream over [W_p | B] (bf16 [rows][R] per block, R = rb + rl): one row per
//   thread, R / 8 16-byte loads, T outputs per row from the T interpolated v's kept in LDS. Bytes per
//   call: blocks * rows * (2 R + 4 [bias] + 4 T [out]) -- HBM-bound.
#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int kMaxRl = 32;

__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + __expf(-z)); }

constexpr int kSamplesPerWave = 4;  // 16 per workgroup: grid y = ceil(S / 16) <= 65535

// 8 consecutive values of one embedding row through silu (zeros past E).
__device__ __forceinline__ void silu8(const float* row, int E, int k0, float (&s)[8]) {
  if (k0 + 8 <= E && (E & 3) == 0) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(row + k0);
    const f32x4 b = *reinterpret_cast<const f32x4*>(row + k0 + 4);
    s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w; s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) s[e] = k0 + e < E ? row[k0 + e] : 0.0f;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s[e] = silu_f32(s[e]);
}

// 8 consecutive bf16 of one A row as fp32 (zeros past E).
__device__ __forceinline__ void a8(const uint16_t* row, int E, int k0, float (&a)[8]) {
  if (k0 + 8 <= E && (E & 7) == 0) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(row + k0);
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[2 * e] = bf16_bits_to_f32(ws[e] & 0xffffu);
      a[2 * e + 1] = bf16_bits_to_f32(ws[e] >> 16);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = k0 + e < E ? bf16_bits_to_f32(row[k0 + e]) : 0.0f;
  }
}

// One wave per kSamplesPerWave samples of one block: lane l takes the 8-column chunks l, l + 64, ...
// of the embedding rows and of every A_b row (16-byte loads), so each A value loaded serves all the
// wave's samples; then a butterfly sum over the lanes.
__global__ __launch_bounds__(256) void adaln_table_kernel(AdalnTableParams p) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.x;
  const int i0 = (blockIdx.y * 4 + wave) * kSamplesPerWave;
  if (i0 >= p.S) return;
  const int ns = min(kSamplesPerWave, p.S - i0);
  const int R = p.rb + p.rl;
  float acc[kSamplesPerWave][kMaxRl];
#pragma unroll
  for (int s = 0; s < kSamplesPerWave; ++s)
#pragma unroll
    for (int j = 0; j < kMaxRl; ++j) acc[s][j] = 0.0f;
  const uint16_t* Ab = p.A + static_cast<int64_t>(b) * p.rl * p.E;
  for (int k0 = lane * 8; k0 < p.E; k0 += 64 * 8) {
    float sv[kSamplesPerWave][8];
#pragma unroll
    for (int s = 0; s < kSamplesPerWave; ++s) silu8(p.emb + static_cast<int64_t>(min(i0 + s, p.S - 1)) * p.E, p.E, k0, sv[s]);
    const uint16_t* ap = Ab;
#pragma unroll
    for (int j = 0; j < kMaxRl; ++j) {
      if (j < p.rl) {
        float a[8];
        a8(ap, p.E, k0, a);
        ap += p.E;
#pragma unroll
        for (int s = 0; s < kSamplesPerWave; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[s][j] = fmaf(a[e], sv[s][e], acc[s][j]);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kMaxRl; ++j) {
    if (j < p.rl) {
#pragma unroll
      for (int s = 0; s < kSamplesPerWave; ++s)
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) acc[s][j] += __shfl_xor(acc[s][j], off);
    }
  }
#pragma unroll
  for (int s = 0; s < kSamplesPerWave; ++s) {
    if (s >= ns) break;
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
  const int per_wg = 4 * kSamplesPerWave;
  const dim3 grid(static_cast<uint32_t>(p.blocks), static_cast<uint32_t>((p.S + per_wg - 1) / per_wg));
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
