// lora_down.hip -- the thin LoRA-down GEMM and the base-path activation prescale, for gfx950.
//
// LoRA-down (FL2VA Turbo, "Implementation": the bf16 branch A(x) on the ORIGINAL activation):
//   t'[s][j] = bf16( f * sum_k x[s][k] * A[j][k] ),   j < r_pad,   fp32 accumulation
// with f = strength * alpha / (rank * ts) (divided on the device by the W4A4 activation scale when
// there is one), so that the main GEMM can add t' x B into the same accumulator as the base term.
// The same pass writes the base path's operand xs = bf16(x * pqs) (same section: pre_quant_scale
// applies to the base path only), since it is already reading every element of x.
//
// Geometry: 256 threads (2x2 wave64s), 128 rows of x per workgroup and all r_pad (<= 512) columns,
// K staged 64 at a time through double-buffered LDS; wave (wm, wn) owns rows wm*64..+64 and
// columns wn*r_pad/2..+r_pad/2 as 2 x (r_pad/64) tiles of v_mfma_f32_32x32x16_bf16.
//
// Prescale: the elementwise xs = bf16(x * pqs) on its own, for calls without an adapter.
#include <mutex>

#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int kThreads = 256;
constexpr int BM = kLoraBM;  // 128
constexpr int BK = 64;

// Loads 8 bf16 of x at (row, k) -- zeros past K (K is a multiple of 16, so chunks never straddle).
__device__ __forceinline__ u32x4 load_x_chunk(const uint16_t* x, int64_t row, int64_t K, int64_t k) {
  if (k >= K) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(x + row * K + k);
}

// bf16(x * pqs) for 8 consecutive elements starting at k (pqs null = 1; past K: zero).
__device__ __forceinline__ u32x4 prescale_chunk(u32x4 xv, const float* pqs, int64_t K, int64_t k) {
  if (!pqs || k >= K) return xv;
  const f32x4 p0 = *reinterpret_cast<const f32x4*>(pqs + k);
  const f32x4 p1 = *reinterpret_cast<const f32x4*>(pqs + k + 4);
  const float ps[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = bf16_bits_to_f32(xv[i] & 0xffffu) * ps[2 * i];
    const float hi = bf16_bits_to_f32(xv[i] >> 16) * ps[2 * i + 1];
    out[i] = f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
  }
  return out;
}

template <int RT2>  // r_pad = 64 * RT2
__global__ __launch_bounds__(kThreads, 1) void lora_down_kernel(LoraDownParams p) {
  constexpr int R = 64 * RT2;
  constexpr uint32_t kXBytes = BM * BK * 2;       // 16 KiB
  constexpr uint32_t kABytes = R * BK * 2;        // 8 KiB per 64 ranks
  constexpr uint32_t kStage = kXBytes + kABytes;
  constexpr int kAChunks = R * BK / 8 / kThreads; // chunks of A per thread per stage = 2*RT2
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * BM;
  const int k_tiles = static_cast<int>(p.K_pad / BK);

  f32x16 acc[2][RT2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < RT2; ++j) acc[i][j] = f32x16{};

  u32x4 xr[4], ar[kAChunks];
  auto load = [&](int kt) {
    const int64_t k0 = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      int64_t row = m0 + (c >> 3);
      row = row < p.S ? row : p.S - 1;
      xr[i] = load_x_chunk(p.x, row, p.K, k0 + (c & 7) * 8);
    }
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = tid + kThreads * i;
      ar[i] = *reinterpret_cast<const u32x4*>(p.A + (c >> 3) * p.K_pad + k0 + (c & 7) * 8);
    }
  };
  auto store = [&](int kt, uint8_t* stage) {
    const int64_t k0 = static_cast<int64_t>(kt) * BK;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(stage + lds_chunk_offset(c >> 3, c & 7)) = xr[i];
      const int64_t row = m0 + (c >> 3);
      if (p.xs_out && row < p.S) {
        const int64_t k = k0 + (c & 7) * 8;
        *reinterpret_cast<u32x4*>(p.xs_out + row * p.K_pad + k) = prescale_chunk(xr[i], p.pqs, p.K, k);
      }
    }
#pragma unroll
    for (int i = 0; i < kAChunks; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(stage + kXBytes + lds_chunk_offset(c >> 3, c & 7)) = ar[i];
    }
  };

  load(0);
  store(0, smem);
  __syncthreads();

  const uint32_t a_row0 = wm * 64 + (lane & 31);
  const uint32_t b_row0 = wn * (R / 2) + (lane & 31);
  const uint32_t khalf = lane >> 5;
  for (int kt = 0; kt < k_tiles; ++kt) {
    const bool more = kt + 1 < k_tiles;
    if (more) load(kt + 1);
    const uint8_t* Xs = smem + (kt & 1) * kStage;
    const uint8_t* As = Xs + kXBytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[2], b[RT2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(Xs + lds_chunk_offset(a_row0 + i * 32, kk * 2 + khalf));
#pragma unroll
      for (int j = 0; j < RT2; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(As + lds_chunk_offset(b_row0 + j * 32, kk * 2 + khalf));
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < RT2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if (more) store(kt + 1, smem + ((kt + 1) & 1) * kStage);
    __syncthreads();
  }

  const float f = p.f_div_dev ? p.f / *p.f_div_dev : p.f;
  const int col_lane = lane & 31, row_lane = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 64 + i * 32 + (r >> 2) * 8 + row_lane + (r & 3);
      if (row >= p.S) continue;
#pragma unroll
      for (int j = 0; j < RT2; ++j) {
        const int col = wn * (R / 2) + j * 32 + col_lane;
        p.t_out[row * R + col] = static_cast<uint16_t>(f32_to_bf16_rne(f * acc[i][j][r]));
      }
    }
}

__global__ __launch_bounds__(256) void prescale_kernel(PrescaleParams p) {
  const int64_t chunks_per_row = p.K_pad / 8;
  const int64_t total = p.S * chunks_per_row;
  for (int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; idx < total;
       idx += static_cast<int64_t>(gridDim.x) * blockDim.x) {
    const int64_t row = idx / chunks_per_row;
    const int64_t k = (idx - row * chunks_per_row) * 8;
    const u32x4 xv = load_x_chunk(p.x, row, p.K, k);
    *reinterpret_cast<u32x4*>(p.xs_out + row * p.K_pad + k) = prescale_chunk(xv, p.pqs, p.K, k);
  }
}

template <int RT2>
hipError_t launch_rt(const LoraDownParams& p, hipStream_t stream) {
  constexpr uint32_t lds = 2 * (BM * BK * 2 + 64 * RT2 * BK * 2);
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lora_down_kernel<RT2>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  const int64_t grid = (p.S + BM - 1) / BM;
  hipLaunchKernelGGL(lora_down_kernel<RT2>, dim3(grid), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_lora_down(const LoraDownParams& p, hipStream_t stream) {
  if (p.S == 0) return hipSuccess;
  switch (p.r_pad / 64) {
    case 1: return launch_rt<1>(p, stream);
    case 2: return launch_rt<2>(p, stream);
    case 3: return launch_rt<3>(p, stream);
    case 4: return launch_rt<4>(p, stream);
    case 5: return launch_rt<5>(p, stream);
    case 6: return launch_rt<6>(p, stream);
    case 7: return launch_rt<7>(p, stream);
    case 8: return launch_rt<8>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prescale(const PrescaleParams& p, hipStream_t stream) {
  const int64_t total = p.S * (p.K_pad / 8);
  if (total == 0) return hipSuccess;
  int64_t grid = (total + 255) / 256;
  if (grid > 256 * 64) grid = 256 * 64;
  hipLaunchKernelGGL(prescale_kernel, dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace h3q
