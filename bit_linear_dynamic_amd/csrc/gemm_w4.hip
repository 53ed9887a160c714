// gemm_w4.hip -- the main W4 + LoRA GEMM for gfx950.
//
//   acc[s][n] = sum_{k<K} act[s][k] * Wq[n][k]  +  sum_{j<r_pad} t'[s][j] * B[n][j]
//   y[s][n]   = bf16( ts * acc[s][n] )                       (plain epilogue)
//   h[s][j]   = bf16( SiLU(ts*acc[s][j]) * ts*acc[s][F+j] )  (gate/up epilogue)
//
// The base term is the NVFP4 projection of FL2VA Turbo, "Implementation"; Wq = E2M1 * E4M3 is
// decoded into LDS as exact bf16. The LoRA-up is folded into the same accumulator as r_pad extra
// K-columns (the concatenation identity W u + B (A s) = [W | B] [u ; A s] of the MiniMax-H3 Turbo
// CMF card, "What the conversion did"), with t' = strength*alpha/(rank*ts) * (A x) so that one
// scale by ts finishes both terms. The gate/up epilogue is the in-place SiLU x up of MiniMax-H3
// Ultra Fast, "Kernel path".
//
// Geometry: 256 threads (4 wave64s in a 2x2 grid), a 256x256 output tile per workgroup, K staged
// 64 at a time through double-buffered LDS (2 x (32 KiB activation + 32 KiB weight)); each wave owns
// a 128x128 quarter as 4x4 tiles of v_mfma_f32_32x32x16_bf16 with fp32 accumulators. Rows past S
// are computed from a clamped (repeated) input row and never stored.
//
// Weight layout (written by h3q_pack_weight): for tile column block nt and K-tile kt, the 256 rows'
// 32 code bytes are contiguous ([nt][kt][256][32]) and so are their 4 scale bytes ([nt][kt][256][4]);
// one thread loads and decodes one row. The LoRA B factor is stored the same way in bf16
// ([nt][rt][256][64]).
//
// Workgroup -> tile order: the hardware hands workgroup b to XCD b % 8. Work item w is mapped so
// that each XCD walks a contiguous range of the (M-tile major, N-tile minor) order: the ~32
// workgroups resident on one XCD then share one activation M-tile in that XCD's L2 while they
// stream different weight tiles.
#include <mutex>

#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int kThreads = 256;
constexpr uint32_t kTileBytes = BM * BK * 2;            // 32 KiB per operand per stage
constexpr uint32_t kStageBytes = 2 * kTileBytes;
constexpr uint32_t kLdsBytes = 2 * kStageBytes;          // 128 KiB

struct Staged {
  u32x4 a[8];   // activation: 8 chunks of 8 bf16
  u32x4 b[8];   // LoRA B: 8 chunks of 8 bf16; W4: b[0..1] = 32 code bytes, b[2].x = 4 scale codes
};

__device__ __forceinline__ void load_stage(const GemmParams& p, int64_t m0, int nt, int kt, int tid,
                                           Staged& st) {
  const bool lora = kt >= p.k_tiles;
  // activation (x*pqs or t'): chunk c = tid + 256 i covers row c/8, 8 bf16 at k-chunk c%8
  const uint16_t* src = lora ? p.lora_t : p.act;
  const int64_t ld = lora ? p.lora_t_ld : p.act_ld;
  const int64_t k0 = static_cast<int64_t>(lora ? kt - p.k_tiles : kt) * BK;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + kThreads * i;
    int64_t row = m0 + (c >> 3);
    row = row < p.S ? row : p.S - 1;
    st.a[i] = *reinterpret_cast<const u32x4*>(src + row * ld + k0 + (c & 7) * 8);
  }
  if (lora) {
    const uint16_t* bt = p.lora_b + (static_cast<int64_t>(nt) * p.r_tiles + (kt - p.k_tiles)) * (BN * BK);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i;
      st.b[i] = *reinterpret_cast<const u32x4*>(bt + (c >> 3) * BK + (c & 7) * 8);
    }
  } else {
    const int64_t tile = static_cast<int64_t>(nt) * p.k_tiles + kt;
    const uint8_t* cp = p.wcodes + (tile * BN + tid) * kCodeBytesPerRowTile;
    st.b[0] = *reinterpret_cast<const u32x4*>(cp);
    st.b[1] = *reinterpret_cast<const u32x4*>(cp + 16);
    st.b[2].x = *reinterpret_cast<const uint32_t*>(p.wscales + (tile * BN + tid) * kScaleBytesPerRowTile);
  }
}

__device__ __forceinline__ void store_stage(uint8_t* stage, bool lora, int tid, const Staged& st) {
  uint8_t* As = stage;
  uint8_t* Bs = stage + kTileBytes;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = tid + kThreads * i;
    *reinterpret_cast<u32x4*>(As + lds_chunk_offset(c >> 3, c & 7)) = st.a[i];
  }
  if (lora) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int c = tid + kThreads * i;
      *reinterpret_cast<u32x4*>(Bs + lds_chunk_offset(c >> 3, c & 7)) = st.b[i];
    }
  } else {
    // one weight row per thread: 4 scale blocks of 16 elements = 8 chunks of 8 elements
    const uint32_t sc = st.b[2].x;
    const uint32_t words[8] = {st.b[0].x, st.b[0].y, st.b[0].z, st.b[0].w,
                               st.b[1].x, st.b[1].y, st.b[1].z, st.b[1].w};
#pragma unroll
    for (int ch = 0; ch < 8; ++ch) {
      const float s = e4m3_to_f32((sc >> (8 * (ch >> 1))) & 0xffu);
      *reinterpret_cast<u32x4*>(Bs + lds_chunk_offset(tid, ch)) = nvfp4_word_to_bf16x8(words[ch], s);
    }
  }
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware work index (gridDim.x is a multiple of 8)
  const int per_xcd = gridDim.x >> 3;
  const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (w >= p.m_tiles * p.n_tiles) return;
  const int mt = w / p.n_tiles, nt = w - mt * p.n_tiles;
  const int64_t m0 = static_cast<int64_t>(mt) * BM;
  const int total = p.k_tiles + p.r_tiles;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  Staged st;
  load_stage(p, m0, nt, 0, tid, st);
  store_stage(smem, 0 >= p.k_tiles, tid, st);
  __syncthreads();

  const uint32_t a_row0 = wm * 128 + (lane & 31);
  const uint32_t b_row0 = wn * 128 + (lane & 31);
  const uint32_t khalf = lane >> 5;

  for (int kt = 0; kt < total; ++kt) {
    const bool more = kt + 1 < total;
    if (more) load_stage(p, m0, nt, kt + 1, tid, st);

    const uint8_t* As = smem + (kt & 1) * kStageBytes;
    const uint8_t* Bs = As + kTileBytes;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(As + lds_chunk_offset(a_row0 + i * 32, kk * 2 + khalf));
#pragma unroll
      for (int j = 0; j < 4; ++j)
        b[j] = *reinterpret_cast<const bf16x8*>(Bs + lds_chunk_offset(b_row0 + j * 32, kk * 2 + khalf));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }

    if (more) store_stage(smem + ((kt + 1) & 1) * kStageBytes, kt + 1 >= p.k_tiles, tid, st);
    __syncthreads();
  }

  // Epilogue. Accumulator register r of lane l in a 32x32 tile holds
  // row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  const float scale = p.ts * (p.ts_dev ? *p.ts_dev : 1.0f);
  const int col_lane = lane & 31;
  const int row_lane = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + wm * 128 + i * 32 + (r >> 2) * 8 + row_lane + (r & 3);
      if (row >= p.S) continue;
      uint16_t* orow = p.out + row * p.out_ld;
      if (EPI == 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int c = wn * 128 + j * 32 + col_lane;
          const int64_t n = p.gate_up ? packed_row_source(nt, c, true, p.n_out) : static_cast<int64_t>(nt) * BN + c;
          if (n >= 0 && n < p.n_out) orow[n] = static_cast<uint16_t>(f32_to_bf16_rne(scale * acc[i][j][r]));
        }
      } else {
        // tile columns alternate in 32-wide groups: gate j0..j0+31, then up j0..j0+31
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
          const int64_t n = static_cast<int64_t>(nt) * (BN / 2) + (wn * 2 + j / 2) * 32 + col_lane;
          if (n < p.n_out) {
            const float g = scale * acc[i][j][r];
            const float u = scale * acc[i][j + 1][r];
            orow[n] = static_cast<uint16_t>(f32_to_bf16_rne(silu(g) * u));
          }
        }
      }
    }
  }
}

}  // namespace

size_t gemm_w4_lds_bytes() { return kLdsBytes; }

hipError_t launch_gemm_w4(const GemmParams& p, Epilogue epi, hipStream_t stream) {
  const int64_t items = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  const int64_t grid = (items + 7) / 8 * 8;
  if (grid == 0) return hipSuccess;
  const void* fn = epi == Epilogue::Plain ? reinterpret_cast<const void*>(&gemm_w4_kernel<0>)
                                          : reinterpret_cast<const void*>(&gemm_w4_kernel<1>);
  static std::once_flag once[2];
  static hipError_t attr_err[2] = {hipSuccess, hipSuccess};
  const int e = static_cast<int>(epi);
  std::call_once(once[e], [&] {
    attr_err[e] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  });
  if (attr_err[e] != hipSuccess) return attr_err[e];
  if (epi == Epilogue::Plain)
    hipLaunchKernelGGL(gemm_w4_kernel<0>, dim3(grid), dim3(kThreads), kLdsBytes, stream, p);
  else
    hipLaunchKernelGGL(gemm_w4_kernel<1>, dim3(grid), dim3(kThreads), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace h3q
