// gemm_w4.hip -- the main W4 + LoRA GEMM for gfx950.
//
//   acc[s][n] = sum_{k<K} act[s][k] * Wq[n][k]  +  sum_{j<r_pad} t'[s][j] * B[n][j]
//   y[s][n]   = bf16( ts * acc[s][n] )                       (plain epilogue)
//   h[s][j]   = bf16( SiLU(ts*acc[s][j]) * ts*acc[s][F+j] )  (gate/up epilogue)
//
// The base term is the NVFP4 projection of FL2VA Turbo, "Implementation"; Wq = E2M1 * E4M3 is
// exact in bf16, so it is decoded without rounding and fed to bf16 matrix cores. The LoRA-up is
// folded into the same accumulator as r_pad extra K-columns (the concatenation identity
// W u + B (A s) = [W | B] [u ; A s] of the MiniMax-H3 Turbo CMF card, "What the conversion did"),
// with t' = strength*alpha/(rank*ts) * (A x) so that one scale by ts finishes both terms. The gate/up
// epilogue is the in-place SiLU x up of MiniMax-H3 Ultra Fast, "Kernel path".
//
// Geometry: 256 threads = 4 wave64s side by side (1 x 4), a 256 x 256 output tile per workgroup;
// wave w owns all 256 rows and columns [64w, 64w+64) as 8 x 2 tiles of v_mfma_f32_32x32x16_bf16
// with fp32 accumulators. K is staged through three LDS stages of 42 KiB, two tiles ahead:
//   base K-tile (64 deep)  activation 256 x 64 bf16, 16-byte chunks XOR-swizzled     32 KiB
//                          8 runs of 256 code dwords (+32 dwords padding each)        9 KiB
//                          256 scale dwords                                            1 KiB
//   LoRA K-tile (32 deep)  t' 256 x 32 bf16 and B 256 x 32 bf16, same swizzle     2 x 16 KiB
// Every global->LDS copy is a buffer_load ... lds (16 bytes per lane, no registers, out-of-range
// offsets read as zero). The weight stays 4-bit in LDS: each wave decodes the B operand of its own 64
// columns straight into MFMA registers -- one code dword (8 consecutive k of one column) and one
// E4M3 scale per lane per 32x32x16 step -- so no column is decoded twice and no bf16 weight tile is
// written to LDS. Rows past S lie outside the activation buffer, load as zero and are never stored.
//
// Workgroup -> tile order: the hardware hands workgroup b to XCD b % 8; work item w is mapped so that
// each XCD walks a contiguous range of the (M-tile major, N-tile minor) order, so the workgroups
// resident on one XCD share one activation M-tile in that XCD's L2 while streaming weight tiles.
#include <algorithm>
#include <mutex>

#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int kThreads = 256;
constexpr uint32_t kCodeRun = (kGemmBN + 32) * 4;        // one code run in LDS, padded: 1152 B
constexpr uint32_t kLdsA = 0;                            // activation / t' tile
constexpr uint32_t kLdsCodes = 32768;                    // base tile: code runs
constexpr uint32_t kLdsScales = kLdsCodes + kCodeChunksPerTile * kCodeRun;  // 41984
constexpr uint32_t kLdsLoraB = kLoraTileBytes;           // LoRA tile: B after the 16 KiB t' tile
constexpr uint32_t kStage = kLdsScales + kScaleTileBytes; // 43008
constexpr int kStages = 3;
constexpr uint32_t kLdsBytes = kStages * kStage;         // 129024
static_assert(kLdsLoraB + kLoraTileBytes <= kStage, "LoRA tile must fit a stage");
// DMA instructions per wave per K-tile (every wave issues the same number, so that a wave can wait
// for all but the newest tile with one vmcnt)
constexpr int kCopiesBase = 8 + 2 + 1;  // activation, codes, a quarter of the scales
constexpr int kCopiesLora = 4 + 4;      // t', B

typedef __attribute__((address_space(3))) void* lds_void_ptr;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}

// 16 bytes per lane from buffer offset voff + soff to LDS at lds + 16 * lane.
__device__ __forceinline__ void copy16(__amdgpu_buffer_rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_ptr)(lds), 16, voff, soff, 0, 0);
}

// s_waitcnt vmcnt(N) (expcnt and lgkmcnt left unconstrained), gfx9 encoding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Stage handover: this wave's copies into the next stage have landed (all but the newest `N`
// DMA instructions), its LDS reads have returned, then all waves meet. Written as one asm block so
// the compiler adds no fence: a fence would wait for every copy, including the tile still in flight.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  wait_vmcnt<N>();
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS slot of (row, 16-byte chunk) in a 64-deep tile (128-byte rows): chunk XOR (row/2)%8.
__device__ __forceinline__ uint32_t slot64(uint32_t row, uint32_t chunk) { return lds_chunk_offset(row, chunk); }
// ... in a 32-deep tile (64-byte rows): rows are paired into 128-byte lines, then as above.
__device__ __forceinline__ uint32_t slot32(uint32_t row, uint32_t chunk) {
  return lds_chunk_offset(row >> 1, ((row & 1u) << 2) | chunk);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

struct Ctx {
  __amdgpu_buffer_rsrc_t act, lt, codes, scales, lb;
  // Base tile: copy i (of 8 per wave) fills LDS slots (8w + i)*64 + lane, i.e. tile rows
  // (8w + i)*8 + lane/8; the chunk depends on i only through i & 1, so the per-lane offset is
  // vact[i & 1] plus a uniform (i & ~1) * 8 rows.
  // LoRA tile: copy i (of 4 per wave) fills slots (4w + i)*64 + lane of a 64-byte-row tile, i.e.
  // 128-byte lines (4w + i)*8 + lane/8 holding 16 rows; again the per-lane part depends on i & 1
  // only, and (i & ~1) adds 16 rows per unit.
  uint32_t vact[2], vlt[2], vlb[2];
  uint32_t act_rows8, lt_rows16;
  int k_tiles, wave, lane;
};

// Issues the copies of K-tile kt (base tiles first, then LoRA tiles) into an LDS stage.
__device__ __forceinline__ void issue_tile(const Ctx& c, int kt, uint8_t* stage) {
  const int w = c.wave;
  if (kt < c.k_tiles) {
    const uint32_t k_bytes = static_cast<uint32_t>(kt) * BK * 2;
#pragma unroll
    for (int i = 0; i < 8; ++i)
      copy16(c.act, stage + kLdsA + (w * 8 + i) * 1024, c.vact[i & 1], k_bytes + (i & ~1) * c.act_rows8);
    const uint32_t ct = static_cast<uint32_t>(kt) * kCodeTileBytes;
    copy16(c.codes, stage + kLdsCodes + w * kCodeRun, c.lane * 16, ct + w * 1024);
    copy16(c.codes, stage + kLdsCodes + (w + 4) * kCodeRun, c.lane * 16, ct + (w + 4) * 1024);
    if (c.lane < 16)
      copy16(c.scales, stage + kLdsScales + w * 256, c.lane * 16,
             static_cast<uint32_t>(kt) * kScaleTileBytes + w * 256);
  } else {
    const uint32_t rt = static_cast<uint32_t>(kt - c.k_tiles);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      copy16(c.lt, stage + kLdsA + (w * 4 + i) * 1024, c.vlt[i & 1], rt * kLoraBK * 2 + (i & ~1) * c.lt_rows16);
      copy16(c.lb, stage + kLdsLoraB + (w * 4 + i) * 1024, c.vlb[i & 1],
             rt * kLoraTileBytes + (i & ~1) * (16 * kLoraBK * 2));
    }
  }
}

// A operand of K-step KK (16 k) for the 8 row tiles: row i*32 + lane%32, chunk 2KK + lane/32.
template <int KK>
__device__ __forceinline__ void load_a64(const uint8_t* stage, uint32_t lane, bf16x8 (&a)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(stage + kLdsA + slot64(i * 32 + (lane & 31), KK * 2 + (lane >> 5)));
}
template <int KK>
__device__ __forceinline__ void load_a32(const uint8_t* stage, uint32_t lane, bf16x8 (&a)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(stage + kLdsA + slot32(i * 32 + (lane & 31), KK * 2 + (lane >> 5)));
}

// 4-bit B operand of K-step KK: one code dword (8 consecutive k) per lane and column tile.
template <int KK>
__device__ __forceinline__ void load_codes(const uint8_t* stage, uint32_t lane, const uint32_t (&ncol)[2],
                                           uint32_t (&cw)[2]) {
  const uint32_t run = kLdsCodes + (KK * 2 + (lane >> 5)) * kCodeRun;
#pragma unroll
  for (int j = 0; j < 2; ++j) cw[j] = *reinterpret_cast<const uint32_t*>(stage + run + ncol[j] * 4);
}

// bf16 B operand of LoRA K-step KK.
template <int KK>
__device__ __forceinline__ void load_b32(const uint8_t* stage, uint32_t lane, const uint32_t (&ncol)[2],
                                         bf16x8 (&b)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    b[j] = *reinterpret_cast<const bf16x8*>(stage + kLdsLoraB + slot32(ncol[j], KK * 2 + (lane >> 5)));
}

// Decode: 8 E2M1 codes times the block scale (byte KK of the row's scale dword) -> bf16 operand.
template <int KK>
__device__ __forceinline__ void decode_b(const uint32_t (&cw)[2], const uint32_t (&sdw)[2], bf16x8 (&b)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j)
    b[j] = __builtin_bit_cast(bf16x8, nvfp4_dword_to_bf16x8(cw[j], e4m3_byte_to_f32<KK>(sdw[j])));
}

__device__ __forceinline__ void mfma_block(const bf16x8 (&a)[8], const bf16x8 (&b)[2], f32x16 (&acc)[8][2]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[0], acc[i][0], 0, 0, 0);
    acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[1], acc[i][1], 0, 0, 0);
  }
}

// One 64-deep base K-tile: the A operand and codes of step KK+1 are read from LDS while step KK's
// 16 MFMAs run (two register sets), and each step's B operand is decoded just before use.
__device__ __forceinline__ void base_tile(const uint8_t* stage, uint32_t lane, const uint32_t (&ncol)[2],
                                          f32x16 (&acc)[8][2]) {
  const uint32_t sdw[2] = {*reinterpret_cast<const uint32_t*>(stage + kLdsScales + ncol[0] * 4),
                           *reinterpret_cast<const uint32_t*>(stage + kLdsScales + ncol[1] * 4)};
  bf16x8 a0[8], a1[8], b[2];
  uint32_t c0[2], c1[2];
  load_a64<0>(stage, lane, a0);
  load_codes<0>(stage, lane, ncol, c0);
  load_a64<1>(stage, lane, a1);
  load_codes<1>(stage, lane, ncol, c1);
  decode_b<0>(c0, sdw, b);
  mfma_block(a0, b, acc);
  load_a64<2>(stage, lane, a0);
  load_codes<2>(stage, lane, ncol, c0);
  decode_b<1>(c1, sdw, b);
  mfma_block(a1, b, acc);
  load_a64<3>(stage, lane, a1);
  load_codes<3>(stage, lane, ncol, c1);
  decode_b<2>(c0, sdw, b);
  mfma_block(a0, b, acc);
  decode_b<3>(c1, sdw, b);
  mfma_block(a1, b, acc);
}

// One 32-deep LoRA K-tile (t' x B in bf16).
__device__ __forceinline__ void lora_tile(const uint8_t* stage, uint32_t lane, const uint32_t (&ncol)[2],
                                          f32x16 (&acc)[8][2]) {
  bf16x8 a0[8], a1[8], b0[2], b1[2];
  load_a32<0>(stage, lane, a0);
  load_b32<0>(stage, lane, ncol, b0);
  load_a32<1>(stage, lane, a1);
  load_b32<1>(stage, lane, ncol, b1);
  mfma_block(a0, b0, acc);
  mfma_block(a1, b1, acc);
}

// Waits for every copy except the newest tile's (`newest` = the tile just issued, -1 if none),
// then barriers.
__device__ __forceinline__ void handover(int newest, int k_tiles) {
  if (newest < 0)
    stage_barrier<0>();
  else if (newest < k_tiles)
    stage_barrier<kCopiesBase>();
  else
    stage_barrier<kCopiesLora>();
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: keep it scalar

  // XCD-aware work index (gridDim.x is a multiple of 8)
  const int per_xcd = gridDim.x >> 3;
  const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (w >= p.m_tiles * p.n_tiles) return;
  const int mt = __builtin_amdgcn_readfirstlane(w / p.n_tiles);
  const int nt = __builtin_amdgcn_readfirstlane(w - mt * p.n_tiles);
  const int64_t m0 = static_cast<int64_t>(mt) * BM;

  Ctx c;
  c.k_tiles = p.k_tiles;
  c.wave = wave;
  c.lane = lane;
  c.act = rsrc(p.act, static_cast<uint32_t>(p.S * p.act_ld * 2));
  c.codes = rsrc(p.wcodes + static_cast<int64_t>(nt) * p.k_tiles * kCodeTileBytes,
                 static_cast<uint32_t>(p.k_tiles) * kCodeTileBytes);
  c.scales = rsrc(p.wscales + static_cast<int64_t>(nt) * p.k_tiles * kScaleTileBytes,
                  static_cast<uint32_t>(p.k_tiles) * kScaleTileBytes);
  c.lt = rsrc(p.lora_t, p.r_tiles ? static_cast<uint32_t>(p.S * p.lora_t_ld * 2) : 0u);
  c.lb = rsrc(reinterpret_cast<const uint8_t*>(p.lora_b) + static_cast<int64_t>(nt) * p.r_tiles * kLoraTileBytes,
              static_cast<uint32_t>(p.r_tiles) * kLoraTileBytes);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    {  // base tile slot (8w + h)*64 + lane -> row, chunk (see Ctx)
      const uint32_t row = (wave * 8 + h) * 8 + (lane >> 3);
      const uint32_t chunk = (lane & 7) ^ ((row >> 1) & 7);
      c.vact[h] = (static_cast<uint32_t>(m0) + row) * static_cast<uint32_t>(p.act_ld * 2) + chunk * 16;
    }
    {  // LoRA tile slot (4w + h)*64 + lane -> 128-byte line, then (row, chunk) of the 64-byte rows
      const uint32_t line = (wave * 4 + h) * 8 + (lane >> 3);
      const uint32_t cl = (lane & 7) ^ ((line >> 1) & 7);
      const uint32_t row = line * 2 + (cl >> 2), chunk = cl & 3;
      c.vlt[h] = (static_cast<uint32_t>(m0) + row) * static_cast<uint32_t>(p.lora_t_ld * 2) + chunk * 16;
      c.vlb[h] = row * (kLoraBK * 2) + chunk * 16;
    }
  }
  c.act_rows8 = static_cast<uint32_t>(p.act_ld * 16);
  c.lt_rows16 = static_cast<uint32_t>(p.lora_t_ld * 32);

  f32x16 acc[8][2];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i][0] = acc[i][1] = f32x16{};

  const uint32_t ncol[2] = {static_cast<uint32_t>(wave * 64) + (lane & 31),
                            static_cast<uint32_t>(wave * 64 + 32) + (lane & 31)};
  const int total = p.k_tiles + p.r_tiles;

  // prologue: tiles 0 and 1 in flight; wait for tile 0
  issue_tile(c, 0, smem);
  if (total > 1) issue_tile(c, 1, smem + kStage);
  handover(total > 1 ? 1 : -1, p.k_tiles);

  // tile kt is read from stage kt % 3 while tile kt + 2 is copied into stage (kt + 2) % 3
  int s_cur = 0;
  for (int kt = 0; kt < p.k_tiles; ++kt) {
    const int s_next = s_cur >= 1 ? s_cur - 1 : 2;  // (kt + 2) % 3
    const bool issue = kt + 2 < total;
    if (issue) issue_tile(c, kt + 2, smem + s_next * kStage);
    base_tile(smem + s_cur * kStage, lane, ncol, acc);
    handover(issue ? kt + 2 : -1, p.k_tiles);
    s_cur = s_cur == 2 ? 0 : s_cur + 1;
  }
  for (int kt = p.k_tiles; kt < total; ++kt) {
    const int s_next = s_cur >= 1 ? s_cur - 1 : 2;
    const bool issue = kt + 2 < total;
    if (issue) issue_tile(c, kt + 2, smem + s_next * kStage);
    lora_tile(smem + s_cur * kStage, lane, ncol, acc);
    handover(issue ? kt + 2 : -1, p.k_tiles);
    s_cur = s_cur == 2 ? 0 : s_cur + 1;
  }

  // Epilogue. Accumulator register r of lane l in a 32x32 tile holds
  // row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  const float scale = p.ts * (p.ts_dev ? *p.ts_dev : 1.0f);
  const int row_lane = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + i * 32 + (r >> 2) * 8 + row_lane + (r & 3);
      if (row >= p.S) continue;
      uint16_t* orow = p.out + row * p.out_ld;
      if (EPI == 0) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cl = static_cast<int>(ncol[j]);
          const int64_t n = p.gate_up ? packed_row_source(nt, cl, true, p.n_out) : static_cast<int64_t>(nt) * BN + cl;
          if (n >= 0 && n < p.n_out) orow[n] = static_cast<uint16_t>(f32_to_bf16_rne(scale * acc[i][j][r]));
        }
      } else {
        // this wave's 64 tile columns are 32 gate columns then the 32 matching up columns
        const int64_t n = static_cast<int64_t>(nt) * (BN / 2) + wave * 32 + (lane & 31);
        if (n < p.n_out) {
          const float g = scale * acc[i][0][r];
          const float u = scale * acc[i][1][r];
          orow[n] = static_cast<uint16_t>(f32_to_bf16_rne(silu(g) * u));
        }
      }
    }
  }
}

}  // namespace

size_t gemm_w4_lds_bytes() { return kLdsBytes; }

hipError_t launch_gemm_w4(const GemmParams& p0, Epilogue epi, hipStream_t stream) {
  const void* fn = epi == Epilogue::Plain ? reinterpret_cast<const void*>(&gemm_w4_kernel<0>)
                                          : reinterpret_cast<const void*>(&gemm_w4_kernel<1>);
  static std::once_flag once[2];
  static hipError_t attr_err[2] = {hipSuccess, hipSuccess};
  const int e = static_cast<int>(epi);
  std::call_once(once[e], [&] {
    attr_err[e] = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  });
  if (attr_err[e] != hipSuccess) return attr_err[e];

  // Buffer offsets are 32-bit: launch row ranges whose activation and t' spans stay below 2 GiB.
  const int64_t row_bytes = std::max<int64_t>(p0.act_ld, p0.lora_t_ld) * 2;
  const int64_t rows_per_launch = ((int64_t{1} << 31) - 1) / row_bytes / BM * BM;
  for (int64_t r0 = 0; r0 < p0.S; r0 += rows_per_launch) {
    GemmParams p = p0;
    p.S = std::min<int64_t>(rows_per_launch, p0.S - r0);
    p.act = p0.act + r0 * p0.act_ld;
    p.lora_t = p0.lora_t ? p0.lora_t + r0 * p0.lora_t_ld : nullptr;
    p.out = p0.out + r0 * p0.out_ld;
    p.m_tiles = static_cast<int32_t>((p.S + BM - 1) / BM);
    const int64_t items = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
    const int64_t grid = (items + 7) / 8 * 8;
    if (epi == Epilogue::Plain)
      hipLaunchKernelGGL(gemm_w4_kernel<0>, dim3(grid), dim3(kThreads), kLdsBytes, stream, p);
    else
      hipLaunchKernelGGL(gemm_w4_kernel<1>, dim3(grid), dim3(kThreads), kLdsBytes, stream, p);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace h3q
