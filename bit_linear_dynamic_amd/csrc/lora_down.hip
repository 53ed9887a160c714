// lora_down.hip -- the thin LoRA-down GEMM and the base-path activation prescale, for gfx950.
//
// LoRA-down (FL2VA Turbo, "Implementation": the bf16 branch A(x) on the ORIGINAL activation):
//   t'[s][j] = bf16( f * sum_k x[s][k] * A[j][k] ),   j < r_pad,   fp32 accumulation
// with f = strength * alpha / (rank * ts) (divided on the device by the W4A4 activation scale when
// there is one), so that the main GEMM can add t' x B into the same accumulator as the base term.
// The same pass writes the base path's operand xs = bf16(x * pqs) (same section: pre_quant_scale
// applies to the base path only), since it is already reading every element of x.
//
// Geometry: one workgroup of 4 wave64s per CU, bm = ceil(S / CUs) rows per workgroup (at least 32,
// at most what the accumulators hold) so that the rows spread evenly over the CUs in one round, in
// RTM = ceil(bm / 32) row tiles of 32 (rows of the last tile past bm read as zero and are not
// written). Every wave computes all RTM row tiles for its columns: the r_pad/32 column tiles of 32
// go to the waves round-robin, at most NC per wave, as RTM x NC tiles of v_mfma_f32_32x32x16_bf16.
// x is read once from HBM, so this is a streaming kernel: K is staged BK (64, or 32 when the A tile
// is large) at a time through as many LDS stages as fit (up to 8) by buffer->LDS copies of the x
// tile (RTM*32 x BK), the A tile (r_pad x BK) and BK pqs values, and the global latency is hidden by
// the bytes in flight rather than by compute. Each wave waits for its own copies with one vmcnt and
// a barrier hands the stage over. The waves also write xs = bf16(x * pqs), reading the tile back
// from LDS row by row so that every store covers whole 128-byte row segments (8 rows per store of a
// wave; stores of 32-byte pieces of 32 rows, straight from the MFMA operand registers, ran the write
// stream at a fraction of the read rate). Every vector-memory operation of the K loop is issued by
// the asm helpers of h3q_device.hpp in a fixed number per wave per tile (copies without a real
// source re-read into a spare LDS area, stores without a real target go past the buffer's end and
// are dropped), so one vmcnt value per iteration waits exactly for the tile about to be read.
//
// Prescale: the elementwise xs = bf16(x * pqs) on its own, for calls without an adapter.
#include <algorithm>
#include <mutex>

#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxRTM = 6;
constexpr uint32_t kLdsBudget = 150 * 1024;

// Stage bytes for K-tiles of depth bk: x tile, A tile, pqs (256 B), 1 KiB target of padding copies.
constexpr uint32_t ld_stage_bytes(int rtm, int nc, int bk) {
  return static_cast<uint32_t>(rtm * 32 * bk * 2 + 4 * nc * 32 * bk * 2 + 256 + 1024);
}

template <int RTM, int NC>
struct LdGeo {
  // 64-deep tiles (128-byte row segments) when three stages of them fit, else 32-deep
  static constexpr int BK = 3 * ld_stage_bytes(RTM, NC, 64) <= kLdsBudget ? 64 : 32;
  static constexpr int CT = 4 * NC;                      // column tiles the A stage is sized for
  static constexpr uint32_t kX = 0;                      // x tile: RTM*32 rows x 2*BK bytes
  static constexpr uint32_t kA = RTM * 32 * BK * 2;      // A tile: CT*32 rows x 2*BK bytes
  static constexpr uint32_t kP = kA + CT * 32 * BK * 2;  // BK pqs values
  static constexpr uint32_t kSpare = kP + 256;           // 1 KiB target of padding copies
  static constexpr uint32_t kStage = kSpare + 1024;
  static constexpr int kStagesFit = static_cast<int>(kLdsBudget / kStage);
  static constexpr int kStages = kStagesFit < 8 ? kStagesFit : 8;
  static constexpr int L = kStages - 1;                  // tiles in flight ahead of the one read
  static constexpr uint32_t kLds = kStages * kStage;
  static constexpr int kCopiesX = (RTM * BK / 16 + 3) / 4;  // 1 KiB copies per wave (RTM*BK/16 per tile)
  static constexpr int kCopiesA = NC * BK / 16;             // (at most CT*BK/16 per tile)
  static constexpr int kPqsLanes = BK / 16;                 // 16 bytes each, per wave
  static constexpr int CPT = kCopiesX + kCopiesA + 1;
  static constexpr int kChunks = RTM * 32 * (BK / 8);       // 16-byte xs chunks per tile
  static constexpr int NS = (kChunks + 255) / 256;          // xs stores per wave per tile
  static_assert(ld_stage_bytes(RTM, NC, BK) == kStage, "stage layout");
  static_assert(kStages >= 3, "at least two tiles in flight");
  static_assert((L - 1) * CPT + L * NS < 64, "vmcnt range");
};

// Loads 8 bf16 of x at (row, k) -- zeros past K (K is a multiple of 16, so chunks never straddle).
__device__ __forceinline__ u32x4 load_x_chunk(const uint16_t* x, int64_t row, int64_t K, int64_t k) {
  if (k >= K) return u32x4{0u, 0u, 0u, 0u};
  return *reinterpret_cast<const u32x4*>(x + row * K + k);
}

// bf16(x * pqs) of 8 consecutive elements (pqs values given), rounded by the hardware pair
// conversion: the bit-level rounding (5 VALU per value) sat on the LoRA-down's critical path.
__device__ __forceinline__ u32x4 scale_chunk(u32x4 xv, const float (&ps)[8]) {
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    out[i] = bf16x2_hw(bf16_bits_to_f32(xv[i] & 0xffffu) * ps[2 * i],
                       __uint_as_float(xv[i] & 0xffff0000u) * ps[2 * i + 1]);
  return out;
}

// bf16(x * pqs) for 8 consecutive elements starting at k (pqs null = 1; past K: zero).
__device__ __forceinline__ u32x4 prescale_chunk(u32x4 xv, const float* pqs, int64_t K, int64_t k) {
  if (!pqs || k >= K) return xv;
  const f32x4 p0 = *reinterpret_cast<const f32x4*>(pqs + k);
  const f32x4 p1 = *reinterpret_cast<const f32x4*>(pqs + k + 4);
  const float ps[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
  return scale_chunk(xv, ps);
}

// Per-lane source offset of 1 KiB copy q of a BK-deep tile whose rows are `row_bytes` apart; the
// copy fills LDS slots q*64 + lane of 128-byte lines, line L = q*8 + lane/8.
//   BK = 64: line L is row L, position lane % 8 holds chunk (lane % 8) ^ ((L / 2) % 8) -- the
//            layout lds_chunk_offset reads;
//   BK = 32: line L holds rows 2L and 2L + 1, position lane % 8 holds chunk (lane % 8) ^ ((L / 2) % 8)
//            of the pair (bit 2: which row, bits 0..1: which 16 bytes) -- lds_chunk_offset32.
template <int BK>
__device__ __forceinline__ uint32_t copy_src_offset(uint32_t q, uint32_t lane, uint32_t row_bytes) {
  const uint32_t line = q * 8 + (lane >> 3);
  const uint32_t cl = (lane & 7) ^ ((line >> 1) & 7);
  if constexpr (BK == 64) return line * row_bytes + cl * 16;
  else return (line * 2 + (cl >> 2)) * row_bytes + (cl & 3) * 16;
}

// Column within the tile (0 .. BK - 8) of the 16 bytes that copy q brings to this lane's slot.
template <int BK>
__device__ __forceinline__ uint32_t copy_src_column(uint32_t q, uint32_t lane) {
  const uint32_t line = q * 8 + (lane >> 3);
  const uint32_t cl = (lane & 7) ^ ((line >> 1) & 7);
  if constexpr (BK == 64) return cl * 8;
  else return (cl & 3) * 8;
}

// A per-lane offset past the end of the x descriptor (which spans under 2^31 bytes): the copy reads
// zeros. Adding the tile's column offset (under 2^21 bytes) cannot wrap it past 2^32.
constexpr uint32_t kOutOfRange = 0x80000000u;

template <int BK>
__device__ __forceinline__ uint32_t tile_offset(uint32_t row, uint32_t chunk) {
  if constexpr (BK == 64) return lds_chunk_offset(row, chunk);
  else return lds_chunk_offset32(row, chunk);
}

struct LdCtx {
  u32x4 x, A, pq, xs;
  uint32_t x_row_bytes, A_row_bytes;
  uint32_t K;
  uint32_t wave, lane;
  int k_tiles, x_copies, A_copies;  // real copies per tile for the whole workgroup
};

// Issues this wave's copies of K-tile kt (a re-read of the last tile when kt is past the end).
template <int RTM, int NC>
__device__ __forceinline__ void issue_tile(const LdCtx& c, int kt, uint32_t stage) {
  using G = LdGeo<RTM, NC>;
  constexpr int BK = G::BK;
  const uint32_t k0 = static_cast<uint32_t>(kt < c.k_tiles ? kt : c.k_tiles - 1) * BK;
#pragma unroll
  for (int i = 0; i < G::kCopiesX; ++i) {
    const uint32_t q = c.wave + 4 * i;
    const bool real = static_cast<int>(q) < c.x_copies;
    const uint32_t qs = real ? q : 0;
    // x rows are K elements apart, so the 16 bytes past a row's end are the next row's first
    // elements: columns at or past K read as zero instead (A is zero there, but 0 * inf is not 0).
    const uint32_t voff = k0 + copy_src_column<BK>(qs, c.lane) < c.K ? copy_src_offset<BK>(qs, c.lane, c.x_row_bytes)
                                                                    : kOutOfRange;
    dma16(c.x, stage + (real ? G::kX + q * 1024 : G::kSpare), voff, k0 * 2);
  }
#pragma unroll
  for (int i = 0; i < G::kCopiesA; ++i) {
    const uint32_t q = c.wave + 4 * i;
    const bool real = static_cast<int>(q) < c.A_copies;
    dma16(c.A, stage + (real ? G::kA + q * 1024 : G::kSpare), copy_src_offset<BK>(real ? q : 0, c.lane, c.A_row_bytes),
          k0 * 2);
  }
  dma16_lanes<G::kPqsLanes>(c.pq, stage + G::kP + c.wave * (BK * 1), c.lane * 16, k0 * 4 + c.wave * (BK * 1));
}

// Waits for tile kt: newer than its copies are those of the L - 1 tiles after it and the xs
// stores of the min(kt, L) iterations since it was issued.
template <int L, int CPT, int NS>
__device__ __forceinline__ void wait_tile(int kt) {
  switch (kt < L ? kt : L) {
    case 0: stage_barrier<(L - 1) * CPT>(); break;
    case 1: stage_barrier<(L - 1) * CPT + 1 * NS>(); break;
    case 2: stage_barrier<(L - 1) * CPT + 2 * NS>(); break;
    case 3: stage_barrier<(L - 1) * CPT + 3 * NS>(); break;
    case 4: stage_barrier<(L - 1) * CPT + 4 * NS>(); break;
    case 5: stage_barrier<(L - 1) * CPT + 5 * NS>(); break;
    case 6: stage_barrier<(L - 1) * CPT + 6 * NS>(); break;
    default: stage_barrier<(L - 1) * CPT + 7 * NS>(); break;
  }
}

template <int RTM, int NC, bool XS>
__global__ __launch_bounds__(kThreads, 1) void lora_down_kernel(LoraDownParams p) {
  using G = LdGeo<RTM, NC>;
  constexpr int L = G::L, CPT = G::CPT, NS = XS ? G::NS : 0, NST = G::kStages, BK = G::BK;
  static_assert(L <= 7, "wait_tile covers up to 7 tiles in flight");
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t m0 = static_cast<int64_t>(blockIdx.x) * p.bm;
  const int64_t rows = std::min<int64_t>(p.bm, p.S - m0);  // <= 32 * RTM
  const int ct = p.r_pad / 32;  // column tiles: wave w owns tiles w, w + 4, ... (< ct)

  LdCtx c;
  c.wave = wave;
  c.lane = lane;
  // K_pad / BK tiles (K_pad is a multiple of 64): with 32-deep tiles that can be one tile past
  // ceil(K / BK), whose x columns are all padding, so xs is written with zeros out to K_pad -- the
  // GEMM reads K_pad columns of it, and the workspace holds whatever an earlier call left there.
  c.k_tiles = static_cast<int>(p.K_pad / BK);
  c.K = static_cast<uint32_t>(p.K);
  c.x_copies = RTM * BK / 16;
  c.A_copies = ct * BK / 16;
  c.x_row_bytes = static_cast<uint32_t>(p.K * 2);
  c.A_row_bytes = static_cast<uint32_t>(p.K_pad * 2);
  c.x = buf_rsrc(p.x + m0 * p.K, static_cast<uint32_t>(rows * p.K * 2));
  c.A = buf_rsrc(p.A, static_cast<uint32_t>(int64_t{p.r_pad} * p.K_pad * 2));
  c.pq = buf_rsrc(p.pqs, p.pqs ? static_cast<uint32_t>(p.K * 4) : 0u);
  c.xs = buf_rsrc(p.xs_out + m0 * p.K_pad,
                  XS ? static_cast<uint32_t>(rows * p.K_pad * 2) : 0u);

  f32x16 acc[RTM][NC];
#pragma unroll
  for (int i = 0; i < RTM; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[i][j] = f32x16{};

  const uint32_t smem0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)(smem)));
  const uint32_t r32 = lane & 31, h32 = lane >> 5;

#pragma unroll
  for (int t = 0; t < L; ++t) issue_tile<RTM, NC>(c, t, smem0 + t * G::kStage);
  int s_cur = 0;
  // Not unrolled: unrolled by the stage count, some shapes had their accumulators moved between
  // AGPRs and VGPRs hundreds of times per tile and ran at a third of the copy rate.
#pragma unroll 1
  for (int kt = 0; kt < c.k_tiles; ++kt) {
    wait_tile<L, CPT, NS>(kt);
    const int s_iss = s_cur == 0 ? NST - 1 : s_cur - 1;  // (kt + L) % NST: the stage of tile kt - 1
    issue_tile<RTM, NC>(c, kt + L, smem0 + s_iss * G::kStage);
    const uint8_t* st = smem + s_cur * G::kStage;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      // Column tile jt = wave + 4j is always inside the stage's A area (CT = 4 NC tiles); a tile at or
      // past ct holds no copy of A, and its accumulator is computed but never stored. No branch: with
      // one, the compiler moved the accumulators between AGPRs and VGPRs around every MFMA.
      bf16x8 a[RTM], b[NC];
#pragma unroll
      for (int i = 0; i < RTM; ++i)
        a[i] = *reinterpret_cast<const bf16x8*>(st + G::kX + tile_offset<BK>(i * 32 + r32, kk * 2 + h32));
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int jt = static_cast<int>(wave) + 4 * j;
        b[j] = *reinterpret_cast<const bf16x8*>(st + G::kA + tile_offset<BK>(jt * 32 + r32, kk * 2 + h32));
      }
#pragma unroll
      for (int i = 0; i < RTM; ++i)
#pragma unroll
        for (int j = 0; j < NC; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
    if constexpr (XS) {
      // xs = bf16(x * pqs) of the whole tile from its LDS copy, row-major: chunk q of the workgroup
      // (16 bytes) is row q / (BK/8), chunk q % (BK/8), so one store of a wave covers 8 (BK = 64) or
      // 16 (BK = 32) rows of full row segments. A lane's chunks all sit at the same column
      // (lane % (BK/8)), so its 8 pqs values are read once; all NS chunks are read before the first
      // store, so the LDS latency is paid once. Every wave issues NS stores; chunks past the tile go
      // past the buffer's end and are dropped.
      constexpr bool kAllReal = G::kChunks % 256 == 0;
      const uint32_t cc = lane % (BK / 8);
      float ps[8];
      if (p.pqs) {
        const f32x4 q0 = *reinterpret_cast<const f32x4*>(st + G::kP + cc * 32);
        const f32x4 q1 = *reinterpret_cast<const f32x4*>(st + G::kP + cc * 32 + 16);
        ps[0] = q0.x; ps[1] = q0.y; ps[2] = q0.z; ps[3] = q0.w;
        ps[4] = q1.x; ps[5] = q1.y; ps[6] = q1.z; ps[7] = q1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) ps[e] = 1.0f;
      }
      u32x4 xv[NS];
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const uint32_t row = (wave * 64 + lane + 256u * q) / (BK / 8);
        const bool real = kAllReal || static_cast<int>(wave * 64 + lane + 256u * q) < G::kChunks;
        xv[q] = real ? *reinterpret_cast<const u32x4*>(st + G::kX + tile_offset<BK>(row, cc)) : u32x4{0u, 0u, 0u, 0u};
      }
      if (static_cast<int64_t>(kt + 1) * BK > p.K) {  // the last tile: padding columns become zero
        const bool pad = static_cast<uint32_t>(kt) * BK + cc * 8 >= p.K;
#pragma unroll
        for (int q = 0; q < NS; ++q)
          if (pad) xv[q] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (pad) ps[e] = 1.0f;
      }
#pragma unroll
      for (int q = 0; q < NS; ++q) {
        const uint32_t chunk = wave * 64 + lane + 256u * q;
        const bool real = kAllReal || static_cast<int>(chunk) < G::kChunks;
        const u32x4 out = scale_chunk(xv[q], ps);
        // (the dummy offset stays out of range with the tile's column offset added: < 2^31 + 2^21)
        buf_store16(out, c.xs, real ? (chunk / (BK / 8)) * static_cast<uint32_t>(p.K_pad * 2) + cc * 16 : 0x7ffffff0u,
                    static_cast<uint32_t>(kt) * BK * 2);
      }
    }
    s_cur = s_cur == NST - 1 ? 0 : s_cur + 1;
  }
  wait_vmcnt<0>();  // drain the trailing copies and stores before the workgroup can end

  const float f = p.f_div_dev ? p.f / *p.f_div_dev : p.f;
  const int row_lane = (lane >> 5) * 4;
  const int R = p.r_pad;
#pragma unroll
  for (int i = 0; i < RTM; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t rl = i * 32 + (r >> 2) * 8 + row_lane + (r & 3);
      if (rl >= rows) continue;
      const int64_t row = m0 + rl;
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int jt = static_cast<int>(wave) + 4 * j;
        if (jt < ct) p.t_out[row * R + jt * 32 + r32] = static_cast<uint16_t>(f32_to_bf16_hw(f * acc[i][j][r]));
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

template <int RTM, int NC, bool XS>
hipError_t launch_rt(const LoraDownParams& p, int64_t blocks, hipStream_t stream) {
  constexpr uint32_t lds = LdGeo<RTM, NC>::kLds;
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&lora_down_kernel<RTM, NC, XS>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  });
  if (attr_err != hipSuccess) return attr_err;
  hipLaunchKernelGGL((lora_down_kernel<RTM, NC, XS>), dim3(blocks), dim3(kThreads), lds, stream, p);
  return hipGetLastError();
}

template <int RTM, int NC>
hipError_t launch_x(const LoraDownParams& p, int64_t blocks, hipStream_t stream) {
  return p.xs_out ? launch_rt<RTM, NC, true>(p, blocks, stream) : launch_rt<RTM, NC, false>(p, blocks, stream);
}

// Row tiles per workgroup allowed with NC column tiles per wave: the RTM x NC accumulator tiles
// (16 registers each) must stay within the 256 accumulation registers.
constexpr int max_rtm(int nc) { return nc <= 2 ? kMaxRTM : (nc == 3 ? 5 : 3); }

template <int RTM, int NC>
hipError_t launch_fit(const LoraDownParams& p, int64_t blocks, hipStream_t stream) {
  if constexpr (RTM <= max_rtm(NC)) return launch_x<RTM, NC>(p, blocks, stream);
  else return hipErrorInvalidValue;  // never chosen by launch_lora_down
}

template <int RTM>
hipError_t launch_nc(const LoraDownParams& p, int nc, int64_t blocks, hipStream_t stream) {
  switch (nc) {  // column tiles per wave
    case 1: return launch_fit<RTM, 1>(p, blocks, stream);
    case 2: return launch_fit<RTM, 2>(p, blocks, stream);
    case 3: return launch_fit<RTM, 3>(p, blocks, stream);
    case 4: return launch_fit<RTM, 4>(p, blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_lora_down(const LoraDownParams& p, hipStream_t stream) {
  if (p.S == 0) return hipSuccess;
  if (p.r_pad <= 0 || p.r_pad % 32 != 0 || p.r_pad > 512) return hipErrorInvalidValue;
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  if (cus <= 0) return hipErrorInvalidValue;
  // rows per workgroup: spread the rows evenly over the CUs in one round (at least one row tile of
  // 32, at most the row tiles whose accumulators fit beside the column tiles each wave holds)
  const int nc = (p.r_pad / 32 + 3) / 4;
  LoraDownParams q = p;
  q.bm = std::min<int64_t>(32 * max_rtm(nc), std::max<int64_t>(32, (p.S + cus - 1) / cus));
  const int rtm = static_cast<int>((q.bm + 31) / 32);
  const int64_t blocks = (p.S + q.bm - 1) / q.bm;
  switch (rtm) {
    case 1: return launch_nc<1>(q, nc, blocks, stream);
    case 2: return launch_nc<2>(q, nc, blocks, stream);
    case 3: return launch_nc<3>(q, nc, blocks, stream);
    case 4: return launch_nc<4>(q, nc, blocks, stream);
    case 5: return launch_nc<5>(q, nc, blocks, stream);
    default: return launch_nc<6>(q, nc, blocks, stream);
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
