// lora_down.hip -- the thin LoRA-down GEMM and the base-path activation prescale, for gfx950.
//
// LoRA-down (FL2VA Turbo, "Implementation": the bf16 branch A(x) on the ORIGINAL activation):
//   t'[s][j] = bf16( f * sum_k x[s][k] * A[j][k] ),   j < r_pad,   fp32 accumulation
// with f = strength * alpha / (rank * ts) (divided on the device by the W4A4 activation scale when
// there is one), so that the main GEMM can add t' x B into the same accumulator as the base term.
// The same pass writes the base path's operand xs = bf16(x * pqs) (same section: pre_quant_scale
// applies to the base path only), since it is already reading every element of x.
//
// Geometry: one workgroup of 4 wave64s per CU. The r_pad/32 column tiles of A are split into
// `groups` column groups (1, 2 or 4, chosen by the launcher); each row block of bm rows (at least
// 32, at most what the accumulators hold) has one workgroup per group, so the row blocks times the
// groups spread over the CUs in one round. A workgroup holds RTM = ceil(bm / 32) row tiles of 32
// (rows of the last tile past bm read as zero and are not written); every wave computes all RTM row
// tiles for its columns: the group's column tiles go to the waves round-robin, at most NC per wave,
// as RTM x NC tiles of v_mfma_f32_32x32x16_bf16. Each group writes its columns of t' and its slice of
// the block's xs rows.
//
// x is read once from HBM and xs written once, while every workgroup copies all of its group's A tiles
// from L2 into LDS; those byte streams, not the MFMAs, set the kernel's time (without the MFMAs it
// runs as fast; without the A copies or the xs stores, a quarter faster). K goes through in BK-deep tiles (64, or 32 when each wave holds more than one column tile) on
// two separate rings of LDS slots, both filled by buffer->LDS copies (no registers): the adapter tile
// A (r_pad x BK, from L2, where every workgroup reads it) one tile ahead in two slots, and the x tile
// (RTM*32 x BK) with its BK pqs values L tiles ahead in L + 2 slots -- all the LDS the two A slots
// leave is x in flight (80 KiB at r = 384 and at r = 128, against 30 and 60 KiB when every stage held
// an A tile and its x tile). Each step issues the A tile first and the x tile after it, so waiting
// for the A tile it is about to read never waits for the x tiles behind it; the x tile it reads is
// older than that A tile, so it has landed too. One vmcnt value per step parity and a barrier hand
// the slots over. xs = bf16(x * pqs) is written from the LDS copy of each 64-deep tile, or of two
// 32-deep tiles after the second, so that each 16-byte store is one chunk of a 128-byte row segment
// and a wave's store covers 8 whole segments.
// Every vector-memory operation of the K loop is issued by the asm helpers of h3q_device.hpp in a
// fixed number per wave (copies without a real source go to a spare LDS area, stores without a real
// target go past the buffer's end and are dropped), so the counts behind each vmcnt are exact.
//
// Prescale: the elementwise xs = bf16(x * pqs) on its own, for calls without an adapter.
#include <algorithm>
#include <mutex>

#include "h3q_device.hpp"
#include "h3q_kernels.hpp"

namespace h3q {

namespace {

constexpr int kThreads = 256;
constexpr uint32_t kLdsBudget = 160 * 1024;
constexpr int kMaxAhead = 10;            // x tiles in flight at most

template <int RTM, int NC>
struct LdGeo {
  // K per tile: 64 (128-byte row segments of x and xs) when the adapter tile is small (one column
  // tile per wave), else 32, which leaves room for more x tiles in flight beside the two A tiles.
  // (Measured at S = 37726: r = 384 0.374 -> 0.301 ms against A staged as deep as x; 32-deep tiles
  // at r = 128 were 3-7 % slower than 64-deep ones, and a second A tile ahead at r = 384, which takes
  // two x tiles out of flight, was 20 % slower.)
  static constexpr int BK = NC == 1 ? 64 : 32;
  static constexpr int LA = 1;                                // A tiles issued ahead
  static constexpr int NA = LA + 1;                           // A slots
  static constexpr int CT = 4 * NC;                           // column tiles the A slots hold
  static constexpr uint32_t kASlot = CT * 32 * BK * 2;        // A tile: CT*32 rows x 2*BK bytes
  static constexpr uint32_t kXTile = RTM * 32 * BK * 2;       // x tile: RTM*32 rows x 2*BK bytes
  static constexpr uint32_t kXSlot = kXTile + BK * 4;         // + the tile's pqs values
  static constexpr uint32_t kSpare = NA * kASlot;             // 1 KiB target of copies without a source
  static constexpr uint32_t kX0 = kSpare + 1024;              // first x slot
  static constexpr int kCX = (RTM * BK / 16 + 3) / 4;         // 1 KiB x copies per wave (RTM*BK/16 per tile)
  static constexpr int kCA = NC * BK / 16;                    // 1 KiB A copies per wave (CT*BK/16 per tile)
  static constexpr int kXOps = kCX + 1;                       // + one pqs copy (BK/16 lanes per wave)
  // xs stores per wave: 64-deep tiles store each tile (RTM per step); 32-deep tiles store two tiles
  // at once after the odd step, so that every store is a chunk of a 128-byte row segment
  static constexpr int kStEven = BK == 64 ? RTM : 0, kStOdd = RTM;
  static constexpr int kFit = static_cast<int>((kLdsBudget - kX0) / kXSlot) - 2;
  // Operations a wave can have in flight: LA A tiles, L x tiles, two xs store rounds; kept below 64
  // so that every count stays within the vmcnt field.
  static constexpr int kVm = (63 - LA * kCA - 2 * RTM) / kXOps;
  static constexpr int kL0 = kFit < kVm ? kFit : kVm;
  static constexpr int L = kL0 < kMaxAhead ? kL0 : kMaxAhead;  // x tiles issued ahead
  static constexpr int NX = L + 2;                            // x slots: L in flight, 2 being read
  static constexpr uint32_t kLds = kX0 + NX * kXSlot;
  static_assert(L > LA, "x tiles must be issued further ahead than A tiles");
  static_assert(kLds <= kLdsBudget, "LDS");
  static_assert(LA * kCA + L * kXOps + 2 * RTM < 64, "vmcnt range");
  // vmcnt to wait for A tile kt at the top of step kt: everything issued after it -- the x tile
  // that step kt - 1 issued after A(kt) and that step's xs stores (none without an xs output);
  static constexpr int wait_steady(int parity, bool xs) {  // parity of kt
    return kXOps + (xs ? (parity ? kStEven : kStOdd) : 0);
  }
  // at step 0, the x tiles 1 .. L - 1 that the prologue issued after A(0).
  static constexpr int wait_first0 = (L - 1) * kXOps;
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

template <int BK>
__device__ __forceinline__ uint32_t tile_offset(uint32_t row, uint32_t chunk) {
  if constexpr (BK == 64) return lds_chunk_offset(row, chunk);
  else return lds_chunk_offset32(row, chunk);
}

// A per-lane offset past the end of the x descriptor (which spans under 2^31 bytes): the copy reads
// zeros. Adding the tile's column offset (under 2^21 bytes) cannot wrap it past 2^32.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct LdCtx {
  u32x4 x, A, pq, xs;
  uint32_t x_row_bytes, A_row_bytes, xs_row_bytes;
  uint32_t K;
  uint32_t wave, lane;
  int k_tiles, x_copies;  // real x copies per tile for the whole workgroup
  uint32_t smem0;
  uint32_t xs_lo, xs_hi;  // rows of the block whose xs this workgroup writes
};

// This wave's copies of A tile kt into A slot `slot` (to the spare area past the last tile).
template <int RTM, int NC>
__device__ __forceinline__ void issue_A(const LdCtx& c, int kt, int slot) {
  using G = LdGeo<RTM, NC>;
  const bool real = kt < c.k_tiles;
  const uint32_t k0 = static_cast<uint32_t>(real ? kt : 0) * G::BK;
#pragma unroll
  for (int i = 0; i < G::kCA; ++i) {
    const uint32_t q = c.wave + 4 * i;
    dma16(c.A, c.smem0 + (real ? slot * G::kASlot + q * 1024 : G::kSpare),
          copy_src_offset<G::BK>(q, c.lane, c.A_row_bytes), k0 * 2);
  }
}

// This wave's copies of x tile kt and its pqs values into x slot `slot` (to the spare area past the
// last tile).
template <int RTM, int NC>
__device__ __forceinline__ void issue_x(const LdCtx& c, int kt, int slot) {
  using G = LdGeo<RTM, NC>;
  constexpr int BK = G::BK;
  const bool tile = kt < c.k_tiles;
  const uint32_t k0 = static_cast<uint32_t>(tile ? kt : 0) * BK;
  const uint32_t base = c.smem0 + G::kX0 + static_cast<uint32_t>(slot) * G::kXSlot;
#pragma unroll
  for (int i = 0; i < G::kCX; ++i) {
    const uint32_t q = c.wave + 4 * i;
    const bool real = tile && static_cast<int>(q) < c.x_copies;
    const uint32_t qs = real ? q : 0;
    // x rows are K elements apart, so the 16 bytes past a row's end are the next row's first
    // elements: columns at or past K read as zero instead (A is zero there, but 0 * inf is not 0).
    const uint32_t voff = k0 + copy_src_column<BK>(qs, c.lane) < c.K ? copy_src_offset<BK>(qs, c.lane, c.x_row_bytes)
                                                                     : kOutOfRange;
    dma16(c.x, real ? base + q * 1024 : c.smem0 + G::kSpare, voff, k0 * 2);
  }
  // the tile's BK pqs values: lanes 0 .. BK/16 - 1 of every wave copy BK bytes
  dma16_lanes<BK / 16>(c.pq, tile ? base + G::kXTile + c.wave * BK : c.smem0 + G::kSpare, c.lane * 16,
                       k0 * 4 + c.wave * BK);
}

// The MFMAs of one tile: x operand from x slot xb, A operand from A slot ab.
template <int RTM, int NC>
__device__ __forceinline__ void mfma_tile(f32x16 (&acc)[RTM][NC], const uint8_t* xb, const uint8_t* ab,
                                          uint32_t wave, uint32_t r32, uint32_t h32) {
  constexpr int BK = LdGeo<RTM, NC>::BK;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    // Column tile jt = wave + 4j is always inside the A slot (CT = 4 NC tiles); a tile at or past ct
    // holds zeros (rows past r_pad read as zero) and its accumulator is never stored. No branch: with
    // one, the compiler moved the accumulators between AGPRs and VGPRs around every MFMA.
    bf16x8 a[RTM], b[NC];
#pragma unroll
    for (int i = 0; i < RTM; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(xb + tile_offset<BK>(i * 32 + r32, kk * 2 + h32));
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const uint32_t jt = wave + 4 * j;
      b[j] = *reinterpret_cast<const bf16x8*>(ab + tile_offset<BK>(jt * 32 + r32, kk * 2 + h32));
    }
#pragma unroll
    for (int i = 0; i < RTM; ++i)
#pragma unroll
      for (int j = 0; j < NC; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// xs = bf16(x * pqs) of 64 columns from the LDS copies of the x tile(s) -- columns [64 kp, 64 kp + 64)
// -- row-major: chunk q of the workgroup (16 bytes) is row q / 8, chunk q % 8 of the 128-byte row
// segment, so one store of a wave covers 8 whole segments. With 32-deep tiles chunks 0..3 come from
// the tile in slot x0 and chunks 4..7 from the next tile in slot x1; with 64-deep tiles all from x0.
// A lane's chunks all sit at the same 8 columns, so its pqs values are read once; all RTM chunks are
// read before the first store. Rows past the workgroup's rows go past the buffer's end and are
// dropped; columns past K are zero (x and pqs read as zero there).
template <int RTM, int NC>
__device__ __forceinline__ void xs_store(const LdCtx& c, const uint8_t* x0, const uint8_t* x1, int kp, bool has_pqs) {
  using G = LdGeo<RTM, NC>;
  constexpr int BK = G::BK;
  const uint32_t cc = c.lane & 7;
  const uint8_t* xb = (BK == 64 || cc < 4) ? x0 : x1;
  const uint32_t ch = BK == 64 ? cc : (cc & 3);
  float ps[8];
  if (has_pqs) {
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(xb + G::kXTile + ch * 32);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(xb + G::kXTile + ch * 32 + 16);
    ps[0] = q0.x; ps[1] = q0.y; ps[2] = q0.z; ps[3] = q0.w;
    ps[4] = q1.x; ps[5] = q1.y; ps[6] = q1.z; ps[7] = q1.w;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) ps[e] = 1.0f;
  }
  u32x4 xv[RTM];
#pragma unroll
  for (int q = 0; q < RTM; ++q) {
    const uint32_t row = (c.wave * 64 + c.lane + 256u * q) >> 3;
    xv[q] = *reinterpret_cast<const u32x4*>(xb + tile_offset<BK>(row, ch));
  }
#pragma unroll
  for (int q = 0; q < RTM; ++q) {
    const uint32_t row = (c.wave * 64 + c.lane + 256u * q) >> 3;
    const uint32_t voff = row >= c.xs_lo && row < c.xs_hi ? (row - c.xs_lo) * c.xs_row_bytes + cc * 16 : kOutOfRange;
    buf_store16(scale_chunk(xv[q], ps), c.xs, voff, static_cast<uint32_t>(kp) * 128);
  }
}

template <int RTM, int NC, bool XS>
__global__ __launch_bounds__(kThreads, 1) void lora_down_kernel(LoraDownParams p) {
  using G = LdGeo<RTM, NC>;
  constexpr int BK = G::BK, L = G::L, LA = G::LA, NX = G::NX, NA = G::NA;
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const uint32_t lane = threadIdx.x & 63;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Workgroup -> (row block, column group): the groups of one row block run on one XCD (consecutive
  // workgroups go to different XCDs), so x is fetched from HBM once for all of them.
  const int groups = p.groups;
  const int64_t rb = static_cast<int64_t>(blockIdx.x / (8 * groups)) * 8 + blockIdx.x % 8;
  const int grp = static_cast<int>((blockIdx.x / 8) % groups);
  const int64_t m0 = rb * p.bm;
  if (m0 >= p.S) return;  // padding of the grid to whole groups of 8 row blocks
  const int64_t rows = std::min<int64_t>(p.bm, p.S - m0);  // <= 32 * RTM
  const int ctg = p.r_pad / 32 / groups;  // column tiles of this group: [grp * ctg, grp * ctg + ctg)
  // xs: each group of the row block writes its own slice of the rows
  const int64_t xs_slice = (rows + groups - 1) / groups;
  const int64_t xs_lo = std::min<int64_t>(rows, grp * xs_slice), xs_hi = std::min<int64_t>(rows, xs_lo + xs_slice);

  LdCtx c;
  c.wave = wave;
  c.lane = lane;
  // K_pad / BK tiles (K_pad is a multiple of 64: the count is even for 32-deep tiles and may be odd
  // for 64-deep ones): xs is written with zeros out to K_pad -- the GEMM reads K_pad columns of it,
  // and the workspace holds whatever an earlier call left there.
  c.k_tiles = static_cast<int>(p.K_pad / BK);
  c.K = static_cast<uint32_t>(p.K);
  c.x_copies = RTM * BK / 16;
  c.x_row_bytes = static_cast<uint32_t>(p.K * 2);
  c.A_row_bytes = static_cast<uint32_t>(p.K_pad * 2);
  c.xs_row_bytes = static_cast<uint32_t>(p.K_pad * 2);
  c.x = buf_rsrc(p.x + m0 * p.K, static_cast<uint32_t>(rows * p.K * 2));
  c.A = buf_rsrc(p.A + static_cast<int64_t>(grp) * ctg * 32 * p.K_pad, static_cast<uint32_t>(int64_t{ctg} * 32 * p.K_pad * 2));
  c.pq = buf_rsrc(p.pqs, p.pqs ? static_cast<uint32_t>(p.K * 4) : 0u);
  c.xs = buf_rsrc(p.xs_out + (m0 + xs_lo) * p.K_pad, XS ? static_cast<uint32_t>((xs_hi - xs_lo) * p.K_pad * 2) : 0u);
  c.xs_lo = static_cast<uint32_t>(xs_lo);
  c.xs_hi = static_cast<uint32_t>(xs_hi);
  c.smem0 = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)(smem)));
  const bool has_pqs = p.pqs != nullptr;

  f32x16 acc[RTM][NC];
#pragma unroll
  for (int i = 0; i < RTM; ++i)
#pragma unroll
    for (int j = 0; j < NC; ++j) acc[i][j] = f32x16{};

  const uint32_t r32 = lane & 31, h32 = lane >> 5;
  const uint8_t* xslot0 = smem + G::kX0;

  // Prologue: x(0), A(0), then x(1) .. x(L - 1): every A tile follows the x tile of the same index,
  // so waiting for an A tile also waits for its x tile.
  issue_x<RTM, NC>(c, 0, 0);
  issue_A<RTM, NC>(c, 0, 0);
#pragma unroll
  for (int t = 1; t < L; ++t) issue_x<RTM, NC>(c, t, t);

  // Step kt reads x slot kt % NX and A slot kt % 2; it first issues A tile kt + 1 into the A slot
  // read at step kt - 1, then x tile kt + L into x slot (kt + L) % NX, that of tile kt - 2, whose
  // MFMAs and xs stores were issued before the barrier that opened step kt - 1 or kt.
  int sx = 0, sa = 0;  // kt % NX, kt % NA
  // Steps go in pairs (even, odd) so that each wait count is a constant; the pair loop is not
  // unrolled further: unrolled by the stage count, some shapes had their accumulators moved between
  // AGPRs and VGPRs hundreds of times per tile.
  int kt = 0;
#pragma unroll 1
  for (; kt + 1 < c.k_tiles; kt += 2) {
    const int sx1 = sx + 1 == NX ? 0 : sx + 1;
    const int sa1 = sa + 1 == NA ? 0 : sa + 1;
    const int sal = sa + LA >= NA ? sa + LA - NA : sa + LA;     // (kt + LA) % NA
    const int sal1 = sa1 + LA >= NA ? sa1 + LA - NA : sa1 + LA;
    const int sxl = sx + L >= NX ? sx + L - NX : sx + L;         // (kt + L) % NX
    const int sxl1 = sxl + 1 == NX ? 0 : sxl + 1;
    // even step kt
    if (kt == 0) stage_barrier<G::wait_first0>();
    else stage_barrier<G::wait_steady(0, XS)>();
    issue_A<RTM, NC>(c, kt + LA, sal);
    issue_x<RTM, NC>(c, kt + L, sxl);
    mfma_tile<RTM, NC>(acc, xslot0 + sx * G::kXSlot, smem + sa * G::kASlot, wave, r32, h32);
    if constexpr (XS && BK == 64) xs_store<RTM, NC>(c, xslot0 + sx * G::kXSlot, nullptr, kt, has_pqs);
    // odd step kt + 1
    stage_barrier<G::wait_steady(1, XS)>();
    issue_A<RTM, NC>(c, kt + 1 + LA, sal1);
    issue_x<RTM, NC>(c, kt + 1 + L, sxl1);
    mfma_tile<RTM, NC>(acc, xslot0 + sx1 * G::kXSlot, smem + sa1 * G::kASlot, wave, r32, h32);
    if constexpr (XS) {
      if constexpr (BK == 64) xs_store<RTM, NC>(c, xslot0 + sx1 * G::kXSlot, nullptr, kt + 1, has_pqs);
      else xs_store<RTM, NC>(c, xslot0 + sx * G::kXSlot, xslot0 + sx1 * G::kXSlot, kt / 2, has_pqs);
    }
    sx = sx1 + 1 == NX ? 0 : sx1 + 1;
    sa = sa1 + 1 == NA ? 0 : sa1 + 1;
  }
  if constexpr (BK == 64) {
    // an odd number of 64-deep tiles (K_pad / 64 is odd): the last one is an even step on its own;
    // nothing is issued after it
    if (kt < c.k_tiles) {
      if (kt == 0) stage_barrier<G::wait_first0>();
      else stage_barrier<G::wait_steady(0, XS)>();
      mfma_tile<RTM, NC>(acc, xslot0 + sx * G::kXSlot, smem + sa * G::kASlot, wave, r32, h32);
      if constexpr (XS) xs_store<RTM, NC>(c, xslot0 + sx * G::kXSlot, nullptr, kt, has_pqs);
    }
  }
  wait_vmcnt<0>();  // drain the trailing copies and stores before the workgroup can end

  const float f = p.f_div_dev ? p.f / *p.f_div_dev : p.f;
  const int row_lane = (lane >> 5) * 4;
  const int R = p.r_pad;
  // this group's column tiles: wave w owns tiles w, w + 4, ... (< ctg), t' columns from grp * ctg * 32
  uint16_t* t_grp = p.t_out + static_cast<int64_t>(grp) * ctg * 32;
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
        if (jt < ctg) t_grp[row * R + jt * 32 + r32] = static_cast<uint16_t>(f32_to_bf16_hw(f * acc[i][j][r]));
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

constexpr int max_rtm(int nc) { return lora_max_rtm(nc); }

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
  const LoraSplit sp = lora_down_split(p.S, p.r_pad, p.K, p.K_pad, p.xs_out != nullptr, cus);
  LoraDownParams q = p;
  q.bm = sp.bm;
  q.groups = sp.groups;
  const int nc = sp.nc;
  const int rtm = static_cast<int>((q.bm + 31) / 32);
  const int64_t blocks = sp.blocks;
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
