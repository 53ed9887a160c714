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
// with fp32 accumulators (256 AGPRs), so one workgroup fills a CU and each SIMD runs one wave that
// issues its own decode, LDS reads and copies between its MFMAs. Every decoded weight value feeds
// eight MFMAs (256 rows), which halves the decode and copy work per flop against a 128-row tile;
// under the board's power limit that work is paid for in clock. K is staged through three LDS
// stages of 42 KiB, two tiles ahead:
//   base K-tile (64 deep)  activation 256 x 64 bf16, 16-byte chunks XOR-swizzled     32 KiB
//                          8 runs of 256 code dwords (+32 dwords padding each)        9 KiB
//                          256 scale dwords                                            1 KiB
//   LoRA K-tile (32 deep)  t' 256 x 32 bf16 (16 KiB) and B 256 x 32 bf16 (16 KiB), same swizzle
// Every global->LDS copy is a buffer_load ... lds (16 bytes per lane, no registers, out-of-range
// offsets read as zero). The weight stays 4-bit in LDS: each wave decodes the B operand of its own 64
// columns straight into MFMA registers -- one code dword (8 consecutive k of one column) and one
// E4M3 scale per lane per 32x32x16 step -- so no column is decoded twice and no bf16 weight tile is
// written to LDS. Rows past S lie outside the activation buffer, load as zero and are never stored.
//
// Workgroup -> tile order: the hardware hands workgroup b to XCD b % 8; work item w is mapped so that
// each XCD walks a contiguous range of a grouped order (kGroupM M-tiles sweep the N-tiles together),
// so the workgroups resident on one XCD share a few activation M-tiles in that XCD's L2 and fetch each
// weight tile once per group.
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
constexpr int RT = BM / 32;  // row tiles per wave
constexpr uint32_t kLdsCodes = BM * BK * 2;              // base tile: code runs (32768)
constexpr uint32_t kLdsScales = kLdsCodes + kCodeChunksPerTile * kCodeRun;  // 41984
constexpr uint32_t kLdsLoraB = BM * kLoraBK * 2;         // LoRA tile: B after the 16 KiB t' tile
constexpr uint32_t kStage = kLdsScales + kScaleTileBytes; // 43008
constexpr int kStages = 3;
constexpr int kGroupM = 2;  // row tiles per group in the work order
// The plain output staging (128 row pairs x 264 dwords, below) is larger than the three stages.
constexpr int kPairPitch = 264;
constexpr uint32_t kOutStaging = BM / 2 * kPairPitch * 4;
constexpr uint32_t kLdsBytes = kStages * kStage > kOutStaging ? kStages * kStage : kOutStaging;
static_assert(kLdsLoraB + kLoraTileBytes <= kLdsCodes, "LoRA tile must leave the code and scale areas free");
static_assert(kLdsBytes <= 160 * 1024, "the workgroup must fit a CU's LDS");
// DMA instructions per wave per copy window (every window issues the same number, so that a wave can
// wait for all but the newest tile with one vmcnt): 8 of activation (LoRA: 4 of t', 4 of B), 2 code
// runs, 1 of scales
constexpr int kCopies = 8 + 2 + 1;

__device__ __forceinline__ u32x4 rsrc(const void* base, uint32_t bytes) { return buf_rsrc(base, bytes); }

// LDS slot of (row, 16-byte chunk) in a 64-deep tile (128-byte rows): chunk XOR (row/2)%8.
__device__ __forceinline__ uint32_t slot64(uint32_t row, uint32_t chunk) { return lds_chunk_offset(row, chunk); }
// ... in a 32-deep tile (64-byte rows): rows are paired into 128-byte lines, then as above.
__device__ __forceinline__ uint32_t slot32(uint32_t row, uint32_t chunk) { return lds_chunk_offset32(row, chunk); }

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

struct Ctx {
  u32x4 act, lt, codes, scales, lb;
  // Base tile: copy i (of 8 per wave) fills LDS slots (8w + i)*64 + lane, i.e. tile rows
  // (8w + i)*8 + lane/8; the chunk depends on i only through i & 1, so the per-lane offset is
  // vact[i & 1] plus a uniform (i & ~1) * 8 rows.
  // LoRA tile: t' copy i (of 4 per wave) fills slots (4w + i)*64 + lane of a 64-byte-row tile, i.e.
  // 128-byte lines (4w + i)*8 + lane/8 holding 16 rows, per-lane part vlt[i & 1], and (i & ~1) adds
  // 16 rows per unit; B copy i (of 4) fills lines (4w + i)*8 + lane/8 the same way (vlb[i & 1]).
  uint32_t vact[2], vlt[2], vlb[2];
  uint32_t lane16;  // lane * 16
  uint32_t act_rows8, lt_rows16;
  int k_tiles, total, wave, lane;
};

// Copies are issued in windows: the copies of K-tile T are spread over the K-steps between the
// handover that frees T's stage (that of tile T - 3) and the next handover. A window has 11 copy
// slots per wave:
//   base tile   slots 0..7 activation (two per 16-row pair), 8 and 9 the two code runs of this
//               wave's 64 columns, 10 this wave's 256 bytes of block scales (lanes 0..15)
//   LoRA tile   slots 0..3 t', 4..7 B (two per 32-row pair of each), 8..10 re-reads of the last
//               base tile's code runs and scales into the code and scale areas, which LoRA steps
//               never read
// Every slot of a window past the last tile re-reads the last base tile into the stage just left,
// so every window issues the same number of copies and a handover waits with one vmcnt.
struct Win {
  uint32_t gA, gB, gC, gS;     // LDS: slots 0..3 at gA + i KiB, 4..7 at gB + (i - 4) KiB, 8 and 9 at
                               // gC and gC + 4 code runs, 10 at gS
  uint32_t s0, s2, s4, s6;     // uniform offsets of slot pairs (0, 1), (2, 3), (4, 5), (6, 7)
  uint32_t sC, sS;             // uniform offsets of slot 8 (slot 9: + 4 KiB) and slot 10
  u32x4 rA, rB;                // descriptors of slots 0..3 and 4..7
  uint32_t v0, v1, v4, v5;     // per-lane offsets: slots 0..3 alternate v0 / v1, slots 4..7 v4 / v5
};

template <bool LORA>
__device__ __forceinline__ Win plan(const Ctx& c, int T, uint32_t stage) {
  Win w;
  const uint32_t wv = static_cast<uint32_t>(c.wave);
  const uint32_t kb = static_cast<uint32_t>(T < c.k_tiles ? T : c.k_tiles - 1);
  // code runs and scales of base tile kb (for a LoRA tile: of the last base tile, into areas that
  // LoRA steps do not read)
  w.gC = stage + kLdsCodes + wv * kCodeRun;
  w.gS = stage + kLdsScales + wv * 256;
  w.sC = kb * kCodeTileBytes + wv * 1024;
  w.sS = kb * kScaleTileBytes + wv * 256;
  if (!LORA || T < c.k_tiles || T >= c.total) {  // base tile kb (a harmless re-read past the end)
    const uint32_t k_bytes = kb * BK * 2;
    w.gA = stage + kLdsA + wv * 8192;
    w.gB = w.gA + 4096;
    w.s0 = k_bytes;
    w.s2 = k_bytes + 2 * c.act_rows8;
    w.s4 = k_bytes + 4 * c.act_rows8;
    w.s6 = k_bytes + 6 * c.act_rows8;
    w.rA = c.act;
    w.rB = c.act;
    w.v0 = c.vact[0]; w.v1 = c.vact[1]; w.v4 = c.vact[0]; w.v5 = c.vact[1];
  } else {  // LoRA tile rt: t' then B
    const uint32_t rt = static_cast<uint32_t>(T - c.k_tiles);
    w.gA = stage + kLdsA + wv * 4096;
    w.gB = stage + kLdsLoraB + wv * 4096;
    w.s0 = rt * kLoraBK * 2;
    w.s2 = w.s0 + 2 * c.lt_rows16;
    w.s4 = rt * kLoraTileBytes;
    w.s6 = w.s4 + 2 * (16 * kLoraBK * 2);
    w.rA = c.lt;
    w.rB = c.lb;
    w.v0 = c.vlt[0]; w.v1 = c.vlt[1]; w.v4 = c.vlb[0]; w.v5 = c.vlb[1];
  }
  return w;
}

template <int I> __device__ __forceinline__ uint32_t slot_m0(const Win& w) {
  if constexpr (I < 4) return w.gA + I * 1024;
  else if constexpr (I < 8) return w.gB + (I - 4) * 1024;
  else if constexpr (I == 8) return w.gC;
  else if constexpr (I == 9) return w.gC + 4 * kCodeRun;
  else return w.gS;
}
template <int I> __device__ __forceinline__ uint32_t slot_soff(const Win& w) {
  if constexpr (I < 2) return w.s0;
  else if constexpr (I < 4) return w.s2;
  else if constexpr (I < 6) return w.s4;
  else if constexpr (I < 8) return w.s6;
  else if constexpr (I == 8) return w.sC;
  else if constexpr (I == 9) return w.sC + 4 * 1024;
  else return w.sS;
}
template <int I> __device__ __forceinline__ uint32_t slot_voff(const Ctx& c, const Win& w) {
  if constexpr (I < 4) return (I & 1) ? w.v1 : w.v0;
  else if constexpr (I < 8) return (I & 1) ? w.v5 : w.v4;
  else return c.lane16;
}
template <int I> __device__ __forceinline__ u32x4 slot_rsrc(const Ctx& c, const Win& w) {
  if constexpr (I < 4) return w.rA;
  else if constexpr (I < 8) return w.rB;
  else if constexpr (I < 10) return c.codes;
  else return c.scales;
}

// Operands of copy j (slot I) of a step block.
#define H3Q_COPY(j, I)                                                                            \
  [cm##j] "s"(slot_m0<I>(w)), [cv##j] "v"(slot_voff<I>(c, w)), [cs##j] "s"(slot_soff<I>(w)),      \
      [cr##j] "s"(slot_rsrc<I>(c, w))

// One copy on its own (prologue). M0 is saved and restored around it. The leading wait covers an SGPR
// operand that the compiler may have just written with a VALU instruction (v_readlane after a spill,
// v_readfirstlane), which a vector-memory instruction must not read for 5 wait states; the compiler
// does not look inside the block to insert them.
template <int I>
__device__ __forceinline__ void copy_slot(const Ctx& c, const Win& w) {
  uint32_t msv;
  if constexpr (I == 10) {
    uint64_t ex;
    asm volatile(
        "s_nop 4\n\ts_mov_b32 %[msv], m0\n\ts_mov_b64 %[ex], exec\n\ts_mov_b32 exec_lo, 0xffff\n\ts_mov_b32 exec_hi, 0\n\t"
        "s_mov_b32 m0, %[cm0]\n\ts_nop 0\n\tbuffer_load_dwordx4 %[cv0], %[cr0], %[cs0] offen lds\n\t"
        "s_mov_b64 exec, %[ex]\n\ts_mov_b32 m0, %[msv]"
        : [msv] "=&s"(msv), [ex] "=&s"(ex)
        : H3Q_COPY(0, I)
        : "memory");
  } else {
    asm volatile(
        "s_nop 4\n\ts_mov_b32 %[msv], m0\n\ts_mov_b32 m0, %[cm0]\n\ts_nop 0\n\t"
        "buffer_load_dwordx4 %[cv0], %[cr0], %[cs0] offen lds\n\ts_mov_b32 m0, %[msv]"
        : [msv] "=&s"(msv)
        : H3Q_COPY(0, I)
        : "memory");
  }
}

template <int I, int N>
__device__ __forceinline__ void copy_slots(const Ctx& c, const Win& w) {
  if constexpr (N > 0) {
    copy_slot<I>(c, w);
    copy_slots<I + 1, N - 1>(c, w);
  }
}

// ------------------------------------------------------------------------------------------------
// K-steps. One asm block per 16-deep K-step (instruction order in gemm_w4_steps.inc); the blocks
// chain through their register operands: a step's "next" outputs are the following step's inputs.
// ------------------------------------------------------------------------------------------------
#include "gemm_w4_steps.inc"

#define H3Q_ACC(acc)                                                                            \
  [c00] "+a"(acc[0][0]), [c01] "+a"(acc[0][1]), [c10] "+a"(acc[1][0]), [c11] "+a"(acc[1][1]),   \
  [c20] "+a"(acc[2][0]), [c21] "+a"(acc[2][1]), [c30] "+a"(acc[3][0]), [c31] "+a"(acc[3][1]),   \
  [c40] "+a"(acc[4][0]), [c41] "+a"(acc[4][1]), [c50] "+a"(acc[5][0]), [c51] "+a"(acc[5][1]),   \
  [c60] "+a"(acc[6][0]), [c61] "+a"(acc[6][1]), [c70] "+a"(acc[7][0]), [c71] "+a"(acc[7][1])
#define H3Q_A_IN(a)                                                                             \
  [a0] "v"(a[0]), [a1] "v"(a[1]), [a2] "v"(a[2]), [a3] "v"(a[3]), [a4] "v"(a[4]), [a5] "v"(a[5]), \
  [a6] "v"(a[6]), [a7] "v"(a[7])
#define H3Q_A_OUT(n)                                                                            \
  [n0] "=&v"(n[0]), [n1] "=&v"(n[1]), [n2] "=&v"(n[2]), [n3] "=&v"(n[3]), [n4] "=&v"(n[4]),    \
  [n5] "=&v"(n[5]), [n6] "=&v"(n[6]), [n7] "=&v"(n[7])
#define H3Q_B_IN(b)                                                                             \
  [bq0] "v"(u32x4{b[0], b[1], b[2], b[3]}), [bq1] "v"(u32x4{b[4], b[5], b[6], b[7]})
#define H3Q_B_OUT(m)                                                                            \
  [m0] "=&v"(m[0]), [m1] "=&v"(m[1]), [m2] "=&v"(m[2]), [m3] "=&v"(m[3]), [m4] "=&v"(m[4]),    \
  [m5] "=&v"(m[5]), [m6] "=&v"(m[6]), [m7] "=&v"(m[7])
#define H3Q_STEP_CLOBBERS                                                                       \
  "v108", "v109", "v110", "v111", "v120", "v121", "v122", "v123", "v124", "v125", "v126", "v127", "memory"
static_assert(RT == 8, "the step blocks and the operand lists above are written for 8 row tiles");

typedef uint32_t bw_t[8];  // a decoded W4 B operand: 2 column tiles x 4 dwords of bf16 pairs
typedef f32x16 acc_t[RT][2];
typedef bf16x8 aop_t[RT];

constexpr uint32_t kPermHighHalves = 0x07060302u;  // v_perm_b32: high 16 bits of each source

// base step, next = K-step of the same base tile (scales s0/s1 of that step given); copies I..I+2
template <int I>
__device__ __forceinline__ void step_bb3(acc_t& acc, const aop_t& a, const bw_t& b, aop_t& n, bw_t& m, float s0,
                                         float s1, uint32_t aaddr, uint32_t caddr, const Ctx& c, const Win& w) {
  uint32_t msv;
  asm volatile(H3Q_STEP_BB_C3_ASM
               : H3Q_ACC(acc), H3Q_A_OUT(n), H3Q_B_OUT(m), [msv] "=&s"(msv)
               : H3Q_A_IN(a), H3Q_B_IN(b), [s0] "v"(s0), [s1] "v"(s1), [aaddr] "v"(aaddr), [caddr] "v"(caddr),
                 [sel] "s"(kPermHighHalves), H3Q_COPY(0, I), H3Q_COPY(1, I + 1), H3Q_COPY(2, I + 2)
               : H3Q_STEP_CLOBBERS);
}
// the same with copies 9 and 10 (the scales, lanes 0..15)
__device__ __forceinline__ void step_bbm(acc_t& acc, const aop_t& a, const bw_t& b, aop_t& n, bw_t& m, float s0,
                                         float s1, uint32_t aaddr, uint32_t caddr, const Ctx& c, const Win& w) {
  uint32_t msv;
  uint64_t ex;
  asm volatile(H3Q_STEP_BB_C1M_ASM
               : H3Q_ACC(acc), H3Q_A_OUT(n), H3Q_B_OUT(m), [msv] "=&s"(msv), [ex] "=&s"(ex)
               : H3Q_A_IN(a), H3Q_B_IN(b), [s0] "v"(s0), [s1] "v"(s1), [aaddr] "v"(aaddr), [caddr] "v"(caddr),
                 [sel] "s"(kPermHighHalves), H3Q_COPY(0, 9), H3Q_COPY(1, 10)
               : H3Q_STEP_CLOBBERS);
}
// base step, next = first K-step of a new base tile (its scale dwords d0/d1 are read here too);
// copies 0..2
__device__ __forceinline__ void step_bbn3(acc_t& acc, const aop_t& a, const bw_t& b, aop_t& n, bw_t& m,
                                          uint32_t (&d)[2], uint32_t aaddr, uint32_t caddr, uint32_t saddr,
                                          const Ctx& c, const Win& w) {
  uint32_t msv;
  asm volatile(H3Q_STEP_BBN_C3_ASM
               : H3Q_ACC(acc), H3Q_A_OUT(n), H3Q_B_OUT(m), [d0] "=&v"(d[0]), [d1] "=&v"(d[1]), [msv] "=&s"(msv)
               : H3Q_A_IN(a), H3Q_B_IN(b), [aaddr] "v"(aaddr), [caddr] "v"(caddr), [saddr] "v"(saddr),
                 [sel] "s"(kPermHighHalves), H3Q_COPY(0, 0), H3Q_COPY(1, 1), H3Q_COPY(2, 2)
               : H3Q_STEP_CLOBBERS);
}
// base step, next = a LoRA K-step; copies 0..2
__device__ __forceinline__ void step_bl3(acc_t& acc, const aop_t& a, const bw_t& b, aop_t& n, bf16x8 (&k)[2],
                                         uint32_t aaddr, uint32_t baddr, const Ctx& c, const Win& w) {
  uint32_t msv;
  asm volatile(H3Q_STEP_BL_C3_ASM
               : H3Q_ACC(acc), H3Q_A_OUT(n), [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [msv] "=&s"(msv)
               : H3Q_A_IN(a), H3Q_B_IN(b), [aaddr] "v"(aaddr), [baddr] "v"(baddr), H3Q_COPY(0, 0), H3Q_COPY(1, 1),
                 H3Q_COPY(2, 2)
               : H3Q_STEP_CLOBBERS);
}
// base step, last of the tile loop
__device__ __forceinline__ void step_bn(acc_t& acc, const aop_t& a, const bw_t& b) {
  asm volatile(H3Q_STEP_BN_ASM : H3Q_ACC(acc) : H3Q_A_IN(a), H3Q_B_IN(b) : H3Q_STEP_CLOBBERS);
}
// LoRA step, next = a LoRA K-step; copies 3..10 (10: lanes 0..15)
__device__ __forceinline__ void step_ll8(acc_t& acc, const aop_t& a, const bf16x8 (&l)[2], aop_t& n,
                                         bf16x8 (&k)[2], uint32_t aaddr, uint32_t baddr, const Ctx& c, const Win& w) {
  uint32_t msv;
  uint64_t ex;
  asm volatile(H3Q_STEP_LL_C7M_ASM
               : H3Q_ACC(acc), H3Q_A_OUT(n), [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [msv] "=&s"(msv), [ex] "=&s"(ex)
               : H3Q_A_IN(a), [l0] "v"(l[0]), [l1] "v"(l[1]), [aaddr] "v"(aaddr), [baddr] "v"(baddr),
                 H3Q_COPY(0, 3), H3Q_COPY(1, 4), H3Q_COPY(2, 5), H3Q_COPY(3, 6), H3Q_COPY(4, 7), H3Q_COPY(5, 8),
                 H3Q_COPY(6, 9), H3Q_COPY(7, 10)
               : H3Q_STEP_CLOBBERS);
}
// LoRA step, next = a LoRA K-step; copies 0..2
__device__ __forceinline__ void step_ll3(acc_t& acc, const aop_t& a, const bf16x8 (&l)[2], aop_t& n,
                                         bf16x8 (&k)[2], uint32_t aaddr, uint32_t baddr, const Ctx& c, const Win& w) {
  uint32_t msv;
  asm volatile(H3Q_STEP_LL_C3_ASM
               : H3Q_ACC(acc), H3Q_A_OUT(n), [k0] "=&v"(k[0]), [k1] "=&v"(k[1]), [msv] "=&s"(msv)
               : H3Q_A_IN(a), [l0] "v"(l[0]), [l1] "v"(l[1]), [aaddr] "v"(aaddr), [baddr] "v"(baddr),
                 H3Q_COPY(0, 0), H3Q_COPY(1, 1), H3Q_COPY(2, 2)
               : H3Q_STEP_CLOBBERS);
}
// LoRA step, last of the tile loop
__device__ __forceinline__ void step_ln(acc_t& acc, const aop_t& a, const bf16x8 (&l)[2]) {
  asm volatile(H3Q_STEP_LN_ASM : H3Q_ACC(acc) : H3Q_A_IN(a), [l0] "v"(l[0]), [l1] "v"(l[1]) : H3Q_STEP_CLOBBERS);
}

// LDS byte address of a pointer into the dynamic shared array.
__device__ __forceinline__ uint32_t lds_addr(const uint8_t* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) uint8_t*)(p)));
}


// Plain output through LDS: the tile goes into the freed stages as row pairs -- dword [q][c] holds
// column c of rows 2q (low half) and 2q + 1 (high half), 264 dwords per pair (8 of padding) -- so
// that each lane writes its accumulator registers r, r + 1 (two consecutive rows of one column) with
// one conversion and one 4-byte write. Then every thread reads 8 dwords of a row pair (two 16-byte
// reads), splits them into the two rows' chunks of 8 consecutive columns (v_perm_b32) and stores both
// with 16-byte stores. Needs the output rows 16-byte aligned (n_out a multiple of 8, or of 16 for a
// gate/up weight, and out aligned).
static_assert(kOutStaging <= kLdsBytes, "output staging must fit the LDS");
constexpr uint32_t kPermLowHalves = 0x05040100u;   // v_perm_b32: low 16 bits of each source

__device__ __forceinline__ void plain_epilogue_staged(const GemmParams& p, const acc_t& acc,
                                                      uint8_t* smem, float scale, int64_t m0, int nt, int wave,
                                                      uint32_t lane) {
  uint32_t* tile = reinterpret_cast<uint32_t*>(smem);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const int row = i * 32 + (r >> 2) * 8 + static_cast<int>(lane >> 5) * 4 + (r & 3);  // even
        const int col = wave * 64 + j * 32 + static_cast<int>(lane & 31);
        tile[(row >> 1) * kPairPitch + col] = bf16x2_hw(scale * acc[i][j][r], scale * acc[i][j][r + 1]);
      }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int q = 0; q < BM * BN / 16 / kThreads; ++q) {
    const int c = static_cast<int>(threadIdx.x) + kThreads * q;
    const int rp = c >> 5, c8 = (c & 31) * 8;
    const u32x4 d0 = *reinterpret_cast<const u32x4*>(tile + rp * kPairPitch + c8);
    const u32x4 d1 = *reinterpret_cast<const u32x4*>(tile + rp * kPairPitch + c8 + 4);
    const u32x4 even = {__builtin_amdgcn_perm(d0.y, d0.x, kPermLowHalves), __builtin_amdgcn_perm(d0.w, d0.z, kPermLowHalves),
                        __builtin_amdgcn_perm(d1.y, d1.x, kPermLowHalves), __builtin_amdgcn_perm(d1.w, d1.z, kPermLowHalves)};
    const u32x4 odd = {__builtin_amdgcn_perm(d0.y, d0.x, kPermHighHalves), __builtin_amdgcn_perm(d0.w, d0.z, kPermHighHalves),
                       __builtin_amdgcn_perm(d1.y, d1.x, kPermHighHalves), __builtin_amdgcn_perm(d1.w, d1.z, kPermHighHalves)};
    const int64_t grow = m0 + 2 * rp;
    const int64_t n = packed_row_source(nt, c8, p.gate_up != 0, p.n_out);
    if (n >= 0) {
      if (grow < p.S) __builtin_nontemporal_store(even, reinterpret_cast<u32x4*>(p.out + grow * p.out_ld + n));
      if (grow + 1 < p.S) __builtin_nontemporal_store(odd, reinterpret_cast<u32x4*>(p.out + (grow + 1) * p.out_ld + n));
    }
  }
}

// SwiGLU output through LDS: h = bf16(SiLU(gate) * up) staged as row pairs like the plain output
// (dword [q][c] = h column c of rows 2q and 2q + 1; 128 h columns + 8 of padding per pair; wave w holds
// h columns [32w, 32w + 32)), then 16-byte stores of 8 consecutive h columns of both rows. With an
// emit target the same pass also writes the next projection's base operand
// xs = bf16(f32(h) * pqs_next[n]) from the stored h bits, i.e. exactly what prescaling the stored h
// would give (FL2VA Turbo, "Implementation": the producer emitting the base input beside the exact bf16
// LoRA input). Needs n_out % 8 == 0 and 16-byte aligned rows.
constexpr int kHPairPitch = 136;
static_assert(BM / 2 * kHPairPitch * 4 <= kLdsBytes, "SwiGLU staging must fit the stages");

// One 16-byte chunk of h (8 columns from n) of output row grow, and its emitted prescaled copy.
__device__ __forceinline__ void swiglu_store_chunk(const GemmParams& p, const u32x4& hv, int64_t grow, int64_t n) {
  __builtin_nontemporal_store(hv, reinterpret_cast<u32x4*>(p.out + grow * p.out_ld + n));
  if (p.emit_out) {
    const f32x4 q0 = *reinterpret_cast<const f32x4*>(p.emit_pqs + n);
    const f32x4 q1 = *reinterpret_cast<const f32x4*>(p.emit_pqs + n + 4);
    const float pq[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
    const uint32_t hw[4] = {hv.x, hv.y, hv.z, hv.w};
    uint32_t xw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      xw[e] = bf16x2_hw(bf16_bits_to_f32(hw[e] & 0xffffu) * pq[2 * e], __uint_as_float(hw[e] & 0xffff0000u) * pq[2 * e + 1]);
    __builtin_nontemporal_store(u32x4{xw[0], xw[1], xw[2], xw[3]},
                                reinterpret_cast<u32x4*>(p.emit_out + grow * p.emit_ld + n));
  }
}

__device__ __forceinline__ void swiglu_epilogue_staged(const GemmParams& p, const acc_t& acc,
                                                       uint8_t* smem, float scale, int64_t m0, int nt, int wave,
                                                       uint32_t lane) {
  uint32_t* tile = reinterpret_cast<uint32_t*>(smem);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const int row = i * 32 + (r >> 2) * 8 + static_cast<int>(lane >> 5) * 4 + (r & 3);  // even
      const int col = wave * 32 + static_cast<int>(lane & 31);
      const float g0 = scale * acc[i][0][r], u0 = scale * acc[i][1][r];
      const float g1 = scale * acc[i][0][r + 1], u1 = scale * acc[i][1][r + 1];
      tile[(row >> 1) * kHPairPitch + col] = bf16x2_hw(silu(g0) * u0, silu(g1) * u1);
      if ((r & 3) == 2) __builtin_amdgcn_sched_barrier(0);  // 4 values at a time: accumulators stay in AGPRs
    }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
  for (int q = 0; q < BM * (BN / 2) / 16 / kThreads; ++q) {
    const int c = static_cast<int>(threadIdx.x) + kThreads * q;
    const int rp = c >> 4, c8 = (c & 15) * 8;
    const int64_t n = static_cast<int64_t>(nt) * (BN / 2) + c8;
    if (n >= p.n_out) continue;
    const u32x4 d0 = *reinterpret_cast<const u32x4*>(tile + rp * kHPairPitch + c8);
    const u32x4 d1 = *reinterpret_cast<const u32x4*>(tile + rp * kHPairPitch + c8 + 4);
    const int64_t grow = m0 + 2 * rp;
    if (grow < p.S)
      swiglu_store_chunk(p, u32x4{__builtin_amdgcn_perm(d0.y, d0.x, kPermLowHalves), __builtin_amdgcn_perm(d0.w, d0.z, kPermLowHalves),
                                  __builtin_amdgcn_perm(d1.y, d1.x, kPermLowHalves), __builtin_amdgcn_perm(d1.w, d1.z, kPermLowHalves)},
                         grow, n);
    if (grow + 1 < p.S)
      swiglu_store_chunk(p, u32x4{__builtin_amdgcn_perm(d0.y, d0.x, kPermHighHalves), __builtin_amdgcn_perm(d0.w, d0.z, kPermHighHalves),
                                  __builtin_amdgcn_perm(d1.y, d1.x, kPermHighHalves), __builtin_amdgcn_perm(d1.w, d1.z, kPermHighHalves)},
                         grow + 1, n);
  }
}

// Q/K tiles of the fused QKV projection (MiniMax-H3 Ultra Fast, "Active optimization stack",
// attention projections, and "Kernel path" item 2: three-axis split-half rotary; 96 of 128 head
// dimensions rotate: MiniMax-H3 Turbo CMF card, "On parity"). The tile's 256 columns are two heads of
// 128. Per row and head:
//   u_i = v_i / sqrt(mean_j v_j^2 + eps) * gamma_i            (v = ts * acc, fp32)
// then the first rot dims, as consecutive sections of widths w_j, each rotated in split halves
// within itself (section at dims [o, o + w), h = w / 2, table column o/2 + i for its pair i):
//   out_{o+i} = u_{o+i} c - u_{o+i+h} s,  out_{o+i+h} = u_{o+i+h} c + u_{o+i} s
//   out_i = u_i                                               (rot <= i < 128)
// with c, s the caller's per-row angle table (one section of rot: pair i is dims i and i + rot/2).
// The fp32 tile goes through the freed LDS 128 rows at a time ([128][260] floats: 16-byte aligned
// rows, and 16-byte reads of 8 consecutive rows fall on distinct banks), with the tile's 256 gamma
// values beside it; then one thread per (row, head) sums the head's squares with 16-byte reads, and
// normalizes and rotates 8 pairs at a time in place (one pair at a time when a section's half is not
// a multiple of 8); then the tile is stored as bf16 by 32 threads per row, whole row segments per
// store instruction. The row's angle table is loaded into registers before the pass's staging, so
// its latency hides behind the LDS writes and the barrier.
constexpr int kQkPitch = 260;
constexpr int kQkRows = 128;
constexpr uint32_t kQkGamma = kQkRows * kQkPitch * 4;
static_assert(kQkGamma + BN * 4 <= kLdsBytes, "Q/K staging must fit the LDS");
static_assert(BN == kThreads, "one gamma value per thread");

__device__ __forceinline__ void load8(const float* src, float (&v)[8]) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(src), b = *reinterpret_cast<const f32x4*>(src + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(float* dst, const float (&v)[8]) {
  *reinterpret_cast<f32x4*>(dst) = f32x4{v[0], v[1], v[2], v[3]};
  *reinterpret_cast<f32x4*>(dst + 4) = f32x4{v[4], v[5], v[6], v[7]};
}
__device__ __forceinline__ void store8_bf16(uint16_t* dst, const float (&v)[8]) {
  u32x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = bf16x2_hw(v[2 * e], v[2 * e + 1]);
  *reinterpret_cast<u32x4*>(dst) = o;
}

__device__ __forceinline__ void qk_norm_rope_epilogue(const GemmParams& p, const acc_t& acc, uint8_t* smem,
                                                      float scale, int64_t m0, int nt, int wave, uint32_t lane,
                                                      bool is_q) {
  float* tile = reinterpret_cast<float*>(smem);
  float* gam = reinterpret_cast<float*>(smem + kQkGamma);
  const int tid = threadIdx.x;
  const float* gamma_tile = is_q ? p.qk_gamma_q + static_cast<int64_t>(nt) * BN
                                 : p.qk_gamma_k + static_cast<int64_t>(nt - p.q_tiles) * BN;
  const int half = p.rope_half;  // angle table columns per row (rot / 2)
  const int head = __builtin_amdgcn_readfirstlane(tid >> 7);  // waves 0, 1: head 0; waves 2, 3: head 1
  const int row_l = tid & (kQkRows - 1);
  const bool vec = p.rope_vec != 0;
  const bool vec_tab = vec && ((reinterpret_cast<uintptr_t>(p.rope_cos) | reinterpret_cast<uintptr_t>(p.rope_sin)) & 15) == 0;
#pragma unroll
  for (int pass = 0; pass < BM / kQkRows; ++pass) {
    const int64_t row = m0 + pass * kQkRows + row_l;
    const float* cr = p.rope_cos + row * half;
    const float* sr = p.rope_sin + row * half;
    f32x4 cpre[16], spre[16];  // the row's angle table, 4 pairs per entry (h <= 64)
    if (vec_tab && row < p.S) {
#pragma unroll
      for (int q = 0; q < 16; ++q)
        if (4 * q < half) {
          cpre[q] = *reinterpret_cast<const f32x4*>(cr + 4 * q);
          spre[q] = *reinterpret_cast<const f32x4*>(sr + 4 * q);
        }
    }
    // every wave is past its last LDS read (pass 0: the last stage handover; pass 1: the barrier
    // after the row threads below), so the tile can be overwritten
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (pass == 0) gam[tid] = gamma_tile[tid];
#pragma unroll
    for (int ii = 0; ii < kQkRows / 32; ++ii)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int rl = ii * 32 + (r >> 2) * 8 + static_cast<int>(lane >> 5) * 4 + (r & 3);
          const int col = wave * 64 + j * 32 + static_cast<int>(lane & 31);
          tile[rl * kQkPitch + col] = scale * acc[pass * (kQkRows / 32) + ii][j][r];
        }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (row < p.S) {
      float* t = tile + row_l * kQkPitch + head * 128;
      const float* g = gam + head * 128;
      float ss = 0.0f;
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(t + 4 * q);
        ss += v.x * v.x;
        ss += v.y * v.y;
        ss += v.z * v.z;
        ss += v.w * v.w;
      }
      const float inv = 1.0f / sqrtf(ss * (1.0f / 128.0f) + p.qk_eps);
      if (vec) {
#pragma unroll
        for (int gi = 0; gi < 8; ++gi) {
          const int i = gi * 8;  // table columns i .. i + 7
          if (i >= half) break;
          const int dlo = p.rope_lo[gi], dhi = p.rope_hi[gi];
          float tv[8], th[8], gv[8], gh[8], cs[8], sn[8], lo[8], hi[8];
          load8(t + dlo, tv);
          load8(t + dhi, th);
          load8(g + dlo, gv);
          load8(g + dhi, gh);
          if (vec_tab) {
            const f32x4 c0 = cpre[2 * gi], c1 = cpre[2 * gi + 1], s0 = spre[2 * gi], s1 = spre[2 * gi + 1];
            cs[0] = c0.x; cs[1] = c0.y; cs[2] = c0.z; cs[3] = c0.w; cs[4] = c1.x; cs[5] = c1.y; cs[6] = c1.z; cs[7] = c1.w;
            sn[0] = s0.x; sn[1] = s0.y; sn[2] = s0.z; sn[3] = s0.w; sn[4] = s1.x; sn[5] = s1.y; sn[6] = s1.z; sn[7] = s1.w;
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              cs[e] = cr[i + e];
              sn[e] = sr[i + e];
            }
          }
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float a = tv[e] * inv * gv[e], b = th[e] * inv * gh[e];
            lo[e] = a * cs[e] - b * sn[e];
            hi[e] = b * cs[e] + a * sn[e];
          }
          store8(t + dlo, lo);
          store8(t + dhi, hi);
        }
        for (int k = 2 * half; k < 128; k += 8) {
          float tv[8], gv[8], u[8];
          load8(t + k, tv);
          load8(g + k, gv);
#pragma unroll
          for (int e = 0; e < 8; ++e) u[e] = tv[e] * inv * gv[e];
          store8(t + k, u);
        }
      } else {  // a section's half is not a multiple of 8: one pair at a time
        int o = 0;
        for (int j = 0; j < p.rope_nsec; ++j) {
          const int h = p.rope_sec[j] / 2;
          for (int i = 0; i < h; ++i) {
            const int lo = o + i, hi = o + i + h;
            const float a = t[lo] * inv * g[lo], b = t[hi] * inv * g[hi];
            const float c = cr[o / 2 + i], sv = sr[o / 2 + i];
            t[lo] = a * c - b * sv;
            t[hi] = b * c + a * sv;
          }
          o += p.rope_sec[j];
        }
        for (int k = 2 * half; k < 128; ++k) t[k] = t[k] * inv * g[k];
      }
    }
    // The results overwrote their own inputs in the tile; now 32 threads per row store 8 consecutive
    // columns each, so every store instruction covers whole 512-byte row segments.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
    for (int k = 0; k < kQkRows * BN / 8 / kThreads; ++k) {
      const int cidx = tid + kThreads * k;
      const int rl = cidx >> 5, c8 = (cidx & 31) * 8;
      const int64_t grow = m0 + pass * kQkRows + rl;
      if (grow < p.S) {
        float v[8];
        load8(tile + rl * kQkPitch + c8, v);
        store8_bf16(p.out + grow * p.out_ld + static_cast<int64_t>(nt) * BN + c8, v);
      }
    }
  }
}

template <int EPI, bool LORA>
__global__ __launch_bounds__(kThreads, 1) void gemm_w4_kernel(GemmParams p) {
  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];

  const int tid = threadIdx.x;
  const uint32_t lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: keep it scalar

  // XCD-aware work index (gridDim.x is a multiple of 8; consecutive workgroups go to different
  // XCDs): each XCD takes one contiguous run of w. Within the run, tiles go in groups of kGroupM row
  // tiles that sweep all column tiles together, so an XCD's L2 holds two activation row blocks
  // and each weight column tile is fetched once per pair of row tiles.
  const int per_xcd = gridDim.x >> 3;
  const int w = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (w >= p.m_tiles * p.n_tiles) return;
  const int grp_items = kGroupM * p.n_tiles;
  const int grp = w / grp_items, idx = w - grp * grp_items;
  const int gm = min(kGroupM, p.m_tiles - grp * kGroupM);  // the last group may be short
  const int mt = __builtin_amdgcn_readfirstlane(grp * kGroupM + idx % gm);
  const int nt = __builtin_amdgcn_readfirstlane(idx / gm);
  const int64_t m0 = static_cast<int64_t>(mt) * BM;

  Ctx c;
  c.k_tiles = p.k_tiles;
  c.total = p.k_tiles + p.r_tiles;
  c.wave = wave;
  c.lane = lane;
  c.lane16 = lane * 16;
  // The activation and t' descriptors start at the tile's first row, so every offset stays within
  // 32 bits whatever S is (rows past S read as zero: the range ends with the tile's last real row).
  const int64_t tile_rows = min(static_cast<int64_t>(BM), p.S - m0);
  c.act = rsrc(p.act + m0 * p.act_ld, static_cast<uint32_t>(tile_rows * p.act_ld * 2));
  c.codes = rsrc(p.wcodes + static_cast<int64_t>(nt) * p.k_tiles * kCodeTileBytes,
                 static_cast<uint32_t>(p.k_tiles) * kCodeTileBytes);
  c.scales = rsrc(p.wscales + static_cast<int64_t>(nt) * p.k_tiles * kScaleTileBytes,
                  static_cast<uint32_t>(p.k_tiles) * kScaleTileBytes);
  c.lt = rsrc(p.r_tiles ? p.lora_t + m0 * p.lora_t_ld : nullptr,
              p.r_tiles ? static_cast<uint32_t>(tile_rows * p.lora_t_ld * 2) : 0u);
  c.lb = rsrc(reinterpret_cast<const uint8_t*>(p.lora_b) + static_cast<int64_t>(nt) * p.r_tiles * kLoraTileBytes,
              static_cast<uint32_t>(p.r_tiles) * kLoraTileBytes);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    {  // base tile slot (8w + h)*64 + lane -> row, chunk (see Ctx)
      const uint32_t row = (wave * 8 + h) * 8 + (lane >> 3);
      const uint32_t chunk = (lane & 7) ^ ((row >> 1) & 7);
      c.vact[h] = row * static_cast<uint32_t>(p.act_ld * 2) + chunk * 16;
    }
    {  // LoRA t' slot (4w + h)*64 + lane -> 128-byte line, then (row, chunk) of the 64-byte rows
      const uint32_t line = (wave * 4 + h) * 8 + (lane >> 3);
      const uint32_t cl = (lane & 7) ^ ((line >> 1) & 7);
      const uint32_t row = line * 2 + (cl >> 2), chunk = cl & 3;
      c.vlt[h] = row * static_cast<uint32_t>(p.lora_t_ld * 2) + chunk * 16;
    }
    {  // LoRA B slot (4w + h)*64 + lane, the same mapping over B's 256 rows
      const uint32_t line = (wave * 4 + h) * 8 + (lane >> 3);
      const uint32_t cl = (lane & 7) ^ ((line >> 1) & 7);
      const uint32_t row = line * 2 + (cl >> 2), chunk = cl & 3;
      c.vlb[h] = row * (kLoraBK * 2) + chunk * 16;
    }
  }
  c.act_rows8 = static_cast<uint32_t>(p.act_ld * 16);
  c.lt_rows16 = static_cast<uint32_t>(p.lora_t_ld * 32);

  // accumulators: zeroed in place in AGPRs (an MFMA of zero operands with C = 0), so that they live
  // in AGPRs from the first to the last K-step
  // One asm block: the compiler writes z just before it and does not see the MFMAs inside, so the
  // block itself waits out the VALU-write -> MFMA-read hazard (s_nop 4) before the first MFMA (without
  // it, a schedule that put the write of z right before the block left acc[0][0] holding garbage).
  acc_t acc;
  {
    const bf16x8 z = {};
    asm volatile(
        "s_nop 4\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c00], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c01], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c10], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c11], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c20], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c21], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c30], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c31], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c40], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c41], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c50], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c51], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c60], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c61], %[z], %[z], 0\n\t"
        "v_mfma_f32_32x32x16_bf16 %[c70], %[z], %[z], 0\n\tv_mfma_f32_32x32x16_bf16 %[c71], %[z], %[z], 0"
        : [c00] "=a"(acc[0][0]), [c01] "=a"(acc[0][1]), [c10] "=a"(acc[1][0]), [c11] "=a"(acc[1][1]),
          [c20] "=a"(acc[2][0]), [c21] "=a"(acc[2][1]), [c30] "=a"(acc[3][0]), [c31] "=a"(acc[3][1]),
          [c40] "=a"(acc[4][0]), [c41] "=a"(acc[4][1]), [c50] "=a"(acc[5][0]), [c51] "=a"(acc[5][1]),
          [c60] "=a"(acc[6][0]), [c61] "=a"(acc[6][1]), [c70] "=a"(acc[7][0]), [c71] "=a"(acc[7][1])
        : [z] "v"(z));
  }

  const uint32_t ncol[2] = {static_cast<uint32_t>(wave * 64) + (lane & 31),
                            static_cast<uint32_t>(wave * 64 + 32) + (lane & 31)};
  const int total = p.k_tiles + p.r_tiles;

  // Per-lane LDS offsets of the MFMA operands inside a stage (see slot64 / slot32 / the code runs):
  // row tile i adds i*4096 (base A) or i*2048 (LoRA A), column tile 1 adds 128 (codes, scales) or
  // 2048 (LoRA B); those constant parts are immediate offsets inside the step blocks.
  const uint32_t r = lane & 31, h = lane >> 5;
  uint32_t off_a64[4], off_a32[2];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) off_a64[kk] = slot64(r, 2 * kk + h);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) off_a32[kk] = slot32(r, 2 * kk + h);
  const uint32_t off_codes = kLdsCodes + h * kCodeRun + wave * 256 + r * 4;
  const uint32_t off_scales = kLdsScales + wave * 256 + r * 4;
  const uint32_t off_lora_b = kLdsLoraB + wave * 4096;
  const uint32_t smem0 = lds_addr(smem);

  // Prologue: tiles 0 and 1 (11 copies each, tile 1 possibly a LoRA tile or a re-read), then the
  // first three copies of tile 2's window; wait for tile 0, read and decode its first K-step in C++.
  copy_slots<0, kCopies>(c, plan<LORA>(c, 0, smem0));
  copy_slots<0, kCopies>(c, plan<LORA>(c, 1, smem0 + kStage));
  Win win = plan<LORA>(c, 2, smem0 + 2 * kStage);
  copy_slots<0, 3>(c, win);
  stage_barrier<kCopies + 3>();

  aop_t aX, aY;
  bf16x8 lX[2], lY[2];
  uint32_t bX[8], bY[8], sdw[2];
  {
    const uint8_t* st = smem;
#pragma unroll
    for (int i = 0; i < RT; ++i) aX[i] = *reinterpret_cast<const bf16x8*>(st + off_a64[0] + i * 4096);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      sdw[j] = *reinterpret_cast<const uint32_t*>(st + off_scales + j * 128);
      const uint32_t cw = *reinterpret_cast<const uint32_t*>(st + off_codes + j * 128);
      const u32x4 v = nvfp4_dword_to_bf16x8(cw, e4m3_byte_to_f32<0>(sdw[j]));
      bX[4 * j] = v.x; bX[4 * j + 1] = v.y; bX[4 * j + 2] = v.z; bX[4 * j + 3] = v.w;
    }
  }

  // Tile t lives in stage t % 3. A base tile runs K-steps 0..2 (carrying copies 3..10 of the
  // window of tile t + 2), then the handover waits for tile t + 1 and plans tile t + 3 into the
  // stage t just left, and K-step 3 runs (copies 0..2) while it reads tile t + 1's first K-step.
  // A LoRA tile runs K-step 0 (copies 3..10), the handover, and K-step 1 (copies 0..2). The last
  // base tile and the last LoRA tile are peeled so that each loop carries one step shape.
  int s_cur = 0;
  auto base_steps_012 = [&](uint32_t st) {
    step_bb3<3>(acc, aX, bX, aY, bY, e4m3_byte_to_f32<1>(sdw[0]), e4m3_byte_to_f32<1>(sdw[1]), st + off_a64[1],
                st + off_codes + 1 * 2 * kCodeRun, c, win);
    step_bb3<6>(acc, aY, bY, aX, bX, e4m3_byte_to_f32<2>(sdw[0]), e4m3_byte_to_f32<2>(sdw[1]), st + off_a64[2],
                st + off_codes + 2 * 2 * kCodeRun, c, win);
    step_bbm(acc, aX, bX, aY, bY, e4m3_byte_to_f32<3>(sdw[0]), e4m3_byte_to_f32<3>(sdw[1]), st + off_a64[3],
             st + off_codes + 3 * 2 * kCodeRun, c, win);
  };
  int kt = 0;
  for (; kt + 1 < p.k_tiles; ++kt) {
    const int s_nxt = s_cur == 2 ? 0 : s_cur + 1;
    const uint32_t st = smem0 + s_cur * kStage, sn = smem0 + s_nxt * kStage;
    base_steps_012(st);
    stage_barrier<kCopies>();  // tile kt+1 has landed; tile kt+2's window may still be in flight
    win = plan<LORA>(c, kt + 3, st);
    step_bbn3(acc, aY, bY, aX, bX, sdw, sn + off_a64[0], sn + off_codes, sn + off_scales, c, win);
    s_cur = s_nxt;
  }
  {  // last base tile
    const int s_nxt = s_cur == 2 ? 0 : s_cur + 1;
    const uint32_t st = smem0 + s_cur * kStage, sn = smem0 + s_nxt * kStage;
    base_steps_012(st);
    if (LORA) {
      stage_barrier<kCopies>();
      win = plan<LORA>(c, kt + 3, st);
      step_bl3(acc, aY, bY, aX, lX, sn + off_a32[0], sn + off_lora_b + off_a32[0], c, win);
    } else {
      stage_barrier<0>();  // drain every copy before the workgroup can end
      step_bn(acc, aY, bY);
    }
    s_cur = s_nxt;
    ++kt;
  }
  if (LORA) {
    for (; kt + 1 < total; ++kt) {
      const int s_nxt = s_cur == 2 ? 0 : s_cur + 1;
      const uint32_t st = smem0 + s_cur * kStage, sn = smem0 + s_nxt * kStage;
      step_ll8(acc, aX, lX, aY, lY, st + off_a32[1], st + off_lora_b + off_a32[1], c, win);
      stage_barrier<kCopies>();
      win = plan<LORA>(c, kt + 3, st);
      step_ll3(acc, aY, lY, aX, lX, sn + off_a32[0], sn + off_lora_b + off_a32[0], c, win);
      s_cur = s_nxt;
    }
    const uint32_t st = smem0 + s_cur * kStage;  // last LoRA tile
    step_ll8(acc, aX, lX, aY, lY, st + off_a32[1], st + off_lora_b + off_a32[1], c, win);
    stage_barrier<0>();
    step_ln(acc, aY, lY);
  }
  // the last MFMAs must retire before their accumulators are read by ordinary instructions (the
  // accumulators are operands, so no read of them can be scheduled above the wait)
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : H3Q_ACC(acc)::"memory");

  // Epilogue. Accumulator register r of lane l in a 32x32 tile holds
  // row (r/4)*8 + (l/32)*4 + r%4, column l%32.
  const float scale = p.ts * (p.ts_dev ? *p.ts_dev : 1.0f);
  const int row_lane = (lane >> 5) * 4;
  if constexpr (EPI == 2) {
    if (nt < 2 * p.q_tiles) {
      qk_norm_rope_epilogue(p, acc, smem, scale, m0, nt, wave, lane, nt < p.q_tiles);
      return;
    }
  }
  if constexpr (EPI != 1) {
    const bool rows16 = (p.out_ld & 7) == 0 && (p.n_out & (p.gate_up ? 15 : 7)) == 0 &&
                        (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
    if (rows16) {
      plain_epilogue_staged(p, acc, smem, scale, m0, nt, wave, lane);
      return;
    }
  } else {
    // an emit target is only accepted with aligned rows, so the 2-byte path below never needs it
    const bool rows16 = (p.out_ld & 7) == 0 && (p.n_out & 7) == 0 && (reinterpret_cast<uintptr_t>(p.out) & 15) == 0;
    if (rows16 || p.emit_out) {
      swiglu_epilogue_staged(p, acc, smem, scale, m0, nt, wave, lane);
      return;
    }
  }
#pragma unroll
  for (int i = 0; i < RT; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t row = m0 + i * 32 + (r >> 2) * 8 + row_lane + (r & 3);
      if (row >= p.S) continue;
      uint16_t* orow = p.out + row * p.out_ld;
      if (EPI != 1) {  // plain (also the v columns of the Q/K epilogue)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int cl = static_cast<int>(ncol[j]);
          const int64_t n = p.gate_up ? packed_row_source(nt, cl, true, p.n_out) : static_cast<int64_t>(nt) * BN + cl;
          if (n >= 0 && n < p.n_out) orow[n] = static_cast<uint16_t>(f32_to_bf16_hw(scale * acc[i][j][r]));
        }
      } else {
        // this wave's 64 tile columns are 32 gate columns then the 32 matching up columns
        const int64_t n = static_cast<int64_t>(nt) * (BN / 2) + wave * 32 + (lane & 31);
        if (n < p.n_out) {
          const float g = scale * acc[i][0][r];
          const float u = scale * acc[i][1][r];
          orow[n] = static_cast<uint16_t>(f32_to_bf16_hw(silu(g) * u));
        }
      }
    }
  }
}

template <int EPI, bool LORA>
hipError_t launch_variant(const GemmParams& p0, hipStream_t stream) {
  static std::once_flag once;
  static hipError_t attr_err = hipSuccess;
  std::call_once(once, [] {
    attr_err = hipFuncSetAttribute(reinterpret_cast<const void*>(&gemm_w4_kernel<EPI, LORA>),
                                   hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
  });
  if (attr_err != hipSuccess) return attr_err;

  // One launch covers every row: the activation and t' descriptors start at each tile's first row,
  // so their 32-bit offsets stay within one tile whatever S is.
  GemmParams p = p0;
  p.m_tiles = static_cast<int32_t>((p.S + BM - 1) / BM);
  const int64_t items = static_cast<int64_t>(p.m_tiles) * p.n_tiles;
  const int64_t grid = (items + 7) / 8 * 8;
  hipLaunchKernelGGL((gemm_w4_kernel<EPI, LORA>), dim3(grid), dim3(kThreads), kLdsBytes, stream, p);
  return hipGetLastError();
}

}  // namespace

size_t gemm_w4_lds_bytes() { return kLdsBytes; }

hipError_t launch_gemm_w4(const GemmParams& p, Epilogue epi, hipStream_t stream) {
  const bool lora = p.r_tiles > 0;
  if (epi == Epilogue::Plain) return lora ? launch_variant<0, true>(p, stream) : launch_variant<0, false>(p, stream);
  if (epi == Epilogue::QkNormRope)
    return lora ? launch_variant<2, true>(p, stream) : launch_variant<2, false>(p, stream);
  return lora ? launch_variant<1, true>(p, stream) : launch_variant<1, false>(p, stream);
}

}  // namespace h3q
