// h3q_layout.hpp -- the device layout of packed NVFP4 weights and of resident adapters, and the host
// loops that build them. Packing only moves bytes and nibbles (no arithmetic), so the GPU decode of a
// packed weight equals the canonical decode bit for bit. Plain C++ (no HIP types), so that a
// host-only program can run these loops under the address and undefined-behaviour sanitizers.
#pragma once

#include <stdint.h>

#include <cstring>

#if defined(__HIPCC__)
#define H3Q_HOST_DEVICE __host__ __device__
#else
#define H3Q_HOST_DEVICE
#endif

namespace h3q {

// Tile geometry of the main GEMM and of the packed weight layout (see gemm_w4.hip).
constexpr int kGemmBM = 256;   // rows of x per workgroup tile
constexpr int kGemmBN = 256;   // output columns (packed weight rows) per workgroup tile
constexpr int kGemmBK = 64;    // K per pipeline stage
// Packed codes: for column tile nt and K-tile kt, chunk kc (8 consecutive k) of all 256 rows is one
// run of 256 dwords: dword [((nt*k_tiles + kt)*8 + kc)*256 + c] holds row c's 8 codes, element i in
// nibble i. Packed scales: dword [(nt*k_tiles + kt)*256 + c] holds row c's 4 E4M3 block scales.
constexpr int kCodeChunksPerTile = kGemmBK / 8;          // 8
constexpr int kCodeTileBytes = kCodeChunksPerTile * kGemmBN * 4;  // 8 KiB per (nt, kt)
constexpr int kScaleTileBytes = kGemmBN * 4;              // 1 KiB per (nt, kt)
// LoRA K-tiles are 32 deep (bf16 B and t' tiles of 16 KiB each fit the base tile's LDS stage).
constexpr int kLoraBK = 32;
constexpr int kLoraTileBytes = kGemmBN * kLoraBK * 2;     // 16 KiB per (nt, rank tile)

// Row of the caller's weight that row c of packed column tile nt holds, or -1 for padding.
// Plain: nt*256 + c. Gate/up (F = N/2): the tile interleaves 32-row groups of gate rows
// nt*128 + (c/64)*32 + c%32 and the matching up rows F + (same), so that one workgroup holds both
// halves of every output column of SiLU(gate) * up.
H3Q_HOST_DEVICE inline int64_t packed_row_source(int64_t nt, int64_t c, bool gate_up, int64_t N) {
  if (!gate_up) {
    const int64_t n = nt * kGemmBN + c;
    return n < N ? n : -1;
  }
  const int64_t F = N / 2;
  const int64_t j = nt * (kGemmBN / 2) + (c / 64) * 32 + (c % 32);
  if (j >= F) return -1;
  return ((c / 32) % 2) ? F + j : j;
}

// Column tiles and K-tiles of a packed [N][K] weight (K padded to a whole K-tile).
inline int64_t packed_n_tiles(int64_t N, bool gate_up) {
  return gate_up ? (N / 2 + kGemmBN / 2 - 1) / (kGemmBN / 2) : (N + kGemmBN - 1) / kGemmBN;
}
inline int64_t packed_k_tiles(int64_t K) { return (K + kGemmBK - 1) / kGemmBK; }

// Canonical codes [N][K/2] (element k in the low nibble of byte k/2 when k is even) and scales
// [N][K/16] -> the packed layout above. tc: n_tiles*k_tiles*8*256 dwords, tsc: n_tiles*k_tiles*256
// dwords, both zero on entry (padding rows and columns stay zero).
inline void tile_weight(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K, bool gate_up,
                        uint32_t* tc, uint32_t* tsc) {
  const int64_t n_tiles = packed_n_tiles(N, gate_up), k_tiles = packed_k_tiles(K);
  for (int64_t nt = 0; nt < n_tiles; ++nt)
    for (int64_t c = 0; c < kGemmBN; ++c) {
      const int64_t n = packed_row_source(nt, c, gate_up, N);
      if (n < 0) continue;
      const uint8_t* crow = codes + n * (K / 2);
      const uint8_t* srow = scales + n * (K / 16);
      for (int64_t kt = 0; kt < k_tiles; ++kt) {
        const int64_t tile = nt * k_tiles + kt;
        for (int64_t kc = 0; kc < kCodeChunksPerTile && kt * kGemmBK + kc * 8 < K; ++kc)
          std::memcpy(&tc[(tile * kCodeChunksPerTile + kc) * kGemmBN + c], crow + (kt * kGemmBK + kc * 8) / 2, 4);
        uint32_t sw = 0;
        for (int64_t b = 0; b < kGemmBK / 16 && kt * (kGemmBK / 16) + b < K / 16; ++b)
          sw |= static_cast<uint32_t>(srow[kt * (kGemmBK / 16) + b]) << (8 * b);
        tsc[tile * kGemmBN + c] = sw;
      }
    }
}

// Adapter factors A bf16 [rank][K] and B bf16 [N][rank] -> the resident layouts: Ah [r_pad][K_pad]
// (zero padded) and Bh [n_tiles][r_pad/32][256][32] (32-deep K-tiles of the GEMM's folded operand,
// rows in the packed tile order). Ah and Bh are zero on entry.
inline void tile_adapter(const uint16_t* A, const uint16_t* B, int64_t rank, int64_t r_pad, int64_t N, int64_t K,
                         int64_t K_pad, bool gate_up, uint16_t* Ah, uint16_t* Bh) {
  for (int64_t j = 0; j < rank; ++j) std::memcpy(&Ah[j * K_pad], A + j * K, K * sizeof(uint16_t));
  const int64_t n_tiles = packed_n_tiles(N, gate_up), r_tiles = r_pad / kLoraBK;
  for (int64_t nt = 0; nt < n_tiles; ++nt)
    for (int64_t c = 0; c < kGemmBN; ++c) {
      const int64_t n = packed_row_source(nt, c, gate_up, N);
      if (n < 0) continue;
      for (int64_t j = 0; j < rank; ++j)
        Bh[((nt * r_tiles + j / kLoraBK) * kGemmBN + c) * kLoraBK + j % kLoraBK] = B[n * rank + j];
    }
}

// ---- LoRA-down work split (lora_down.hip) ----
// Row tiles of 32 a LoRA-down workgroup can hold with nc column tiles per wave: the RTM x nc
// accumulator tiles (16 registers each) stay within the 256 accumulation registers.
constexpr int lora_max_rtm(int nc) { return nc <= 2 ? 6 : (nc == 3 ? 5 : 3); }

struct LoraSplit {
  int64_t bm;       // rows per workgroup
  int32_t groups;   // column groups of A per row block (1, 2 or 4)
  int32_t nc;       // column tiles per wave
  int64_t blocks;   // workgroups: row blocks padded to whole groups of 8, times groups
};

// Every workgroup copies all of its group's A tiles from L2, so a CU moves |A| / g + bm * K * 2 *
// (1 + 1/g) bytes (x read by every group, xs written once). Among g in {1, 2, 4} dividing the column
// tiles, take the fewest bytes per CU times rounds, where g > 1 must take the rows in one round with
// rows that fit the accumulators (ties: the smaller g).
inline LoraSplit lora_down_split(int64_t S, int32_t r_pad, int64_t K, int64_t K_pad, bool xs, int cus) {
  const int ct_all = r_pad / 32;
  const double a_bytes = static_cast<double>(r_pad) * static_cast<double>(K_pad) * 2.0;
  const double row_bytes = static_cast<double>(K) * 2.0;
  LoraSplit best{0, 0, 0, 0};
  double best_cost = 0.0;
  for (int g = 1; g <= 4; g *= 2) {
    if (ct_all % g != 0) continue;
    const int nc = (ct_all / g + 3) / 4;
    const int64_t bm_max = 32 * lora_max_rtm(nc);
    int64_t bm = (S * g + cus - 1) / cus;
    if (bm < 32) bm = 32;
    if (bm > bm_max) {
      if (g > 1) continue;  // the rows would need more than one round: keep the columns together
      bm = bm_max;
    }
    const int64_t row_blocks = (S + bm - 1) / bm;
    const double rounds = static_cast<double>((row_blocks * g + cus - 1) / cus);
    const double cost = rounds * (a_bytes / g + static_cast<double>(bm) * row_bytes * (1.0 + (xs ? 1.0 / g : 0.0)));
    if (best.groups == 0 || cost < best_cost) {
      best = LoraSplit{bm, g, nc, (row_blocks + 7) / 8 * 8 * g};
      best_cost = cost;
    }
  }
  return best;
}

}  // namespace h3q
