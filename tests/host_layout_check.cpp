// Host-only check of the packing loops in bit_linear_dynamic_amd/csrc/h3q_layout.hpp, built by
// tests/test_sanitizers_cpu.py with the address and undefined-behaviour sanitizers. For ragged shapes,
// plain and gate/up, it packs random codes, scales and adapter factors and reads every element back
// from the packed buffers through the layout as the comments define it, written out here a second
// time (the inverse direction: from a caller's row to its packed tile and column), so that an index
// slip in either the loops or this check shows as a mismatch, and any access outside the buffers as a
// sanitizer report. It also checks the LoRA-down work split (lora_down_split). Prints "ok" and exits 0
// when everything matches.
#include <cstdint>
#include <cstdio>
#include <random>
#include <vector>

#include "../bit_linear_dynamic_amd/csrc/h3q_layout.hpp"

using namespace h3q;

namespace {

// Packed tile and column of caller row n (the inverse of packed_row_source).
void packed_position(int64_t n, int64_t N, bool gate_up, int64_t* nt, int64_t* c) {
  if (!gate_up) {
    *nt = n / 256;
    *c = n % 256;
    return;
  }
  const int64_t F = N / 2;
  const bool up = n >= F;
  const int64_t j = up ? n - F : n;           // output column of SiLU(gate) * up
  *nt = j / 128;
  const int64_t w = j % 128;                  // a tile holds 128 output columns in 4 groups of 32,
  *c = (w / 32) * 64 + (up ? 32 : 0) + w % 32;  // each as 32 gate rows then the 32 matching up rows
}

int check(int64_t N, int64_t K, int64_t rank, bool gate_up, std::mt19937& rng) {
  std::uniform_int_distribution<int> byte(0, 255), scale(0, 0x7E);
  std::vector<uint8_t> codes(N * (K / 2)), scales(N * (K / 16));
  for (auto& v : codes) v = static_cast<uint8_t>(byte(rng));
  for (auto& v : scales) v = static_cast<uint8_t>(scale(rng));
  const int64_t n_tiles = packed_n_tiles(N, gate_up), k_tiles = packed_k_tiles(K);
  std::vector<uint32_t> tc(n_tiles * k_tiles * 8 * 256, 0u), tsc(n_tiles * k_tiles * 256, 0u);
  tile_weight(codes.data(), scales.data(), N, K, gate_up, tc.data(), tsc.data());
  int bad = 0;
  std::vector<char> seen(n_tiles * 256, 0);
  for (int64_t n = 0; n < N; ++n) {
    int64_t nt, c;
    packed_position(n, N, gate_up, &nt, &c);
    if (nt >= n_tiles || packed_row_source(nt, c, gate_up, N) != n) ++bad;
    seen[nt * 256 + c] = 1;
    for (int64_t k = 0; k < K; ++k) {
      const int want = (k % 2 == 0) ? (codes[n * (K / 2) + k / 2] & 0xF) : (codes[n * (K / 2) + k / 2] >> 4);
      const int64_t kt = k / 64, kc = (k % 64) / 8, i = k % 8;
      const uint32_t dw = tc[((nt * k_tiles + kt) * 8 + kc) * 256 + c];
      if (static_cast<int>((dw >> (4 * i)) & 0xF) != want) ++bad;
    }
    for (int64_t b = 0; b < K / 16; ++b) {
      const uint32_t dw = tsc[(nt * k_tiles + b / 4) * 256 + c];
      if (((dw >> (8 * (b % 4))) & 0xFF) != scales[n * (K / 16) + b]) ++bad;
    }
  }
  // padding rows and padding K columns hold zeros
  for (int64_t p = 0; p < n_tiles * 256; ++p)
    if (!seen[p]) {
      const int64_t nt = p / 256, c = p % 256;
      for (int64_t kt = 0; kt < k_tiles; ++kt) {
        for (int64_t kc = 0; kc < 8; ++kc) bad += tc[((nt * k_tiles + kt) * 8 + kc) * 256 + c] != 0u;
        bad += tsc[(nt * k_tiles + kt) * 256 + c] != 0u;
      }
    }
  for (int64_t nt = 0; nt < n_tiles; ++nt)
    for (int64_t c = 0; c < 256; ++c)
      for (int64_t k = K; k < k_tiles * 64; ++k) {
        const uint32_t dw = tc[((nt * k_tiles + k / 64) * 8 + (k % 64) / 8) * 256 + c];
        bad += ((dw >> (4 * (k % 8))) & 0xF) != 0u;
      }
  // adapter
  const int64_t r_pad = (rank + 31) / 32 * 32, K_pad = k_tiles * 64;
  std::vector<uint16_t> A(rank * K), B(N * rank);
  for (auto& v : A) v = static_cast<uint16_t>(byte(rng) | (byte(rng) << 8));
  for (auto& v : B) v = static_cast<uint16_t>(byte(rng) | (byte(rng) << 8));
  std::vector<uint16_t> Ah(r_pad * K_pad, 0), Bh(n_tiles * r_pad * 256, 0);
  tile_adapter(A.data(), B.data(), rank, r_pad, N, K, K_pad, gate_up, Ah.data(), Bh.data());
  for (int64_t j = 0; j < r_pad; ++j)
    for (int64_t k = 0; k < K_pad; ++k) bad += Ah[j * K_pad + k] != ((j < rank && k < K) ? A[j * K + k] : 0);
  for (int64_t n = 0; n < N; ++n) {
    int64_t nt, c;
    packed_position(n, N, gate_up, &nt, &c);
    for (int64_t j = 0; j < r_pad; ++j)
      bad += Bh[((nt * (r_pad / 32) + j / 32) * 256 + c) * 32 + j % 32] != (j < rank ? B[n * rank + j] : 0);
  }
  if (bad) std::printf("N=%lld K=%lld rank=%lld gate_up=%d: %d mismatches\n", (long long)N, (long long)K,
                       (long long)rank, gate_up ? 1 : 0, bad);
  return bad;
}

}  // namespace

// The LoRA-down work split (lora_down_split): rows per workgroup within what the accumulators hold,
// one round whenever the columns are split, every (row block, column group) of the workgroup mapping
// that lora_down_kernel uses (block b: row block (b / 8g) * 8 + b % 8, group (b / 8) % g) exactly once
// with the groups of a row block on one XCD (b % 8), and one group at the block's S = 37726.
int check_split(int64_t S, int32_t r_pad, int64_t K, bool xs, int cus) {
  const int64_t K_pad = (K + 63) / 64 * 64;
  const LoraSplit sp = lora_down_split(S, r_pad, K, K_pad, xs, cus);
  int bad = 0;
  const int ct = r_pad / 32;
  if (sp.groups < 1 || ct % sp.groups != 0 || sp.nc != (ct / sp.groups + 3) / 4) ++bad;
  if (sp.bm < 32 || sp.bm > 32 * lora_max_rtm(sp.nc)) ++bad;
  const int64_t row_blocks = (S + sp.bm - 1) / sp.bm;
  if (sp.groups > 1 && row_blocks * sp.groups > cus) ++bad;
  if (sp.blocks != (row_blocks + 7) / 8 * 8 * sp.groups) ++bad;
  std::vector<char> seen(static_cast<size_t>(row_blocks * sp.groups), 0);
  for (int64_t b = 0; b < sp.blocks; ++b) {
    const int64_t rb = (b / (8 * sp.groups)) * 8 + b % 8, grp = (b / 8) % sp.groups;
    if (rb % 8 != b % 8) ++bad;
    if (rb * sp.bm >= S) continue;  // padding workgroups return at once
    char& v = seen[static_cast<size_t>(rb * sp.groups + grp)];
    if (v) ++bad;
    v = 1;
  }
  for (char v : seen) bad += v ? 0 : 1;
  if (bad) std::printf("lora_down_split S=%lld r_pad=%d K=%lld: %d mismatches\n", (long long)S, r_pad, (long long)K, bad);
  return bad;
}

int main() {
  std::mt19937 rng(2024);
  int bad = 0;
  const int64_t shapes[][3] = {{1, 16, 1}, {300, 208, 65}, {256, 64, 32}, {520, 1040, 384}, {70, 96, 16},
                               {2 * 116, 96, 16}, {2 * 200, 320, 128}, {2 * 128, 64, 7}, {257, 16, 512}};
  for (const auto& s : shapes) {
    bad += check(s[0], s[1], s[2], false, rng);
    if (s[0] % 2 == 0) bad += check(s[0], s[1], s[2], true, rng);
  }
  for (int64_t S : {1, 31, 77, 256, 300, 1000, 8192, 16384, 37726, 37728, 65836, 140000, 4200000})
    for (int32_t r_pad : {32, 64, 128, 160, 320, 384, 512})
      for (int64_t K : {512, 1040, 6144, 16384})
        for (bool xs : {true, false}) bad += check_split(S, r_pad, K, xs, 256);
  for (int32_t r_pad : {128, 384})
    for (int64_t K : {6144, 16384})
      if (lora_down_split(37726, r_pad, K, K, true, 256).groups != 1) ++bad;
  if (bad) return 1;
  std::printf("ok\n");
  return 0;
}
