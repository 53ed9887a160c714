// h3q_kernels.hpp -- launch interface between the C-ABI layer (h3q_api.cpp) and the gfx950 kernels.
// Host-side only: parameter blocks and launcher functions; every launcher returns the HIP error of
// its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "h3q_layout.hpp"

namespace h3q {

struct GemmParams {
  const uint16_t* act;      // bf16 [S][act_ld]: activation operand (x, x*pqs, or decoded NVFP4 x)
  int64_t act_ld;
  const uint16_t* lora_t;   // bf16 [S][r_pad]: f * (A x), folded in as extra K-columns; or null
  int64_t lora_t_ld;
  const uint8_t* wcodes;    // packed codes (layout above)
  const uint8_t* wscales;   // packed scales (layout above)
  const uint16_t* lora_b;   // bf16 [n_tiles][r_tiles][256][32], rows in the weight's tile order
  int64_t S;
  int32_t k_tiles;          // K_pad / 64
  int32_t r_tiles;          // r_pad / 32 (0: no adapter)
  int32_t m_tiles, n_tiles;
  int64_t n_out;            // valid output columns (N, or N/2 for SwiGLU)
  int32_t gate_up;          // weight packed with interleaved gate/up column tiles
  float ts;                 // weight tensor scale
  const float* ts_dev;      // optional device scalar multiplying ts (W4A4 activation scale)
  uint16_t* out;            // bf16 [S][n_out]
  int64_t out_ld;
  // Q/K RMSNorm + rotary epilogue only: column tiles [0, q_tiles) are q, [q_tiles, 2 q_tiles) are k
  const float* qk_gamma_q;  // fp32 [q_tiles * 256]
  const float* qk_gamma_k;  // fp32 [q_tiles * 256]
  const float* rope_cos;    // fp32 [S][rope_half]
  const float* rope_sin;    // fp32 [S][rope_half]
  int32_t q_tiles;
  int32_t rope_half;        // rotated pairs per 128-wide head (rot_dim / 2): the angle table's columns
  float qk_eps;
  // the rotated dims as consecutive sections, each rotated in split halves within itself; table
  // columns follow the sections in order (one section of rot_dim: pair i is dims i and i + rot_dim/2)
  int32_t rope_nsec;        // 1..4
  int32_t rope_sec[4];      // section widths (even, summing to rot_dim)
  // when every section's half is a multiple of 8 (rope_vec), pair group g (table columns 8g..8g+7)
  // rotates dims rope_lo[g] + e with rope_hi[g] + e, e < 8
  int32_t rope_vec;
  int32_t rope_lo[8], rope_hi[8];
  // SwiGLU epilogue only, optional: also write the next projection's base operand
  // emit_out[s][n] = bf16(f32(h[s][n]) * emit_pqs[n]) (16-byte aligned rows, n_out % 8 == 0)
  const float* emit_pqs;    // fp32 [n_out]
  uint16_t* emit_out;       // bf16 [S][emit_ld] or null
  int64_t emit_ld;
};

enum class Epilogue { Plain = 0, SwiGLU = 1, QkNormRope = 2 };

hipError_t launch_gemm_w4(const GemmParams& p, Epilogue epi, hipStream_t stream);
size_t gemm_w4_lds_bytes();

struct LoraDownParams {
  const uint16_t* x;        // bf16 [S][K] (caller's activation)
  const float* pqs;         // fp32 [K] or null
  const uint16_t* A;        // bf16 [r_pad][K_pad], zero padded
  int64_t S, K, K_pad;
  int32_t r_pad;
  float f;                  // t' = bf16(f / (*f_div_dev or 1) * (A x))
  const float* f_div_dev;
  uint16_t* t_out;          // bf16 [S][r_pad]
  uint16_t* xs_out;         // bf16 [S][K_pad] = x * pqs, or null
  int64_t bm;               // rows per workgroup (set by launch_lora_down)
  int32_t groups;           // column groups of A per row block (set by launch_lora_down)
};
hipError_t launch_lora_down(const LoraDownParams& p, hipStream_t stream);

struct PrescaleParams {
  const uint16_t* x;        // bf16 [S][K]
  const float* pqs;         // fp32 [K] or null
  int64_t S, K, K_pad;
  uint16_t* xs_out;         // bf16 [S][K_pad]
};
hipError_t launch_prescale(const PrescaleParams& p, hipStream_t stream);

struct ActQuantParams {
  const uint16_t* x;        // bf16 [S][K]
  const float* pqs;         // fp32 [K] or null
  int64_t S, K;
  uint32_t* amax_bits;      // device scratch: global amax as fp32 bits
  float* ts_out;            // device fp32 [1]
  uint8_t* codes;           // [S][K/2] or null
  uint8_t* scales;          // [S][K/16] or null
  uint16_t* xq_out;         // bf16 [S][xq_ld] = E2M1 * E4M3 (no ts), or null
  int64_t xq_ld;            // >= K; columns [K, xq_ld) are written as zero
  const float* xf = nullptr; // fp32 [S][K] input used as v instead of x * pqs (x, pqs unused), or null
};
hipError_t launch_act_quant(const ActQuantParams& p, hipStream_t stream);

struct DequantParams {
  const uint32_t* wcodes_dw;
  const uint32_t* wscales_dw;
  int32_t n_tiles, k_tiles;
  bool gate_up;
  int64_t N, K;
  uint16_t* out;            // bf16 [N][K]
};
hipError_t launch_debug_dequant(const DequantParams& p, hipStream_t stream);
// 64 MFMAs of 32x32x16 per wave and iteration; ops_a, ops_b: bf16 [8][256][8]; sink: [workgroups * 256]
hipError_t launch_mfma_loop(const uint16_t* ops_a, const uint16_t* ops_b, int32_t iters, int32_t workgroups,
                            float* sink, hipStream_t stream);

// Merged route (merge.hip): m = f32(Wq * ts + c * (B A) / pqs) in fp64, rows in the caller's order.
struct MergeParams {
  const uint16_t* wq;       // bf16 [N][K] = E2M1 * E4M3 (from the dequant kernel)
  const uint16_t* A;        // adapter A, bf16 [r_pad][K_pad] (unused when r_pad == 0)
  const uint16_t* B;        // adapter B, bf16 [n_tiles][r_pad/32][256][32]
  const float* pqs;         // [K] or null (ones)
  float* m;                 // fp32 [N][K]
  double ts, c;             // weight tensor scale; strength * alpha / rank (0 without an adapter)
  int64_t N, K, K_pad;
  int32_t n_tiles, r_pad;
  bool gate_up;
};
hipError_t launch_lora_merge(const MergeParams& p, hipStream_t stream);

// AdaLN modulation curve (adaln.hip).
struct AdalnTableParams {
  const float* u;           // fp32 [S][rb], shared by the blocks
  const float* emb;         // fp32 [S][E]
  const uint16_t* A;        // bf16 [blocks][rl][E] (unused when rl == 0)
  float c;                  // strength * alpha / rank
  int32_t blocks, S, E, rb, rl;  // rl <= 32
  float* table;             // fp32 [blocks][S][rb + rl]
};
hipError_t launch_adaln_table(const AdalnTableParams& p, hipStream_t stream);

struct AdalnApplyParams {
  const uint16_t* M;        // bf16 [blocks][rows][R], 16-byte aligned, R % 8 == 0, R <= 64
  const float* bias;        // fp32 [blocks][rows] or null
  const float* table;       // fp32 [blocks][S][R]
  const float* t;           // fp32 [T], T <= 8
  int32_t T, blocks, S, R;
  int64_t rows;
  float* out;               // fp32 [T][blocks][rows]
};
hipError_t launch_adaln_apply(const AdalnApplyParams& p, hipStream_t stream);

}  // namespace h3q
