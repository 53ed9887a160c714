/* h3q.h -- C ABI of the MI355X (gfx950) W4 + dynamic LoRA linear.
 *
 * Each entry point below either cites the passage of the pages that defines what it computes, or
 * says that it is a library convention (handles, introspection, diagnostics, timing), which the
 * pages do not describe.
 *
 * The operation (FL2VA Turbo page, section "Implementation"):
 *
 *     y = NVFP4_base(x (*) pre_quant_scale) + strength * (alpha / rank) * B(A x)
 *
 *   - the base weight W [N][K] is NVFP4: E2M1 element codes, one E4M3 ("FN": bias 7, no inf,
 *     NaN = 0x7F/0xFF) scale per 16 consecutive K-elements, and one fp32 tensor scale that
 *     multiplies on decode (the pages name only "NVFP4"; the layout below is this library's);
 *   - pre_quant_scale (pqs) multiplies the activation on the base path only; the bf16 LoRA branch
 *     receives the original activation (same section);
 *   - adapters stay resident and are selected per call; the LoRA delta is never merged into the
 *     packed weight, which no call ever writes (FL2VA Turbo, opening paragraph and "Hot API":
 *     "none" selects the base path);
 *   - fused QKV and fused gate/up are single matrices; gate/up output may be reduced in the same
 *     call to SiLU(gate) * up (MiniMax-H3 Ultra Fast, "Active optimization stack", MLP row, and
 *     "Kernel path");
 *   - W4A4 variant: the base path's activation is itself quantized to NVFP4 on every call
 *     (MiniMax-H3 Ultra Fast, "Kernel path", item 1).
 *
 * Conventions for every entry point:
 *   - bf16 tensors are passed as uint16_t bit patterns; all 2-D arrays are row-major and dense.
 *   - "host" pointers are read before the call returns; "device" pointers must stay valid until
 *     the work enqueued on `stream` (a hipStream_t; NULL = the null stream) has run.
 *   - every call returns H3Q_OK (0) or a positive H3Q_E_* code and on error sets h3q_last_error().
 *     Arguments, shapes, formats, adapter ids, the device and the workspace are all checked before
 *     the first launch, so every code except H3Q_E_HIP means that nothing has been enqueued and no
 *     output has been written. H3Q_E_HIP reports a launch that the runtime refused: the kernels of
 *     the same call enqueued before it may still run, but they write only the library's own
 *     workspace and temporaries (and, for h3q_merge_adapter, its `merged` output), never the
 *     caller's other outputs, which each call writes in its last kernel.
 *   - a weight handle belongs to the device that was current when it was packed; calls that use it
 *     must be made with that device current.
 *   - calls on different streams may run concurrently; registering or unregistering an adapter
 *     while a call that uses the same handle is in flight is not allowed.
 *   - the linear entry points use a device workspace per (device, stream), grown when a call needs
 *     more (t', the prescaled or quantized activation); growing synchronizes that stream.
 *   - stream capture (HIP graphs): the linear entry points may be captured once the same call (same
 *     or larger S) has run on the capturing stream outside the capture, so that its workspace is
 *     sized; a capture that would need a larger workspace fails with H3Q_E_ARG. A workspace a
 *     capture has used is never freed (if it must grow later, it is retired until the process ends),
 *     so graphs stay valid. Timing (h3q_timing_enable) must be off while capturing. Pack, register,
 *     merge, checksum and the AdaLN table build are not meant for capture.
 */
#ifndef H3Q_H
#define H3Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t h3q_status;
typedef struct h3q_weight_s* h3q_weight; /* opaque; owns its device memory */

enum {
  H3Q_OK = 0,
  H3Q_E_ARG = 1,         /* null pointer, non-finite scalar, bad flag */
  H3Q_E_SHAPE = 2,       /* dimensions out of range or inconsistent */
  H3Q_E_FORMAT = 3,      /* invalid NVFP4 scale code (sign bit set or NaN) */
  H3Q_E_ADAPTER = 4,     /* unknown or duplicate adapter id */
  H3Q_E_NOMEM = 5,       /* device or host allocation failed */
  H3Q_E_HIP = 6,         /* HIP runtime error (message carries hipGetErrorString) */
  H3Q_E_UNSUPPORTED = 7  /* current device is not gfx950 */
};

#define H3Q_ADAPTER_NONE (-1)

/* h3q_pack_weight flags */
enum { H3Q_PACK_GATE_UP = 1u << 0 }; /* rows [0, N/2) are gate, [N/2, N) are up (N even) */

/* h3q_linear_ex flags */
enum {
  H3Q_ACT_NVFP4 = 1u << 0,  /* W4A4: quantize x (*) pqs to NVFP4 per call for the base path */
  H3Q_EPI_SWIGLU = 1u << 1  /* output SiLU(gate) * up, [S][N/2]; needs an H3Q_PACK_GATE_UP weight */
};

/* Limits: 1 <= N, K <= 2^20 with K % 16 == 0 (and N even for H3Q_PACK_GATE_UP);
 * 1 <= rank <= 512; 0 <= S <= 2^24. */

/* Pack an NVFP4 weight (FL2VA Turbo, opening paragraph: the packed base that adapters are switched
 * over without rebuilding).
 *   codes  host  uint8 [N][K/2]  E2M1 codes, element k in the low nibble of byte k/2 when k is even
 *   scales host  uint8 [N][K/16] E4M3FN block scales; codes with the sign bit set or 0x7F -> E_FORMAT
 *   tensor_scale  fp32 > 0, finite; the decoded weight is E2M1 * E4M3 * tensor_scale
 * Copies into a device layout tiled for the GEMM (byte moves only; the values are untouched),
 * synchronizes `stream`, and returns a handle in *out. The caller may free codes/scales after. */
h3q_status h3q_pack_weight(void* stream, const uint8_t* codes, const uint8_t* scales, float tensor_scale,
                           int64_t N, int64_t K, uint32_t flags, h3q_weight* out);

/* Release a handle and every adapter registered on it (no call using it may be in flight).
 * Library convention (handle lifetime), not on the pages. */
h3q_status h3q_free_weight(h3q_weight w);

/* Register a resident LoRA adapter on one projection (FL2VA Turbo, "Implementation": A, B, rank and
 * alpha per target, validated at load).
 *   id     >= 0, unique on this handle (else E_ADAPTER); ids are scoped per handle
 *   A      host  bf16 [rank][K];   B  host  bf16 [N][rank];   alpha finite
 * Copies to device memory and synchronizes; the caller may free A and B after. */
h3q_status h3q_register_adapter(h3q_weight w, int32_t id, const uint16_t* A, const uint16_t* B, int32_t rank,
                                float alpha);

/* Drop an adapter (E_ADAPTER if unknown). No call using it may be in flight. Library convention
 * (the pages register adapters at start-up and never unload them). */
h3q_status h3q_unregister_adapter(h3q_weight w, int32_t id);

/* Registered ids of a handle: writes up to `cap` ids to `ids` (host) and the total to *count.
 * Library convention (introspection), not on the pages. */
h3q_status h3q_list_adapters(h3q_weight w, int32_t* ids, int32_t cap, int32_t* count);

/* Dimensions and flags of a handle (any out-pointer may be NULL). Library convention
 * (introspection), not on the pages. */
h3q_status h3q_weight_info(h3q_weight w, int64_t* N, int64_t* K, uint32_t* flags);

/* The projection (FL2VA Turbo, "Implementation"):
 *   x    device bf16 [S][K]     the original activation
 *   pqs  device fp32 [K]        pre_quant_scale of the base path, or NULL for all ones
 *   adapter_id                  a registered id, or H3Q_ADAPTER_NONE for the base path
 *   strength                    finite; 0 runs the base path (bit-identical to adapter none)
 *   y    device bf16 [S][N]     every element written; must not overlap x
 * Asynchronous on `stream`. S == 0 is a no-op. */
h3q_status h3q_linear(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                      int32_t adapter_id, float strength, uint16_t* y);

/* Fused gate/up projection followed by SiLU(gate) * up (MiniMax-H3 Ultra Fast, "Kernel path"):
 * w must be packed with H3Q_PACK_GATE_UP; h device bf16 [S][N/2]. Otherwise as h3q_linear. */
h3q_status h3q_linear_swiglu(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                             int32_t adapter_id, float strength, uint16_t* h);

/* h3q_linear with flags (H3Q_ACT_NVFP4, H3Q_EPI_SWIGLU): the projection of FL2VA Turbo,
 * "Implementation", with the activation quantized to NVFP4 per call for the base path (MiniMax-H3
 * Ultra Fast, "Kernel path", item 1) and/or the SiLU(gate) * up output. out is [S][N] or, with
 * H3Q_EPI_SWIGLU, [S][N/2]. With H3Q_ACT_NVFP4 the LoRA branch still receives the original bf16 x. */
h3q_status h3q_linear_ex(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                         int32_t adapter_id, float strength, uint32_t flags, uint16_t* out);

/* h3q_linear_ex for callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels and the same results bit for
 * bit, but the per-call workspace (the prescaled or quantized activation, t', the W4A4 scale) lives in
 * a fixed device array of H3Q_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, so the call allocates nothing, frees nothing and never synchronizes.
 * A call needs 256 + S * K_pad * 2 (unless pqs is NULL, K % 64 == 0 and the W4A4 flag is off) +
 * S * r_pad * 2 (with an active adapter) bytes, K_pad = K rounded up to 64 and r_pad = rank rounded
 * up to 32; a call that needs more fails with H3Q_E_SHAPE before anything is enqueued. Every call
 * on one GPU shares that GPU's array, whatever its stream: calls that overlap in time on one GPU race
 * on it, so the caller orders them (one stream, or events). Otherwise as h3q_linear_ex. */
#define H3Q_NOALLOC_SCRATCH_BYTES (64u << 20)
h3q_status h3q_linear_ex_noalloc(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                                 int32_t adapter_id, float strength, uint32_t flags, uint16_t* out);

/* Producer fusion across the MLP (FL2VA Turbo, "Implementation": a producer that emits the next
 * projection's base input together with the exact bf16 LoRA input; on the pages' hardware it was
 * bit-exact and 3.08% slower, and the runtime kept the materialized path).
 *
 * h3q_linear_swiglu_emit: h3q_linear_swiglu (flags: 0 or H3Q_ACT_NVFP4) whose epilogue also writes
 *   xs_next[s][j] = bf16( f32(h[s][j]) * pqs_next[j] )
 * -- the down projection's base operand, from the bf16 h it stores (so it equals what that projection
 * would compute from h itself). h and xs_next: device bf16 [S][N/2]; pqs_next: device fp32 [N/2];
 * all three 16-byte aligned, N/2 a multiple of 8; xs_next must not overlap h or x.
 *
 * h3q_linear_prescaled: h3q_linear with the base operand given: xs (device bf16 [S][K], 16-byte
 * aligned) is the GEMM's activation operand as it stands, x (device bf16 [S][K]) only feeds the LoRA
 * branch; there is no pre_quant_scale argument (it is inside xs). K must be a multiple of 64. With
 * xs = bf16(x * pqs) the result is bit-identical to h3q_linear(x, pqs). Otherwise as h3q_linear. */
h3q_status h3q_linear_swiglu_emit(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                                  int32_t adapter_id, float strength, uint32_t flags, uint16_t* h,
                                  const float* pqs_next, uint16_t* xs_next);
h3q_status h3q_linear_prescaled(void* stream, const uint16_t* x, const uint16_t* xs, int64_t S, h3q_weight w,
                                int32_t adapter_id, float strength, uint16_t* y);

/* Fused QKV projection followed by per-head Q/K RMSNorm and partial split-half rotary embedding
 * (MiniMax-H3 Ultra Fast, "Active optimization stack", attention projections: one fused QKV matrix
 * and one fused in-place Q/K RMSNorm + partial split-half RoPE; "Kernel path", item 2; 96 of the 128
 * head dimensions rotate: MiniMax-H3 Turbo CMF card, "On parity"). The projection is h3q_linear_ex
 * (flags: 0 or H3Q_ACT_NVFP4); its output columns are [q: q_width | k: q_width | v: the rest], q and
 * k in heads of 128. For each row and each q or k head, with v = the projection's fp32 value:
 *   u_i       = v_i / sqrt(mean_j v_j^2 + eps) * gamma_i        (gamma_q for q heads, gamma_k for k)
 *   y_i       = u_i * c_i - u_{i+h} * s_i,  y_{i+h} = u_{i+h} * c_i + u_i * s_i    (i < h = rot_dim/2)
 *   y_i       = u_i                                              (rot_dim <= i < 128)
 * with c = rope_cos[row][i], s = rope_sin[row][i]; v columns are the plain projection.
 *   q_width   multiple of 256 with 2 * q_width <= N (N a multiple of 8); weight not gate/up
 *   rot_dim   even, 0..128                  eps  finite, > 0
 *   gamma_q, gamma_k  device fp32 [q_width]
 *   rope_cos, rope_sin  device fp32 [S][rot_dim/2] (may be NULL when rot_dim is 0)
 *   y         device bf16 [S][N], 16-byte aligned, must not overlap x
 * Otherwise as h3q_linear. */
h3q_status h3q_linear_qk_norm_rope(void* stream, const uint16_t* x, int64_t S, const float* pqs, h3q_weight w,
                                   int32_t adapter_id, float strength, uint32_t flags, int64_t q_width,
                                   int32_t rot_dim, float eps, const float* gamma_q, const float* gamma_k,
                                   const float* rope_cos, const float* rope_sin, uint16_t* y);

/* The same with the rotated dims split into axis sections (MiniMax-H3 Ultra Fast, "Kernel path",
 * item 2: a three-axis split-half rotary). The pages do not say whether the split halves pair over
 * all rotated dims or within each axis's dims; this call serves either reading. The first rot_dim
 * dims of a head are n_sections consecutive sections of widths sections[0..n_sections) (host
 * int32, each even and > 0, summing to rot_dim, 1 <= n_sections <= 4; ignored when rot_dim is 0), and
 * each section is rotated in split halves within itself: for the section at dims [o, o + w) with
 * h = w / 2 and its table columns [o/2, o/2 + h),
 *   y_{o+i} = u_{o+i} * c - u_{o+i+h} * s,  y_{o+i+h} = u_{o+i+h} * c + u_{o+i} * s,
 *   c = rope_cos[row][o/2 + i], s = rope_sin[row][o/2 + i]      (i < h)
 * One section of rot_dim is h3q_linear_qk_norm_rope; three sections of 32 pair each axis's dims
 * within the axis. Bad sections -> H3Q_E_SHAPE. Otherwise as h3q_linear_qk_norm_rope. */
h3q_status h3q_linear_qk_norm_rope_sections(void* stream, const uint16_t* x, int64_t S, const float* pqs,
                                            h3q_weight w, int32_t adapter_id, float strength, uint32_t flags,
                                            int64_t q_width, int32_t rot_dim, const int32_t* sections,
                                            int32_t n_sections, float eps, const float* gamma_q,
                                            const float* gamma_k, const float* rope_cos, const float* rope_sin,
                                            uint16_t* y);

/* The merged route, for comparison with the dynamic path only: the adapter's update folded into the
 * weight before quantizing, as a converter that bakes a LoRA into a 4-bit checkpoint does (MiniMax-H3
 * Turbo CMF card, "What the conversion did", backbone item; "Which file"), where the dynamic path
 * keeps base and adapter apart on every call (FL2VA Turbo, "Implementation"). With Wq the packed
 * weight's E2M1 * E4M3 values, ts its tensor scale and c = strength * alpha / rank:
 *   m[n][k] = f32( Wq[n][k] * ts + (c * sum_j B[n][j] * A[j][k]) / pqs[k] )   fp64, j ascending
 * (pqs NULL -> ones; the division keeps m (x * pqs) = base + c B (A x) up to m's fp32 rounding), then
 * m is quantized exactly as h3q_quantize_nvfp4 quantizes v. adapter_id H3Q_ADAPTER_NONE, or strength
 * 0, merges nothing (a plain re-quantization of the decoded weight). Outputs, device pointers in the
 * caller's row order (gate/up weights: rows [0, N/2) gate, [N/2, N) up), ready for h3q_pack_weight
 * after a copy to the host:
 *   codes uint8 [N][K/2] (8-byte aligned), scales uint8 [N][K/16], ts fp32 [1],
 *   merged fp32 [N][K] (16-byte aligned) or NULL -- the unquantized m, if wanted.
 * pqs: device fp32 [K] (16-byte aligned) or NULL. Allocates N * K * 2 (+ N * K * 4 when merged is
 * NULL) bytes of temporary device memory and synchronizes `stream` before returning. The handle and
 * its adapter are not modified. Errors: unknown adapter -> H3Q_E_ADAPTER; null or misaligned output,
 * non-finite strength -> H3Q_E_ARG; allocation -> H3Q_E_NOMEM. */
h3q_status h3q_merge_adapter(void* stream, h3q_weight w, int32_t adapter_id, float strength, const float* pqs,
                             uint8_t* codes, uint8_t* scales, float* ts, float* merged);

/* The AdaLN modulation curve with the adapter folded in by the same K-concatenation as the main GEMM
 * (MiniMax-H3 Turbo CMF card, "What the conversion did": the pruned modulation W_p u(t) plus the
 * adapter's B (A silu(e(t))) become one rank-24 curve [W_p | B] [u(t) ; A silu(e(t))] driven by a
 * per-block table; MiniMax-H3 Ultra Fast, "Why the pruned transformer matters": u is an 8-value
 * coordinate sampled at 1025 points and interpolated linearly, the modulation matrix is [96768, 8]).
 *
 * h3q_adaln_table: table[b][i] = [ u[i][0..rb) ; scale * A_b silu(emb[i]) ] for the `samples` points
 * t_i = i / (samples - 1), fp32 accumulation, silu(z) = z / (1 + exp(-z)); scale = strength * alpha /
 * rank of the adapter (rebuild the table to change either). Device pointers:
 *   u      fp32 [samples][base_rank]        (shared by every block)
 *   emb    fp32 [samples][emb_dim]          (the timestep embedding at the sample points)
 *   A      bf16 [blocks][lora_rank][emb_dim] (NULL if lora_rank is 0)
 *   table  fp32 [blocks][samples][base_rank + lora_rank]
 * 1 <= blocks <= 65535, 2 <= samples <= 1048560, 1 <= base_rank, 0 <= lora_rank <= 32,
 * base_rank + lora_rank <= 64, samples * emb_dim <= 2^31.
 * Asynchronous.
 *
 * h3q_adaln_apply: for each of the T requested times (clamped to [0, 1]), with p = t (samples - 1),
 * i0 = min(floor(p), samples - 2), th = p - i0 and v = (1 - th) table[b][i0] + th table[b][i0 + 1]:
 *   out[tau][b][r] = bias[b][r] + sum_q M[b][r][q] v[q]          (fp32)
 *   M      bf16 [blocks][rows][R], row r = [W_p row | B row], 16-byte aligned; R % 8 == 0, 8 <= R <= 64
 *   bias   fp32 [blocks][rows] or NULL;  table  fp32 [blocks][samples][R];  t  fp32 [T], 1 <= T <= 8
 *   out    fp32 [T][blocks][rows]
 * Asynchronous on `stream`. */
h3q_status h3q_adaln_table(void* stream, const float* u, const float* emb, const uint16_t* A, float scale,
                           int32_t blocks, int32_t samples, int32_t emb_dim, int32_t base_rank, int32_t lora_rank,
                           float* table);
h3q_status h3q_adaln_apply(void* stream, const uint16_t* M, const float* bias, const float* table, const float* t,
                           int32_t T, int32_t blocks, int64_t rows, int32_t samples, int32_t R, float* out);

/* Measurement aid (library convention, not on the pages): the matrix-core throughput the board sustains under its power limit, beside which
 * the GEMM's rate is read (the nominal dense bf16 peak assumes the full engine clock). Each of the
 * `workgroups` workgroups of 256 threads (two waves per SIMD, as the main GEMM runs) performs
 * iters x 64 v_mfma_f32_32x32x16_bf16 per wave (32768 flops each) on 8 rotating operand pairs, with no
 * memory traffic in the loop: flops = workgroups * 4 * iters * 64 * 32768. Device pointers: ops_a,
 * ops_b bf16 [8][256][8] (16-byte aligned; the operand values, e.g. activation-like and decoded-weight-
 * like data), sink fp32 [workgroups * 256] (written, meaningless). Asynchronous on `stream`. */
h3q_status h3q_mfma_loop(void* stream, const uint16_t* ops_a, const uint16_t* ops_b, int32_t iters,
                         int32_t workgroups, float* sink);

/* The W4A4 activation quantizer on its own (MiniMax-H3 Ultra Fast, "Kernel path", item 1: the
 * activations are quantized to NVFP4 on every call), as h3q_linear_ex(H3Q_ACT_NVFP4) runs it
 * (the same kernels):
 *   v      = f32(x) * pqs[k] rounded to fp32            (pqs NULL -> v = x)
 *   ts     = amax|v| / (6 * 448) rounded to fp32         (1 when v is all zero)
 *   scale  = E4M3 nearest to amax_block|v| / (6 * ts), ties to even, saturating at 448
 *   code   = E2M1 nearest to v / (E4M3(scale) * ts), ties to even, saturating at 6; 0 if scale is 0
 * Each quotient is the exact quotient rounded once. All pointers are device pointers:
 *   x bf16 [S][K], pqs fp32 [K] or NULL, codes uint8 [S][K/2], scales uint8 [S][K/16], ts fp32 [1].
 * K % 16 == 0. Asynchronous on `stream`. */
h3q_status h3q_debug_quantize_act(void* stream, const uint16_t* x, int64_t S, int64_t K, const float* pqs,
                                  uint8_t* codes, uint8_t* scales, float* ts);
/* The same entry point under its earlier name. */
h3q_status h3q_quantize_nvfp4(void* stream, const uint16_t* x, int64_t S, int64_t K, const float* pqs,
                              uint8_t* codes, uint8_t* scales, float* ts);

/* Diagnostic (library convention): the weight as the GEMM's decode stage sees it, E2M1 * E4M3
 * without the tensor scale (exact in bf16), written to device bf16 [N][K]. Uses the same device
 * decode as the GEMM; it exists so that the decode can be compared with the format's definition
 * bit for bit. */
h3q_status h3q_debug_dequant(void* stream, h3q_weight w, uint16_t* wq);

/* Diagnostic (library convention): 64-bit FNV-1a hash of the packed weight's device bytes
 * (synchronizes `stream`). It makes the pages' rule checkable that the adapter is never merged into
 * the packed base (FL2VA Turbo, "Implementation"): the hash is unchanged across any number of
 * h3q_linear calls. */
h3q_status h3q_weight_checksum(void* stream, h3q_weight w, uint64_t* out);

/* Measurement aid (library convention, not on the pages): kernel timing with HIP events recorded
 * on the call's stream around each launch of one kind.
 * Off by default. h3q_timing_get waits for the recorded events, returns the summed milliseconds
 * and the number of launches of `kind` since the last get (or enable), and resets that kind. */
enum { H3Q_KERNEL_GEMM = 0, H3Q_KERNEL_LORA_DOWN = 1, H3Q_KERNEL_PRESCALE = 2, H3Q_KERNEL_ACT_QUANT = 3 };
h3q_status h3q_timing_enable(int32_t on);
h3q_status h3q_timing_get(int32_t kind, double* total_ms, int64_t* launches);

/* Thread-local description of the last failure on this thread ("" if none). Library convention. */
const char* h3q_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* H3Q_H */
