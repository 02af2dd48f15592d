/*
 * mxmoe.h -- C ABI of the MXFP8 MoE routed-expert hot path on gfx950.
 *
 * What the library computes
 * -------------------------
 * Dynamic MXFP8 quantization followed by a block-scaled grouped GEMM for the
 * routed experts of a Mixture-of-Experts layer, forward, dgrad and wgrad:
 *   - "MXFP8 training for MoEs" article, section "Is MXFP8 Training for MoEs
 *     Actually Stable?": activations and weights are quantized dynamically to
 *     MXFP8, a scaled grouped GEMM runs, the result comes back in the original
 *     precision; section "Why Does MXFP8 Speed Up MoE Training So Much?":
 *     the backward pass mirrors the forward.
 *   - "MXFP8 (Micro-scaling FP8)" page, section "Definition": one shared
 *     power-of-two scale per small block of values; section "Low-precision
 *     Flash Attention (MXFP8 on FA4)": scales are generated along each GEMM's
 *     K dimension, scale factors come from bit manipulation rather than
 *     log2/round/clamp, and 32x32 square blocks (one scale per tile) make the
 *     quantization transpose-invariant.
 *   - "feat(moe): add MoK MXFP8 expert support" PR, review of the
 *     mxfp8_weights argument: every expert weight exists in two quantized
 *     orientations (weight_fp8/weight_scale for the forward, weight_t_fp8/
 *     weight_t_scale for the backward), and a mismatched call raises.  Its
 *     summary: unsupported settings are rejected with a clear error.
 *
 * Encoding (shared by every entry point)
 * --------------------------------------
 *   block    32 consecutive values along the contraction axis (1x32 rowwise,
 *            32x1 colwise) or a 32x32 tile;
 *   scale    one E8M0 byte per block: byte = clamp(floor(log2 amax) - 8,
 *            -127, 127) + 127 (8 is E4M3's largest exponent); 0x00 for an
 *            all-zero block; 0xFF when the block holds NaN or Inf;
 *   element  FP8 E4M3 (bias 7, largest finite 448, 0x7F = NaN) of
 *            value * 2^(127 - byte), rounded to nearest even, saturated to
 *            +-448, subnormals kept, sign kept on values that round to zero;
 *            every element of a NaN/Inf block is 0x7F.
 *   value    decode(q) * 2^(byte - 127).
 * bf16 is passed as uint16_t bit patterns, E4M3 and E8M0 as uint8_t.  All
 * tensors are dense and row-major unless a leading dimension says otherwise.
 *
 * Memory, streams, errors
 * -----------------------
 *   - Every tensor pointer is a DEVICE pointer (hipMalloc'd or a torch CUDA
 *     tensor), 16-byte aligned.  The caller owns all memory, including the
 *     workspace of the bf16 GEMM entry points; the library never allocates,
 *     frees or synchronizes.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Every call only enqueues kernels on it and returns.
 *   - Inputs are read-only.  Outputs are overwritten in full (an expert with
 *     no tokens gets an all-zero weight gradient).
 *   - Host-checkable misuse (null pointers, negative or misaligned sizes, a
 *     too-small workspace) returns a status != MX_OK before anything is
 *     launched; mx_last_error() then describes it (thread-local text).
 *   - Group offsets live on the device and are not checked against the host.
 *     Preconditions: non-decreasing, offs[E-1] == M, and for wgrad every
 *     group start a multiple of 32.  mx_check_offsets tests them on the
 *     device.  Kernels clamp offsets into the operand's extent (the rows of
 *     X in mode 0; the contraction length Kc in mode 1, which the wgrad
 *     entry point pads with zero codes from M up to M rounded to 128) and
 *     round wgrad group bounds down to multiples of 32, so a violation never
 *     reads or writes out of bounds; the values are then unspecified.
 *   - No global state besides the error text: calls are reentrant.
 */
#ifndef MXMOE_H
#define MXMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mx_status {
  MX_OK = 0,
  MX_ERR_NULL = 1,       /* a required pointer is NULL                        */
  MX_ERR_SHAPE = 2,      /* a size is negative or violates a divisibility rule */
  MX_ERR_ALIGN = 3,      /* a pointer is not 16-byte aligned                   */
  MX_ERR_WORKSPACE = 4,  /* workspace smaller than mx_grouped_mm_workspace_bytes */
  MX_ERR_HIP = 5,        /* a kernel launch failed (text has the HIP error)    */
  MX_ERR_LAYOUT = 6      /* scales passed in a layout the callee does not read */
} mx_status;

/* Arrangement of E8M0 scale bytes.  The quantizers write row-major scales
 * [rows][K/32]; the GEMM reads its blocked layout [K/128][rows][4] (see
 * mx_scales_to_gemm_layout).  The GEMM entry points take the layout of the
 * scales they are given and refuse anything but MX_SCALES_GEMM. */
typedef enum mx_scale_layout {
  MX_SCALES_ROWMAJOR = 0,
  MX_SCALES_GEMM = 1
} mx_scale_layout;

/* Text describing the last non-OK status returned on this thread. */
const char* mx_last_error(void);

/* Library version string. */
const char* mx_version(void);

/* ------------------------------------------------------------------------
 * Quantizers.  x is bf16 [batch, rows, cols] (batch >= 1, rows, cols >= 0).
 * ------------------------------------------------------------------------ */

/* 1x32 blocks along cols (the contraction axis of the GEMM that consumes
 * the result).  Requires cols % 32 == 0.
 * Out: q [batch, rows, cols] E4M3, s [batch, rows, cols/32] E8M0. */
mx_status mx_quantize_rowwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                              uint8_t* q, uint8_t* s, void* stream);

/* 32x1 blocks along rows, stored transposed so the block axis is contiguous
 * (the 3D colwise weight quantization of the dgrad path, and the token-axis
 * quantization of wgrad).  Requires rows % 32 == 0 and cols % 8 == 0.
 * Out: q_t [batch, cols, rows] E4M3, s_t [batch, cols, rows/32] E8M0. */
mx_status mx_quantize_colwise(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                              uint8_t* q_t, uint8_t* s_t, void* stream);

/* 32x32 square blocks, elements stay in place.  Requires rows % 32 == 0 and
 * cols % 32 == 0.  Out: q [batch, rows, cols], s [batch, rows/32, cols/32]. */
mx_status mx_quantize_32x32(const uint16_t* x, int64_t batch, int64_t rows, int64_t cols,
                            uint8_t* q, uint8_t* s, void* stream);

/* ------------------------------------------------------------------------
 * Scale layout conversion for the GEMM.  The quantizers above write scales
 * row-major, [batch, rows, kblocks].  The GEMM reads them in its blocked
 * layout [batch, kblocks/4, rows, 4]: element (b, r, kb) moves to
 * ((b * kblocks/4 + kb/4) * rows + r) * 4 + kb%4, so the four scale blocks of
 * one 128-element contraction step of consecutive rows are contiguous (the
 * role of the per-group blocked scale conversion in the pytorch/ao PR
 * timeline).  Requires kblocks % 4 == 0; s_gemm 4-byte aligned.
 * ------------------------------------------------------------------------ */
mx_status mx_scales_to_gemm_layout(const uint8_t* s, int64_t batch, int64_t rows, int64_t kblocks,
                                   uint8_t* s_gemm, void* stream);

/* ------------------------------------------------------------------------
 * The block-scaled grouped GEMM on prequantized operands.
 *
 *   C[i, j] = sum_k X[i, k] * Y[j, k] * 2^(sX[i, k/32] + sY[j, k/32] - 254)
 *
 * accumulated in fp32, stored as bf16 (round to nearest even).
 *   mode 0: groups over the rows i of X.  X [I, Kc], sX [I, Kc/32];
 *           Y [E, J, Kc], sY [E, J, Kc/32] (expert e's slice for group e);
 *           C [I, J].  Rows of an empty group do not exist.
 *   mode 1: groups over the contraction index k (weight gradient).
 *           X [I, Kc], Y [J, Kc] (token axis contiguous), C [E, I, J];
 *           expert e sums k in [offs[e-1], offs[e]); an empty group gives
 *           C[e] = 0.  Group starts must be multiples of 32.
 * Scale tensors are passed in the GEMM layout of mx_scales_to_gemm_layout
 * (sX with batch 1 and rows I; sY with batch E and rows J in mode 0, batch 1
 * and rows J in mode 1), and scale_layout must say so (MX_SCALES_GEMM);
 * MX_SCALES_ROWMAJOR returns MX_ERR_LAYOUT.
 * offs: int32 [E] cumulative END offsets on the device (offs[-1] = 0),
 * over rows of X (mode 0) or over k (mode 1).
 * Requires Kc % 128 == 0, J % 8 == 0, E >= 1.
 * Operand mapping: forward X = q(A), Y = q(W) (rowwise along K); dgrad
 * X = q(dOut) (rowwise along N), Y = q_t(W) (colwise along N, [E, K, N]);
 * wgrad X = q_t(dOut) [N, M], Y = q_t(A) [K, M] (colwise along tokens).
 * ------------------------------------------------------------------------ */
mx_status mx_grouped_gemm_mx(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                             int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J, int64_t Kc,
                             int64_t E, uint16_t* C, void* stream);

/* The same GEMM with the fp32 accumulators stored unrounded (C is float,
 * same shapes and rules).  For callers that accumulate results in fp32, e.g.
 * weight gradients summed over micro-batches before the optimizer step. */
mx_status mx_grouped_gemm_mx_f32(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                 int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J, int64_t Kc,
                                 int64_t E, float* C, void* stream);

/* mx_grouped_gemm_mx (bf16 output) with its workgroups dealt to output tiles
 * in a seeded pseudo-random order instead of the library's (XCD-aware)
 * order; order_seed = 0 is the library's order.  Every tile computes its
 * outputs alone, so the result is bit-identical for every seed: the race
 * check of the test suite compares seeds, which changes which tiles run side
 * by side and in what sequence. */
mx_status mx_grouped_gemm_mx_ordered(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                     int scale_layout, const int32_t* offs, int mode, int64_t I, int64_t J, int64_t Kc,
                                     int64_t E, uint16_t* C, uint64_t order_seed, void* stream);

/* ------------------------------------------------------------------------
 * Validity of group offsets, tested on the device (no host round trip; the
 * caller reads *status when it chooses to).  offs: int32 [E] cumulative END
 * offsets on the device; status: one int32 on the device, set to 0 when
 * every offset is valid, else to the OR of
 *   MX_OFFS_DECREASING  an offset below its predecessor (offs[-1] = 0),
 *   MX_OFFS_RANGE       an offset outside [0, M],
 *   MX_OFFS_LAST        offs[E-1] != M,
 *   MX_OFFS_ALIGN       a group start that is not a multiple of `align`
 *                       (the weight gradient needs align = 32: its 32-token
 *                       blocks must not straddle two experts).
 * Unsupported inputs get a clear error before they reach a GEMM ("feat(moe):
 * add MoK MXFP8 expert support" PR, summary).
 * ------------------------------------------------------------------------ */
#define MX_OFFS_DECREASING 1
#define MX_OFFS_RANGE 2
#define MX_OFFS_LAST 4
#define MX_OFFS_ALIGN 8
mx_status mx_check_offsets(const int32_t* offs, int64_t E, int64_t M, int32_t align, int32_t* status, void* stream);

/* ------------------------------------------------------------------------
 * The grouped GEMMs on bf16 inputs: quantize both operands into the caller's
 * workspace, then run the GEMM above.  M = total rows of A / dOut, grouped by
 * offs (int32 [E] cumulative END offsets on the device).
 * ------------------------------------------------------------------------ */
#define MX_OP_FWD 0
#define MX_OP_DGRAD 1
#define MX_OP_WGRAD 2

/* Bytes of workspace the bf16 entry point `op` needs (0 on invalid sizes). */
size_t mx_grouped_mm_workspace_bytes(int op, int64_t M, int64_t N, int64_t K, int64_t E);

/* out [M, N] = A [M, K] @ W[e] [N, K]^T per group.  Requires K % 128 == 0,
 * N % 8 == 0. */
mx_status mx_grouped_mm_fwd(const uint16_t* A, const uint16_t* W, const int32_t* offs,
                            int64_t M, int64_t N, int64_t K, int64_t E, uint16_t* out,
                            void* ws, size_t ws_bytes, void* stream);

/* dA [M, K] = dOut [M, N] @ W[e] [N, K] per group; W is quantized in 32-blocks
 * along N.  Requires N % 128 == 0, K % 8 == 0. */
mx_status mx_grouped_mm_dgrad(const uint16_t* dOut, const uint16_t* W, const int32_t* offs,
                              int64_t M, int64_t N, int64_t K, int64_t E, uint16_t* dA,
                              void* ws, size_t ws_bytes, void* stream);

/* dW [E, N, K], dW[e] = dOut[g_e]^T @ A[g_e]; both operands quantized in
 * 32-blocks along tokens.  Requires M % 32 == 0, every group start a multiple
 * of 32 (pad groups with zero rows), N % 8 == 0, K % 8 == 0. */
mx_status mx_grouped_mm_wgrad(const uint16_t* dOut, const uint16_t* A, const int32_t* offs,
                              int64_t M, int64_t N, int64_t K, int64_t E, uint16_t* dW,
                              void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Token gather fused into the rowwise quantizer (the rowwise-A quantization
 * done inside the token gather of the MoE dispatch).  Output row r holds the
 * codes of x[rows[r], :]; an index < 0 or >= src_rows gives a zero row (the
 * padding of expert groups to 32 rows).  x [src_rows, cols] bf16, rows int32
 * [M] on the device, q [M, cols], s_gemm in the GEMM scale layout
 * [cols/128, M, 4]: (q, s_gemm) is X of mx_grouped_gemm_mx as it stands.
 * Requires cols % 128 == 0.  Bit-identical to gathering the rows and calling
 * mx_quantize_rowwise then mx_scales_to_gemm_layout.
 * ------------------------------------------------------------------------ */
mx_status mx_quantize_rowwise_gather(const uint16_t* x, int64_t src_rows, const int32_t* rows, int64_t M,
                                     int64_t cols, uint8_t* q, uint8_t* s_gemm, void* stream);

/* ------------------------------------------------------------------------
 * Routed experts end to end on the device: the grouped GEMMs above take the
 * tokens already grouped by expert, with every group padded to a multiple of
 * 32 rows ("MXFP8 training for MoEs", section "Is MXFP8 Training for MoEs
 * Actually Stable?": the scaled grouped GEMM over each expert's routed
 * tokens; the MoK expert PR: routed-expert precision path).  The three calls
 * below build that grouping from the router's expert ids, gather the tokens
 * into it inside the quantizer, and scatter GEMM rows back to token order in
 * the GEMM's epilogue, so no permuted bf16 copy of the tokens exists.
 * ------------------------------------------------------------------------ */

/* Grouping of n routed items (tokens of a top-1 router, or the token-expert
 * pairs of a top-k router flattened token-major, item = token * k + slot).
 * expert_idx int32 [n] (device): the expert of each item.  Each expert's
 * items form one group, in their original order, followed by zero rows up to
 * a multiple of 32.  Outputs (device):
 *   offs [E]   int32 cumulative END offsets of the padded groups (the
 *              grouped GEMMs' offsets; offs[E-1] <= cap);
 *   rows [cap] int32 grouped row -> item; -1 for padding rows and for every
 *              row past offs[E-1];
 *   pos  [n]   int32 item -> grouped row (-1 for an item not routed);
 *   status     one int32: 0, or 1 when some expert id lies outside [0, E)
 *              (such items join no group).
 * Requires 1 <= E <= 1024, 0 <= n < 2^30 and cap >= n + 31*E (the most rows
 * the padded groups can take; round it up to a multiple of 128 to use the
 * rows as the wgrad contraction).  ws: device scratch of at least
 * mx_route_workspace_bytes(n, E) bytes, 4-byte aligned, the caller's; its
 * contents need no initialisation and are not meaningful afterwards.  Three
 * kernels (per-chunk histograms, one scan, per-chunk scatter); every grouped
 * row follows from counts and ranks, so the result is deterministic. */
size_t mx_route_workspace_bytes(int64_t n, int64_t E);
mx_status mx_route(const int32_t* expert_idx, int64_t n, int64_t E, int64_t cap, int32_t* offs, int32_t* rows,
                   int32_t* pos, int32_t* status, void* ws, size_t ws_bytes, void* stream);

/* mx_quantize_dual on gathered rows: row r of the quantized operand is
 * x[rows[r] / topk, :], or a zero row where rows[r] is negative or
 * >= src_rows * topk.  x bf16 [src_rows, cols]; rows int32 [M] (the `rows`
 * of mx_route, or its first M entries); outputs as mx_quantize_dual with
 * rows = M: q [M, cols], s [cols/128, M, 4], q_t [cols, ldq] (32x1 blocks
 * along the grouped rows), s_t [ldq/128, cols, 4].  topk = 1 gathers per
 * item (dOut of the backward, one row per item); topk = k gathers the token
 * of item a = token * k + slot (the forward's tokens).  Requires M % 32 == 0,
 * cols % 128 == 0, ldq % 128 == 0, ldq >= M, 1 <= topk <= 1024 and
 * src_rows * topk < 2^31.  Bit-identical to gathering the rows and calling
 * mx_quantize_dual. */
mx_status mx_quantize_dual_gather(const uint16_t* x, int64_t src_rows, const int32_t* rows, int64_t topk, int64_t M,
                                  int64_t cols, int64_t ldq, uint8_t* q, uint8_t* s, uint8_t* q_t, uint8_t* s_t,
                                  void* stream);

/* mx_grouped_gemm_mx in mode 0 with its rows stored through a map: the
 * result row of grouped row i (i inside a group) goes to C row row_map[i]
 * when 0 <= row_map[i] < c_rows and is dropped otherwise; C rows no entry
 * names are left as they were.  C bf16 [c_rows, J]; row_map int32 [I].
 * With the `rows` of mx_route as the map, the forward's output and the
 * dgrad's input gradient land in item order.  Arguments and rules otherwise
 * as mx_grouped_gemm_mx (mode 0). */
mx_status mx_grouped_gemm_mx_rows(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                  int scale_layout, const int32_t* offs, int64_t I, int64_t J, int64_t Kc, int64_t E,
                                  const int32_t* row_map, uint16_t* C, int64_t c_rows, void* stream);

/* mx_grouped_gemm_mx_rows with fp32 output C [c_rows, J] (accumulators stored
 * unrounded): the per-item input gradients of a top-k router, before
 * mx_topk_sum_rows adds each token's k of them. */
mx_status mx_grouped_gemm_mx_rows_f32(const uint8_t* X, const uint8_t* sX, const uint8_t* Y, const uint8_t* sY,
                                      int scale_layout, const int32_t* offs, int64_t I, int64_t J, int64_t Kc,
                                      int64_t E, const int32_t* row_map, float* C, int64_t c_rows, void* stream);

/* Gradient of the top-k token gather: a token feeds its k items, so its input
 * gradient is the sum of theirs.  out[t, c] = bf16(x[t*k, c] + x[t*k+1, c]
 * + ... + x[t*k+k-1, c]), summed in fp32 in slot order and rounded to nearest
 * even once.  x fp32 [T*k, cols], out bf16 [T, cols], both 16-byte aligned;
 * 1 <= k <= 1024, cols % 8 == 0. */
mx_status mx_topk_sum_rows(const float* x, int64_t T, int64_t k, int64_t cols, uint16_t* out, void* stream);

/* ------------------------------------------------------------------------
 * Prequantized expert weights: the weight 4-tuple of the MoK expert PR
 * review (weight_fp8 / weight_scale feed the forward, weight_t_fp8 /
 * weight_t_scale the backward).  Weights change once per optimizer step, so
 * both orientations are quantized once, in one pass that reads W once, and
 * reused by the forward and the dgrad of that step.
 * ------------------------------------------------------------------------ */

/* W [E, N, K] -> q [E, N, K] (1x32 blocks along K) with s in the GEMM scale
 * layout [E, K/128, N, 4], and q_t [E, K, N] (32x1 blocks along N, stored
 * transposed) with s_t in the GEMM scale layout [E, N/128, K, 4].  Requires
 * N % 128 == 0 and K % 128 == 0.  Bit-identical to mx_quantize_rowwise and
 * mx_quantize_colwise followed by mx_scales_to_gemm_layout.  w, q, q_t
 * 16-byte aligned; s, s_t 4-byte aligned. */
mx_status mx_quantize_weights(const uint16_t* w, int64_t E, int64_t N, int64_t K, uint8_t* q, uint8_t* s,
                              uint8_t* q_t, uint8_t* s_t, void* stream);

/* Activations in both orientations from one read: the forward quantizes its
 * tokens A [M, K] 1x32 along K for its own GEMM and 32x1 along the tokens for
 * the wgrad GEMM of the backward; the backward does the same with dOut [M, N]
 * for dgrad and wgrad ("MXFP8 training for MoEs": the backward mirrors the
 * forward, with each GEMM's operands blocked along its contraction dim).
 * x [rows, cols] bf16 -> q [rows, cols] (1x32 blocks along cols) with s in the
 * GEMM scale layout [cols/128, rows, 4] (X of the rows-grouped GEMM), and
 * q_t [cols, ldq] (32x1 blocks along rows, stored transposed) with s_t in the
 * GEMM scale layout [ldq/128, cols, 4] (an operand of the wgrad GEMM with
 * Kc = ldq).  Columns rows .. ldq-1 of q_t are the codes of zero rows (0x00,
 * scale byte 0).  Requires rows % 32 == 0, cols % 128 == 0, ldq % 128 == 0
 * and ldq >= rows.  Over rows 0 .. rows-1, bit-identical to
 * mx_quantize_rowwise and mx_quantize_colwise followed by
 * mx_scales_to_gemm_layout.  x, q, q_t 16-byte aligned; s, s_t 4-byte
 * aligned. */
mx_status mx_quantize_dual(const uint16_t* x, int64_t rows, int64_t cols, int64_t ldq, uint8_t* q, uint8_t* s,
                           uint8_t* q_t, uint8_t* s_t, void* stream);

/* Workspaces of the two entry points below (they quantize only the
 * activation side). */
#define MX_OP_FWD_Q 3
#define MX_OP_DGRAD_Q 4

/* mx_grouped_mm_fwd with W given as (q, s) of mx_quantize_weights: the
 * result is bit-identical.  Requires K % 128 == 0, N % 8 == 0. */
mx_status mx_grouped_mm_fwd_q(const uint16_t* A, const uint8_t* qW, const uint8_t* sW, const int32_t* offs,
                              int64_t M, int64_t N, int64_t K, int64_t E, uint16_t* out,
                              void* ws, size_t ws_bytes, void* stream);

/* mx_grouped_mm_dgrad with W given as (q_t, s_t) of mx_quantize_weights: the
 * result is bit-identical.  Requires N % 128 == 0, K % 8 == 0. */
mx_status mx_grouped_mm_dgrad_q(const uint16_t* dOut, const uint8_t* qWt, const uint8_t* sWt,
                                const int32_t* offs, int64_t M, int64_t N, int64_t K, int64_t E,
                                uint16_t* dA, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * mx_grouped_mm_fwd_q without a workspace, for callers that cannot allocate
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments as mx_grouped_mm_fwd_q minus the workspace,
 * same kernels and bit-identical results.  The MX codes and scales of A go
 * to a static device array of MX_NOALLOC_SCRATCH_BYTES (128 MiB) that the
 * library holds on every GPU it runs on until the process ends; inputs whose
 * quantized activations do not fit (256-aligned M*K codes plus M*K/32 scale
 * bytes) return MX_ERR_WORKSPACE.  Nothing is allocated or freed.  Every call
 * on one GPU shares that array: calls that overlap on one GPU (two streams,
 * or two host threads) race and must be ordered by the caller. */
#define MX_NOALLOC_SCRATCH_BYTES (128u << 20)
mx_status mx_grouped_mm_fwd_q_noalloc(const uint16_t* A, const uint8_t* qW, const uint8_t* sW,
                                      const int32_t* offs, int64_t M, int64_t N, int64_t K, int64_t E,
                                      uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MXMOE_H */
