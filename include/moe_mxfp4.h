/*
 * moe_mxfp4.h -- C ABI of the MXFP4 routed-expert mixture-of-experts layer
 * for AMD MI355X (gfx950).
 *
 * The layer (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the
 * specific optimisations; VibeSys "Qwen3.5-397B on 4x MI300A" post, sections
 * "Goal" and "Baseline"; MiniMax M3 on MI355X post, sections "Local shape
 * and tiling" and "Shared expert fusion"):
 *
 *   0. (optional) the router GEMM producing the logits   moe_route_topk_gemm
 *   1. softmax top-K routing over E experts, the shared expert folded in as
 *      expert E in slot K                              moe_route_topk
 *   2. permute: group the (token, slot) assignments by expert   moe_align_sort
 *   1 and 2 in one call (one launch for a small batch)  moe_route_align
 *   3. (W4A4 only) MXFP4-quantise the activations      moe_mxfp4_quantize
 *   4. grouped gate/up GEMM on MXFP4 weights + SwiGLU  moe_expert_gate_up
 *   5. grouped down GEMM                               moe_expert_down
 *   6. weighted combine back into token order          moe_combine
 *   all six in one call                                moe_mxfp4_forward
 *   0-6 in one call                                    moe_mxfp4_forward_router
 *   L layers of 0-6 in one call (a decode step's MoE layers)
 *                                                      moe_mxfp4_forward_layers
 *   the same with the residual add and RMSNorm after each layer
 *                                                      moe_mxfp4_forward_layers_norm
 *   after the layer: partial outputs summed (tensor parallelism), residual
 *   added, RMSNorm                                     moe_residual_rmsnorm
 *
 * The same layer over MXFP8 expert weights (bf16 activations; the pages
 * serve MoE models in MXFP8 next to MXFP4: MiniMax M3 on MI355X post,
 * section on its MI355X performance benchmarks): moe_mxfp8_quantize,
 * moe_mxfp8_expert_gate_up, moe_mxfp8_expert_down, moe_mxfp8_forward, with
 * steps 1, 2 and 6 shared.
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers (HBM of the current HIP device),
 *     owned by the caller; the library reads/writes them only during the
 *     enqueued work and keeps no reference.  Scalars are passed by value.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call
 *     only enqueues work on it and returns; it never synchronises, never
 *     allocates device memory and never reads device memory on the host, so
 *     a call can be captured in a HIP graph.  Faults inside kernels surface
 *     at the caller's next synchronisation.
 *   - All argument checks happen before anything is enqueued; on an error
 *     nothing is enqueued and no output is touched.  T = 0 is valid and
 *     enqueues nothing (moe_align_sort and moe_route_align still write
 *     their zero tables).
 *   - Vector-loaded buffers (activations, packed weights, y, quantiser
 *     input and output) must be 16-byte aligned.
 *   - Shapes: H and I multiples of 128; E <= 1024; K + shared <= 32.
 *     The kernels address the activations, h and each expert's weight
 *     codes with 32-bit offsets: x (T*H*2 bytes bf16, T*H/2 MXFP4), h
 *     (T*K'*I*2 or T*K'*I/2) and one expert's codes (2I*H/2, 2I*H for MXFP8;
 *     the same for W2) each stay below 2 GiB, else UNSUPPORTED.
 *
 * MXFP4 (OCP Microscaling v1.0): per 32 consecutive elements along the
 * reduction axis one E8M0 scale byte b (value 2^(b-127)) and 32 E2M1 codes
 * (s|ee|m, values +-{0, .5, 1, 1.5, 2, 3, 4, 6}), two codes per byte with
 * element 2j in the low nibble.  Scale bytes 1..254 are supported; 0 only
 * for all-zero blocks; 255 (NaN) is outside the contract.
 *
 * Weight matrices (expert e in [0, E'), E' = E + shared; the shared expert
 * is expert E), row-major as moe_mxfp4_quantize writes them:
 *   w13       uint8 [E', 2I, H/2]  rows [0, I) gate, rows [I, 2I) up
 *   w13_scale uint8 [E', 2I, H/32]
 *   w2        uint8 [E', H, I/2]
 *   w2_scale  uint8 [E', H, I/32]
 *
 * MXFP8 (OCP Microscaling v1.0): per 32 consecutive elements along the
 * reduction axis one E8M0 scale byte and 32 FP8 E4M3 codes, one per byte
 * (s|eeee|mmm, bias 7, subnormals m/8 * 2^-6, largest 448, S.1111.111 =
 * NaN outside the contract).  Matrices as above with one byte per element:
 *   w13 uint8 [E', 2I, H], w2 uint8 [E', H, I]; the scales as for MXFP4.
 *
 * Native code order.  The GEMM entry points (moe_expert_gate_up,
 * moe_expert_down, the mxfp8 ones and every forward) take the weight CODES
 * (w13, w2) in the kernels' native order, which moe_weights_to_native makes
 * from the row-major matrices once, when the weights are loaded; the scales
 * stay row-major.  Per expert, with K the reduction length (H for w13, I for
 * w2), NQ = 1 (MXFP4) or 2 (MXFP8) and C = K/128 chunks, the codes are
 * 1 KiB blocks: block ((s*C + c)*NQ + q) holds at byte 16*l (l < 64,
 * l = 16*g + n) the 16 row-major bytes of row
 * 32*(s/2) + 8*(n/4) + 4*(s%2) + n%4 starting at byte
 * NQ*(64*c + 16*g) + 16*q.  An expert keeps its size and place (expert e
 * starts at e * rows * K * NQ / 2 bytes), so each expert's codes stay one
 * contiguous range.  (One MFMA operand load of 16 rows x 128 elements is
 * then one contiguous KiB instead of 16 half cache lines; the two 16-row
 * strips of each 32-row group interleave their rows in runs of four so
 * that a lane of the MFMA result holds eight consecutive output columns.)
 */
#ifndef MOE_MXFP4_H
#define MOE_MXFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARGUMENT = 1,   /* null pointer, negative size, bad flag, misaligned buffer */
  MOE_ERR_UNSUPPORTED = 2,        /* a shape outside the compiled kernels' range */
  MOE_ERR_WORKSPACE_TOO_SMALL = 3,
  MOE_ERR_DEVICE = 4              /* a HIP launch error (hipGetLastError) */
} moe_status;

/* Activation formats of the GEMM entry points.  MOE_ACT_MXFP4_BLOCKED is
 * MXFP4 in the blocked row order below, for the LDS-tiled GEMMs only (the
 * forward uses it for W4A4 whenever it picks tiled GEMMs). */
typedef enum {
  MOE_ACT_BF16 = 0 /* W4A16 */,
  MOE_ACT_MXFP4 = 1 /* W4A4, row-major codes and scales */,
  MOE_ACT_MXFP4_BLOCKED = 2 /* W4A4, sorted rows in the blocked order */
} moe_act_fmt;
typedef enum { MOE_SRC_F32 = 0, MOE_SRC_BF16 = 1 } moe_src_dtype;

/* Rows per tile of the weight-streaming (decode) GEMMs: the 32-row tiles of
 * the VibeSys post, section "Prefill, cache and speculation".  The LDS-tiled
 * (prefill) GEMMs take 64- or 128-row tiles. */
#define MOE_TILE_M 32

/* Human-readable name of a status code (static string).  Not a step of the
 * method: the pages describe no error conventions, these are the library's. */
MOE_API const char *moe_status_string(moe_status s);

/*
 * Bound-check results of a debug build of the library (compiled with
 * MOE_DEBUG; libmoe_mxfp4_debug.so).  In such a build every kernel checks the
 * indices it takes from device tables before using them; a failed check skips
 * the access and sets a bit, never traps:
 *   MOE_DEBUG_ALIGN    (1) a grouping position or a tile-table entry out of range
 *   MOE_DEBUG_TILES    (2) a GEMM tile whose rows leave [0, T*Kp)
 *   MOE_DEBUG_COMBINE  (4) a slot row at or past T*Kp read by the combine
 * Returns the OR of the bits set since the last reset (bit 31: the flags
 * could not be read) and clears them when reset != 0.  It synchronises with
 * the device (a blocking copy), so it is for tests, not for captured work.
 * Release builds compile the checks away and return 0 without touching the
 * device.  Not a step of the method.
 */
#define MOE_DEBUG_ALIGN 1u
#define MOE_DEBUG_TILES 2u
#define MOE_DEBUG_COMBINE 4u
MOE_API uint32_t moe_debug_flags(int32_t reset);

/*
 * Softmax top-K routing (InferenceX Qwen3.5 post, fused_topk bullet:
 * softmax-scored top-K selection, E = 512, K = 10; shared-expert bullet: the
 * shared expert as expert top-K+1 of one dispatch).
 *   logits        fp32 [T, E] row-major, router logits
 *   gate_logits   fp32 [T] shared-expert gate logits; required iff shared = 1
 *   topk_ids      out int32 [T, K'] (K' = K + shared)
 *   topk_weights  out fp32  [T, K']
 * Slots 0..K-1: the K experts with the largest logits, ordered by (logit
 * descending, index ascending), -0.0 equal to +0.0.  Weight of slot k:
 * exp(l_k - l_max) / sum exp(l - l_max), the sum over the K selected when
 * renormalize = 1, over all E when 0.  Slot K when shared = 1: expert E with
 * weight 1 / (1 + exp(-g_t)).  NaN or infinite logits are outside the contract.
 * Errors: INVALID_ARGUMENT (null pointers, T < 0, K < 1, K > E, flags not 0/1),
 * UNSUPPORTED (E > 1024, K' > 32).
 */
MOE_API moe_status moe_route_topk(const float *logits, const float *gate_logits, int32_t T, int32_t E,
                          int32_t K, int32_t shared, int32_t renormalize, int32_t *topk_ids,
                          float *topk_weights, void *stream);

/*
 * Router GEMM and routing in one call: the step just before the layer (the
 * router producing the gating output that the InferenceX post's fused_topk
 * consumes) joined to moe_route_topk.
 *   x             bf16 [T, H] activations (16-byte aligned)
 *   router_w      bf16 [E + shared, H] (16-byte aligned): rows [0, E) the
 *                 router; with shared = 1, row E is the shared expert's gate
 *                 vector, so its gate logit is g_t = x_t . router_w[E]
 *   logits_out    out fp32 [T, E + shared] or NULL: the logits routed on
 *   workspace     >= moe_route_gemm_workspace_size(T, H, E, shared) bytes
 * logits = x . router_w^T with fp32 accumulation of the exact bf16 products
 * (the reduction is split over H and the fp32 partial sums are added in a
 * fixed order, so equal inputs give equal logits and selections); then
 * exactly moe_route_topk on them (renormalize as there).
 * Errors: INVALID_ARGUMENT (null or misaligned pointers, T < 0, K < 1,
 * K > E, flags not 0/1), UNSUPPORTED (H not a multiple of 128, E > 1024,
 * K' > 32, T*H or (E + shared)*H bf16 bytes beyond 2^31),
 * WORKSPACE_TOO_SMALL.
 */
MOE_API size_t moe_route_gemm_workspace_size(int32_t T, int32_t H, int32_t E, int32_t shared);
MOE_API moe_status moe_route_topk_gemm(const uint16_t *x, const uint16_t *router_w, int32_t T,
                                       int32_t H, int32_t E, int32_t K, int32_t shared,
                                       int32_t renormalize, int32_t *topk_ids,
                                       float *topk_weights, float *logits_out, void *workspace,
                                       size_t workspace_bytes, void *stream);

/* Scratch bytes moe_align_sort needs for A = T * Kp assignments over Ep experts. */
MOE_API size_t moe_align_workspace_size(int32_t T, int32_t Kp, int32_t Ep);

/*
 * Group the flat assignments a = t*Kp + k by expert id (the "one MoE
 * dispatch" of the InferenceX post's shared-expert bullet; 32-row tiles of
 * the VibeSys post).  A histogram / prefix-scan permute; the result is
 * unique: stable, ascending a inside each expert's group.
 *   topk_ids       int32 [T, Kp], every id in [0, Ep) (other ids are skipped)
 *   expert_counts  out int32 [Ep]      rows per expert
 *   expert_offsets out int32 [Ep + 1]  exclusive scan of counts, last = T*Kp
 *   sorted_assign  out int32 [T*Kp]    flat ids grouped by expert
 *   inv_assign     out int32 [T*Kp] or NULL: position of flat id a in sorted_assign
 *   tile_table     out int32 [ceil(T*Kp/tile_m) + Ep][2] or NULL: (expert,
 *                  first row) of each tile_m-row tile, expert-major, rows ascending
 *   num_tiles      out int32 [1]
 *   workspace      device scratch of moe_align_workspace_size bytes
 * Errors: INVALID_ARGUMENT (null required pointer, T < 0, Kp < 1, Ep < 1,
 * tile_m < 1), UNSUPPORTED (Ep > 2048), WORKSPACE_TOO_SMALL.
 */
MOE_API moe_status moe_align_sort(const int32_t *topk_ids, int32_t T, int32_t Kp, int32_t Ep,
                          int32_t tile_m, int32_t *expert_counts, int32_t *expert_offsets,
                          int32_t *sorted_assign, int32_t *inv_assign, int32_t *tile_table,
                          int32_t *num_tiles, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * Steps 1 and 2 in one call: exactly moe_route_topk followed by
 * moe_align_sort on its ids (Kp = K + shared, Ep = E + shared), the same
 * outputs bit for bit.  A small batch (T <= 32 at E <= 256, T <= 16 at
 * E <= 512, T <= 8 at E <= 1024) runs as ONE launch, one workgroup that
 * routes the tokens and then groups their assignments, the chosen experts
 * passed on in LDS (at most 64 assignments and 16 tokens: one wave per
 * token, the first wave grouping) (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section
 * on the specific optimisations: fused_topk, and the shared expert folded
 * into the one MoE dispatch); larger batches run the two steps' kernels,
 * which route their tokens across the whole chip.  The forwards route and
 * group through the same path.
 *   logits, gate_logits, renormalize, topk_ids, topk_weights  as moe_route_topk
 *   tile_m, expert_counts ... num_tiles                       as moe_align_sort
 *   workspace  >= moe_align_workspace_size(T, K + shared, E + shared) bytes
 * Errors: those of moe_route_topk and of moe_align_sort (tile_m < 1, null
 * output pointers: INVALID_ARGUMENT; WORKSPACE_TOO_SMALL).
 */
MOE_API moe_status moe_route_align(const float *logits, const float *gate_logits, int32_t T,
                                   int32_t E, int32_t K, int32_t shared, int32_t renormalize,
                                   int32_t tile_m, int32_t *topk_ids, float *topk_weights,
                                   int32_t *expert_counts, int32_t *expert_offsets,
                                   int32_t *sorted_assign, int32_t *inv_assign,
                                   int32_t *tile_table, int32_t *num_tiles, void *workspace,
                                   size_t workspace_bytes, void *stream);

/*
 * MXFP4-quantise rows x cols values (OpenRelay "Gemma 4 31B on MI355X" post,
 * sections "Optimisation 3" and "Optimisation 4": activation quantisation to
 * MXFP4 in its own fused kernel).  Per 32-block: X = floor(log2 amax) - 2,
 * clamped to [-127, 127] (-127 for an all-zero block); scale byte X + 127;
 * each v / 2^X rounded to the nearest E2M1 value, ties to the even code,
 * saturating at 6, sign kept.  Used for W4A4 activations and to pack
 * float weights.
 *   src        fp32 or bf16 [rows, cols] (src_dtype), 16-byte aligned
 *   packed     out uint8 [rows, cols/2], 16-byte aligned
 *   scales     out uint8 [rows, cols/32]
 * Errors: INVALID_ARGUMENT (null pointers, rows < 0, cols < 0, bad dtype,
 * misaligned), UNSUPPORTED (cols not a multiple of 32).
 */
MOE_API moe_status moe_mxfp4_quantize(const void *src, int32_t src_dtype, int64_t rows, int64_t cols,
                              uint8_t *packed, uint8_t *scales, void *stream);

/*
 * The same MXFP4 quantisation, written in the blocked row order that the
 * LDS-tiled GEMMs read MXFP4 activations in (a layout for the memory system,
 * not a step of the method: each row gets the codes and scales
 * moe_mxfp4_quantize gives it).  With C = cols/128 chunks per row, output
 * row p's chunk c (elements [128c, 128c + 128)) has its 64 code bytes (the
 * row-major bytes [64c, 64c + 64)) at
 *   packed + ((p/16)*C + c)*1024 + (p%16)*64
 * and its 4 scale bytes (row-major [4c, 4c + 4)) at
 *   scales + ((p/16)*C + c)*64 + (p%16)*4,
 * so 16 consecutive rows' chunk is one contiguous KiB of codes and 64 bytes
 * of scales.
 *   src        fp32 or bf16 [rows, cols] (src_dtype), 16-byte aligned
 *   row_map    NULL: source row t -> output row t (out_rows >= rows);
 *              else int32 [rows, Kp]: source row t -> output rows
 *              row_map[t*Kp + k], k < Kp (e.g. inv_assign: each token into
 *              its sorted slots); values outside [0, out_rows) write nothing
 *   packed     out uint8 [ceil(out_rows/16)*16, cols/2], 16-byte aligned
 *   scales     out uint8 [ceil(out_rows/16)*16, cols/32], 16-byte aligned
 * Output rows no source row goes to are left as they were.
 * Errors: INVALID_ARGUMENT (null or misaligned pointers, negative sizes, bad
 * dtype, Kp < 1 with a map, out_rows < rows without one), UNSUPPORTED (cols
 * not a multiple of 128 or above 2^30, packed at or above 2^31 bytes, a
 * grid above 2^32 - 1 workgroups).
 */
MOE_API moe_status moe_mxfp4_quantize_blocked(const void *src, int32_t src_dtype, int64_t rows,
                                              int64_t cols, const int32_t *row_map, int32_t Kp,
                                              int64_t out_rows, uint8_t *packed, uint8_t *scales,
                                              void *stream);

/*
 * Row-major weight codes -> the native code order the GEMM kernels read
 * (defined above), for rows x cols elements of one or more experts stacked
 * by rows (e.g. all of w13 as [E' * 2I, H]): a pure permutation of 16-byte
 * pieces, done once when weights are loaded.  (A layout for the memory
 * system, not a step of the method: the MoE computes the same either way.)
 *   src        uint8 row-major codes [rows, cols/2] (wfmt 0, MXFP4) or
 *              [rows, cols] (wfmt 1, MXFP8), 16-byte aligned
 *   wfmt       0 = MXFP4, 1 = MXFP8
 *   dst        out, same size, 16-byte aligned, not overlapping src
 * Errors: INVALID_ARGUMENT (null or misaligned pointers, rows < 0, cols < 0,
 * bad wfmt, overlapping buffers), UNSUPPORTED (rows not a multiple of 32,
 * cols not a multiple of 128).
 */
MOE_API moe_status moe_weights_to_native(const uint8_t *src, int32_t wfmt, int64_t rows,
                                         int64_t cols, uint8_t *dst, void *stream);

/*
 * Grouped gate/up GEMM with SwiGLU (VibeSys post, section "Baseline": the
 * fused HIP MoE kernel dequantises MXFP4 weights in registers).
 * For every sorted row r of expert e (token t = sorted_assign[r] / Kp):
 *   acc[n] = sum_h a[t, h] * W13[e, n, h]   (fp32 accumulation), n < 2I
 *   h[r, i] = bf16( silu(acc[i]) * acc[I + i] )
 *   act_fmt = MOE_ACT_BF16:  act = x bf16 [T, H], act_scale = NULL
 *   act_fmt = MOE_ACT_MXFP4: act = packed uint8 [T, H/2], act_scale uint8 [T, H/32]
 *   act_fmt = MOE_ACT_MXFP4_BLOCKED (tile_m 64, 128, 256): act, act_scale =
 *              the activations of the SORTED rows r < T*Kp (token
 *              sorted_assign[r] / Kp) in the blocked order, ceil(T*Kp/16)*16
 *              rows (moe_mxfp4_quantize_blocked with row_map = inv_assign);
 *              act_scale 16-byte aligned
 *   sorted_assign, expert_offsets, tile_table, num_tiles: moe_align_sort's
 *     outputs built with the same tile_m
 *   tile_m     rows per tile: 32 selects the weight-streaming kernel (small
 *              groups, decode); 64 or 128 the LDS-tiled kernel (large
 *              groups, prefill; needs H a multiple of 256 and H, I at most
 *              4096 for bf16 activations, 6144 (64-row) or 8192 (128-row)
 *              for MXFP4 ones: the weight scales of a workgroup's rows sit
 *              in LDS for the whole reduction); 256 the LDS-tiled kernel
 *              for MXFP4 activations only (H, I at most 6144)
 *   w13        codes [E', 2I, H/2] in the native order; w13_scale [E', 2I, H/32]
 *   h          out bf16 [T*Kp, I], sorted row order
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (H or I not a multiple of 128, or a
 * tile_m / shape the kernels do not cover; with tile_m 32, H above 13,568 for
 * bf16 activations: the kernel's LDS would exceed 160 KiB).
 */
MOE_API moe_status moe_expert_gate_up(const void *act, const uint8_t *act_scale, int32_t act_fmt,
                              const int32_t *sorted_assign, const int32_t *expert_offsets,
                              const int32_t *tile_table, const int32_t *num_tiles, int32_t tile_m,
                              const uint8_t *w13, const uint8_t *w13_scale, int32_t T, int32_t H,
                              int32_t I, int32_t Ep, int32_t Kp, uint16_t *h, void *stream);

/*
 * The W4A4 gate/up GEMM with the MXFP4 quantisation of h in its epilogue
 * (OpenRelay "Gemma 4 31B on MI355X" post, section "Optimisation 4": one
 * kernel for the activation, the up projection and the MXFP4 quantisation).
 * Computes moe_expert_gate_up's h and writes, instead of the bf16 h, what
 * moe_mxfp4_quantize_blocked (row_map NULL) writes from it: the same bits,
 * without h's round trip through HBM.  moe_mxfp4_forward takes this path
 * whenever it runs W4A4 on the tiled kernels.
 *   act_fmt    MOE_ACT_MXFP4 (per-token rows) or MOE_ACT_MXFP4_BLOCKED
 *   act ... w13_scale, T ... Kp   as moe_expert_gate_up with that act_fmt
 *              (tile_m 64, 128 or 256)
 *   h_packed   out uint8, the blocked order, ceil(T*Kp/16)*16 rows of I/2
 *              bytes (rows from T*Kp on are not written), 16-byte aligned
 *   h_scale    out uint8, the blocked order, same rows of I/32 bytes,
 *              16-byte aligned
 * Errors: as moe_expert_gate_up; INVALID_ARGUMENT also for another act_fmt
 * or a null or misaligned h_packed / h_scale; UNSUPPORTED for tile_m 32.
 */
MOE_API moe_status moe_expert_gate_up_quant(const void *act, const uint8_t *act_scale,
                                    int32_t act_fmt, const int32_t *sorted_assign, const int32_t *expert_offsets,
                                    const int32_t *tile_table, const int32_t *num_tiles,
                                    int32_t tile_m, const uint8_t *w13, const uint8_t *w13_scale,
                                    int32_t T, int32_t H, int32_t I, int32_t Ep, int32_t Kp,
                                    uint8_t *h_packed, uint8_t *h_scale, void *stream);

/*
 * Grouped down GEMM: y[r, j] = sum_i h[r, i] * W2[e, j, i], fp32 accumulation,
 * staged for moe_combine (VibeSys "Qwen3.5-397B on 4x MI300A" post, section
 * "Baseline": the down projection of the fused MoE kernel).
 * Staged y format: fp16 [A, H] holding y / 2^e, then uint8 [A, H/32] holding
 * e + 127, one e per row and 32-column group, chosen so that the group's
 * largest magnitude lands in [2^14, 2^15): every element keeps 11
 * significant bits (a bf16 y, 8 bits, measured up to 3 output ulps of error
 * where a token's slots cancel) in MOE_STAGED_Y_BYTES(A, H) bytes, half of
 * fp32's.
 *   act_fmt = MOE_ACT_BF16:  h bf16 [A, I], h_scale = NULL
 *   act_fmt = MOE_ACT_MXFP4: h packed uint8 [A, I/2], h_scale uint8 [A, I/32]
 *   act_fmt = MOE_ACT_MXFP4_BLOCKED (tile_m 64, 128, 256): h, h_scale in the
 *              blocked order, ceil(A/16)*16 rows; h_scale 16-byte aligned
 *   tile_m     as for moe_expert_gate_up
 *   w2         codes [E', H, I/2] in the native order; w2_scale [E', H, I/32]
 *   y          out staged y of MOE_STAGED_Y_BYTES(A, H) bytes, rows in
 *              sorted order (A = T*Kp), 16-byte aligned
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (H or I not a multiple of 128, or a
 * tile_m / shape the kernels do not cover; with tile_m 32, I above 13,568 for
 * bf16 activations: the kernel's LDS would exceed 160 KiB).
 */
#define MOE_STAGED_Y_BYTES(A, H) ((size_t)(A) * (size_t)(H) * 2 + (size_t)(A) * ((size_t)(H) / 32))
MOE_API moe_status moe_expert_down(const void *h, const uint8_t *h_scale, int32_t act_fmt,
                           const int32_t *expert_offsets, const int32_t *tile_table,
                           const int32_t *num_tiles, int32_t tile_m, const uint8_t *w2,
                           const uint8_t *w2_scale, int32_t T, int32_t H, int32_t I, int32_t Ep,
                           int32_t Kp, void *y, void *stream);

/*
 * Weighted combine back into token order (the shared expert is slot K, so
 * no separate dense MLP is added: MiniMax M3 post, section "Shared expert
 * fusion"):  out[t, j] = bf16( sum_{k < Kp} w[t, k] * y[inv[t*Kp + k], j] ),
 * slots summed in order in fp32 (y decoded from its staged fp16 format), one
 * rounding to bf16.
 *   y staged y of T*Kp rows (moe_expert_down; 16-byte aligned);
 *   topk_weights fp32 [T, Kp]; inv_assign int32 [T*Kp]; out bf16 [T, H]
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (H not a multiple of 128).
 */
MOE_API moe_status moe_combine(const void *y, const float *topk_weights, const int32_t *inv_assign,
                       int32_t T, int32_t H, int32_t Kp, uint16_t *out, void *stream);

/*
 * The step after the layer in a tensor-parallel decode, on one GPU's rows:
 * the G ranks' partial outputs summed, the residual stream added, then
 * RMSNorm.  The pages replace the per-layer all-reduce with a one-shot one
 * fused with the residual add and RMSNorm (VibeSys "Qwen3.5-397B on 4x
 * MI300A" post, section "Communication and concurrency"): each GPU reads
 * every rank's partial output and normalises the rows itself.  This call is
 * that epilogue over G buffers this GPU can address (on one GPU, the outputs
 * of G shard layers; the library makes no inter-GPU mapping).  RMSNorm in
 * its textbook form (the pages do not define it):
 *   h[t, j] = bf16( residual[t, j] + sum_{g < G} partials[g][t, j] ),
 *             summed in fp32 in that order;
 *   out[t, j] = bf16( h[t, j] / sqrt(mean_j h[t, j]^2 + eps) * gamma[j] ),
 *             the mean of squares in fp32 over h's bf16 values.
 *   partials      HOST array of G (1..MOE_NORM_MAX_RANKS) device pointers,
 *                 each bf16 [T, H], 16-byte aligned
 *   residual      bf16 [T, H] or NULL (zeros)
 *   gamma         bf16 [H]
 *   eps           >= 0, finite
 *   residual_out  out bf16 [T, H] = h, or NULL; may be `residual` itself
 *   out           out bf16 [T, H]; may be partials[0] itself
 * Buffers 16-byte aligned; H a multiple of 8, at most 16384.  T = 0 returns
 * MOE_OK without reading any data pointer (the host array must still hold G).
 * The kernel's fp32 arithmetic follows the definition while |h| <= 2^56 and
 * mean_j h^2 + eps stays a normal fp32 number (eps > 0 keeps zero rows finite).
 * Errors: INVALID_ARGUMENT (null or misaligned pointer, G outside
 * 1..MOE_NORM_MAX_RANKS, negative T, bad eps), UNSUPPORTED (H).
 */
#define MOE_NORM_MAX_RANKS 8
MOE_API moe_status moe_residual_rmsnorm(const uint16_t *const *partials, int32_t G,
                                        const uint16_t *residual, const uint16_t *gamma,
                                        float eps, int32_t T, int32_t H, uint16_t *residual_out,
                                        uint16_t *out, void *stream);

/*
 * MXFP8-quantise rows x cols values (packing float expert weights).  Per
 * 32-block: X = floor(log2 amax) - 8, clamped to [-127, 127] (-127 for an
 * all-zero block); scale byte X + 127; each v / 2^X rounded to the nearest
 * E4M3 value, ties to the even code, saturating at 448, sign kept.
 *   src        fp32 or bf16 [rows, cols] (src_dtype), 16-byte aligned
 *   codes      out uint8 [rows, cols], 16-byte aligned
 *   scales     out uint8 [rows, cols/32]
 * Errors: as moe_mxfp4_quantize.
 */
MOE_API moe_status moe_mxfp8_quantize(const void *src, int32_t src_dtype, int64_t rows, int64_t cols,
                              uint8_t *codes, uint8_t *scales, void *stream);

/*
 * Grouped gate/up GEMM + SwiGLU over MXFP8 weights, bf16 activations
 * (W8A16): as moe_expert_gate_up with act_fmt = MOE_ACT_BF16, the weights
 * dequantised to bf16 in registers by the scaled FP8 converter.  tile_m 32
 * (weight-streaming kernel) or 64 / 128 (LDS-tiled kernel; H a multiple of
 * 256, H and I at most 4096); the tile table from moe_align_sort with the
 * same tile_m.
 *   x          bf16 [T, H];  w13 uint8 [E', 2I, H] (native code order),
 *              w13_scale uint8 [E', 2I, H/32]
 *   h          out bf16 [T*Kp, I] in sorted row order
 * Errors: INVALID_ARGUMENT, UNSUPPORTED (H or I not a multiple of 128, a
 * tile_m / shape the kernels do not cover, an expert's 2I x H code bytes
 * at or above 2^31).
 */
MOE_API moe_status moe_mxfp8_expert_gate_up(const uint16_t *x, const int32_t *sorted_assign,
                                    const int32_t *expert_offsets, const int32_t *tile_table,
                                    const int32_t *num_tiles, int32_t tile_m, const uint8_t *w13,
                                    const uint8_t *w13_scale, int32_t T, int32_t H, int32_t I,
                                    int32_t Ep, int32_t Kp, uint16_t *h, void *stream);

/*
 * Grouped down GEMM over MXFP8 weights (W8A16): as moe_expert_down with
 * act_fmt = MOE_ACT_BF16; tile_m as for moe_mxfp8_expert_gate_up.
 *   h          bf16 [T*Kp, I];  w2 uint8 [E', H, I] (native code order),
 *              w2_scale uint8 [E', H, I/32]
 *   y          out staged y (as moe_expert_down), sorted row order
 * Errors: as moe_mxfp8_expert_gate_up.
 */
MOE_API moe_status moe_mxfp8_expert_down(const uint16_t *h, const int32_t *expert_offsets,
                                 const int32_t *tile_table, const int32_t *num_tiles,
                                 int32_t tile_m, const uint8_t *w2, const uint8_t *w2_scale,
                                 int32_t T, int32_t H, int32_t I, int32_t Ep, int32_t Kp,
                                 void *y, void *stream);

/* The tile_m moe_mxfp4_forward uses for these shapes and activation format
 * (A = T*Kp assignments over Ep experts): 32 up to an average of 3 rows per
 * expert (W4A16; 8 for W4A4), else 64 or 128 (see moe_expert_gate_up;
 * 256-row tiles are used only when a caller of the per-step entry points
 * asks for them).  The pages keep separate small-M
 * (decode) and large-M (prefill) GEMM launchers chosen by the local shape
 * (MiniMax M3 on MI355X post, section "Local shape and tiling") and use
 * 32-row tiles for the MoE kernel (VibeSys post, section "Prefill, cache and
 * speculation"). */
MOE_API int32_t moe_gemm_tile_m(int32_t T, int32_t Kp, int32_t Ep, int32_t H, int32_t I,
                                int32_t act_fmt);

/* Workspace bytes moe_mxfp4_forward needs (0 for T = 0): the routing
 * tables, the grouping, the quantised activations, h and the staged y.  The
 * pages say nothing of memory management; a caller-owned workspace keeps
 * every call free of allocation and so capturable in a HIP graph, which the
 * pages' graph-captured decode steps need (VibeSys post, section "Kernels
 * and graph capture"). */
MOE_API size_t moe_mxfp4_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                int32_t shared, int32_t act_fmt);

/*
 * The whole layer in one call: the MoE layer of 512 routed experts with
 * MXFP4 weights (VibeSys "Qwen3.5-397B on 4x MI300A" post, section "Goal")
 * run as one MoE dispatch over the top-K routed experts plus the shared
 * expert as slot K (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section
 * on the specific optimisations, shared-expert fusion bullet; MiniMax M3 on
 * MI355X post, section "Shared expert fusion"): route, align, [quantise x],
 * gate/up + SwiGLU [+ the quantisation of h, in the tiled W4A4 GEMM's
 * epilogue], down, combine, all enqueued on `stream`.  The GEMM kernels
 * are chosen on the host from the shapes alone (no device read): average
 * rows per expert T*K'/E' <= 8 -> 32-row weight-streaming tiles, else
 * 64-row LDS-tiled tiles (bf16 activations; MXFP4 activations: 64 up to 48
 * rows, 128 above) when the shapes fit the tiled kernels (see
 * moe_expert_gate_up; otherwise 32).
 *   x              bf16 [T, H]
 *   router_logits  fp32 [T, E];  shared_gate_logits fp32 [T] (shared = 1) or NULL
 *   w13, w13_scale, w2, w2_scale: the MXFP4 weights of E + shared experts
 *                  (codes in the native order, scales row-major)
 *   act_fmt        MOE_ACT_BF16 (W4A16) or MOE_ACT_MXFP4 (W4A4: x and h are
 *                  MXFP4-quantised before their GEMM; with tiled GEMMs into
 *                  the blocked sorted-row order, x into each of its token's
 *                  slots and h by the gate/up GEMM itself, as
 *                  moe_expert_gate_up_quant)
 *   out            out bf16 [T, H]
 *   topk_ids_out, topk_weights_out: optional copies of the routing [T, K']
 *   workspace      caller-owned device scratch of moe_mxfp4_workspace_size bytes
 * Errors: any of the stage errors, WORKSPACE_TOO_SMALL.
 */
MOE_API moe_status moe_mxfp4_forward(const uint16_t *x, const float *router_logits,
                             const float *shared_gate_logits, const uint8_t *w13,
                             const uint8_t *w13_scale, const uint8_t *w2, const uint8_t *w2_scale,
                             int32_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared,
                             int32_t act_fmt, uint16_t *out, int32_t *topk_ids_out,
                             float *topk_weights_out, void *workspace, size_t workspace_bytes,
                             void *stream);

/*
 * moe_mxfp4_forward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same layer, arguments and results, with no workspace
 * argument.  The workspace is a library-owned device array of
 * MOE_NOALLOC_SCRATCH_BYTES per GPU, held until the process ends; its
 * address on the current device is looked up on the first call on that
 * device (make that first call outside graph capture).  Nothing is
 * allocated or freed by any call.
 *   Limit: the call's workspace (moe_mxfp4_workspace_size) must fit the
 *   scratch, else WORKSPACE_TOO_SMALL: e.g. T up to 587 at H = 4096,
 *   I = 1024, E = 512, K' = 11 (about 114 KB of workspace per token there:
 *   each assignment's bf16 h and staged y), enough for decode batches.
 *   Every call on one GPU uses that GPU's one scratch: calls that overlap
 *   on one GPU (different streams, or host threads) race; serialise them.
 *   No part of the scratch needs to start at zero.
 * Errors: as moe_mxfp4_forward; WORKSPACE_TOO_SMALL beyond the limit;
 * DEVICE if the scratch's address cannot be looked up.
 */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
MOE_API moe_status moe_mxfp4_forward_noalloc(const uint16_t *x, const float *router_logits,
                                     const float *shared_gate_logits, const uint8_t *w13,
                                     const uint8_t *w13_scale, const uint8_t *w2,
                                     const uint8_t *w2_scale, int32_t T, int32_t H, int32_t I,
                                     int32_t E, int32_t K, int32_t shared, int32_t act_fmt,
                                     uint16_t *out, int32_t *topk_ids_out,
                                     float *topk_weights_out, void *stream);

/*
 * The whole layer routed from x: moe_route_topk_gemm's router GEMM and
 * routing, then everything moe_mxfp4_forward does after its routing.
 *   router_w     bf16 [E + shared, H] (16-byte aligned); row E = the shared
 *                expert's gate vector (see moe_route_topk_gemm)
 *   logits_out   out fp32 [T, E + shared] or NULL
 *   workspace    >= moe_mxfp4_workspace_size(...) bytes (the same size as
 *                for moe_mxfp4_forward)
 * Other arguments, outputs and errors as moe_mxfp4_forward (router_w
 * replaces router_logits and shared_gate_logits).
 */
MOE_API moe_status moe_mxfp4_forward_router(const uint16_t *x, const uint16_t *router_w,
                                            const uint8_t *w13, const uint8_t *w13_scale,
                                            const uint8_t *w2, const uint8_t *w2_scale, int32_t T,
                                            int32_t H, int32_t I, int32_t E, int32_t K,
                                            int32_t shared, int32_t act_fmt, uint16_t *out,
                                            int32_t *topk_ids_out, float *topk_weights_out,
                                            float *logits_out, void *workspace,
                                            size_t workspace_bytes, void *stream);

/* One layer of a multi-layer pass: its router rows and MXFP4 expert weights
 * (device pointers, layouts as for moe_mxfp4_forward_router). */
typedef struct {
  const uint16_t *router_w;      /* bf16 [E + shared, H], 16-byte aligned */
  const uint8_t *w13;            /* [E', 2I, H/2], native code order */
  const uint8_t *w13_scale;      /* [E', 2I, H/32] */
  const uint8_t *w2;             /* [E', H, I/2], native code order */
  const uint8_t *w2_scale;       /* [E', H, I/32] */
} moe_mxfp4_layer;

/*
 * L MoE layers back to back, as the MoE part of a decode step (the pages
 * capture whole decode steps in HIP graphs, one launch per step: VibeSys
 * post, section "Kernels and graph capture"; OpenRelay "Gemma 4 31B on
 * MI355X" post, "Optimisation 2", the GPU waiting on the CPU): layer l computes
 * moe_mxfp4_forward_router on its input with layers[l]'s weights; layer 0
 * reads x, layer l > 0 reads layer l-1's output.  All layers write `out` in
 * place (a layer's combine, its only write, runs after all its reads), so
 * out holds the last layer's output.  With prefetch = 1 the combine of
 * layer l also reads layer l+1's router rows and shared expert's weights
 * (the only weights of the next layer known before its routing) into the
 * caches while it runs; results are identical either way.  The call only
 * enqueues work, so the whole pass can be captured in one HIP graph.
 *   layers     host array of L layer descriptors (read during the call only)
 *   workspace  >= moe_mxfp4_workspace_size(T, H, I, E, K, shared, act_fmt)
 * Errors: INVALID_ARGUMENT (L < 1, null or misaligned layer pointers, bad
 * prefetch flag), and those of moe_mxfp4_forward_router; every check runs
 * before the first enqueue.
 */
MOE_API moe_status moe_mxfp4_forward_layers(const uint16_t *x, int32_t L,
                                            const moe_mxfp4_layer *layers, int32_t T, int32_t H,
                                            int32_t I, int32_t E, int32_t K, int32_t shared,
                                            int32_t act_fmt, int32_t prefetch, uint16_t *out,
                                            void *workspace, size_t workspace_bytes, void *stream);

/*
 * The same L layers as the MoE sub-layers of a pre-norm decode step: after
 * each layer the residual stream is updated and normalised in one pass (the
 * pages fuse the residual add and RMSNorm into the step after the layer:
 * VibeSys post, section "Communication and concurrency"; see
 * moe_residual_rmsnorm, here with the layer's output as the one partial):
 *   y_l = layer l on x_l (x_0 = x);  residual += y_l (bf16);
 *   x_{l+1} = RMSNorm(residual) * gammas[l]  (written to out)
 * so out holds the last layer's normalised output and residual the stream
 * after all L layers.  Layer l > 0 reads out; every step writes in place.
 *   gammas     host array of L device pointers, bf16 [H] each, 16-byte aligned
 *   eps        >= 0, finite
 *   residual   in/out bf16 [T, H], 16-byte aligned, not overlapping out
 * Other arguments as moe_mxfp4_forward_layers.  Errors: those of
 * moe_mxfp4_forward_layers and moe_residual_rmsnorm, all checked before the
 * first enqueue.
 */
MOE_API moe_status moe_mxfp4_forward_layers_norm(const uint16_t *x, int32_t L,
                                                 const moe_mxfp4_layer *layers,
                                                 const uint16_t *const *gammas, float eps,
                                                 uint16_t *residual, int32_t T, int32_t H,
                                                 int32_t I, int32_t E, int32_t K, int32_t shared,
                                                 int32_t act_fmt, int32_t prefetch, uint16_t *out,
                                                 void *workspace, size_t workspace_bytes,
                                                 void *stream);

/* The tile_m moe_mxfp8_forward uses for these shapes: 32 up to an average
 * of 4 rows per expert, else 64 (128-row tiles only when a caller of the
 * per-step entry points asks for them). */
MOE_API int32_t moe_mxfp8_gemm_tile_m(int32_t T, int32_t Kp, int32_t Ep, int32_t H, int32_t I);

/* Workspace bytes moe_mxfp8_forward needs (0 for T = 0). */
MOE_API size_t moe_mxfp8_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                int32_t shared);

/*
 * The whole layer over MXFP8 expert weights with bf16 activations (W8A16):
 * route, align (moe_mxfp8_gemm_tile_m), gate/up + SwiGLU, down, combine, enqueued on
 * `stream`.  Arguments, outputs and errors as moe_mxfp4_forward with
 * act_fmt = MOE_ACT_BF16, except the weights (MXFP8 layout above) and the
 * workspace (moe_mxfp8_workspace_size bytes); UNSUPPORTED also when an
 * expert's 2I x H code bytes reach 2^31.
 */
MOE_API moe_status moe_mxfp8_forward(const uint16_t *x, const float *router_logits,
                             const float *shared_gate_logits, const uint8_t *w13,
                             const uint8_t *w13_scale, const uint8_t *w2, const uint8_t *w2_scale,
                             int32_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared,
                             uint16_t *out, int32_t *topk_ids_out, float *topk_weights_out,
                             void *workspace, size_t workspace_bytes, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MXFP4_H */
