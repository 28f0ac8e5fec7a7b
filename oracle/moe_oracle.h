/*
 * moe_oracle.h -- CPU oracle of the MXFP4 routed-expert mixture-of-experts
 * layer: plain C++17, fp64 arithmetic, no GPU headers.
 *
 * TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
 * cpu_baseline leg may load this library (through oracle/__init__.py) or run
 * its command-line tool.  It shares no code with the HIP path: no header,
 * kernel, table or helper; the GPU library never links or loads it.
 *
 * What it computes (each function below names the passage it follows):
 *
 *   route   softmax-scored top-K over E experts, ties to the lower index;
 *           the weights renormalised over the K routed experts; the shared
 *           expert folded in as expert E in slot K with weight sigmoid(g)
 *           (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the
 *           specific optimisations: the fused_topk and shared-expert fusion
 *           bullets; MiniMax M3 on MI355X post, section "Shared expert fusion")
 *   align   a stable counting sort of the assignments t*K'+k by expert, with
 *           per-expert counts and offsets and a list of tile_m-row tiles
 *           (VibeSys "Qwen3.5-397B on 4x MI300A" post, section "Prefill,
 *           cache and speculation": 32-row tiles in the MoE kernel)
 *   expert  MLP_e(a) = dq(W2) . bf16( silu(dq(W13)_gate . a) * (dq(W13)_up . a) )
 *           over exactly decoded MXFP4 (or MXFP8) weights, fp64 dot
 *           products (VibeSys post, section "Baseline": MXFP4 weights
 *           dequantised inside the MoE kernel; the SwiGLU expert MLP)
 *   norm    the residual add and RMSNorm after the layer's partial outputs
 *           are summed (oracle_residual_rmsnorm below)
 *   forward out[t] = bf16( sum_k w[t,k] * MLP_{ids[t,k]}(x_t) ), slots summed
 *           in order (optionally each MLP output rounded to bf16 first).  For W4A4 the activations and h go through
 *           MXFP4 quantise-then-decode before their GEMM (OpenRelay "Gemma 4
 *           31B on MI355X" post, sections "Optimisation 3" and
 *           "Optimisation 4": activation + MXFP4 quantisation fused).
 *
 * Number formats (OCP Microscaling v1.0; the pages name "MXFP4" and "MXFP8"
 * weights and give no bits): 32 consecutive elements along the reduction
 * axis share one E8M0 scale byte b (2^(b-127), 255 = NaN).  MXFP4 elements
 * are E2M1 codes s|ee|m (values +-{0, .5, 1, 1.5, 2, 3, 4, 6}), two per
 * byte, element 2j in the low nibble.  MXFP8 elements are E4M3 bytes
 * s|eeee|mmm (bias 7, subnormals m/8 * 2^-6, largest 448, S.1111.111 NaN).
 * Quantisation: X = floor(log2 amax) - emax (emax 2 for E2M1, 8 for E4M3)
 * clamped to [-127, 127] (-127 for an all-zero block), each v / 2^X to the
 * nearest element value with ties to the even code, saturating, sign kept.
 *
 * Conventions: every pointer is host memory owned by the caller; arrays are
 * row-major; bf16 values travel as their uint16 bit patterns.  `threads` <= 0
 * means the number of CPUs in the process's affinity mask.  Functions return
 * 0 on success and a negative number on a bad argument (nothing written).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { ORACLE_ACT_BF16 = 0, ORACLE_ACT_MXFP4 = 1 };
enum { ORACLE_W_MXFP4 = 0, ORACLE_W_MXFP8 = 1 };

/* ---- number formats ---------------------------------------------------- */

/* Value of one E2M1 code (0..15): (-1)^s * 0.5m for e = 0, else
 * (-1)^s * (1 + 0.5m) * 2^(e-1). */
double oracle_e2m1_value(int code);
/* Value of one E4M3 code (0..255); NaN for S.1111.111. */
double oracle_e4m3_value(int code);
/* 2^(b-127) for a scale byte b; NaN for 255. */
double oracle_e8m0_value(int b);

/* Round v to the nearest bf16 value, ties to even, in one step (never
 * through float32); overflow (|result| >= 2^128) gives +-inf. */
double oracle_round_bf16(double v);
/* The same rounding, returned as the bf16 bit pattern. */
uint16_t oracle_bf16_bits(double v);
/* bf16 bit pattern -> its exact value. */
double oracle_bf16_value(uint16_t bits);

/* n values -> rounded bf16 values / bit patterns (array forms of the above). */
void oracle_round_bf16_array(const double *v, int64_t n, double *out);
void oracle_bf16_bits_array(const double *v, int64_t n, uint16_t *out);

/* MXFP4: rows x K values (K a multiple of 32) -> packed codes [rows, K/2]
 * and scales [rows, K/32].  src_f32 = 1 reads float32 input instead of
 * fp64 (every float is exactly a double, so the result is the same). */
int oracle_mxfp4_quantize(const void *v, int src_f32, int64_t rows, int64_t K, uint8_t *packed,
                          uint8_t *scales, int threads);
/* MXFP4 -> fp64 [rows, K], exact. */
int oracle_mxfp4_decode(const uint8_t *packed, const uint8_t *scales, int64_t rows, int64_t K,
                        double *out);
/* MXFP8 quantise / decode, as above with one code byte per element. */
int oracle_mxfp8_quantize(const void *v, int src_f32, int64_t rows, int64_t K, uint8_t *codes,
                          uint8_t *scales, int threads);
int oracle_mxfp8_decode(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                        double *out);

/* ---- the layer's steps ------------------------------------------------- */

/* Routing.  logits float [T, E]; gate float [T] (read when shared = 1).
 * ids int32 [T, K'], w float [T, K'] (K' = K + shared).  Slots 0..K-1 hold
 * the K experts ordered by (logit descending, index ascending), -0.0 equal
 * to +0.0; weights in fp64, rounded once to float:
 *   renormalize = 1: exp(l_k - l_max) / sum_{k' < K} exp(l_k' - l_max)
 *   renormalize = 0: exp(l_k - l_max) / sum_{all e} exp(l_e - l_max)
 * Slot K (shared = 1): id E, weight 1 / (1 + exp(-g)). */
int oracle_route(const float *logits, const float *gate, int64_t T, int32_t E, int32_t K,
                 int32_t shared, int32_t renormalize, int32_t *ids, float *w);

/* Grouping.  ids int32 [A] (A = T*K', values in [0, Ep)).  counts [Ep],
 * offsets [Ep+1] (exclusive scan, offsets[Ep] = A), sorted [A] (flat ids
 * grouped by expert, ascending inside a group), inv [A] (the position of
 * each flat id in sorted), tiles [max_tiles, 2] (expert, first row) for
 * the tile_m-row tiles of each group, expert-major; *n_tiles their number.
 * tiles may be NULL; otherwise max_tiles must be >= the number of tiles. */
int oracle_align(const int32_t *ids, int64_t A, int32_t Ep, int32_t tile_m, int32_t *counts,
                 int32_t *offsets, int32_t *sorted_ids, int32_t *inv, int32_t *tiles,
                 int64_t max_tiles, int64_t *n_tiles);

/* Router GEMM (the gating output the top-K consumes): x bf16 [T, H], router
 * rows bf16 [R, H] -> fp64 [T, R] = x . W^T, each entry a sum over h of
 * exact products, in fp64. */
int oracle_router_logits(const uint16_t *x_bits, const uint16_t *w_bits, int64_t T, int64_t R,
                         int64_t H, double *out, int threads);

/* One expert on n rows a (fp64 [n, H], values already bf16- or
 * MXFP4-exact): acc = a . dq(W13)^T; h = bf16(silu(acc_gate) * acc_up);
 * hin = h, or for act_fmt = MXFP4 h quantised to MXFP4 along I and decoded;
 * y = hin . dq(W2)^T (fp64, before any rounding).  Weights in wfmt
 * (MXFP4: w13 [2I, H/2], w2 [H, I/2]; MXFP8: w13 [2I, H], w2 [H, I]);
 * scales [2I, H/32] and [H, I/32].  y [n, H] and h [n, I] (may be NULL). */
int oracle_expert_mlp(const double *a, int64_t n, int64_t H, int64_t I, const uint8_t *w13,
                      const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s, int act_fmt,
                      int wfmt, double *y, double *h, int threads);

/* The whole layer.
 *   x_bits bf16 [T, H]; logits float [T, E]; gate float [T] or NULL
 *   w13[e], w13s[e], w2[e], w2s[e]: expert e's arrays (e < E + shared) as in
 *     oracle_expert_mlp; an expert no selected token uses may be NULL
 *   tokens: n_tokens token indices whose outputs are computed (NULL: all T;
 *     routing and grouping always cover every token)
 *   round_y: 1 rounds each slot's expert output y to bf16 before the
 *     combine (a path that stores y in bf16 between the down GEMM and the
 *     combine), 0 keeps it (a path whose combine adds the unrounded products)
 * Outputs (any may be NULL): ids int32 [T, K'], w float [T, K'];
 *   out_bits bf16 [n, H] and out_f64 [n, H] (the fp64 sum before its
 *   rounding), n = n_tokens or T; h_bits bf16 [T*K', I]: each assignment's
 *   h, rows in the grouping's sorted order (only with tokens = NULL).
 * seconds (may be NULL) receives the wall time of the call. */
int oracle_forward(const uint16_t *x_bits, const float *logits, const float *gate,
                   const uint8_t *const *w13, const uint8_t *const *w13s,
                   const uint8_t *const *w2, const uint8_t *const *w2s, int64_t T, int64_t H,
                   int64_t I, int32_t E, int32_t K, int32_t shared, int act_fmt, int wfmt,
                   int32_t renormalize, int32_t round_y, const int64_t *tokens, int64_t n_tokens,
                   int threads, int32_t *ids, float *w, uint16_t *out_bits, double *out_f64,
                   uint16_t *h_bits, double *seconds);

/* The layer from a given h onward: routing and grouping as oracle_forward,
 * then each assignment's down projection of h_bits [T*K', I] (bf16, rows in
 * the grouping's sorted order; for W4A4 quantised to MXFP4 and decoded
 * first) and the combine.  Only the W2 arrays are read.  Tests use it to
 * take the h-dependent steps on the h a GPU produced, so that a rounding
 * decision taken differently on the two sides upstream does not propagate.
 * out_bits / out_f64 [T, H] as in oracle_forward (either may be NULL). */
int oracle_forward_from_h(const uint16_t *h_bits, const float *logits, const float *gate,
                          const uint8_t *const *w2, const uint8_t *const *w2s, int64_t T,
                          int64_t H, int64_t I, int32_t E, int32_t K, int32_t shared, int act_fmt,
                          int wfmt, int32_t renormalize, int32_t round_y, int threads,
                          uint16_t *out_bits, double *out_f64);

/* The step after the layer in a tensor-parallel decode: the G ranks' partial
 * outputs summed (the all-reduce), the residual stream added, then RMSNorm;
 * the pages replace the all-reduce with a one-shot one fused with the
 * residual add and RMSNorm (VibeSys post, section "Communication and
 * concurrency").  RMSNorm is not defined on the pages; the textbook form:
 *   h[t, j] = bf16( residual[t, j] + sum_g partial[g][t, j] )   (new residual)
 *   y[t, j] = bf16( h[t, j] / sqrt(mean_j h[t, j]^2 + eps) * gamma[j] )
 * with the sum and the norm in fp64 on h's bf16 values.  partials: G arrays
 * of T x H bf16 bits one after another ([G][T][H]); residual [T, H] and
 * gamma [H] bf16 bits (residual may be NULL: zeros); G >= 1.  rstd_out [T]
 * (may be NULL) receives 1 / sqrt(mean_j h^2 + eps). */
int oracle_residual_rmsnorm(const uint16_t *partials, int32_t G, const uint16_t *residual,
                            const uint16_t *gamma, double eps, int64_t T, int64_t H,
                            uint16_t *h_out, uint16_t *y_out, double *rstd_out);

/* The thread count `threads` <= 0 resolves to. */
int oracle_default_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ORACLE_H */
