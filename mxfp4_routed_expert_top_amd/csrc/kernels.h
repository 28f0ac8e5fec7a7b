// Host-side launchers of the HIP kernels (internal to the library).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

hipError_t launch_route_topk(const float* logits, const float* gate, int T, int E, int K,
                             int shared, int renormalize, int32_t* ids, float* weights,
                             hipStream_t stream);
// The same on logits of row stride ld, the gate logit of token t at
// gate[t * gate_stride].
hipError_t launch_route_topk_rows(const float* logits, int ld, const float* gate,
                                  int gate_stride, int T, int E, int K, int shared,
                                  int renormalize, int32_t* ids, float* weights,
                                  hipStream_t stream);

// Adds the router GEMM's S partial sums into logits [T, E + shared] (in
// split order), then routes on them (the gate logit is column E).
int route_max_splits();
hipError_t launch_route_topk_split(const float* partial, int S, int T, int E, int K, int shared,
                                   int renormalize, int32_t* ids, float* weights, float* logits,
                                   hipStream_t stream);

// Adds the router GEMM's S partial sums into logits [T, Ep] (nothing for S = 1).
hipError_t launch_sum_splits(const float* partial, int S, int T, int Ep, float* logits,
                             hipStream_t stream);

int router_splits(int T, int H, int Ep);
size_t router_workspace_bytes(int T, int H, int Ep);   // partial sums + summed logits
// S = router_splits(...) > 1: partial sums into partial [S, T, Ep] (added by
// launch_route_topk_split); S = 1: the logits straight into logits [T, Ep].
hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w, int T, int H, int Ep,
                              float* partial, float* logits, hipStream_t stream);

// Routing then grouping (route_align.hip): the results of
// launch_route_topk_rows followed by launch_align_sort (scratch of
// align_scratch_bytes), in one launch when route_align_fits (a small batch).
bool route_align_fits(int T, int E, int K, int shared);
hipError_t launch_route_align(const float* logits, int ld, const float* gate, int gate_stride,
                              int T, int E, int K, int shared, int renormalize, int tile_m,
                              int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                              int32_t* sorted, int32_t* inv, int32_t* tiles, int32_t* num_tiles,
                              int32_t* scratch, hipStream_t stream);

size_t align_scratch_bytes(int A, int Ep);
hipError_t launch_align_sort(const int32_t* ids, int A, int Ep, int tile_m, int32_t* counts,
                             int32_t* offsets, int32_t* sorted, int32_t* inv, int32_t* tiles,
                             int32_t* num_tiles, int32_t* scratch, hipStream_t stream);

hipError_t launch_mxfp4_quant(const void* src, int src_is_bf16, int64_t rows, int64_t cols,
                              uint8_t* packed, uint8_t* scales, hipStream_t stream);
// MXFP4 quantisation into the blocked row order of the tiled GEMMs' MXFP4
// activations (cols a multiple of 128): source row t to output rows
// map[t * Kp + k] < out_rows, k < Kp (or to row t without a map).
hipError_t launch_mxfp4_quant_blocked(const void* src, int src_is_bf16, int64_t rows, int64_t cols,
                                      const int32_t* map, int Kp, int64_t out_rows,
                                      uint8_t* packed, uint8_t* scales, hipStream_t stream);
hipError_t launch_mxfp8_quant(const void* src, int src_is_bf16, int64_t rows, int64_t cols,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream);
// row-major weight codes -> native code order (nq = 1 MXFP4, 2 MXFP8)
hipError_t launch_weights_native(const uint8_t* src, int nq, int64_t rows, int64_t cols,
                                 uint8_t* dst, hipStream_t stream);

int expert_gemm_tile_m();
// Dynamic LDS bytes of the 32-row kernels for a reduction of K elements
// (act_fmt 0: bf16 activations staged too); at most kMaxLdsBytes.
size_t expert_gemm_lds_bytes(int K, int act_fmt);
constexpr size_t kMaxLdsBytes = 160 * 1024;
int expert_gemm_phase(int nch);
// wfmt: 0 = MXFP4 weights, 1 = MXFP8 weights (bf16 activations only)
hipError_t launch_gate_up(int act_fmt, int wfmt, const void* act, const uint8_t* act_scale,
                          const int32_t* sorted, const int32_t* offsets, const int32_t* tiles,
                          const int32_t* num_tiles, int max_tiles, const uint8_t* w13,
                          const uint8_t* w13s, int T, int H, int I, int Kp, uint16_t* h,
                          hipStream_t stream);
// y: each sorted row's down-projection in the staged fp16 format of
// common.h: fp16 [A, H] followed by the group exponent bytes [A, H / 32]
// (staged_y_bytes(A, H) bytes in all)
inline size_t staged_y_bytes(size_t A, size_t H) { return A * H * 2 + A * (H / 32); }
hipError_t launch_down(int act_fmt, int wfmt, const void* h, const uint8_t* h_scale,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                       int max_tiles, const uint8_t* w2, const uint8_t* w2s, int A, int H, int I,
                       uint16_t* y, hipStream_t stream);
// Byte ranges the combine's extra workgroups read into the caches (the next
// layer's weights that are known before its routing); n = 0 for none.
struct Prefetch {
  static constexpr int kMax = 5;
  const void* p[kMax];
  uint32_t bytes[kMax];
  int n;
};
// y as written by launch_down / launch_down_tiled for A = T * Kp rows
hipError_t launch_combine(const uint16_t* y, const float* w, const int32_t* inv, int T, int H,
                          int Kp, uint16_t* out, hipStream_t stream, const Prefetch* pf = nullptr);

// Debug builds: each source file's bound-check flags (0 in release builds).
uint32_t debug_flags_align(bool reset);
uint32_t debug_flags_expert_gemm(bool reset);
uint32_t debug_flags_expert_gemm_tiled(bool reset);
uint32_t debug_flags_route_align(bool reset);

bool expert_gemm_tiled_supported(int tile_m, int act_fmt, int H, int I, int wfmt = 0);
hipError_t launch_gate_up_tiled(int tile_m, int act_fmt, int wfmt, const void* act,
                                const uint8_t* act_scale,
                                const int32_t* sorted, const int32_t* offsets,
                                const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                                const uint8_t* w13, const uint8_t* w13s, int T, int H, int I,
                                int Kp, uint16_t* h, hipStream_t stream, uint8_t* hq = nullptr,
                                uint8_t* hs = nullptr);
// (hq, hs given, MXFP4 activations only: h is written MXFP4-quantised
// in the blocked row order, as launch_mxfp4_quant_blocked would write it from
// the bf16 h, and h itself is not written)
// y in sorted order, as launch_down
hipError_t launch_down_tiled(int tile_m, int act_fmt, int wfmt, const void* h,
                             const uint8_t* h_scale,
                             const int32_t* offsets, const int32_t* tiles,
                             const int32_t* num_tiles, int max_tiles, const uint8_t* w2,
                             const uint8_t* w2s, int A, int H, int I, uint16_t* y,
                             hipStream_t stream);

// G partial outputs summed, the residual added, RMSNorm (residual_norm.hip):
// partials is a host array of G <= kMaxNormRanks device pointers (bf16
// [T, H] each); H a multiple of 8, at most residual_rmsnorm_max_h();
// residual and residual_out may be null.
constexpr int kMaxNormRanks = 8;
int residual_rmsnorm_max_h();
hipError_t launch_residual_rmsnorm(const uint16_t* const* partials, int G, const uint16_t* residual,
                                   const uint16_t* gamma, float eps, int T, int H,
                                   uint16_t* residual_out, uint16_t* out, hipStream_t stream);
