// C ABI of the MXFP4 routed-expert MoE layer: argument checks, workspace
// carving and the launch sequence.  Every check runs before the first
// enqueue; nothing here allocates, synchronises or reads device memory.
#include "../../include/moe_mxfp4.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxKp = 32;
constexpr size_t kAlign = 256;

inline size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The GEMM kernels address each expert's weight codes, the activation rows
// and h with 32-bit buffer offsets in which bit 31 marks a row that is not
// there (the load returns zeros): every such buffer stays below 2 GiB.
constexpr int64_t kMaxBufferBytes = (int64_t)1 << 31;
inline hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }
inline moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

inline int64_t max_tiles_for(int64_t A, int64_t Ep, int64_t tile_m = MOE_TILE_M) {
  return (A + tile_m - 1) / tile_m + Ep;
}

// Rows per GEMM tile for a call, from the shapes alone: small groups stream
// weights through 32-row tiles; larger groups use the LDS-tiled kernels.
// bf16 activations (MXFP4 or MXFP8 weights) take 64-row tiles at any group
// size: two workgroups fit a CU (two waves per SIMD), which beats the
// weight reuse of 128-row tiles even on the skewed T = 8192 batch (~176
// rows per expert: step 2.92 -> 2.53 ms).  MXFP4 activations keep 128-row
// tiles above 48 rows (64-row tiles are 5% slower on the W4A4 batch).
// The 32-row weight-streaming kernels up to an average group of `small`
// rows (whole passes at E = 512, H = 4096, I = 1024 cross over at ~3.4 rows
// for W4A16: 64-row tiles 5% faster at 4.1 rows and 10% at 5.5; at ~5 rows
// with MXFP8 weights; at ~9.6 rows for W4A4, 6% faster at 11.8), the tiled
// kernels above.
int choose_tile_m(int64_t A, int64_t Ep, int H, int I, int act_fmt, int wfmt = 0) {
  const int64_t avg = A / Ep;
  const int64_t small = act_fmt != MOE_ACT_BF16 ? 8 : wfmt == 1 ? 4 : 3;
  if (avg <= small) return MOE_TILE_M;
  // (256-row tiles, MXFP4 activations only, are taken on request: on the
  // W4A4 batch, ~143 rows per expert, 128-row tiles are faster even though
  // they stream most experts' weights twice, the second time mostly from L2.
  // bf16 activations keep 64-row tiles at two workgroups per CU even for
  // large groups: the 8-wave 128-row kernel, which fetches each weight slice
  // once for 128 rows, runs the skewed 8,192-token batch's gate/up 1.48 ms
  // and down 1.00 ms against 1.36 and 0.85.)
  // (MXFP4 activations: 64- and 128-row tiles equal at ~28 rows per expert
  // on the W4A4 shapes, 128 faster by 1.6% at 38 rows, 3% at 49, 16% at 84)
  const int tm = (act_fmt == MOE_ACT_BF16 || avg <= 32) ? 64 : 128;
  return expert_gemm_tiled_supported(tm, act_fmt, H, I, wfmt) ? tm : MOE_TILE_M;
}

bool tile_m_ok(int32_t tile_m, int32_t act_fmt, int32_t H, int32_t I, int wfmt = 0) {
  return tile_m == MOE_TILE_M || expert_gemm_tiled_supported(tile_m, act_fmt, H, I, wfmt);
}

moe_status check_shape_HI(int32_t H, int32_t I) {
  if (H <= 0 || I <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128 || I % 128) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

// Forward workspace layout, in this order, each piece 256-byte aligned.
struct FwdLayout {
  size_t ids, w, counts, offsets, sorted, inv, tiles, ntiles, scratch, xq, xs, h, hq, hs, y, total;
};

FwdLayout forward_layout(int64_t T, int64_t H, int64_t I, int64_t E, int64_t K, int64_t shared,
                         int32_t act_fmt) {
  const int64_t Kp = K + shared, Ep = E + shared, A = T * Kp;
  FwdLayout L{};
  size_t p = 0;
  auto take = [&](size_t bytes) {
    size_t at = p;
    p += round_up(bytes);
    return at;
  };
  L.ids = take(A * 4);
  L.w = take(A * 4);
  L.counts = take(Ep * 4);
  L.offsets = take((Ep + 1) * 4);
  L.sorted = take(A * 4);
  L.inv = take(A * 4);
  L.tiles = take(max_tiles_for(A, Ep) * 2 * 4);
  L.ntiles = take(4);
  L.scratch = take(align_scratch_bytes((int)A, (int)Ep));
  // MXFP4 activations: per token (decode kernels) or per sorted row in the
  // blocked order (tiled kernels), A16 >= T rows either way
  const bool q = act_fmt == MOE_ACT_MXFP4;
  const int64_t A16 = (A + 15) / 16 * 16;
  L.xq = take(q ? A16 * H / 2 : 0);
  L.xs = take(q ? A16 * H / 32 : 0);
  L.h = take(A * I * 2);
  L.hq = take(q ? A16 * I / 2 : 0);
  L.hs = take(q ? A16 * I / 32 : 0);
  // staged y (fp16 [A, H] + group exponents); the router GEMM's partial sums
  // (when the call routes from x) live in the same bytes: routing consumes
  // them before the down GEMM writes y
  L.y = take(std::max(staged_y_bytes(A, H), router_workspace_bytes((int)T, (int)H, (int)Ep)));
  L.total = p;
  return L;
}

// Routing shapes and flags.
moe_status check_route_shape(int32_t T, int32_t E, int32_t K, int32_t shared,
                             int32_t renormalize) {
  if (T < 0 || E < 1 || K < 1 || K > E || (shared != 0 && shared != 1) ||
      (renormalize != 0 && renormalize != 1))
    return MOE_ERR_INVALID_ARGUMENT;
  if (E > kMaxE || K + shared > kMaxKp) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

moe_status check_route(const float* logits, const float* gate, int32_t T, int32_t E, int32_t K,
                       int32_t shared, int32_t renormalize) {
  moe_status st = check_route_shape(T, E, K, shared, renormalize);
  if (st != MOE_OK) return st;
  if (T > 0 && (!logits || (shared && !gate))) return MOE_ERR_INVALID_ARGUMENT;
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
    case MOE_ERR_DEVICE: return "MOE_ERR_DEVICE";
  }
  return "MOE_ERR_UNKNOWN";
}

uint32_t moe_debug_flags(int32_t reset) {
  return debug_flags_align(reset != 0) | debug_flags_expert_gemm(reset != 0) |
         debug_flags_expert_gemm_tiled(reset != 0) | debug_flags_route_align(reset != 0);
}

moe_status moe_route_topk(const float* logits, const float* gate_logits, int32_t T, int32_t E,
                          int32_t K, int32_t shared, int32_t renormalize, int32_t* topk_ids,
                          float* topk_weights, void* stream) {
  moe_status st = check_route(logits, gate_logits, T, E, K, shared, renormalize);
  if (st != MOE_OK) return st;
  if (T > 0 && (!topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARGUMENT;
  if (T == 0) return MOE_OK;
  return from_hip(launch_route_topk(logits, gate_logits, T, E, K, shared, renormalize, topk_ids,
                                    topk_weights, as_stream(stream)));
}

size_t moe_route_gemm_workspace_size(int32_t T, int32_t H, int32_t E, int32_t shared) {
  if (T <= 0 || H <= 0 || H % 128 || E < 1 || (shared != 0 && shared != 1)) return 0;
  return round_up(router_workspace_bytes(T, H, E + shared));
}

moe_status moe_route_topk_gemm(const uint16_t* x, const uint16_t* router_w, int32_t T, int32_t H,
                               int32_t E, int32_t K, int32_t shared, int32_t renormalize,
                               int32_t* topk_ids, float* topk_weights, float* logits_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  moe_status st = check_route_shape(T, E, K, shared, renormalize);
  if (st != MOE_OK) return st;
  if (H <= 0) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  const int Ep = E + shared;
  if ((int64_t)T * H * 2 >= INT32_MAX || (int64_t)Ep * H * 2 >= INT32_MAX)
    return MOE_ERR_UNSUPPORTED;                          // 32-bit buffer ranges
  if (T == 0) return MOE_OK;
  if (!x || !router_w || !topk_ids || !topk_weights || !workspace) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(router_w)) return MOE_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < router_workspace_bytes(T, H, Ep)) return MOE_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = as_stream(stream);
  float* partial = (float*)workspace;
  const int S = router_splits(T, H, Ep);
  float* logits = logits_out ? logits_out : partial + (size_t)S * T * Ep;
  hipError_t e = launch_router_gemm(x, router_w, T, H, Ep, partial, logits, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  return from_hip(launch_route_topk_split(partial, S, T, E, K, shared, renormalize, topk_ids,
                                          topk_weights, logits, s));
}

size_t moe_align_workspace_size(int32_t T, int32_t Kp, int32_t Ep) {
  if (T < 0 || Kp < 1 || Ep < 1) return 0;
  return align_scratch_bytes((int)((int64_t)T * Kp), Ep);
}

moe_status moe_align_sort(const int32_t* topk_ids, int32_t T, int32_t Kp, int32_t Ep,
                          int32_t tile_m, int32_t* expert_counts, int32_t* expert_offsets,
                          int32_t* sorted_assign, int32_t* inv_assign, int32_t* tile_table,
                          int32_t* num_tiles, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (T < 0 || Kp < 1 || Ep < 1 || tile_m < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (Ep > 2048) return MOE_ERR_UNSUPPORTED;
  const int64_t A = (int64_t)T * Kp;
  if (A > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (!expert_counts || !expert_offsets || !num_tiles || (A > 0 && (!topk_ids || !sorted_assign)))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = align_scratch_bytes((int)A, Ep);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_align_sort(topk_ids, (int)A, Ep, tile_m, expert_counts, expert_offsets,
                                    sorted_assign, inv_assign, tile_table, num_tiles,
                                    (int32_t*)workspace, as_stream(stream)));
}

moe_status moe_route_align(const float* logits, const float* gate_logits, int32_t T, int32_t E,
                           int32_t K, int32_t shared, int32_t renormalize, int32_t tile_m,
                           int32_t* topk_ids, float* topk_weights, int32_t* expert_counts,
                           int32_t* expert_offsets, int32_t* sorted_assign, int32_t* inv_assign,
                           int32_t* tile_table, int32_t* num_tiles, void* workspace,
                           size_t workspace_bytes, void* stream) {
  moe_status st = check_route(logits, gate_logits, T, E, K, shared, renormalize);
  if (st != MOE_OK) return st;
  if (tile_m < 1) return MOE_ERR_INVALID_ARGUMENT;
  const int Kp = K + shared, Ep = E + shared;
  const int64_t A = (int64_t)T * Kp;
  if (A > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  if (!expert_counts || !expert_offsets || !num_tiles ||
      (T > 0 && (!topk_ids || !topk_weights || !sorted_assign)))
    return MOE_ERR_INVALID_ARGUMENT;
  const size_t need = align_scratch_bytes((int)A, Ep);
  if (workspace_bytes < need) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (!workspace) return MOE_ERR_INVALID_ARGUMENT;
  hipStream_t s = as_stream(stream);
  if (T == 0)     // no assignments: zero counts and offsets, no tiles
    return from_hip(launch_align_sort(nullptr, 0, Ep, tile_m, expert_counts, expert_offsets,
                                      sorted_assign, inv_assign, tile_table, num_tiles,
                                      (int32_t*)workspace, s));
  return from_hip(launch_route_align(logits, E, gate_logits, 1, T, E, K, shared, renormalize,
                                     tile_m, topk_ids, topk_weights, expert_counts,
                                     expert_offsets, sorted_assign, inv_assign, tile_table,
                                     num_tiles, (int32_t*)workspace, s));
}

moe_status moe_mxfp4_quantize(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                              uint8_t* packed, uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || (src_dtype != MOE_SRC_F32 && src_dtype != MOE_SRC_BF16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (cols % 32) return MOE_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!src || !packed || !scales || !aligned16(src) || !aligned16(packed))
    return MOE_ERR_INVALID_ARGUMENT;
  if (rows * (cols / 32) / 256 >= (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  return from_hip(launch_mxfp4_quant(src, src_dtype == MOE_SRC_BF16, rows, cols, packed, scales,
                                     as_stream(stream)));
}

moe_status moe_mxfp4_quantize_blocked(const void* src, int32_t src_dtype, int64_t rows,
                                      int64_t cols, const int32_t* row_map, int32_t Kp,
                                      int64_t out_rows, uint8_t* packed, uint8_t* scales,
                                      void* stream) {
  if (rows < 0 || cols < 0 || out_rows < 0 || (src_dtype != MOE_SRC_F32 && src_dtype != MOE_SRC_BF16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (row_map ? Kp < 1 : out_rows < rows) return MOE_ERR_INVALID_ARGUMENT;
  if (cols % 128) return MOE_ERR_UNSUPPORTED;
  const int64_t out16 = (out_rows + 15) / 16 * 16;
  const int64_t grid = row_map ? (rows * (cols / 32) + 255) / 256 : out16 / 16 * ((cols / 128 + 3) / 4);
  if (out16 * (cols / 2) >= kMaxBufferBytes || (row_map && rows * Kp >= INT32_MAX) ||
      cols > ((int64_t)1 << 30) || grid >= (int64_t)UINT32_MAX)
    return MOE_ERR_UNSUPPORTED;                          // 32-bit offsets, columns and grid
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!src || !packed || !scales || !aligned16(src) || !aligned16(packed) || !aligned16(scales))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_mxfp4_quant_blocked(src, src_dtype == MOE_SRC_BF16, rows, cols, row_map,
                                             row_map ? Kp : 1, out_rows, packed, scales,
                                             as_stream(stream)));
}

moe_status moe_mxfp8_quantize(const void* src, int32_t src_dtype, int64_t rows, int64_t cols,
                              uint8_t* codes, uint8_t* scales, void* stream) {
  if (rows < 0 || cols < 0 || (src_dtype != MOE_SRC_F32 && src_dtype != MOE_SRC_BF16))
    return MOE_ERR_INVALID_ARGUMENT;
  if (cols % 32) return MOE_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!src || !codes || !scales || !aligned16(src) || !aligned16(codes))
    return MOE_ERR_INVALID_ARGUMENT;
  if (rows * (cols / 32) / 256 >= (int64_t)UINT32_MAX) return MOE_ERR_UNSUPPORTED;
  return from_hip(launch_mxfp8_quant(src, src_dtype == MOE_SRC_BF16, rows, cols, codes, scales,
                                     as_stream(stream)));
}

moe_status moe_weights_to_native(const uint8_t* src, int32_t wfmt, int64_t rows, int64_t cols,
                                 uint8_t* dst, void* stream) {
  if (rows < 0 || cols < 0 || (wfmt != 0 && wfmt != 1)) return MOE_ERR_INVALID_ARGUMENT;
  if (rows % 32 || cols % 128) return MOE_ERR_UNSUPPORTED;
  if (rows == 0 || cols == 0) return MOE_OK;
  if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t bytes = rows * (wfmt == 1 ? cols : cols / 2);
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + (uintptr_t)bytes && d0 < s0 + (uintptr_t)bytes) return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_weights_native(src, wfmt == 1 ? 2 : 1, rows, cols, dst,
                                        as_stream(stream)));
}

}  // extern "C"

namespace {

// Weight code bytes of one expert's W13 (2I rows) or W2 (H rows).
bool weights_fit(int wfmt, int64_t rows, int64_t k) {
  return rows * (wfmt == 1 ? k : k / 2) < kMaxBufferBytes;
}

// rows x cols activations (bf16, or MXFP4 codes; blocked rows come in whole
// 16-row blocks).
bool acts_fit(int act_fmt, int64_t rows, int64_t cols) {
  if (act_fmt == MOE_ACT_MXFP4_BLOCKED) rows = (rows + 15) / 16 * 16;
  return rows * (act_fmt == MOE_ACT_BF16 ? cols * 2 : cols / 2) < kMaxBufferBytes;
}

bool act_fmt_ok(int32_t act_fmt) {
  return act_fmt == MOE_ACT_BF16 || act_fmt == MOE_ACT_MXFP4 || act_fmt == MOE_ACT_MXFP4_BLOCKED;
}

moe_status gate_up_impl(const void* act, const uint8_t* act_scale, int32_t act_fmt, int wfmt,
                        const int32_t* sorted_assign, const int32_t* expert_offsets,
                        const int32_t* tile_table, const int32_t* num_tiles, int32_t tile_m,
                        const uint8_t* w13, const uint8_t* w13_scale, int32_t T, int32_t H,
                        int32_t I, int32_t Ep, int32_t Kp, uint16_t* h, void* stream,
                        uint8_t* hq = nullptr, uint8_t* hs = nullptr) {
  if (T < 0 || Ep < 1 || Kp < 1 || !act_fmt_ok(act_fmt)) return MOE_ERR_INVALID_ARGUMENT;
  const bool quant = hq || hs;                              // h written as blocked MXFP4
  moe_status st = check_shape_HI(H, I);
  if (st != MOE_OK) return st;
  const bool blk = act_fmt == MOE_ACT_MXFP4_BLOCKED;
  if (Ep > 2048 || !weights_fit(wfmt, 2 * (int64_t)I, H) ||
      !acts_fit(act_fmt, blk ? (int64_t)T * Kp : T, H))
    return MOE_ERR_UNSUPPORTED;
  if (!tile_m_ok(tile_m, act_fmt, H, I, wfmt) || (blk && tile_m == MOE_TILE_M))
    return MOE_ERR_UNSUPPORTED;
  if (tile_m == MOE_TILE_M && expert_gemm_lds_bytes(H, act_fmt) > kMaxLdsBytes)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!act || !sorted_assign || !expert_offsets || !tile_table || !num_tiles || !w13 ||
      !w13_scale || (quant ? (!hq || !hs) : !h) || (act_fmt != MOE_ACT_BF16 && !act_scale))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(act) || !aligned16(w13) || (blk && !aligned16(act_scale)))
    return MOE_ERR_INVALID_ARGUMENT;
  if (quant && (!aligned16(hq) || !aligned16(hs))) return MOE_ERR_INVALID_ARGUMENT;
  const int64_t mt = max_tiles_for((int64_t)T * Kp, Ep, tile_m);
  if (mt * (I / 16) >= INT32_MAX) return MOE_ERR_UNSUPPORTED;
  hipStream_t s = as_stream(stream);
  if (tile_m != MOE_TILE_M)
    return from_hip(launch_gate_up_tiled(tile_m, act_fmt, wfmt, act, act_scale, sorted_assign,
                                         expert_offsets, tile_table, num_tiles, (int)mt, w13,
                                         w13_scale, T, H, I, Kp, h, s, hq, hs));
  return from_hip(launch_gate_up(act_fmt, wfmt, act, act_scale, sorted_assign, expert_offsets,
                                 tile_table, num_tiles, (int)mt, w13, w13_scale, T, H, I, Kp, h,
                                 s));
}

moe_status down_impl(const void* h, const uint8_t* h_scale, int32_t act_fmt, int wfmt,
                     const int32_t* expert_offsets, const int32_t* tile_table,
                     const int32_t* num_tiles, int32_t tile_m, const uint8_t* w2,
                     const uint8_t* w2_scale, int32_t T, int32_t H, int32_t I, int32_t Ep,
                     int32_t Kp, void* y, void* stream) {
  if (T < 0 || Ep < 1 || Kp < 1 || !act_fmt_ok(act_fmt)) return MOE_ERR_INVALID_ARGUMENT;
  moe_status st = check_shape_HI(H, I);
  if (st != MOE_OK) return st;
  const bool blk = act_fmt == MOE_ACT_MXFP4_BLOCKED;
  if (Ep > 2048 || !weights_fit(wfmt, H, I) || !acts_fit(act_fmt, (int64_t)T * Kp, I))
    return MOE_ERR_UNSUPPORTED;
  if (!tile_m_ok(tile_m, act_fmt, H, I, wfmt) || (blk && tile_m == MOE_TILE_M))
    return MOE_ERR_UNSUPPORTED;
  if (tile_m == MOE_TILE_M && expert_gemm_lds_bytes(I, act_fmt) > kMaxLdsBytes)
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!h || !expert_offsets || !tile_table || !num_tiles || !w2 || !w2_scale || !y ||
      (act_fmt != MOE_ACT_BF16 && !h_scale))
    return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(h) || !aligned16(w2) || !aligned16(y) || (blk && !aligned16(h_scale)))
    return MOE_ERR_INVALID_ARGUMENT;
  const int64_t mt = max_tiles_for((int64_t)T * Kp, Ep, tile_m);
  if (mt * (H / 128) >= INT32_MAX) return MOE_ERR_UNSUPPORTED;
  uint16_t* y16 = static_cast<uint16_t*>(y);
  hipStream_t s = as_stream(stream);
  if (tile_m != MOE_TILE_M)
    return from_hip(launch_down_tiled(tile_m, act_fmt, wfmt, h, h_scale, expert_offsets, tile_table,
                                      num_tiles, (int)mt, w2, w2_scale, T * Kp, H, I, y16, s));
  return from_hip(launch_down(act_fmt, wfmt, h, h_scale, expert_offsets, tile_table, num_tiles,
                              (int)mt, w2, w2_scale, T * Kp, H, I, y16, s));
}

}  // namespace

extern "C" {

moe_status moe_expert_gate_up(const void* act, const uint8_t* act_scale, int32_t act_fmt,
                              const int32_t* sorted_assign, const int32_t* expert_offsets,
                              const int32_t* tile_table, const int32_t* num_tiles, int32_t tile_m,
                              const uint8_t* w13, const uint8_t* w13_scale, int32_t T, int32_t H,
                              int32_t I, int32_t Ep, int32_t Kp, uint16_t* h, void* stream) {
  return gate_up_impl(act, act_scale, act_fmt, 0, sorted_assign, expert_offsets, tile_table,
                      num_tiles, tile_m, w13, w13_scale, T, H, I, Ep, Kp, h, stream);
}

moe_status moe_expert_gate_up_quant(const void* act, const uint8_t* act_scale, int32_t act_fmt,
                                    const int32_t* sorted_assign, const int32_t* expert_offsets,
                                    const int32_t* tile_table, const int32_t* num_tiles,
                                    int32_t tile_m, const uint8_t* w13, const uint8_t* w13_scale,
                                    int32_t T, int32_t H, int32_t I, int32_t Ep, int32_t Kp,
                                    uint8_t* h_packed, uint8_t* h_scale, void* stream) {
  if (act_fmt != MOE_ACT_MXFP4 && act_fmt != MOE_ACT_MXFP4_BLOCKED) return MOE_ERR_INVALID_ARGUMENT;
  if (tile_m == MOE_TILE_M) return MOE_ERR_UNSUPPORTED;
  return gate_up_impl(act, act_scale, act_fmt, 0, sorted_assign, expert_offsets, tile_table,
                      num_tiles, tile_m, w13, w13_scale, T, H, I, Ep, Kp, nullptr, stream,
                      h_packed, h_scale);
}

moe_status moe_mxfp8_expert_gate_up(const uint16_t* x, const int32_t* sorted_assign,
                                    const int32_t* expert_offsets, const int32_t* tile_table,
                                    const int32_t* num_tiles, int32_t tile_m, const uint8_t* w13,
                                    const uint8_t* w13_scale, int32_t T, int32_t H, int32_t I,
                                    int32_t Ep, int32_t Kp, uint16_t* h, void* stream) {
  return gate_up_impl(x, nullptr, MOE_ACT_BF16, 1, sorted_assign, expert_offsets, tile_table,
                      num_tiles, tile_m, w13, w13_scale, T, H, I, Ep, Kp, h, stream);
}

moe_status moe_expert_down(const void* h, const uint8_t* h_scale, int32_t act_fmt,
                           const int32_t* expert_offsets, const int32_t* tile_table,
                           const int32_t* num_tiles, int32_t tile_m, const uint8_t* w2,
                           const uint8_t* w2_scale, int32_t T, int32_t H, int32_t I, int32_t Ep,
                           int32_t Kp, void* y, void* stream) {
  return down_impl(h, h_scale, act_fmt, 0, expert_offsets, tile_table, num_tiles, tile_m, w2,
                   w2_scale, T, H, I, Ep, Kp, y, stream);
}

moe_status moe_mxfp8_expert_down(const uint16_t* h, const int32_t* expert_offsets,
                                 const int32_t* tile_table, const int32_t* num_tiles,
                                 int32_t tile_m, const uint8_t* w2, const uint8_t* w2_scale,
                                 int32_t T, int32_t H, int32_t I, int32_t Ep, int32_t Kp,
                                 void* y, void* stream) {
  return down_impl(h, nullptr, MOE_ACT_BF16, 1, expert_offsets, tile_table, num_tiles, tile_m, w2,
                   w2_scale, T, H, I, Ep, Kp, y, stream);
}

moe_status moe_combine(const void* y, const float* topk_weights, const int32_t* inv_assign,
                       int32_t T, int32_t H, int32_t Kp, uint16_t* out, void* stream) {
  if (T < 0 || H <= 0 || Kp < 1) return MOE_ERR_INVALID_ARGUMENT;
  if (H % 128) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!y || !topk_weights || !inv_assign || !out || !aligned16(y) || !aligned16(out))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_combine(static_cast<const uint16_t*>(y), topk_weights, inv_assign, T, H,
                                 Kp, out, as_stream(stream)));
}

static_assert(MOE_NORM_MAX_RANKS == kMaxNormRanks, "the header's rank limit is the kernel's");

moe_status moe_residual_rmsnorm(const uint16_t* const* partials, int32_t G,
                                const uint16_t* residual, const uint16_t* gamma, float eps,
                                int32_t T, int32_t H, uint16_t* residual_out, uint16_t* out,
                                void* stream) {
  if (!partials || G < 1 || G > MOE_NORM_MAX_RANKS || T < 0 || H <= 0 || !(eps >= 0.f) ||
      !std::isfinite(eps))
    return MOE_ERR_INVALID_ARGUMENT;
  if (H % 8 || H > residual_rmsnorm_max_h()) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!gamma || !out) return MOE_ERR_INVALID_ARGUMENT;
  for (int32_t g = 0; g < G; ++g)
    if (!partials[g] || !aligned16(partials[g])) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(gamma) || !aligned16(out) || (residual && !aligned16(residual)) ||
      (residual_out && !aligned16(residual_out)))
    return MOE_ERR_INVALID_ARGUMENT;
  return from_hip(launch_residual_rmsnorm(partials, G, residual, gamma, eps, T, H, residual_out,
                                          out, as_stream(stream)));
}

int32_t moe_gemm_tile_m(int32_t T, int32_t Kp, int32_t Ep, int32_t H, int32_t I,
                        int32_t act_fmt) {
  if (T <= 0 || Kp < 1 || Ep < 1 || H <= 0 || I <= 0) return MOE_TILE_M;
  return choose_tile_m((int64_t)T * Kp, Ep, H, I, act_fmt);
}

int32_t moe_mxfp8_gemm_tile_m(int32_t T, int32_t Kp, int32_t Ep, int32_t H, int32_t I) {
  if (T <= 0 || Kp < 1 || Ep < 1 || H <= 0 || I <= 0) return MOE_TILE_M;
  return choose_tile_m((int64_t)T * Kp, Ep, H, I, MOE_ACT_BF16, 1);
}

size_t moe_mxfp4_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                int32_t shared, int32_t act_fmt) {
  if (T <= 0 || H <= 0 || I <= 0 || E < 1 || K < 1 || shared < 0 || shared > 1) return 0;
  return forward_layout(T, H, I, E, K, shared, act_fmt).total;
}

}  // extern "C"

namespace {

// The whole layer.  Routing either from the caller's logits (router_w null)
// or through the router GEMM on x (router_w [E + shared, H] bf16; its
// logits optionally copied to logits_out).
moe_status forward_impl(const uint16_t* x, const float* router_logits,
                        const float* shared_gate_logits, const uint16_t* router_w,
                        float* logits_out, const uint8_t* w13, const uint8_t* w13_scale,
                        const uint8_t* w2, const uint8_t* w2_scale, int32_t T, int32_t H,
                        int32_t I, int32_t E, int32_t K, int32_t shared, int32_t act_fmt,
                        int wfmt, uint16_t* out, int32_t* topk_ids_out, float* topk_weights_out,
                        void* workspace, size_t workspace_bytes, void* stream,
                        const Prefetch* pf = nullptr, bool check_only = false) {
  moe_status st = router_w ? check_route_shape(T, E, K, shared, 1)
                           : check_route(router_logits, shared_gate_logits, T, E, K, shared, 1);
  if (st != MOE_OK) return st;
  if (router_w && ((int64_t)T * H * 2 >= INT32_MAX || (int64_t)(E + shared) * H * 2 >= INT32_MAX))
    return MOE_ERR_UNSUPPORTED;                          // 32-bit buffer ranges
  if (router_w && !aligned16(router_w)) return MOE_ERR_INVALID_ARGUMENT;
  if (act_fmt != MOE_ACT_BF16 && act_fmt != MOE_ACT_MXFP4) return MOE_ERR_INVALID_ARGUMENT;
  if (wfmt == 1 && act_fmt != MOE_ACT_BF16) return MOE_ERR_INVALID_ARGUMENT;
  st = check_shape_HI(H, I);
  if (st != MOE_OK) return st;
  if (!weights_fit(wfmt, 2 * (int64_t)I, H) || !weights_fit(wfmt, H, I)) return MOE_ERR_UNSUPPORTED;
  // x and the bf16 h (the larger of each pair of formats)
  if (!acts_fit(MOE_ACT_BF16, T, H) || !acts_fit(MOE_ACT_BF16, (int64_t)T * (K + shared), I))
    return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !w13 || !w13_scale || !w2 || !w2_scale || !out) return MOE_ERR_INVALID_ARGUMENT;
  if (!aligned16(x) || !aligned16(w13) || !aligned16(w2) || !aligned16(out))
    return MOE_ERR_INVALID_ARGUMENT;
  const int Kp = K + shared, Ep = E + shared;
  const int64_t A = (int64_t)T * Kp;
  if (A * (int64_t)H >= ((int64_t)1 << 40) || A > INT32_MAX / 2) return MOE_ERR_UNSUPPORTED;
  const FwdLayout L = forward_layout(T, H, I, E, K, shared, act_fmt);
  const int tm = choose_tile_m(A, Ep, H, I, act_fmt, wfmt);
  const int mt = (int)max_tiles_for(A, Ep, tm);
  // the 32-row kernels' LDS (weight scales, staged activation rows) must fit
  if (tm == MOE_TILE_M && (expert_gemm_lds_bytes(H, act_fmt) > kMaxLdsBytes ||
                           expert_gemm_lds_bytes(I, act_fmt) > kMaxLdsBytes))
    return MOE_ERR_UNSUPPORTED;
  if (workspace_bytes < L.total) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (check_only) return MOE_OK;
  if (!workspace) return MOE_ERR_INVALID_ARGUMENT;

  char* ws = (char*)workspace;
  int32_t* ids = topk_ids_out ? topk_ids_out : (int32_t*)(ws + L.ids);
  float* wts = topk_weights_out ? topk_weights_out : (float*)(ws + L.w);
  int32_t* counts = (int32_t*)(ws + L.counts);
  int32_t* offsets = (int32_t*)(ws + L.offsets);
  int32_t* sorted = (int32_t*)(ws + L.sorted);
  int32_t* inv = (int32_t*)(ws + L.inv);
  int32_t* tiles = (int32_t*)(ws + L.tiles);
  int32_t* ntiles = (int32_t*)(ws + L.ntiles);
  int32_t* scratch = (int32_t*)(ws + L.scratch);
  uint8_t* xq = (uint8_t*)(ws + L.xq);
  uint8_t* xs = (uint8_t*)(ws + L.xs);
  uint16_t* h = (uint16_t*)(ws + L.h);
  uint8_t* hq = (uint8_t*)(ws + L.hq);
  uint8_t* hs = (uint8_t*)(ws + L.hs);
  uint16_t* y = (uint16_t*)(ws + L.y);
  float* rpart = (float*)(ws + L.y);                       // router partial sums (same bytes)
  hipStream_t s = as_stream(stream);

  // routing: logits of row stride ld, the shared gate logit of token t at
  // gate[t * gate_stride]
  hipError_t e;
  const float* lgt = router_logits;
  const float* gate = shared_gate_logits;
  int ld = E, gate_stride = 1;
  if (router_w) {
    const int S = router_splits(T, H, Ep);
    float* lg = logits_out ? logits_out : rpart + (size_t)S * T * Ep;
    e = launch_router_gemm(x, router_w, T, H, Ep, rpart, lg, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    e = launch_sum_splits(rpart, S, T, Ep, lg, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
    lgt = lg;
    gate = lg + E;
    ld = gate_stride = Ep;
  }
  // (a small batch, a decode step: routing and grouping in one workgroup)
  e = launch_route_align(lgt, ld, gate, gate_stride, T, E, K, shared, 1, tm, ids, wts, counts,
                         offsets, sorted, inv, tiles, ntiles, scratch, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  // W4A4 on the tiled kernels: x quantised once per token and written into
  // each of its sorted slots, h in its sorted rows, both in the blocked order
  // (contiguous per 16 rows and chunk instead of gathered rows)
  const bool q = act_fmt == MOE_ACT_MXFP4;
  const bool blk = q && tm != MOE_TILE_M;
  const int32_t gemm_act = blk ? MOE_ACT_MXFP4_BLOCKED : act_fmt;
  if (q) {
    e = blk ? launch_mxfp4_quant_blocked(x, 1, T, H, inv, Kp, A, xq, xs, s)
            : launch_mxfp4_quant(x, 1, T, H, xq, xs, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }
  const void* a1 = q ? (const void*)xq : (const void*)x;
  const uint8_t* a1s = q ? xs : nullptr;
  // (blocked W4A4: the gate/up epilogue writes h MXFP4-quantised, no bf16 h)
  e = tm != MOE_TILE_M
          ? launch_gate_up_tiled(tm, gemm_act, wfmt, a1, a1s, sorted, offsets, tiles, ntiles, mt, w13,
                                 w13_scale, T, H, I, Kp, h, s, blk ? hq : nullptr,
                                 blk ? hs : nullptr)
          : launch_gate_up(act_fmt, wfmt, a1, a1s, sorted, offsets, tiles, ntiles, mt, w13,
                           w13_scale, T, H, I, Kp, h, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  if (q && !blk) {
    e = launch_mxfp4_quant(h, 1, A, I, hq, hs, s);
    if (e != hipSuccess) return MOE_ERR_DEVICE;
  }
  const void* a2 = q ? (const void*)hq : (const void*)h;
  const uint8_t* a2s = q ? hs : nullptr;
  e = tm != MOE_TILE_M
          ? launch_down_tiled(tm, gemm_act, wfmt, a2, a2s, offsets, tiles, ntiles, mt, w2, w2_scale,
                              (int)A, H, I, y, s)
          : launch_down(act_fmt, wfmt, a2, a2s, offsets, tiles, ntiles, mt, w2, w2_scale, (int)A, H,
                        I, y, s);
  if (e != hipSuccess) return MOE_ERR_DEVICE;
  return from_hip(launch_combine(y, wts, inv, T, H, Kp, out, s, pf));
}

moe_status layers_impl(const uint16_t* x, int32_t L, const moe_mxfp4_layer* layers,
                       const uint16_t* const* gammas, float eps, uint16_t* residual, int32_t T,
                       int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared, int32_t act_fmt,
                       int32_t prefetch, uint16_t* out, void* workspace, size_t workspace_bytes,
                       void* stream);

}  // namespace

extern "C" {

moe_status moe_mxfp4_forward(const uint16_t* x, const float* router_logits,
                             const float* shared_gate_logits, const uint8_t* w13,
                             const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                             int32_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared,
                             int32_t act_fmt, uint16_t* out, int32_t* topk_ids_out,
                             float* topk_weights_out, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return forward_impl(x, router_logits, shared_gate_logits, nullptr, nullptr, w13, w13_scale, w2,
                      w2_scale, T, H, I, E, K, shared, act_fmt, 0, out, topk_ids_out,
                      topk_weights_out, workspace, workspace_bytes, stream);
}

size_t moe_mxfp8_workspace_size(int32_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                int32_t shared) {
  return moe_mxfp4_workspace_size(T, H, I, E, K, shared, MOE_ACT_BF16);
}

moe_status moe_mxfp8_forward(const uint16_t* x, const float* router_logits,
                             const float* shared_gate_logits, const uint8_t* w13,
                             const uint8_t* w13_scale, const uint8_t* w2, const uint8_t* w2_scale,
                             int32_t T, int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared,
                             uint16_t* out, int32_t* topk_ids_out, float* topk_weights_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  return forward_impl(x, router_logits, shared_gate_logits, nullptr, nullptr, w13, w13_scale, w2,
                      w2_scale, T, H, I, E, K, shared, MOE_ACT_BF16, 1, out, topk_ids_out,
                      topk_weights_out, workspace, workspace_bytes, stream);
}

moe_status moe_mxfp4_forward_router(const uint16_t* x, const uint16_t* router_w,
                                    const uint8_t* w13, const uint8_t* w13_scale,
                                    const uint8_t* w2, const uint8_t* w2_scale, int32_t T,
                                    int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared,
                                    int32_t act_fmt, uint16_t* out, int32_t* topk_ids_out,
                                    float* topk_weights_out, float* logits_out, void* workspace,
                                    size_t workspace_bytes, void* stream) {
  if (T > 0 && !router_w) return MOE_ERR_INVALID_ARGUMENT;
  return forward_impl(x, nullptr, nullptr, T > 0 ? router_w : nullptr, logits_out, w13, w13_scale,
                      w2, w2_scale, T, H, I, E, K, shared, act_fmt, 0, out, topk_ids_out,
                      topk_weights_out, workspace, workspace_bytes, stream);
}


moe_status moe_mxfp4_forward_layers(const uint16_t* x, int32_t L, const moe_mxfp4_layer* layers,
                                    int32_t T, int32_t H, int32_t I, int32_t E, int32_t K,
                                    int32_t shared, int32_t act_fmt, int32_t prefetch,
                                    uint16_t* out, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return layers_impl(x, L, layers, nullptr, 0.f, nullptr, T, H, I, E, K, shared, act_fmt,
                     prefetch, out, workspace, workspace_bytes, stream);
}

moe_status moe_mxfp4_forward_layers_norm(const uint16_t* x, int32_t L,
                                         const moe_mxfp4_layer* layers,
                                         const uint16_t* const* gammas, float eps,
                                         uint16_t* residual, int32_t T, int32_t H, int32_t I,
                                         int32_t E, int32_t K, int32_t shared, int32_t act_fmt,
                                         int32_t prefetch, uint16_t* out, void* workspace,
                                         size_t workspace_bytes, void* stream) {
  if (L < 1 || !gammas || !(eps >= 0.f) || !std::isfinite(eps)) return MOE_ERR_INVALID_ARGUMENT;
  if (H > 0 && (H % 8 || H > residual_rmsnorm_max_h())) return MOE_ERR_UNSUPPORTED;
  if (T > 0) {
    // (the norm reads out as its partial and updates residual: two buffers)
    if (!residual || !aligned16(residual) || residual == out) return MOE_ERR_INVALID_ARGUMENT;
    for (int l = 0; l < L; ++l)
      if (!gammas[l] || !aligned16(gammas[l])) return MOE_ERR_INVALID_ARGUMENT;
  }
  return layers_impl(x, L, layers, gammas, eps, residual, T, H, I, E, K, shared, act_fmt,
                     prefetch, out, workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

// The layers of a pass; with gammas, each layer's output then goes through
// the residual add and RMSNorm (one partial: h += out, out = RMSNorm(h)),
// both in place, before the next layer reads out.
moe_status layers_impl(const uint16_t* x, int32_t L, const moe_mxfp4_layer* layers,
                       const uint16_t* const* gammas, float eps, uint16_t* residual, int32_t T,
                       int32_t H, int32_t I, int32_t E, int32_t K, int32_t shared, int32_t act_fmt,
                       int32_t prefetch, uint16_t* out, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (L < 1 || !layers || (prefetch != 0 && prefetch != 1)) return MOE_ERR_INVALID_ARGUMENT;
  // Every layer's pointers are checked before anything is enqueued; the shapes
  // (shared by all layers) are checked by the first layer's call, before its
  // first enqueue.
  for (int l = 0; l < L; ++l) {
    const moe_mxfp4_layer& w = layers[l];
    if (T > 0 && (!w.router_w || !w.w13 || !w.w13_scale || !w.w2 || !w.w2_scale))
      return MOE_ERR_INVALID_ARGUMENT;
    if (!aligned16(w.router_w) || !aligned16(w.w13) || !aligned16(w.w2))
      return MOE_ERR_INVALID_ARGUMENT;
  }
  const int64_t Ep = (int64_t)E + shared;
  for (int l = 0; l < L; ++l) {
    // The next layer's weights known before its routing: its router rows and
    // its shared expert (every token's slot K).
    Prefetch pf{};
    if (prefetch && l + 1 < L && T > 0 && E > 0 && H > 0 && I > 0) {
      const moe_mxfp4_layer& n = layers[l + 1];
      const int64_t w13b = 2 * (int64_t)I * H / 2, w13sb = 2 * (int64_t)I * H / 32;
      const int64_t w2b = (int64_t)H * I / 2, w2sb = (int64_t)H * I / 32;
      auto add = [&](const void* p, int64_t bytes) {
        if (bytes > 0 && bytes < (int64_t)UINT32_MAX) {
          pf.p[pf.n] = p;
          pf.bytes[pf.n++] = (uint32_t)bytes;
        }
      };
      add(n.router_w, Ep * H * 2);
      if (shared) {
        add(n.w13 + (int64_t)E * w13b, w13b);
        add(n.w13_scale + (int64_t)E * w13sb, w13sb);
        add(n.w2 + (int64_t)E * w2b, w2b);
        add(n.w2_scale + (int64_t)E * w2sb, w2sb);
      }
    }
    // Layer 0 reads x; later layers read and rewrite out in place (each
    // layer's combine, its only writer of out, runs after all its reads).
    const moe_mxfp4_layer& w = layers[l];
    moe_status st = forward_impl(l == 0 ? x : out, nullptr, nullptr, T > 0 ? w.router_w : nullptr,
                                 nullptr, w.w13, w.w13_scale, w.w2, w.w2_scale, T, H, I, E, K,
                                 shared, act_fmt, 0, out, nullptr, nullptr, workspace,
                                 workspace_bytes, stream, pf.n ? &pf : nullptr);
    if (st != MOE_OK) return st;
    if (T == 0) return MOE_OK;
    if (gammas) {
      const uint16_t* part = out;
      if (launch_residual_rmsnorm(&part, 1, residual, gammas[l], eps, T, H, residual, out,
                                  as_stream(stream)) != hipSuccess)
        return MOE_ERR_DEVICE;
    }
  }
  return MOE_OK;
}

}  // namespace

// ---- the forward for callers that cannot allocate -------------------------

namespace {

// Workspace of moe_mxfp4_forward_noalloc: one copy per GPU the library runs
// on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: host code uses only the device address
// hipGetSymbolAddress returns for the current device (noalloc_scratch).
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];        // per device, looked up on its first call

// The current device's address of `scratch` (looked up once per device,
// with that device current).
moe_status noalloc_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_ERR_DEVICE;
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status moe_mxfp4_forward_noalloc(const uint16_t* x, const float* router_logits,
                                     const float* shared_gate_logits, const uint8_t* w13,
                                     const uint8_t* w13_scale, const uint8_t* w2,
                                     const uint8_t* w2_scale, int32_t T, int32_t H, int32_t I,
                                     int32_t E, int32_t K, int32_t shared, int32_t act_fmt,
                                     uint16_t* out, int32_t* topk_ids_out,
                                     float* topk_weights_out, void* stream) {
  // every argument check (and the scratch size) before any HIP call
  moe_status st = forward_impl(x, router_logits, shared_gate_logits, nullptr, nullptr, w13,
                               w13_scale, w2, w2_scale, T, H, I, E, K, shared, act_fmt, 0, out,
                               topk_ids_out, topk_weights_out, nullptr,
                               MOE_NOALLOC_SCRATCH_BYTES, stream, nullptr, true);
  if (st != MOE_OK || T == 0) return st;
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st != MOE_OK) return st;
  return forward_impl(x, router_logits, shared_gate_logits, nullptr, nullptr, w13, w13_scale, w2,
                      w2_scale, T, H, I, E, K, shared, act_fmt, 0, out, topk_ids_out,
                      topk_weights_out, ws, MOE_NOALLOC_SCRATCH_BYTES, stream);
}

}  // extern "C"
