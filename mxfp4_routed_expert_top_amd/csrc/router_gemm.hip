// Router GEMM: the logits the routing step consumes, logits = x . Wr^T, with
// Wr bf16 [E', H] (E routed rows, plus the shared expert's gate vector as
// row E when shared = 1) and fp32 accumulation of the exact bf16 products on
// v_mfma_f32_16x16x32_bf16.  The pages' top-K kernel takes the router's
// gating output as its input (InferenceX "MI355X Qwen3.5 SGLang v0.5.12"
// post, section on the specific optimisations, fused_topk bullet); here the
// router GEMM and the routing run as one call.
//
// The reduction over H is cut into S splits so that a small batch still
// spreads the router rows over the GPU; split s writes its partial sums
// P[s][t][e] (fp32 [S, T, E']), which are then added in split order (a
// fixed order: the logits, and the selection, do not depend on timing).
//
// Small batches: workgroup = 4 waves x 16 router rows = 64 rows, 64 tokens
// (four 16-row MFMA sub-tiles), one split of `cps` 128-element chunks.  Lane (row / column
// l % 16, K-group g = l / 16) loads the four 16-byte pieces of elements
// [32 g, 32 g + 32) of the chunk, for its router row and for each of its
// token rows; MFMA step j takes piece j from every lane (a permutation of
// the chunk's K that both operands share).  Rows past E' or T read zeros
// through out-of-range buffer offsets and are not stored.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace {

constexpr uint32_t kOOR = 0x80000000u;
constexpr int kTargetBlocks = 256;     // split the reduction until about one workgroup per CU

__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ w, int T,
                                                          int H, int Ep, int cps, int nEg, int nT,
                                                          float* __restrict__ partial) {
  const int b = blockIdx.x;
  const int eg = b % nEg, tt = (b / nEg) % nT, s = b / (nEg * nT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int e = eg * 64 + wave * 16 + nl;
  const int c0 = s * cps, c1 = min(c0 + cps, H / 128);
  const rsrc_t rw = make_rsrc(w, (uint32_t)((size_t)Ep * H * 2));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
  const uint32_t wo = e < Ep ? (uint32_t)e * H * 2 + 64 * g : kOOR;
  uint32_t xo[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = tt * 64 + 16 * mt + nl;
    xo[mt] = t < T ? (uint32_t)t * H * 2 + 64 * g : kOOR;
  }
  floatx4_t acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) acc[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  for (int c = c0; c < c1; ++c) {
    u32x4_t bw[4], ax[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) bw[j] = bload16(rw, wo, 256 * c + 16 * j);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) ax[mt][j] = bload16(rx, xo[mt], 256 * c + 16 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        acc[mt] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, ax[mt][j]),
                                     __builtin_bit_cast(bf16x8_t, bw[j]), acc[mt]);
  }
  // D: lane holds token rows 4 g + r of router column e
  if (e < Ep) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tt * 64 + 16 * mt + 4 * g + r;
        if (t < T) partial[((size_t)s * T + t) * Ep + e] = acc[mt][r];
      }
  }
}

// Large batches: each wave owns 64 router rows (four 16-row strips) of a
// 256-row workgroup slice, so every token fragment it loads feeds four MFMAs
// instead of one.  No split of the reduction.
__global__ __launch_bounds__(256) void router_gemm_wide_kernel(const uint16_t* __restrict__ x,
                                                               const uint16_t* __restrict__ w,
                                                               int T, int H, int Ep, int nEg,
                                                               float* __restrict__ out) {
  const int b = blockIdx.x;
  const int eg = b % nEg, tt = b / nEg;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const rsrc_t rw = make_rsrc(w, (uint32_t)((size_t)Ep * H * 2));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
  uint32_t wo[4], xo[4];
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = eg * 256 + wave * 64 + 16 * n + nl;
    wo[n] = e < Ep ? (uint32_t)e * H * 2 + 64 * g : kOOR;
  }
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    const int t = tt * 64 + 16 * mt + nl;
    xo[mt] = t < T ? (uint32_t)t * H * 2 + 64 * g : kOOR;
  }
  floatx4_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[mt][n] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  // K-steps of 32 elements (16-byte pieces), NSTEP deep: the loads of step
  // k + NSTEP - 1 are issued before step k's MFMAs run.
  constexpr int NSTEP = 4;
  const int nk = H / 32;                 // 4 pieces per 128-element chunk
  u32x4_t bw[NSTEP][4], ax[NSTEP][4];
  auto load = [&](int k, u32x4_t (&b)[4], u32x4_t (&a)[4]) {
    const uint32_t so = 256 * (k >> 2) + 16 * (k & 3);
#pragma unroll
    for (int n = 0; n < 4; ++n) b[n] = bload16(rw, wo[n], so);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) a[mt] = bload16(rx, xo[mt], so);
  };
#pragma unroll
  for (int k = 0; k < NSTEP - 1; ++k) load(k, bw[k], ax[k]);
  for (int k0 = 0; k0 < nk; k0 += NSTEP) {
#pragma unroll
    for (int u = 0; u < NSTEP; ++u) {
      const int k = k0 + u;
      const int nx = (u + NSTEP - 1) % NSTEP;
      if (k + NSTEP - 1 < nk) load(k + NSTEP - 1, bw[nx], ax[nx]);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int n = 0; n < 4; ++n)
          acc[mt][n] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, ax[u][mt]),
                                          __builtin_bit_cast(bf16x8_t, bw[u][n]), acc[mt][n]);
    }
  }
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = eg * 256 + wave * 64 + 16 * n + nl;
    if (e >= Ep) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tt * 64 + 16 * mt + 4 * g + r;
        if (t < T) out[(size_t)t * Ep + e] = acc[mt][n][r];
      }
  }
}

struct RouterPlan {
  bool wide;
  int nEg, nT, cps, S;
};

RouterPlan router_plan(int T, int H, int Ep) {
  RouterPlan p;
  p.nT = (T + 63) / 64;
  const int nch = H / 128;
  p.wide = (long)p.nT * ((Ep + 255) / 256) >= kTargetBlocks / 2;
  if (p.wide) {                      // enough token tiles: wide workgroups, no split
    p.nEg = (Ep + 255) / 256;
    p.cps = nch;
    p.S = 1;
    return p;
  }
  p.nEg = (Ep + 63) / 64;
  const long base = (long)p.nEg * p.nT;
  const long cap = std::min((long)nch, (long)route_max_splits());
  const int want = (int)std::max(1L, std::min(cap, (kTargetBlocks + base - 1) / base));
  p.cps = (nch + want - 1) / want;
  p.S = (nch + p.cps - 1) / p.cps;
  return p;
}

}  // namespace

int router_splits(int T, int H, int Ep) { return router_plan(T, H, Ep).S; }

// The S partial sums, then room for the summed logits [T, Ep].
size_t router_workspace_bytes(int T, int H, int Ep) {
  return (size_t)(router_plan(T, H, Ep).S + 1) * T * Ep * sizeof(float);
}

hipError_t launch_router_gemm(const uint16_t* x, const uint16_t* w, int T, int H, int Ep,
                              float* partial, hipStream_t stream) {
  const RouterPlan p = router_plan(T, H, Ep);
  if (p.wide) {
    hipLaunchKernelGGL(router_gemm_wide_kernel, dim3((unsigned)((long)p.nEg * p.nT)), dim3(256), 0,
                       stream, x, w, T, H, Ep, p.nEg, partial);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)((long)p.nEg * p.nT * p.S);
  hipLaunchKernelGGL(router_gemm_kernel, dim3(grid), dim3(256), 0, stream, x, w, T, H, Ep, p.cps,
                     p.nEg, p.nT, partial);
  return hipGetLastError();
}
