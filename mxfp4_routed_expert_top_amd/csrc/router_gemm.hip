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
// Small batches (T < 256): workgroup = 4 waves x 16 router rows = 64 rows, 64 tokens
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

// Larger batches, LDS-tiled: a workgroup computes 128 tokens x 128 router
// rows over one split of the reduction; wave (wm, wn) of the 2 x 2 grid owns
// tokens [64 wm, +64) and rows [64 wn, +64) (4 x 4 MFMA tiles).  The
// reduction runs in chunks of 64 elements: both operands' chunk rows (128
// bytes each) go to LDS with direct-to-LDS 16-byte loads, two stages deep,
// so every byte of x and Wr a workgroup needs is requested once (a
// register-fed kernel requests a token row once per wave).  With one split
// the workgroup writes the logits themselves.  16-byte piece p of row r sits in slot
// p ^ (r & 7) of the row: the 16 rows an MFMA operand read touches spread
// over all banks.
constexpr int kLdsBT = 128, kLdsBE = 128, kLdsKC = 64;
constexpr int kLdsStage = (kLdsBT + kLdsBE) * kLdsKC * 2;          // 32 KiB

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void lds_load16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, (int)soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void router_wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__global__ __launch_bounds__(256) void router_gemm_lds_kernel(const uint16_t* __restrict__ x,
                                                              const uint16_t* __restrict__ w,
                                                              int T, int H, int Ep, int nE, int nT,
                                                              int cps, float* __restrict__ out) {
  __shared__ __align__(16) uint8_t st0[kLdsStage];
  __shared__ __align__(16) uint8_t st1[kLdsStage];
  const int b = blockIdx.x;
  const int et = b % nE, tt = (b / nE) % nT, sp = b / (nE * nT);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int nl = lane & 15, g = lane >> 4;
  const rsrc_t rw = make_rsrc(w, (uint32_t)((size_t)Ep * H * 2));
  const rsrc_t rx = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
  // Loads: the stage holds 256 rows (x rows 0..127, then W rows) of 8
  // pieces; wave v's instruction i fills rows 64 v + 8 i .. + 8 (waves 0-1:
  // x rows, waves 2-3: W rows), lane l row + l / 8, slot l % 8 (from piece
  // (l % 8) ^ (row & 7)).
  uint32_t src[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int row = 8 * (8 * wave + i) + (lane >> 3);        // 0..255
    const int piece = (lane & 7) ^ (row & 7);
    if (row < kLdsBT) {
      const int t = tt * kLdsBT + row;
      src[i] = t < T ? (uint32_t)t * H * 2 + 16 * piece : kOOR;
    } else {
      const int e = et * kLdsBE + row - kLdsBT;
      src[i] = e < Ep ? (uint32_t)e * H * 2 + 16 * piece : kOOR;
    }
  }
  const int c0 = sp * cps, c1 = min(c0 + cps, H / kLdsKC);   // this split's chunks
  auto issue = [&](uint8_t* st, int c) {
    const uint32_t oor = c < c1 ? 0u : kOOR;
    const uint32_t so = c < c1 ? (uint32_t)(kLdsKC * 2 * c) : 0u;
    const rsrc_t r = wave < 2 ? rx : rw;                   // wave-uniform
#pragma unroll
    for (int i = 0; i < 8; ++i) lds_load16(r, src[i] | oor, so, st + (8 * wave + i) * 1024);
  };
  floatx4_t acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[mt][n] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  auto frag = [&](const uint8_t* st, int row, int piece) {
    return *reinterpret_cast<const bf16x8_t*>(st + row * 128 + 16 * (piece ^ (row & 7)));
  };
  auto compute = [&](const uint8_t* st) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {                           // two 32-element MFMA K-steps
      bf16x8_t a[4], b[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) a[mt] = frag(st, 64 * wm + 16 * mt + nl, 4 * k + g);
#pragma unroll
      for (int n = 0; n < 4; ++n) b[n] = frag(st, kLdsBT + 64 * wn + 16 * n + nl, 4 * k + g);
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int n = 0; n < 4; ++n) acc[mt][n] = mfma_bf16_16x16x32(a[mt], b[n], acc[mt][n]);
    }
  };
  // Wait rules: direct-to-LDS loads are counted by vmcnt; a wave waits for
  // its own loads of the stage it is about to read and for its own LDS reads
  // (lgkmcnt), then the barrier makes every wave's loads of that stage
  // visible and retires every read of the other stage before its refill.
  issue(st0, c0);
  for (int c = c0; c < c1; c += 2) {
    router_wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(st1, c + 1);
    compute(st0);
    router_wait_vmcnt<0>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    issue(st0, c + 2);
    if (c + 1 < c1) compute(st1);
  }
  router_wait_vmcnt<0>();
#pragma unroll
  for (int n = 0; n < 4; ++n) {
    const int e = et * kLdsBE + 64 * wn + 16 * n + nl;
    if (e >= Ep) continue;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tt * kLdsBT + 64 * wm + 16 * mt + 4 * g + r;
        if (t < T) out[((size_t)sp * T + t) * Ep + e] = acc[mt][n][r];
      }
  }
}

struct RouterPlan {
  bool lds;            // the LDS-tiled kernel (else the register-fed small-batch one)
  int nE, nT, cps, S;  // row tiles, token tiles, chunks per split, splits
};

// Small batches (T < 256): 64 x 64 register-fed tiles; larger: 128 x 128
// LDS tiles.  Either way the reduction is split until about kTargetBlocks
// workgroups exist (at most route_max_splits(), at least two chunks each).
RouterPlan router_plan(int T, int H, int Ep) {
  RouterPlan p;
  p.lds = T >= 256;
  const int bt = p.lds ? kLdsBT : 64, be = p.lds ? kLdsBE : 64;
  const int kc = p.lds ? kLdsKC : 128;                   // elements per chunk
  p.nT = (T + bt - 1) / bt;
  p.nE = (Ep + be - 1) / be;
  const int nch = H / kc;
  const long base = (long)p.nE * p.nT;
  const long cap = std::min((long)std::max(1, nch / 2), (long)route_max_splits());
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
                              float* partial, float* logits, hipStream_t stream) {
  const RouterPlan p = router_plan(T, H, Ep);
  float* out = p.S == 1 ? logits : partial;
  const unsigned grid = (unsigned)((long)p.nE * p.nT * p.S);
  if (p.lds)
    hipLaunchKernelGGL(router_gemm_lds_kernel, dim3(grid), dim3(256), 0, stream, x, w, T, H, Ep,
                       p.nE, p.nT, p.cps, out);
  else
    hipLaunchKernelGGL(router_gemm_kernel, dim3(grid), dim3(256), 0, stream, x, w, T, H, Ep, p.cps,
                       p.nE, p.nT, out);
  return hipGetLastError();
}
