// Grouped expert GEMMs over MXFP4 weights, one workgroup per (32-row tile,
// N-slice).  The tiles come from the align step's tile table; a tile holds up
// to 32 consecutive rows of one expert's group (VibeSys "Qwen3.5-397B on 4x
// MI300A" post, section "Prefill, cache and speculation": 32-row tiles).
//
// W4A16 (bf16 activations): the fused HIP MoE kernel dequantises MXFP4 in
// registers (same post, section "Baseline"); here each lane loads 16 bytes
// (32 codes, one scale block) of a weight row, expands them to bf16 with the
// gfx950 scaled converter (exact: an E2M1 value times a power of two) and
// feeds v_mfma_f32_16x16x32_bf16.  W4A4 (MXFP4 activations): both operands
// go straight into the scaled MFMA v_mfma_scale_f32_16x16x128_f8f6f4 with
// their E8M0 scales.
//
// MFMA operand layout (16x16 tiles, wave64): lane l supplies row / column
// (l % 16) and K-group (l / 16).  A lane's 16 weight bytes cover K-elements
// [k0 + 32g, k0 + 32g + 32): for bf16 they feed four 16x16x32 MFMAs, K-slice
// j = elements [k0 + 32g + 8j, +8), and the activation operand takes the
// same elements, so every MFMA sums matching products.  D: lane l holds rows
// 4*(l/16) + r, r < 4, of column l % 16.
//
// gate_up: rows [0, I) of W13 are the gate projection, rows [I, 2I) the up
// projection; a wave owns 16 intermediate columns i and both projections, so
// SwiGLU h = silu(gate) * up runs in registers and h is stored as bf16 in
// the sorted row order.  down: a wave owns 32 output columns j; y is stored
// as fp32 in the sorted row order.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kTileM = 32;        // rows per workgroup (= the tile table's tile_m)
constexpr int kMT = kTileM / 16;  // 16-row MFMA subtiles per tile

struct TileInfo {
  int expert, row0, rows;
};

__device__ __forceinline__ bool load_tile(const int32_t* tiles, const int32_t* num_tiles,
                                          const int32_t* offsets, int tile, TileInfo* ti) {
  if (tile >= *num_tiles) return false;
  ti->expert = tiles[2 * tile];
  ti->row0 = tiles[2 * tile + 1];
  ti->rows = min(kTileM, offsets[ti->expert + 1] - ti->row0);
  return true;
}

// ---------------------------------------------------------------- W4A16 ----

__global__ __launch_bounds__(256) void gate_up_w4a16_kernel(
    const uint16_t* __restrict__ x, const int32_t* __restrict__ sorted,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ w13,
    const uint8_t* __restrict__ w13s, int T, int H, int I, int Kp, int nsl,
    uint16_t* __restrict__ h) {
  TileInfo ti;
  if (!load_tile(tiles, num_tiles, offsets, blockIdx.x / nsl, &ti)) return;
  const int s = blockIdx.x % nsl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int i = s * 64 + wave * 16 + nl;
  const size_t rb = (size_t)H / 2, rs = (size_t)H / 32;
  const size_t erow = (size_t)ti.expert * 2 * I;
  const uint8_t* wg = w13 + (erow + i) * rb + 16 * g;
  const uint8_t* wu = w13 + (erow + I + i) * rb + 16 * g;
  const uint8_t* sg = w13s + (erow + i) * rs + g;
  const uint8_t* su = w13s + (erow + I + i) * rs + g;

  const uint16_t* xr[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int m = min(16 * mt + nl, ti.rows - 1);          // padded rows reuse a valid row
    const int tok = min((unsigned)(sorted[ti.row0 + m] / Kp), (unsigned)(T - 1));
    xr[mt] = x + (size_t)tok * H + 32 * g;
  }
  const int mtn = (ti.rows + 15) / 16;

  floatx4_t accg[kMT], accu[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) accg[mt] = accu[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += 128) {
    const u32x4_t qg = load16(wg + k0 / 2);
    const u32x4_t qu = load16(wu + k0 / 2);
    const float scg = e8m0_to_f32(sg[k0 / 32]);
    const float scu = e8m0_to_f32(su[k0 / 32]);
    bf16x8_t a[kMT][4];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      if (mt < mtn)
#pragma unroll
        for (int j = 0; j < 4; ++j) a[mt][j] = load_bf16x8(xr[mt] + k0 + 8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t bg = dequant8_bf16(qg[j], scg);
      const bf16x8_t bu = dequant8_bf16(qu[j], scu);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
        if (mt < mtn) {
          accg[mt] = mfma_bf16_16x16x32(a[mt][j], bg, accg[mt]);
          accu[mt] = mfma_bf16_16x16x32(a[mt][j], bu, accu[mt]);
        }
    }
  }

#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * g + r;
      if (m < ti.rows)
        h[(size_t)(ti.row0 + m) * I + i] = f32_to_bf16_rne(swiglu(accg[mt][r], accu[mt][r]));
    }
}

__global__ __launch_bounds__(256) void down_w4a16_kernel(
    const uint16_t* __restrict__ h, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const uint8_t* __restrict__ w2, const uint8_t* __restrict__ w2s, int H, int I, int nsl,
    float* __restrict__ y) {
  TileInfo ti;
  if (!load_tile(tiles, num_tiles, offsets, blockIdx.x / nsl, &ti)) return;
  const int s = blockIdx.x % nsl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int j0 = s * 128 + wave * 32 + nl;                 // strip 0; strip 1 is j0 + 16
  const size_t rb = (size_t)I / 2, rs = (size_t)I / 32;
  const size_t erow = (size_t)ti.expert * H;
  const uint8_t* w0 = w2 + (erow + j0) * rb + 16 * g;
  const uint8_t* w1 = w2 + (erow + j0 + 16) * rb + 16 * g;
  const uint8_t* s0 = w2s + (erow + j0) * rs + g;
  const uint8_t* s1 = w2s + (erow + j0 + 16) * rs + g;

  const uint16_t* hr[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int m = min(16 * mt + nl, ti.rows - 1);
    hr[mt] = h + (size_t)(ti.row0 + m) * I + 32 * g;
  }
  const int mtn = (ti.rows + 15) / 16;

  floatx4_t acc0[kMT], acc1[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) acc0[mt] = acc1[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < I; k0 += 128) {
    const u32x4_t q0 = load16(w0 + k0 / 2);
    const u32x4_t q1 = load16(w1 + k0 / 2);
    const float sc0 = e8m0_to_f32(s0[k0 / 32]);
    const float sc1 = e8m0_to_f32(s1[k0 / 32]);
    bf16x8_t a[kMT][4];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      if (mt < mtn)
#pragma unroll
        for (int j = 0; j < 4; ++j) a[mt][j] = load_bf16x8(hr[mt] + k0 + 8 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bf16x8_t b0 = dequant8_bf16(q0[j], sc0);
      const bf16x8_t b1 = dequant8_bf16(q1[j], sc1);
#pragma unroll
      for (int mt = 0; mt < kMT; ++mt)
        if (mt < mtn) {
          acc0[mt] = mfma_bf16_16x16x32(a[mt][j], b0, acc0[mt]);
          acc1[mt] = mfma_bf16_16x16x32(a[mt][j], b1, acc1[mt]);
        }
    }
  }

#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * g + r;
      if (m < ti.rows) {
        float* yr = y + (size_t)(ti.row0 + m) * H;
        yr[j0] = acc0[mt][r];
        yr[j0 + 16] = acc1[mt][r];
      }
    }
}

// ----------------------------------------------------------------- W4A4 ----

__global__ __launch_bounds__(256) void gate_up_w4a4_kernel(
    const uint8_t* __restrict__ xq, const uint8_t* __restrict__ xs,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s, int T, int H, int I,
    int Kp, int nsl, uint16_t* __restrict__ h) {
  TileInfo ti;
  if (!load_tile(tiles, num_tiles, offsets, blockIdx.x / nsl, &ti)) return;
  const int s = blockIdx.x % nsl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int i = s * 64 + wave * 16 + nl;
  const size_t rb = (size_t)H / 2, rs = (size_t)H / 32;
  const size_t erow = (size_t)ti.expert * 2 * I;
  const uint8_t* wg = w13 + (erow + i) * rb + 16 * g;
  const uint8_t* wu = w13 + (erow + I + i) * rb + 16 * g;
  const uint8_t* sg = w13s + (erow + i) * rs + g;
  const uint8_t* su = w13s + (erow + I + i) * rs + g;

  const uint8_t* ar[kMT];
  const uint8_t* asr[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int m = min(16 * mt + nl, ti.rows - 1);
    const int tok = min((unsigned)(sorted[ti.row0 + m] / Kp), (unsigned)(T - 1));
    ar[mt] = xq + (size_t)tok * rb + 16 * g;
    asr[mt] = xs + (size_t)tok * rs + g;
  }
  const int mtn = (ti.rows + 15) / 16;

  floatx4_t accg[kMT], accu[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) accg[mt] = accu[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < H; k0 += 128) {
    const u32x4_t qg = load16(wg + k0 / 2);
    const u32x4_t qu = load16(wu + k0 / 2);
    const uint32_t scg = sg[k0 / 32];
    const uint32_t scu = su[k0 / 32];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      if (mt < mtn) {
        const u32x4_t qa = load16(ar[mt] + k0 / 2);
        const uint32_t sa = asr[mt][k0 / 32];
        accg[mt] = mfma_fp4_16x16x128(qa, sa, qg, scg, accg[mt]);
        accu[mt] = mfma_fp4_16x16x128(qa, sa, qu, scu, accu[mt]);
      }
  }

#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * g + r;
      if (m < ti.rows)
        h[(size_t)(ti.row0 + m) * I + i] = f32_to_bf16_rne(swiglu(accg[mt][r], accu[mt][r]));
    }
}

__global__ __launch_bounds__(256) void down_w4a4_kernel(
    const uint8_t* __restrict__ hq, const uint8_t* __restrict__ hs,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2s, int H, int I, int nsl, float* __restrict__ y) {
  TileInfo ti;
  if (!load_tile(tiles, num_tiles, offsets, blockIdx.x / nsl, &ti)) return;
  const int s = blockIdx.x % nsl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const int j0 = s * 128 + wave * 32 + nl;
  const size_t rb = (size_t)I / 2, rs = (size_t)I / 32;
  const size_t erow = (size_t)ti.expert * H;
  const uint8_t* w0 = w2 + (erow + j0) * rb + 16 * g;
  const uint8_t* w1 = w2 + (erow + j0 + 16) * rb + 16 * g;
  const uint8_t* s0 = w2s + (erow + j0) * rs + g;
  const uint8_t* s1 = w2s + (erow + j0 + 16) * rs + g;

  const uint8_t* ar[kMT];
  const uint8_t* asr[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    const int m = min(16 * mt + nl, ti.rows - 1);
    ar[mt] = hq + (size_t)(ti.row0 + m) * rb + 16 * g;
    asr[mt] = hs + (size_t)(ti.row0 + m) * rs + g;
  }
  const int mtn = (ti.rows + 15) / 16;

  floatx4_t acc0[kMT], acc1[kMT];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) acc0[mt] = acc1[mt] = (floatx4_t){0.f, 0.f, 0.f, 0.f};

  for (int k0 = 0; k0 < I; k0 += 128) {
    const u32x4_t q0 = load16(w0 + k0 / 2);
    const u32x4_t q1 = load16(w1 + k0 / 2);
    const uint32_t sc0 = s0[k0 / 32];
    const uint32_t sc1 = s1[k0 / 32];
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
      if (mt < mtn) {
        const u32x4_t qa = load16(ar[mt] + k0 / 2);
        const uint32_t sa = asr[mt][k0 / 32];
        acc0[mt] = mfma_fp4_16x16x128(qa, sa, q0, sc0, acc0[mt]);
        acc1[mt] = mfma_fp4_16x16x128(qa, sa, q1, sc1, acc1[mt]);
      }
  }

#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * g + r;
      if (m < ti.rows) {
        float* yr = y + (size_t)(ti.row0 + m) * H;
        yr[j0] = acc0[mt][r];
        yr[j0 + 16] = acc1[mt][r];
      }
    }
}

// -------------------------------------------------------------- combine ----

// out[t, j] = bf16( sum_k w[t, k] * y[inv[t*K' + k], j] ), slots in order.
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ y,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv, int H,
                                                      int Kp, int nbx, uint16_t* __restrict__ out) {
  const int t = blockIdx.x / nbx;
  const int j = ((blockIdx.x % nbx) * 256 + threadIdx.x) * 4;
  if (j >= H) return;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int k = 0; k < Kp; ++k) {
    const float wk = w[(size_t)t * Kp + k];
    const float4 v = *reinterpret_cast<const float4*>(y + (size_t)inv[(size_t)t * Kp + k] * H + j);
    acc.x += wk * v.x;
    acc.y += wk * v.y;
    acc.z += wk * v.z;
    acc.w += wk * v.w;
  }
  uint2 o;
  o.x = (uint32_t)f32_to_bf16_rne(acc.x) | ((uint32_t)f32_to_bf16_rne(acc.y) << 16);
  o.y = (uint32_t)f32_to_bf16_rne(acc.z) | ((uint32_t)f32_to_bf16_rne(acc.w) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * H + j) = o;
}

}  // namespace

int expert_gemm_tile_m() { return kTileM; }

hipError_t launch_gate_up(int act_fmt, const void* act, const uint8_t* act_scale,
                          const int32_t* sorted, const int32_t* offsets, const int32_t* tiles,
                          const int32_t* num_tiles, int max_tiles, const uint8_t* w13,
                          const uint8_t* w13s, int T, int H, int I, int Kp, uint16_t* h,
                          hipStream_t stream) {
  const int nsl = I / 64;
  dim3 grid((unsigned)(max_tiles * nsl)), block(256);
  if (act_fmt == 0)
    hipLaunchKernelGGL(gate_up_w4a16_kernel, grid, block, 0, stream, (const uint16_t*)act, sorted,
                       offsets, tiles, num_tiles, w13, w13s, T, H, I, Kp, nsl, h);
  else
    hipLaunchKernelGGL(gate_up_w4a4_kernel, grid, block, 0, stream, (const uint8_t*)act, act_scale,
                       sorted, offsets, tiles, num_tiles, w13, w13s, T, H, I, Kp, nsl, h);
  return hipGetLastError();
}

hipError_t launch_down(int act_fmt, const void* h, const uint8_t* h_scale, const int32_t* offsets,
                       const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                       const uint8_t* w2, const uint8_t* w2s, int H, int I, float* y,
                       hipStream_t stream) {
  const int nsl = H / 128;
  dim3 grid((unsigned)(max_tiles * nsl)), block(256);
  if (act_fmt == 0)
    hipLaunchKernelGGL(down_w4a16_kernel, grid, block, 0, stream, (const uint16_t*)h, offsets, tiles,
                       num_tiles, w2, w2s, H, I, nsl, y);
  else
    hipLaunchKernelGGL(down_w4a4_kernel, grid, block, 0, stream, (const uint8_t*)h, h_scale, offsets,
                       tiles, num_tiles, w2, w2s, H, I, nsl, y);
  return hipGetLastError();
}

hipError_t launch_combine(const float* y, const float* w, const int32_t* inv, int T, int H, int Kp,
                          uint16_t* out, hipStream_t stream) {
  const int nbx = (H / 4 + 255) / 256;
  dim3 grid((unsigned)(nbx * T)), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, y, w, inv, H, Kp, nbx, out);
  return hipGetLastError();
}
