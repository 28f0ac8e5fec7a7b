// Large-M grouped expert GEMMs (prefill): one workgroup per (BM-row tile of
// one expert's group, 256 weight rows), the activation rows staged through
// LDS and shared by the workgroup's 4 waves, each wave owning 64 weight rows
// (four 16-row strips) over the whole K.  The pages keep separate launchers
// for small-M decode and large-M prefill GEMMs and reorder grouped-MoE
// programs so that neighbours reuse expert-weight tiles from cache (MiniMax
// M3 on MI355X post, section "Local shape and tiling"); here the block order
// is remapped so that each XCD (own L2) walks consecutive tiles of one
// weight slice.
//
// Per 128-element K chunk: every wave loads its four strips' codes (16 bytes
// per lane = one scale block) and scale bytes from HBM, the workgroup
// gathers the tile's activation chunk into LDS (double-buffered, one barrier
// per chunk, the next chunk's loads in flight during the MFMAs).
//   W4A16: codes -> bf16 via v_cvt_scalef32_pk_bf16_fp4, v_mfma_f32_16x16x32_bf16,
//          activations bf16 [rows][128] per chunk in LDS.
//   W4A4:  codes and E8M0 scales straight into v_mfma_scale_f32_16x16x128_f8f6f4,
//          activations MXFP4 ([rows][64 B] codes + [rows][4] scales) in LDS.
// Operand layout as in the streaming kernels: lane l supplies row / column
// l % 16 and K group g = l / 16; its 16 bytes are K-elements [32 g, 32 g + 32)
// of the chunk.
#include "common.h"
#include "kernels.h"

namespace {

constexpr uint32_t kOOR = 0x80000000u;   // out-of-range buffer offset: loads return 0

struct TileT {
  int expert, row0, rows;
};

// Logical block index: the blocks an XCD receives (b = x, x+8, x+16, ...)
// take consecutive logical indices.  The grid is a multiple of 8.
__device__ __forceinline__ int xcd_logical(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

// LDS bytes of one activation row of one chunk (+16 bytes of padding so that
// 16 consecutive rows fall in different banks).
template <bool kFP4A>
constexpr int lds_row_bytes() {
  return kFP4A ? 64 + 16 : 256 + 16;
}

template <int BM, bool kFP4A>
constexpr int lds_buf_bytes() {
  return BM * lds_row_bytes<kFP4A>() + (kFP4A ? BM * 4 : 0);
}

// One wave's GEMM over the tile: acc[mt][st] for 16-row subtile mt and
// 16-row weight strip st.  `rows_act` are the activation rows staged per
// chunk; `fill` gathers chunk c into an LDS buffer.
template <int BM, bool kFP4A>
struct TiledGemm {
  static constexpr int MT = BM / 16;
  static constexpr int RB = lds_row_bytes<kFP4A>();
  static constexpr int NQ = kFP4A ? (BM * 5 + 255) / 256 : BM / 16;   // 16-byte pieces per thread

  // weights
  rsrc_t w, ws;
  uint32_t wo[4], so[4];
  // activations: per thread, NQ pieces of the chunk (offset of the piece in
  // the source row per chunk, or kOOR), and where each lands in LDS
  rsrc_t a, as;
  uint32_t src[NQ];
  uint32_t dst[NQ];
  bool is_scale[NQ];

  __device__ __forceinline__ void load_w(int c, u32x4_t (&q)[4], uint32_t (&s)[4]) const {
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      q[st] = bload16(w, wo[st], 64 * c);
      s[st] = bload1(ws, so[st], 4 * c);
    }
  }

  __device__ __forceinline__ void load_x(int c, u32x4_t (&v)[NQ]) const {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if constexpr (kFP4A) {
        // codes: 64 B per row per chunk; scales: 4 B per row per chunk (one dword)
        if (is_scale[q]) {
          v[q] = (u32x4_t){(uint32_t)__builtin_amdgcn_raw_buffer_load_b32(as, (int)src[q], 4 * c, 0),
                           0u, 0u, 0u};
        } else {
          v[q] = bload16(a, src[q], 64 * c);
        }
      } else {
        v[q] = bload16(a, src[q], 256 * c);
      }
    }
  }

  __device__ __forceinline__ void store_x(uint8_t* buf, const u32x4_t (&v)[NQ]) const {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      if (dst[q] == 0xFFFFFFFFu) continue;
      if (kFP4A && is_scale[q])
        *reinterpret_cast<uint32_t*>(buf + dst[q]) = v[q][0];
      else
        *reinterpret_cast<u32x4_t*>(buf + dst[q]) = v[q];
    }
  }

  __device__ __forceinline__ void compute(const uint8_t* buf, const u32x4_t (&q)[4],
                                          const uint32_t (&s)[4], int nl, int g,
                                          floatx4_t (&acc)[MT][4]) const {
    if constexpr (kFP4A) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * mt + nl;
        const u32x4_t av = *reinterpret_cast<const u32x4_t*>(buf + r * RB + 16 * g);
        const uint32_t sa = buf[BM * RB + r * 4 + g];
#pragma unroll
        for (int st = 0; st < 4; ++st)
          acc[mt][st] = mfma_fp4_16x16x128(av, sa, q[st], s[st], acc[mt][st]);
      }
    } else {
      float sc[4];
#pragma unroll
      for (int st = 0; st < 4; ++st) sc[st] = e8m0_to_f32(s[st]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bf16x8_t b[4];
#pragma unroll
        for (int st = 0; st < 4; ++st) b[st] = dequant8_bf16(q[st][j], sc[st]);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const int r = 16 * mt + nl;
          const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(buf + r * RB + 64 * g + 16 * j);
#pragma unroll
          for (int st = 0; st < 4; ++st) acc[mt][st] = mfma_bf16_16x16x32(av, b[st], acc[mt][st]);
        }
      }
    }
  }

  // The K loop: chunk c+1's weights and activations are loaded while chunk c
  // is computed; the activations go to the other LDS buffer after the MFMAs.
  __device__ __forceinline__ void run(uint8_t* lds, int nch, int nl, int g,
                                      floatx4_t (&acc)[MT][4]) const {
    constexpr int BUF = lds_buf_bytes<BM, kFP4A>();
    u32x4_t q[4], qn[4];
    uint32_t s[4], sn[4];
    u32x4_t v[NQ];
    load_x(0, v);
    load_w(0, q, s);
    store_x(lds, v);
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
      const bool more = c + 1 < nch;
      if (more) {
        load_w(c + 1, qn, sn);
        load_x(c + 1, v);
      }
      compute(lds + (c & 1) * BUF, q, s, nl, g, acc);
      if (more) store_x(lds + ((c + 1) & 1) * BUF, v);
      __syncthreads();
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        q[st] = qn[st];
        s[st] = sn[st];
      }
    }
  }
};

template <int BM>
__device__ __forceinline__ bool tile_of(const int32_t* tiles, const int32_t* num_tiles,
                                        const int32_t* offsets, int tile, TileT* ti) {
  if (tile >= *num_tiles) return false;
  ti->expert = tiles[2 * tile];
  ti->row0 = tiles[2 * tile + 1];
  ti->rows = min(BM, offsets[ti->expert + 1] - ti->row0);
  return true;
}

// Per-thread activation pieces of a chunk.  bf16: BM rows x 16 pieces of 16
// bytes; thread t takes rows t/16 + 16 q, piece t % 16.  MXFP4: BM rows x 4
// code pieces, then BM scale dwords; thread t takes items t + 256 q.
template <int BM, bool kFP4A>
__device__ __forceinline__ void plan_x(TiledGemm<BM, kFP4A>& G, const int32_t* sorted, int Kp,
                                       int T, const TileT& ti, bool gather, uint32_t row_bytes,
                                       uint32_t scale_bytes) {
  constexpr int RB = lds_row_bytes<kFP4A>();
  const int t = threadIdx.x;
#pragma unroll
  for (int q = 0; q < G.NQ; ++q) {
    int r, piece;
    bool sc = false;
    if (kFP4A) {
      const int item = t + 256 * q;
      if (item < BM * 4) {
        r = item >> 2;
        piece = item & 3;
      } else {
        r = item - BM * 4;
        piece = 0;
        sc = true;
      }
    } else {
      r = (t >> 4) + 16 * q;
      piece = t & 15;
    }
    G.is_scale[q] = sc;
    if (r >= BM) {
      G.src[q] = kOOR;
      G.dst[q] = 0xFFFFFFFFu;
      continue;
    }
    G.dst[q] = sc ? (uint32_t)(BM * RB + r * 4) : (uint32_t)(r * RB + 16 * piece);
    if (r >= ti.rows) {
      G.src[q] = kOOR;                     // padded row: zeros
      continue;
    }
    const uint32_t srow = gather ? min((unsigned)(sorted[ti.row0 + r] / Kp), (unsigned)(T - 1))
                                 : (uint32_t)(ti.row0 + r);
    G.src[q] = sc ? srow * scale_bytes : srow * row_bytes + 16 * piece;
  }
}

// gate/up + SwiGLU: weight rows gate [i0, i0 + 128) and up [I + i0, I + i0 + 128),
// i0 = 128 s; wave w owns i in [i0 + 32 w, i0 + 32 w + 32): strips gate lo/hi, up lo/hi.
template <int BM, bool kFP4A>
__global__ __launch_bounds__(256) void gate_up_tiled_kernel(
    const void* __restrict__ act, const uint8_t* __restrict__ act_scale,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s, int T, int H, int I, int Kp,
    int max_tiles, uint16_t* __restrict__ h) {
  __shared__ __align__(16) uint8_t lds[2 * lds_buf_bytes<BM, kFP4A>()];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int s = L / max_tiles;
  if (s >= I / 128) return;
  TileT ti;
  if (!tile_of<BM>(tiles, num_tiles, offsets, L % max_tiles, &ti)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t rb = H / 2, rs = H / 32;
  const size_t wbytes = (size_t)2 * I * rb, sbytes = (size_t)2 * I * rs;
  TiledGemm<BM, kFP4A> G;
  G.w = make_rsrc(w13 + ti.expert * wbytes, (uint32_t)wbytes);
  G.ws = make_rsrc(w13s + ti.expert * sbytes, (uint32_t)sbytes);
  const int i0 = s * 128 + wave * 32;
  const int rows4[4] = {i0 + nl, i0 + 16 + nl, I + i0 + nl, I + i0 + 16 + nl};
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    G.wo[st] = rows4[st] * rb + 16 * g;
    G.so[st] = rows4[st] * rs + g;
  }
  if (kFP4A) {
    G.a = make_rsrc(act, (uint32_t)((size_t)T * rb));
    G.as = make_rsrc(act_scale, (uint32_t)((size_t)T * rs));
  } else {
    G.a = make_rsrc(act, (uint32_t)((size_t)T * H * 2));
  }
  plan_x<BM, kFP4A>(G, sorted, Kp, T, ti, true, kFP4A ? rb : (uint32_t)H * 2, rs);

  floatx4_t acc[BM / 16][4];
#pragma unroll
  for (int mt = 0; mt < BM / 16; ++mt)
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[mt][st] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  G.run(lds, H / 128, nl, g, acc);

#pragma unroll
  for (int mt = 0; mt < BM / 16; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * g + r;
      if (m < ti.rows) {
        uint16_t* hr = h + (size_t)(ti.row0 + m) * I;
        hr[i0 + nl] = f32_to_bf16_rne(swiglu(acc[mt][0][r], acc[mt][2][r]));
        hr[i0 + 16 + nl] = f32_to_bf16_rne(swiglu(acc[mt][1][r], acc[mt][3][r]));
      }
    }
}

// down: weight rows j in [256 s, 256 s + 256); wave w owns [256 s + 64 w, +64).
template <int BM, bool kFP4A>
__global__ __launch_bounds__(256) void down_tiled_kernel(
    const void* __restrict__ hin, const uint8_t* __restrict__ hscale,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2s, int A, int H, int I, int max_tiles, float* __restrict__ y) {
  __shared__ __align__(16) uint8_t lds[2 * lds_buf_bytes<BM, kFP4A>()];
  const int L = xcd_logical(blockIdx.x, gridDim.x);
  const int s = L / max_tiles;
  if (s >= H / 256) return;
  TileT ti;
  if (!tile_of<BM>(tiles, num_tiles, offsets, L % max_tiles, &ti)) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  const uint32_t rb = I / 2, rs = I / 32;
  const size_t wbytes = (size_t)H * rb, sbytes = (size_t)H * rs;
  TiledGemm<BM, kFP4A> G;
  G.w = make_rsrc(w2 + ti.expert * wbytes, (uint32_t)wbytes);
  G.ws = make_rsrc(w2s + ti.expert * sbytes, (uint32_t)sbytes);
  const int j0 = s * 256 + wave * 64;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    G.wo[st] = (j0 + 16 * st + nl) * rb + 16 * g;
    G.so[st] = (j0 + 16 * st + nl) * rs + g;
  }
  if (kFP4A) {
    G.a = make_rsrc(hin, (uint32_t)((size_t)A * rb));
    G.as = make_rsrc(hscale, (uint32_t)((size_t)A * rs));
  } else {
    G.a = make_rsrc(hin, (uint32_t)((size_t)A * I * 2));
  }
  plan_x<BM, kFP4A>(G, nullptr, 1, A, ti, false, kFP4A ? rb : (uint32_t)I * 2, rs);

  floatx4_t acc[BM / 16][4];
#pragma unroll
  for (int mt = 0; mt < BM / 16; ++mt)
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[mt][st] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  G.run(lds, I / 128, nl, g, acc);

#pragma unroll
  for (int mt = 0; mt < BM / 16; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = 16 * mt + 4 * g + r;
      if (m < ti.rows) {
        float* yr = y + (size_t)(ti.row0 + m) * H;
#pragma unroll
        for (int st = 0; st < 4; ++st) yr[j0 + 16 * st + nl] = acc[mt][st][r];
      }
    }
}

template <int BM, bool kFP4A>
hipError_t launch_gate_up_bm(const void* act, const uint8_t* act_scale, const int32_t* sorted,
                             const int32_t* offsets, const int32_t* tiles,
                             const int32_t* num_tiles, int max_tiles, const uint8_t* w13,
                             const uint8_t* w13s, int T, int H, int I, int Kp, uint16_t* h,
                             hipStream_t stream) {
  const long n = (long)max_tiles * (I / 128);
  const unsigned grid = (unsigned)((n + 7) / 8 * 8);
  hipLaunchKernelGGL((gate_up_tiled_kernel<BM, kFP4A>), dim3(grid), dim3(256), 0, stream, act,
                     act_scale, sorted, offsets, tiles, num_tiles, w13, w13s, T, H, I, Kp,
                     max_tiles, h);
  return hipGetLastError();
}

template <int BM, bool kFP4A>
hipError_t launch_down_bm(const void* h, const uint8_t* h_scale, const int32_t* offsets,
                          const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                          const uint8_t* w2, const uint8_t* w2s, int A, int H, int I, float* y,
                          hipStream_t stream) {
  const long n = (long)max_tiles * (H / 256);
  const unsigned grid = (unsigned)((n + 7) / 8 * 8);
  hipLaunchKernelGGL((down_tiled_kernel<BM, kFP4A>), dim3(grid), dim3(256), 0, stream, h,
                     h_scale, offsets, tiles, num_tiles, w2, w2s, A, H, I, max_tiles, y);
  return hipGetLastError();
}

}  // namespace

bool expert_gemm_tiled_supported(int tile_m, int H, int I) {
  return (tile_m == 64 || tile_m == 128) && H % 256 == 0 && I % 128 == 0;
}

hipError_t launch_gate_up_tiled(int tile_m, int act_fmt, const void* act, const uint8_t* act_scale,
                                const int32_t* sorted, const int32_t* offsets,
                                const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                                const uint8_t* w13, const uint8_t* w13s, int T, int H, int I,
                                int Kp, uint16_t* h, hipStream_t stream) {
  if (tile_m == 128)
    return act_fmt ? launch_gate_up_bm<128, true>(act, act_scale, sorted, offsets, tiles,
                                                   num_tiles, max_tiles, w13, w13s, T, H, I, Kp,
                                                   h, stream)
                   : launch_gate_up_bm<128, false>(act, act_scale, sorted, offsets, tiles,
                                                    num_tiles, max_tiles, w13, w13s, T, H, I, Kp,
                                                    h, stream);
  return act_fmt ? launch_gate_up_bm<64, true>(act, act_scale, sorted, offsets, tiles, num_tiles,
                                                max_tiles, w13, w13s, T, H, I, Kp, h, stream)
                 : launch_gate_up_bm<64, false>(act, act_scale, sorted, offsets, tiles, num_tiles,
                                                 max_tiles, w13, w13s, T, H, I, Kp, h, stream);
}

hipError_t launch_down_tiled(int tile_m, int act_fmt, const void* h, const uint8_t* h_scale,
                             const int32_t* offsets, const int32_t* tiles,
                             const int32_t* num_tiles, int max_tiles, const uint8_t* w2,
                             const uint8_t* w2s, int A, int H, int I, float* y,
                             hipStream_t stream) {
  if (tile_m == 128)
    return act_fmt ? launch_down_bm<128, true>(h, h_scale, offsets, tiles, num_tiles, max_tiles,
                                                w2, w2s, A, H, I, y, stream)
                   : launch_down_bm<128, false>(h, h_scale, offsets, tiles, num_tiles, max_tiles,
                                                 w2, w2s, A, H, I, y, stream);
  return act_fmt ? launch_down_bm<64, true>(h, h_scale, offsets, tiles, num_tiles, max_tiles, w2,
                                             w2s, A, H, I, y, stream)
                 : launch_down_bm<64, false>(h, h_scale, offsets, tiles, num_tiles, max_tiles, w2,
                                              w2s, A, H, I, y, stream);
}
