// Grouped expert GEMMs over MXFP4 weights, one workgroup per (32-row tile,
// N-slice).  The tiles come from the align step's tile table; a tile holds up
// to 32 consecutive rows of one expert's group (VibeSys "Qwen3.5-397B on 4x
// MI300A" post, section "Prefill, cache and speculation": 32-row tiles).
//
// W4A16 (bf16 activations): the fused HIP MoE kernel dequantises MXFP4 in
// registers (same post, section "Baseline"); here each lane loads 16 bytes
// (32 codes, one scale block) of a weight row (from the native code order of
// common.h: a strip's chunk is one contiguous KiB), expands them to bf16 with the
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
// the sorted row order.  down: a wave owns 32 output columns j (one
// exponent group); y is stored in the staged fp16 format of common.h in the
// sorted row order.
#include "common.h"
#include "kernels.h"

MOE_DEBUG_FLAGS(debug_flags_expert_gemm)

namespace {

// Tuning constants: the widest pipeline phase (in 128-element chunks) and
// the waves per SIMD the register allocation of the GEMM kernels aims for.
#ifndef MOE_GEMM_PH_MAX
#define MOE_GEMM_PH_MAX 2
#endif
#ifndef MOE_GEMM_WAVES_PER_EU
#define MOE_GEMM_WAVES_PER_EU 3
#endif

constexpr int kTileM = 32;        // rows per workgroup (= the tile table's tile_m)

struct TileInfo {
  int expert, row0, rows;
  bool single;    // the expert's only tile: nothing re-reads its weights
};

// Workgroups take the tile table from its end: block b works on tile
// num_tiles - 1 - b / nsl (blocks past the live tiles exit at once).  The
// shared expert's tiles are last in the table and are the longest-running
// ones (T rows, several 16-row subtiles, where a routed expert of a decode
// batch has 1-3 rows); started first they no longer form the kernel's tail.
__device__ __forceinline__ bool load_tile(const int32_t* tiles, const int32_t* num_tiles,
                                          const int32_t* offsets, int block, TileInfo* ti) {
  const int tile = *num_tiles - 1 - block;
  if (tile < 0) return false;
  ti->expert = tiles[2 * tile];
  ti->row0 = tiles[2 * tile + 1];
  ti->rows = min(kTileM, offsets[ti->expert + 1] - ti->row0);
  ti->single = offsets[ti->expert + 1] - offsets[ti->expert] <= kTileM;
  return true;
}

// A wave computes two 16-row strips of weights against the activation rows of
// its tile over the whole K, in phases of PH chunks of 128 K-elements.  In
// chunk c, lane (row l%16, group g = l/16) holds bytes [64 c + 16 g, +16) of
// its weight row (32 codes) and the scale byte of block 4 c + g.
//
// Software pipeline: phases alternate between two register sets; the loads
// of phase p+1 (weights and activations together) are issued before phase p
// is computed, so the wave always has one phase in flight and waits only for
// the older one (vmcnt counts in issue order).
//
// Operands are read with buffer loads: one resource per tensor (wave-uniform)
// and per-lane byte offsets, so a chunk's position is a scalar offset.  The
// weight scales of the workgroup's rows are first copied to LDS with 16-byte
// loads (one byte per lane per chunk would cost a load instruction per 1 KiB
// of weights); lanes of padded tile rows get an out-of-range activation
// offset, so their loads return zeros without touching memory.
constexpr uint32_t kOutOfRange = 0x80000000u;

struct Operands {
  rsrc_t w, a, as;         // weights, activations, activation scales (MXFP4)
  uint32_t wo[2];          // lane offsets in its two weight strips (native code order)
  uint32_t lso[2];         // LDS offsets of its two weight rows' scales (+g)
  uint32_t ao, aso;        // lane offset of its activation row (+32 g elements or +16 g bytes)
  const uint8_t* lds;      // the workgroup's weight scales
  const uint8_t* ldx;      // bf16 activation rows staged in LDS (small tiles), lane row + 64 g
  bool xvalid;             // the lane's activation row exists (padded rows read zeros)
  bool stream;             // weights read once (the expert's only tile): non-temporal loads
};

template <int PH, bool kFP4A, bool XL, bool kW8>
struct Phase {
  // weight bytes per lane per chunk: 16 (32 E2M1 codes) or 32 (32 E4M3 codes)
  static constexpr int NQ = kW8 ? 2 : 1;
  u32x4_t q[2][PH * NQ];
  u32x4_t a[PH][(kFP4A || XL) ? 1 : 4];
  uint32_t as[PH];

  __device__ __forceinline__ void load(const Operands& o, int c0) {
#pragma unroll
    for (int j = 0; j < PH; ++j)
#pragma unroll
      for (int si = 0; si < 2; ++si)
#pragma unroll
        for (int hq = 0; hq < NQ; ++hq)
          q[si][NQ * j + hq] = o.stream ? bload16_nt(o.w, o.wo[si], wnat_chunk(c0 + j, NQ, hq))
                                        : bload16(o.w, o.wo[si], wnat_chunk(c0 + j, NQ, hq));
#pragma unroll
    for (int j = 0; j < PH; ++j) {
      if constexpr (kFP4A) {
        a[j][0] = bload16(o.a, o.ao, 64 * (c0 + j));
        as[j] = bload1(o.as, o.aso, 4 * (c0 + j));
      } else if constexpr (!XL) {
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) a[j][qq] = bload16(o.a, o.ao + 16 * qq, 256 * (c0 + j));
      }
    }
  }

  __device__ __forceinline__ void compute(const Operands& o, int c0, floatx4_t (&acc)[2]) const {
#pragma unroll
    for (int j = 0; j < PH; ++j) {
      uint32_t sw[2];
#pragma unroll
      for (int si = 0; si < 2; ++si) sw[si] = o.lds[o.lso[si] + 4 * (c0 + j)];
      if constexpr (kFP4A) {
#pragma unroll
        for (int si = 0; si < 2; ++si)
          acc[si] = mfma_fp4_16x16x128(a[j][0], as[j], q[si][j], sw[si], acc[si]);
      } else {
        u32x4_t x[4];
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) {
          if constexpr (XL) {
            const u32x4_t v = *reinterpret_cast<const u32x4_t*>(o.ldx + 256 * (c0 + j) + 16 * qq);
            x[qq] = o.xvalid ? v : (u32x4_t){0u, 0u, 0u, 0u};
          } else {
            x[qq] = a[j][qq];
          }
        }
#pragma unroll
        for (int si = 0; si < 2; ++si) {
          const float sc = e8m0_to_f32(sw[si]);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) {
            bf16x8_t wv;
            if constexpr (kW8) {
              const u32x4_t& d = q[si][2 * j + (qq >> 1)];
              wv = dequant8_bf16_fp8(d[2 * (qq & 1)], d[2 * (qq & 1) + 1], sc);
            } else {
              wv = dequant8_bf16(q[si][j][qq], sc);
            }
            acc[si] = mfma_bf16_16x16x32(__builtin_bit_cast(bf16x8_t, x[qq]), wv, acc[si]);
          }
        }
      }
    }
  }
};

template <int PH, bool kFP4A, bool XL, bool kW8>
__device__ __forceinline__ void wave_gemm(const Operands& o, int nph, floatx4_t (&acc)[2]) {
  Phase<PH, kFP4A, XL, kW8> A, B;
  int p = 0;
  if (nph & 1) {                 // an odd phase first, unpipelined
    A.load(o, 0);
    A.compute(o, 0, acc);
    p = 1;
  }
  if (p < nph) {
    A.load(o, PH * p);
    B.load(o, PH * (p + 1));
    for (; p + 2 < nph; p += 2) {
      A.compute(o, PH * p, acc);
      A.load(o, PH * (p + 2));
      B.compute(o, PH * (p + 1), acc);
      B.load(o, PH * (p + 3));
    }
    A.compute(o, PH * p, acc);
    B.compute(o, PH * (p + 1), acc);
  }
}

// Tiles of at most kXR rows take their bf16 activation rows from LDS (one
// cooperative copy per workgroup instead of 4 loads per lane per chunk).
constexpr int kXR = 4;

// Copy `bytes` (a multiple of 256) from byte off of resource r into LDS with
// direct-to-LDS loads (no registers): 1 KiB per wave instruction when the
// size allows, else 256 bytes; wave w takes every fourth piece.  src maps a
// byte of the copy to its byte in the resource.
template <class Src>
__device__ __forceinline__ void copy_to_lds(rsrc_t r, uint32_t bytes, uint8_t* lds, Src src) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (bytes % 1024 == 0) {
    for (uint32_t p = wave * 1024; p < bytes; p += 4 * 1024)
      load_to_lds16(r, src(p + 16 * lane), 0, lds + p);
  } else {
    for (uint32_t p = wave * 256; p < bytes; p += 4 * 256)
      load_to_lds4(r, src(p + 4 * lane), 0, lds + p);
  }
}

// The common decode tile (bf16 activations, at most kXR rows: one 16-row
// subtile, activations from LDS), with a shorter prologue: the weight scales
// and the activation rows go straight into LDS, the first two phases' weight
// loads go out right after, and the workgroup's barrier waits for the LDS
// copies only (loads complete in issue order), so the scales' and the
// weights' fetches overlap instead of following one another.  copies()
// issues the LDS copies; returns acc for rows 4 g + r of the subtile.
template <int PH, bool kW8, class Copies>
__device__ __forceinline__ void small_tile_gemm(Operands& o, int nph, Copies&& copies,
                                                floatx4_t (&acc)[2]) {
  using PA = Phase<PH, false, true, kW8>;
  constexpr int kOps = PH * 2 * PA::NQ;                  // one phase's weight loads
  copies();
  __builtin_amdgcn_sched_barrier(0);
  PA A, B;
  A.load(o, 0);
  if (nph > 1) {
    B.load(o, PH);
    wait_vmcnt<2 * kOps>();
  } else {
    wait_vmcnt<kOps>();
  }
  stage_barrier();
  int p = 0;
  for (; p + 3 < nph; p += 2) {
    A.compute(o, PH * p, acc);
    A.load(o, PH * (p + 2));
    B.compute(o, PH * (p + 1), acc);
    B.load(o, PH * (p + 3));
  }
  if (nph - p == 3) {
    A.compute(o, PH * p, acc);
    A.load(o, PH * (p + 2));
    B.compute(o, PH * (p + 1), acc);
    A.compute(o, PH * (p + 2), acc);
  } else if (nph - p == 2) {
    A.compute(o, PH * p, acc);
    B.compute(o, PH * (p + 1), acc);
  } else {
    A.compute(o, PH * p, acc);
  }
}

// Copy `bytes` (a multiple of 16) of weight scales starting at byte `off` of
// resource r into LDS, 16 bytes per lane per step.
__device__ __forceinline__ void scales_to_lds(rsrc_t r, uint32_t off, uint32_t bytes,
                                              uint8_t* lds) {
  for (uint32_t v = threadIdx.x * 16; v < bytes; v += blockDim.x * 16)
    *reinterpret_cast<u32x4_t*>(lds + v) = bload16(r, off + v, 0);
}

// gate_up: a workgroup (4 waves) owns one tile and 64 intermediate columns;
// wave w owns strip w of them (16 columns, every other run of four in its
// strip pair's 32, in the native order): 16 gate rows and 16 up rows of W13
// over the whole K = H.  The tile's 16-row subtiles run one after
// the other (the second re-reads the weights, from L2): decode tiles mostly
// have 1-3 rows and this keeps a single subtile's registers live.  SwiGLU in
// registers, bf16 h stored in sorted row order.
//
// The shared expert's tiles (T rows, last in the tile table) are the only
// full ones in a decode batch, and with two subtiles each in turn their
// workgroups run twice as long as the rest: where the whole grid fits on the
// GPU at once (one GPU's tensor-parallel share, I = 128) they alone set the
// kernel's length.  So the first nx * nsl blocks take subtile 1 of the last
// nx tiles (when such a tile has more than 16 rows) and the workgroups of
// those tiles run subtile 0 only: the two halves run side by side.
template <int PH, bool kFP4A, bool kW8>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(MOE_GEMM_WAVES_PER_EU))) void gate_up_kernel(
    const void* __restrict__ act, const uint8_t* __restrict__ act_scale,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s, int T, int H, int I, int Kp,
    int nsl, int nx, uint16_t* __restrict__ h) {
  TileInfo ti;
  // blocks [0, nx * nsl): subtile 1 of tile num_tiles - 1 - r; then every tile
  const int bt = (int)(blockIdx.x / nsl);
  const bool second = bt < nx;
  const int r = second ? bt : bt - nx;
  if (!load_tile(tiles, num_tiles, offsets, r, &ti)) return;
  const bool split = r < nx && ti.rows > 16;
  if (second && !split) return;
  // (debug builds: a tile whose rows leave [0, A) stores nothing)
  if (!MOE_DOK(ti.row0 >= 0 && ti.rows > 0 && (int64_t)ti.row0 + ti.rows <= (int64_t)T * Kp, kDbgTiles))
    return;
  const int s = blockIdx.x % nsl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  // the wave's strip of gate rows (and the matching up strip) and the
  // intermediate column its lane's slot holds in the native order
  const int st = s * 4 + wave;
  const int i = s * 64 + (wave & ~1) * 16 + wnat_row(wave & 1, nl);
  const uint32_t rb = H / 2, rs = H / 32;
  const uint32_t wrb = kW8 ? H : H / 2;                    // weight code bytes per row
  const size_t wbytes = (size_t)2 * I * wrb, sbytes = (size_t)2 * I * rs;
  extern __shared__ uint8_t lds_scales[];                  // [2][64 rows][rs]: gate, up
  Operands o;
  o.lds = lds_scales;
  o.w = make_rsrc(w13 + ti.expert * wbytes, (uint32_t)wbytes);
  o.stream = ti.single && !split;   // (the halves of a split tile share the lines in L2)
  constexpr int NQ = Phase<PH, kFP4A, false, kW8>::NQ;
  o.wo[0] = wnat_lane(st, H, NQ, lane);
  o.wo[1] = wnat_lane(I / 16 + st, H, NQ, lane);
  o.lso[0] = (i - s * 64) * rs + g;
  o.lso[1] = (64 + i - s * 64) * rs + g;
  if (kFP4A) {
    o.a = make_rsrc(act, (uint32_t)((size_t)T * rb));
    o.as = make_rsrc(act_scale, (uint32_t)((size_t)T * rs));
  } else {
    o.a = make_rsrc(act, (uint32_t)((size_t)T * H * 2));
  }
  if (!kFP4A && ti.rows <= kXR) {
    // (the common decode tile; its tokens are wave-uniform loads)
    uint8_t* lds_x = lds_scales + 128 * rs;
    uint32_t tk[kXR];
#pragma unroll
    for (int r = 0; r < kXR; ++r)
      tk[r] = r < ti.rows ? min((unsigned)(sorted[ti.row0 + r] / Kp), (unsigned)(T - 1)) : 0u;
    const uint32_t rowb = (uint32_t)H * 2;
    const rsrc_t rsc = make_rsrc(w13s + ti.expert * sbytes, (uint32_t)sbytes);
    o.ldx = lds_x + min(nl, kXR - 1) * H * 2 + 64 * g;
    o.xvalid = nl < ti.rows;
    floatx4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    small_tile_gemm<PH, kW8>(o, H / 128 / PH, [&] {
      const uint32_t gs = (uint32_t)(s * 64) * rs, us = (uint32_t)(I + s * 64) * rs;
      copy_to_lds(rsc, 64 * rs, lds_scales, [&](uint32_t b) { return gs + b; });
      copy_to_lds(rsc, 64 * rs, lds_scales + 64 * rs, [&](uint32_t b) { return us + b; });
      copy_to_lds(o.a, (uint32_t)ti.rows * rowb, lds_x, [&](uint32_t b) {
        const uint32_t r = b / rowb;
        const uint32_t t = r == 0 ? tk[0] : r == 1 ? tk[1] : r == 2 ? tk[2] : tk[3];
        return t * rowb + (b - r * rowb);
      });
    }, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 4 * g + r;
      if (mm < ti.rows)
        h[(size_t)(ti.row0 + mm) * I + i] = f32_to_bf16_rne(swiglu(acc[0][r], acc[1][r]));
    }
    return;
  }
  {
    const rsrc_t rsc = make_rsrc(w13s + ti.expert * sbytes, (uint32_t)sbytes);
    scales_to_lds(rsc, (uint32_t)(s * 64) * rs, 64 * rs, lds_scales);
    scales_to_lds(rsc, (uint32_t)(I + s * 64) * rs, 64 * rs, lds_scales + 64 * rs);
  }
  uint8_t* lds_x = lds_scales + 128 * rs;                  // [kXR rows][H] bf16 (small tiles)
  const bool xl = !kFP4A && ti.rows <= kXR;
  if (xl) {
    const uint32_t rowb = (uint32_t)H * 2;
    for (uint32_t v = threadIdx.x * 16; v < ti.rows * rowb; v += blockDim.x * 16) {
      const uint32_t r = v / rowb;
      const uint32_t tok = min((unsigned)(sorted[ti.row0 + r] / Kp), (unsigned)(T - 1));
      *reinterpret_cast<u32x4_t*>(lds_x + v) = bload16(o.a, tok * rowb + (v - r * rowb), 0);
    }
  }
  __syncthreads();
  const int mtn = (ti.rows + 15) / 16;
  for (int mt = second ? 1 : 0; mt < (split && !second ? 1 : mtn); ++mt) {
    const int m = 16 * mt + nl;
    floatx4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (xl) {
      o.ldx = lds_x + min(m, kXR - 1) * H * 2 + 64 * g;
      o.xvalid = m < ti.rows;
      wave_gemm<PH, kFP4A, true, kW8>(o, H / 128 / PH, acc);
    } else {
      const uint32_t tok = min((unsigned)(sorted[ti.row0 + min(m, ti.rows - 1)] / Kp),
                               (unsigned)(T - 1));
      o.ao = m >= ti.rows ? kOutOfRange : (kFP4A ? tok * rb + 16 * g : tok * H * 2 + 64 * g);
      o.aso = m >= ti.rows ? kOutOfRange : tok * rs + g;
      wave_gemm<PH, kFP4A, false, kW8>(o, H / 128 / PH, acc);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 16 * mt + 4 * g + r;
      if (mm < ti.rows)
        h[(size_t)(ti.row0 + mm) * I + i] = f32_to_bf16_rne(swiglu(acc[0][r], acc[1][r]));
    }
  }
}

// down: a workgroup (4 waves) owns one tile and 128 output columns j; wave w
// owns [32 w, 32 w + 32) of them (a strip pair of W2) over K = I.  y is
// stored in the staged fp16 format in sorted row order.
template <int PH, bool kFP4A, bool kW8>
__global__ __launch_bounds__(256)
__attribute__((amdgpu_waves_per_eu(MOE_GEMM_WAVES_PER_EU))) void down_kernel(
    const void* __restrict__ hin, const uint8_t* __restrict__ hscale,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2s, int A, int H, int I, int nsl, uint16_t* __restrict__ y,
    uint8_t* __restrict__ ye) {
  TileInfo ti;
  if (!load_tile(tiles, num_tiles, offsets, (int)(blockIdx.x / nsl), &ti)) return;
  // (debug builds: a tile whose rows leave [0, A) stores nothing)
  if (!MOE_DOK(ti.row0 >= 0 && ti.rows > 0 && (int64_t)ti.row0 + ti.rows <= (int64_t)A, kDbgTiles))
    return;
  const int s = blockIdx.x % nsl;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nl = lane & 15, g = lane >> 4;
  // the wave's strip pair 2 st, 2 st + 1 (columns jb .. jb + 31) and the
  // columns its lane's slots hold in the native order
  const int st = s * 4 + wave, jb = 32 * st;
  const int jc[2] = {jb + wnat_row(0, nl), jb + wnat_row(1, nl)};
  const uint32_t rb = I / 2, rs = I / 32;
  const uint32_t wrb = kW8 ? I : I / 2;                    // weight code bytes per row
  const size_t wbytes = (size_t)H * wrb, sbytes = (size_t)H * rs;
  extern __shared__ uint8_t lds_scales[];                  // [128 rows][rs]
  Operands o;
  o.lds = lds_scales;
  o.w = make_rsrc(w2 + ti.expert * wbytes, (uint32_t)wbytes);
  o.stream = ti.single;
  constexpr int NQ = Phase<PH, kFP4A, false, kW8>::NQ;
  o.wo[0] = wnat_lane(2 * st, I, NQ, lane);
  o.wo[1] = wnat_lane(2 * st + 1, I, NQ, lane);
  o.lso[0] = (jc[0] - s * 128) * rs + g;
  o.lso[1] = (jc[1] - s * 128) * rs + g;
  if (kFP4A) {
    o.a = make_rsrc(hin, (uint32_t)((size_t)A * rb));
    o.as = make_rsrc(hscale, (uint32_t)((size_t)A * rs));
  } else {
    o.a = make_rsrc(hin, (uint32_t)((size_t)A * I * 2));
  }
  if (!kFP4A && ti.rows <= kXR) {
    // (the common decode tile: see small_tile_gemm)
    uint8_t* lds_x = lds_scales + 128 * rs;
    const rsrc_t rsc = make_rsrc(w2s + ti.expert * sbytes, (uint32_t)sbytes);
    o.ldx = lds_x + min(nl, kXR - 1) * I * 2 + 64 * g;
    o.xvalid = nl < ti.rows;
    floatx4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    small_tile_gemm<PH, kW8>(o, I / 128 / PH, [&] {
      const uint32_t so = (uint32_t)(s * 128) * rs, xo = (uint32_t)ti.row0 * I * 2;
      copy_to_lds(rsc, 128 * rs, lds_scales, [&](uint32_t b) { return so + b; });
      copy_to_lds(o.a, (uint32_t)ti.rows * I * 2, lds_x, [&](uint32_t b) { return xo + b; });
    }, acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 4 * g + r;
      const int e = y_exponent_of_field(
          row16_max_halves(max_halves(pack_exponents(acc[0][r], 0.f), pack_exponents(acc[1][r], 0.f))) &
          0xFFFFu);
      if (mm < ti.rows) {
        const size_t row = (size_t)(ti.row0 + mm);
        uint16_t* yr = y + row * H;
        yr[jc[0]] = y_encode(acc[0][r], e);
        yr[jc[1]] = y_encode(acc[1][r], e);
        if (nl == 0) ye[row * (H / kYGroup) + jb / kYGroup] = (uint8_t)(e + 127);
      }
    }
    return;
  }
  scales_to_lds(make_rsrc(w2s + ti.expert * sbytes, (uint32_t)sbytes), (uint32_t)(s * 128) * rs,
                128 * rs, lds_scales);
  uint8_t* lds_x = lds_scales + 128 * rs;                  // [kXR rows][I] bf16 (small tiles)
  const bool xl = !kFP4A && ti.rows <= kXR;
  if (xl) {
    const uint32_t rowb = (uint32_t)I * 2;
    for (uint32_t v = threadIdx.x * 16; v < ti.rows * rowb; v += blockDim.x * 16)
      *reinterpret_cast<u32x4_t*>(lds_x + v) = bload16(o.a, ti.row0 * rowb + v, 0);
  }
  __syncthreads();
  const int mtn = (ti.rows + 15) / 16;
  for (int mt = 0; mt < mtn; ++mt) {
    const int m = 16 * mt + nl;
    floatx4_t acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    if (xl) {
      o.ldx = lds_x + min(m, kXR - 1) * I * 2 + 64 * g;
      o.xvalid = m < ti.rows;
      wave_gemm<PH, kFP4A, true, kW8>(o, I / 128 / PH, acc);
    } else {
      const uint32_t row = ti.row0 + m;
      o.ao = m >= ti.rows ? kOutOfRange : (kFP4A ? row * rb + 16 * g : row * I * 2 + 64 * g);
      o.aso = m >= ti.rows ? kOutOfRange : row * rs + g;
      wave_gemm<PH, kFP4A, false, kW8>(o, I / 128 / PH, acc);
    }
    // y in the staged fp16 format: the wave's 32 columns of a row are one
    // group, held by one 16-lane row of the wave
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int mm = 16 * mt + 4 * g + r;
      const int e = y_exponent_of_field(
          row16_max_halves(max_halves(pack_exponents(acc[0][r], 0.f), pack_exponents(acc[1][r], 0.f))) &
          0xFFFFu);
      if (mm < ti.rows) {
        const size_t row = (size_t)(ti.row0 + mm);
        uint16_t* yr = y + row * H;
        yr[jc[0]] = y_encode(acc[0][r], e);
        yr[jc[1]] = y_encode(acc[1][r], e);
        if (nl == 0) ye[row * (H / kYGroup) + jb / kYGroup] = (uint8_t)(e + 127);
      }
    }
  }
}

// -------------------------------------------------------------- combine ----

constexpr int kPrefetchBlocks = 256;

// Workgroups past the combine's own read pf's byte ranges in 4 KiB pages
// (page j of a range goes to prefetch block j % kPrefetchBlocks) and discard
// the data: the reads leave the lines in L2 and the memory-side cache for the
// next kernels.  Buffer loads, so nothing outside a range is touched.
__device__ __forceinline__ void prefetch_ranges(const Prefetch& pf, int b) {
  uint32_t acc = 0;
  for (int r = 0; r < pf.n; ++r) {
    const rsrc_t rs = make_rsrc(pf.p[r], pf.bytes[r]);
    const uint32_t pages = (pf.bytes[r] + 4095) / 4096;
    for (uint32_t j = b; j < pages; j += kPrefetchBlocks) {
      const u32x4_t v = bload16(rs, j * 4096 + threadIdx.x * 16, 0);
      acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
  }
  asm volatile("" ::"v"(acc));                 // keeps the loads; no memory effect
}

// out[t, j] = bf16( sum_k w[t, k] * y[inv[t*K' + k], j] ), slots in order,
// fp32 sums of the staged fp16 y (times its group's power of two); 8 outputs
// per thread (a 16-byte load of each slot's y and its group exponent byte, a
// 16-byte store).  The eight slots' row indices are read first, then their y
// rows, so the loads are independent (waiting for each slot's index before
// its y load cost 20% on the skewed batch).
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ y,
                                                      const uint8_t* __restrict__ ye,
                                                      const float* __restrict__ w,
                                                      const int32_t* __restrict__ inv, int H,
                                                      int Kp, int nbx, uint16_t* __restrict__ out,
                                                      int T, Prefetch pf) {
  if ((int)blockIdx.x >= nbx * T) {
    prefetch_ranges(pf, (int)blockIdx.x - nbx * T);
    return;
  }
  const int t = blockIdx.x / nbx;
  const int j = ((blockIdx.x % nbx) * 256 + threadIdx.x) * 8;
  if (j >= H) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // Eight slots at a time: their row indices and weights, then their y
  // rows (independent loads, non-temporal: each y row is read once), then
  // the sums in slot order.
  for (int k0 = 0; k0 < Kp; k0 += 8) {
    int r[8];
    float wk[8];
    bool live[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool ok = k0 + i < Kp;
      r[i] = ok ? inv[(size_t)t * Kp + k0 + i] : 0;
      wk[i] = ok ? w[(size_t)t * Kp + k0 + i] : 0.f;
      live[i] = ok && MOE_DOK((unsigned)r[i] < (unsigned)(T * Kp), kDbgCombine);
    }
    u32x4_t v[8];
    int ex[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (live[i]) {
        v[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(y + (size_t)r[i] * H + j));
        ex[i] = (int)ye[(size_t)r[i] * (H / kYGroup) + j / kYGroup] - 127;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i)
      if (live[i])
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += wk[i] * y_decode((uint16_t)(v[i][q] & 0xFFFFu), ex[i]);
          acc[2 * q + 1] += wk[i] * y_decode((uint16_t)(v[i][q] >> 16), ex[i]);
        }
  }
  u32x4_t o;
#pragma unroll
  for (int q = 0; q < 4; ++q)
    o[q] = (uint32_t)f32_to_bf16_rne(acc[2 * q]) | ((uint32_t)f32_to_bf16_rne(acc[2 * q + 1]) << 16);
  *reinterpret_cast<u32x4_t*>(out + (size_t)t * H + j) = o;
}

}  // namespace

int expert_gemm_tile_m() { return kTileM; }

// Dynamic LDS of the 32-row kernels over a reduction of K: the weight scales
// of 128 rows, plus (bf16 activations) kXR activation rows.
size_t expert_gemm_lds_bytes(int K, int act_fmt) {
  return (size_t)128 * (K / 32) + (act_fmt == 0 ? (size_t)kXR * K * 2 : 0);
}

// Phase width (chunks of 128 K-elements per pipeline stage): 2 when the chunk
// count is even, else 1.  MXFP8 weights (32 bytes per lane per chunk) use 1,
// which keeps the same bytes in flight per phase as MXFP4 with 2.
int expert_gemm_phase(int nch) { return (MOE_GEMM_PH_MAX >= 2 && nch % 2 == 0) ? 2 : 1; }

namespace {
template <int PH, bool kFP4A, bool kW8>
struct GateUpLaunch {
  static hipError_t run(dim3 grid, hipStream_t stream, const void* act, const uint8_t* act_scale,
                        const int32_t* sorted, const int32_t* offsets, const int32_t* tiles,
                        const int32_t* num_tiles, const uint8_t* w13, const uint8_t* w13s, int T,
                        int H, int I, int Kp, int nsl, int nx, uint16_t* h) {
    const size_t lds = (size_t)128 * (H / 32) + (kFP4A ? 0 : (size_t)kXR * H * 2);
    hipLaunchKernelGGL((gate_up_kernel<PH, kFP4A, kW8>), grid, dim3(256), lds, stream,
                       act, act_scale,
                       sorted, offsets, tiles, num_tiles, w13, w13s, T, H, I, Kp, nsl, nx, h);
    return hipGetLastError();
  }
};

template <int PH, bool kFP4A, bool kW8>
struct DownLaunch {
  static hipError_t run(dim3 grid, hipStream_t stream, const void* hin, const uint8_t* hscale,
                        const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                        const uint8_t* w2, const uint8_t* w2s, int A, int H, int I, int nsl,
                        uint16_t* y) {
    const size_t lds = (size_t)128 * (I / 32) + (kFP4A ? 0 : (size_t)kXR * I * 2);
    uint8_t* ye = reinterpret_cast<uint8_t*>(y) + (size_t)A * H * 2;   // the group exponents
    hipLaunchKernelGGL((down_kernel<PH, kFP4A, kW8>), grid, dim3(256), lds, stream,
                       hin, hscale, offsets,
                       tiles, num_tiles, w2, w2s, A, H, I, nsl, y, ye);
    return hipGetLastError();
  }
};

// (activation format, weight format, phase width) -> kernel instance.  MXFP8
// weights come with bf16 activations only (checked by the caller).
template <template <int, bool, bool> class Launch, typename... Args>
hipError_t dispatch(int act_fmt, int wfmt, int nch, Args... args) {
  if (wfmt == 1) return Launch<1, false, true>::run(args...);
  const int ph = expert_gemm_phase(nch);
  if (act_fmt == 0)
    return ph == 2 ? Launch<2, false, false>::run(args...) : Launch<1, false, false>::run(args...);
  return ph == 2 ? Launch<2, true, false>::run(args...) : Launch<1, true, false>::run(args...);
}
}  // namespace

hipError_t launch_gate_up(int act_fmt, int wfmt, const void* act, const uint8_t* act_scale,
                          const int32_t* sorted, const int32_t* offsets, const int32_t* tiles,
                          const int32_t* num_tiles, int max_tiles, const uint8_t* w13,
                          const uint8_t* w13s, int T, int H, int I, int Kp, uint16_t* h,
                          hipStream_t stream) {
  const int nsl = I / 64;
  // the last tiles of a T-row group (the shared expert's) split in two
  const int nx = max_tiles < (T + kTileM - 1) / kTileM ? max_tiles : (T + kTileM - 1) / kTileM;
  dim3 grid((unsigned)((max_tiles + nx) * nsl));
  return dispatch<GateUpLaunch>(act_fmt, wfmt, H / 128, grid, stream, act, act_scale, sorted,
                                offsets, tiles, num_tiles, w13, w13s, T, H, I, Kp, nsl, nx, h);
}

hipError_t launch_down(int act_fmt, int wfmt, const void* h, const uint8_t* h_scale,
                       const int32_t* offsets, const int32_t* tiles, const int32_t* num_tiles,
                       int max_tiles, const uint8_t* w2, const uint8_t* w2s, int A, int H, int I,
                       uint16_t* y, hipStream_t stream) {
  const int nsl = H / 128;
  dim3 grid((unsigned)(max_tiles * nsl));
  return dispatch<DownLaunch>(act_fmt, wfmt, I / 128, grid, stream, h, h_scale, offsets, tiles,
                              num_tiles, w2, w2s, A, H, I, nsl, y);
}

hipError_t launch_combine(const uint16_t* y, const float* w, const int32_t* inv, int T, int H,
                          int Kp, uint16_t* out, hipStream_t stream, const Prefetch* pf) {
  const int nbx = (H / 8 + 255) / 256;
  Prefetch none{};
  const Prefetch& p = pf ? *pf : none;
  const uint8_t* ye = reinterpret_cast<const uint8_t*>(y) + (size_t)T * Kp * H * 2;
  dim3 grid((unsigned)(nbx * T + (p.n > 0 ? kPrefetchBlocks : 0))), block(256);
  hipLaunchKernelGGL(combine_kernel, grid, block, 0, stream, y, ye, w, inv, H, Kp, nbx, out, T, p);
  return hipGetLastError();
}
