// Large-M grouped expert GEMMs (prefill): one workgroup per (BM-row tile of
// one expert's group, 256 weight rows), the activation rows staged through
// LDS and shared by the workgroup's 4 waves, each wave owning 64 weight rows
// (four 16-row strips) over the whole K.  The pages keep separate launchers
// for small-M decode and large-M prefill GEMMs and reorder grouped-MoE
// programs so that neighbours reuse expert-weight tiles from cache (MiniMax
// M3 on MI355X post, section "Local shape and tiling"); here the block order
// is remapped so that each XCD (own L2) runs every weight slice of a tile
// together and an expert's tiles back to back.
//
// The weight scales of the workgroup's rows (whole K) go to LDS once, up
// front.  Per 128-element K chunk: every wave loads its four strips' codes
// (16 bytes per lane = one scale block; one contiguous KiB per strip in the
// native code order of common.h) from HBM into registers and the
// workgroup gathers the tile's activation chunk into LDS (a 3- or 4-stage
// pipeline, one barrier per chunk, later chunks' loads in flight during the
// MFMAs).
//   W4A16: codes -> bf16 via v_cvt_scalef32_pk_bf16_fp4, v_mfma_f32_16x16x32_bf16,
//          activations bf16 [rows][128] per chunk in LDS.
//   W4A4:  codes and E8M0 scales straight into v_mfma_scale_f32_16x16x128_f8f6f4,
//          activations MXFP4 ([rows][64 B] codes + [rows][4] scales) in LDS.
// Operand layout as in the streaming kernels: lane l supplies row / column
// l % 16 and K group g = l / 16; its 16 bytes are K-elements [32 g, 32 g + 32)
// of the chunk.  Here the weights are the A operand and the activation rows
// the B operand, so D lane l holds strip slots 4 g .. 4 g + 3 of tile row
// l % 16, and with the native order's strip pairs that is eight consecutive
// output columns: the epilogues write h and y in 16-byte stores (with the
// activations as A a lane held one column of four rows, stored 2 bytes at a
// time).
#include "common.h"
#include "kernels.h"

MOE_DEBUG_FLAGS(debug_flags_expert_gemm_tiled)

namespace {

constexpr uint32_t kOOR = 0x80000000u;   // out-of-range buffer offset: loads return 0

struct TileT {
  int expert, row0, rows;
  bool single;    // the expert's only tile: nothing re-reads its weights
};

// Block -> (tile, weight slice).  The hardware hands workgroup b to XCD
// b % 8, and an XCD runs the pairs it is given in order.
//
// MXFP4 activations (bandwidth-bound): the num_tiles * nslices live pairs
// are cut into 8 contiguous runs, one per XCD.  Inside a run an expert's
// tiles are taken G at a time and each group goes slice by slice: its tiles
// read one weight slice back to back, so all but the first find the slice in
// L2, and each tile's activation rows are re-read from L2 by the next slice
// G pairs later.  G = 1 is the plain tile-major order (an XCD runs all
// slices of a tile back to back).  On the W4A4 batch (experts of ~128 rows,
// about half of them with a second, nearly empty 128-row tile) the down GEMM
// takes G = 4: fetched bytes 1.74 -> 1.36 GB per launch, 1-2% faster.  The
// gate/up GEMM takes G = 4 on blocked activations (1% faster than 1) and
// G = 1 on gathered per-token rows (2.5% faster than 4 there).
//
// bf16 activations (bound by the MFMA work, which grows with a tile's rows):
// runs of equal pair counts leave the XCD holding a hot expert's full tiles
// (or the shared expert's) with more work than the others, so chunks of
// kDeal consecutive tiles are dealt to the XCDs in turn instead, each chunk
// tile-major; on the skewed 8,192-token batch this shortens both GEMMs by
// 5-7%.
//
// Blocks past the live pairs exit.
constexpr int kDeal = 4;

template <int BM, bool kFP4A, int G = 1>
__device__ __forceinline__ bool tile_slice(int b, const int32_t* tiles, const int32_t* offsets,
                                           int num_tiles, int nslices, TileT* ti, int* slice) {
  const int j = b >> 3;
  int tile;
  if constexpr (kFP4A) {
    const int live = num_tiles * nslices;
    const int per = (live + 7) >> 3;
    const int L = (b & 7) * per + j;
    if (j >= per || L >= live) return false;
    // The pairs of group [t_g, t_g + n) are [t_g * nslices, (t_g + n) * nslices),
    // so tile L / nslices lies in L's group.
    const int t0 = L / nslices;
    const int e = tiles[2 * t0];
    const int o0 = offsets[e], o1 = offsets[e + 1];
    const int k0 = (tiles[2 * t0 + 1] - o0) / BM;         // t0's place among e's tiles
    const int kg = k0 - k0 % G;                             // its group's first place
    const int n = min(G, (o1 - o0 + BM - 1) / BM - kg);
    const int local = L - (t0 - k0 + kg) * nslices;
    const int k = kg + local % n;
    *slice = local / n;
    ti->expert = e;
    ti->row0 = o0 + k * BM;
    ti->rows = min(BM, o1 - ti->row0);
    ti->single = o1 - o0 <= BM;
    return true;
  } else {
    const int q = j / (kDeal * nslices), p = j - q * kDeal * nslices;
    tile = (q * 8 + (b & 7)) * kDeal + p / nslices;
    if (tile >= num_tiles) return false;
    *slice = p % nslices;
  }
  ti->expert = tiles[2 * tile];
  ti->row0 = tiles[2 * tile + 1];
  ti->rows = min(BM, offsets[ti->expert + 1] - ti->row0);
  ti->single = offsets[ti->expert + 1] - offsets[ti->expert] <= BM;
  return true;
}

// Blocks for up to max_tiles tiles of nslices slices each under tile_slice.
template <bool kFP4A>
unsigned tile_slice_grid(int max_tiles, int nslices) {
  if (kFP4A) return (unsigned)(((long)max_tiles * nslices + 7) / 8 * 8);
  return (unsigned)((long)(max_tiles + 8 * kDeal - 1) / (8 * kDeal) * (8 * kDeal) * nslices);
}

// Per-configuration constants.  NS: pipeline stages.  KMAX: the largest
// reduction length whose scales fit the LDS left over by the stages (256
// weight rows x KMAX/32 bytes, plus the tile's activation rows for MXFP4).
// Totals: bf16 128-row 128 KiB (one 8-wave workgroup per CU; MXFP8 weights
// 160 KiB), bf16 64-row 80 KiB (two per CU), MXFP4 256-row 145 KiB (three stages), MXFP4 128-row
// 128 KiB (48.5 KiB for reductions up to 2048: two per CU), MXFP4 64-row
// 76 KiB (two per CU).  256-row tiles exist for MXFP4
// activations only: an expert of the W4A4 batch (~143 rows) then streams its
// weights once instead of once per 128-row tile.
template <int BM, bool kFP4A, bool kW8 = false, int KV = 0, bool kBlk = false>
struct TileCfg {
  static_assert(BM == 64 || BM == 128 || (BM == 256 && kFP4A), "tile sizes");
  static_assert(!(kW8 && kFP4A), "MXFP8 weights take bf16 activations");
  // (MXFP8 weights: twice the weight registers per stage, so 128-row tiles
  // keep three stages in flight instead of four)
  // KV (MXFP4 activations, 128-row tiles only) picks a variant that fits two
  // workgroups per CU (three stages, under 256 VGPRs):
  //   1: reductions up to 2048 (the W4A4 layer's down GEMM, I = 1536): the
  //      scale arrays shrink (48.5 KiB of LDS); W4A4 down 0.476 -> 0.409 ms
  //   2: reductions up to 6144 (its gate/up, H = 6144): the activation
  //      scales come with each stage (4 bytes per row) instead of for the
  //      whole K, leaving the weight scales' 48 KiB (74 KiB of LDS)
  static_assert(KV == 0 || (kFP4A && BM == 128), "variants: MXFP4 128-row tiles");
  // kBlk: MXFP4 activations in the blocked row order (sorted rows, 16-row
  // blocks: per block and chunk 1 KiB of codes and 64 bytes of scales, each
  // contiguous); their scales then always come with each stage
  static_assert(!kBlk || kFP4A, "blocked rows: MXFP4 activations");
  // bf16 activations and MXFP4 weights at 128 rows: two 64-row halves, each
  // on four waves with the weight strips of the 64-row tile (8 waves, one
  // workgroup per CU: the same two waves per SIMD as two 64-row workgroups,
  // but one weight fetch for the 128 rows)
  static constexpr bool kM2 = BM == 128 && !kFP4A && !kW8;
  static constexpr int kThreads = kM2 ? 512 : 256;
  static constexpr int NS =
      ((BM == 64 && !kFP4A) || BM == 256 || (kW8 && BM == 128) || (KV && BM == 128) || kM2) ? 3 : 4;
  static constexpr int KMAX =
      KV == 1 ? 2048 : KV == 2 ? 6144 : kFP4A ? (BM == 128 ? 8192 : 6144) : 4096;
  static constexpr int SCB = 256 * (KMAX / 32);             // weight scales
  // MXFP4 activation scales of the tile's rows (whole K), BM/4 rows per wave
  // (KV 2 or blocked rows: NS stage slots of BM rows x 4 bytes, plus 256
  // bytes the waves that load no scales write their zeros to)
  static constexpr int ASB = (KV == 2 || kBlk) ? NS * BM * 4 + 256
                             : kFP4A ? 4 * ((BM / 4 * (KMAX / 128) + 63) / 64) * 256 : 0;
  // activation bytes per stage:
  //   bf16:  256 bytes per row, 16-byte slot p of row r holds piece p ^ (r & 15)
  //   MXFP4: 64 bytes of codes per row, slot p holds piece p ^ ((r >> 2) & 3)
  // (the XOR swizzle spreads the 16 rows an MFMA operand read touches over all
  // LDS banks)
  static constexpr int XB = kFP4A ? BM * 64 : BM * 256;
};

// Weight scales in LDS: the workgroup's 256 weight rows (wave w's strips are
// rows [64 w, 64 w + 64)), each Q = K/128 dwords for the whole K, dword c
// holding chunk c's four scale bytes (K-groups 0..3).  They are loaded once,
// before the K loop (one request per cache line), not per chunk.  Dword c of
// row r sits at slot c ^ scale_swizzle(r): the 16 rows one read touches then
// fall in 16 different banks whatever Q is (for Q = 2^v * odd the rows'
// natural offsets already differ mod 64 when v <= 2; otherwise the XOR
// separates the rows that would share a bank).
__device__ __forceinline__ int scale_swizzle(int r, int Q) {
  const int v = __builtin_ctz(Q);
  const int rr = r & 15;
  return v <= 2 ? 0 : (v < 6 ? rr >> (6 - v) : rr);
}

// The K loop as an NS-stage pipeline.  Stage u holds one 128-element chunk:
// the tile's activation rows in LDS (written by direct-to-LDS buffer loads,
// no registers) and each wave's four weight strips (16 bytes per lane) in
// registers.  Iteration c waits for stage c % NS, meets the other waves at
// the barrier (which also retires every read of the stage about to be
// refilled), issues chunk c + NS - 1 into that stage and runs the MFMAs of
// chunk c; NS - 1 chunks stay in flight.  Loads beyond the tile's rows or
// past the last chunk use an out-of-range offset: they move no data and
// every wave issues the same number of loads per stage, so the wait counts
// are constants.  MFMAs run only on the tile's live 16-row sub-tiles.
template <int BM, bool kFP4A, bool kW8 = false, int KV = 0, bool kBlk = false>
struct TiledGemm {
  static constexpr int NS = TileCfg<BM, kFP4A, kW8, KV, kBlk>::NS;
  static constexpr int XB = TileCfg<BM, kFP4A, kW8, KV, kBlk>::XB;
  static constexpr bool kM2 = TileCfg<BM, kFP4A, kW8, KV, kBlk>::kM2;
  static constexpr int MT = kM2 ? 4 : BM / 16;           // 16-row sub-tiles per wave
  // code / row loads per wave per stage (kM2: the 128 rows over 8 waves)
  static constexpr int XI = kFP4A ? BM / 64 : kM2 ? BM / 32 : BM / 16;
  // weight registers per strip and stage: 16 bytes (32 E2M1 codes) or 32 (32 E4M3 codes)
  static constexpr int NQ = kW8 ? 2 : 1;
  static constexpr bool kAS = KV == 2 || kBlk;            // activation scales per stage
  // per-chunk step of the activation code / scale offsets
  static constexpr uint32_t kXStep = kBlk ? 1024 : kFP4A ? 64 : 256, kSStep = kBlk ? 64 : 4;
  static constexpr int LPS = XI + 4 * NQ + (kAS ? 1 : 0);  // vmem ops per wave per stage

  rsrc_t w, ws, a, as;
  uint32_t wo[4];               // lane's offsets in its four weight strips (native code order)
  uint32_t wsd, ssd;            // (two slices) code and scale-row byte distance of the next slice
  uint32_t xo[XI];              // lane's activation source offsets (or kOOR)
  uint32_t sro;                 // lane's scale byte offset in LDS for strip 0 (row 64 wv + nl, + g)
  uint32_t aso;                 // (kAS) lane's activation scale row offset, or kOOR
  int wave, lane, nl, g, nch, Q, swz;
  int wv, half;                 // weight rows [64 wv, 64 wv + 64); tile rows from 64 half (kM2)
  bool stream;                  // weights read once: non-temporal loads

  // Scale rows (Q dwords each, whole K) into LDS: wave w fills rows
  // [RW w, RW w + RW), its region padded to whole 64-lane loads (size-4
  // direct-to-LDS loads); dword c of row r lands at slot c ^ swizzle(r).
  // src(r) = byte offset of row r in the resource, or kOOR (row of zeros).
  template <int RW, class SrcFn>
  __device__ __forceinline__ void stage_rows(uint8_t* lds, rsrc_t rsrc, SrcFn src) const {
    const int per = (RW * Q + 63) / 64;
    const int step_r = 64 / Q, step_s = 64 % Q;
    int r = lane / Q, sl = lane % Q;
    uint8_t* dst = lds + 256 * per * wave;
    for (int i = 0; i < per; ++i) {
      const int row = RW * wave + r;
      // row offset + dword offset (kOOR + a small offset stays out of range)
      const uint32_t base = r < RW ? src(row) : kOOR;
      load_to_lds4(rsrc, base + (uint32_t)(4 * (sl ^ scale_swizzle(row, Q))), 0, dst + 256 * i);
      r += step_r;
      sl += step_s;
      if (sl >= Q) {
        sl -= Q;
        ++r;
      }
    }
  }

  // LDS byte of scale row `row` (of an array filled with RW rows per wave),
  // chunk c, K-group g.
  template <int RW>
  __device__ __forceinline__ uint32_t scale_at(int row, int c) const {
    const int per = (RW * Q + 63) / 64;
    return 4 * ((row / RW) * per * 64 + (row % RW) * Q + (c ^ scale_swizzle(row, Q))) + g;
  }

  // Issue chunk c: the weight codes into this wave's registers q (strip t's
  // 16-byte pieces at q[NQ t .. NQ t + NQ)), then the activations into a
  // stage of LDS (kAS: adst = where this wave's activation-scale load lands).
  // Past the last chunk both move no data.
  // With NSL weight slices per workgroup, chunk c of the run is chunk
  // c % nch of slice c / nch (the next slice's weights sit wsd bytes further,
  // the activation chunk is the same).
  template <int NSL = 1>
  __device__ __forceinline__ void issue_w(int c, u32x4_t (&q)[4 * NQ]) const {
    const bool ok = c < NSL * nch;
    const bool hi = NSL > 1 && c >= nch;
    const uint32_t oor = ok ? 0u : kOOR;
    const uint32_t cc = ok ? (uint32_t)(hi ? c - nch : c) : 0u;
    const uint32_t so = hi ? wsd : 0u;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int hq = 0; hq < NQ; ++hq)
        q[NQ * t + hq] = stream ? bload16_nt(w, wo[t] | oor, wnat_chunk(cc, NQ, hq) + so)
                                : bload16(w, wo[t] | oor, wnat_chunk(cc, NQ, hq) + so);
  }
  template <int NSL = 1>
  __device__ __forceinline__ void issue_x(uint8_t* base, int c, uint8_t* adst = nullptr) const {
    const bool ok = c < NSL * nch;
    const uint32_t oor = ok ? 0u : kOOR;
    const uint32_t cc = ok ? (uint32_t)(NSL > 1 && c >= nch ? c - nch : c) : 0u;
    if constexpr (kAS) load_to_lds4(as, aso | oor, kSStep * cc, adst);
#pragma unroll
    for (int i = 0; i < XI; ++i)
      load_to_lds16(a, xo[i] | oor, kXStep * cc, base + (wave * XI + i) * 1024);
  }

  // MFMAs of one chunk on the first NMT 16-row sub-tiles (the live ones).
  template <int NMT>
  __device__ __forceinline__ void compute(const uint8_t* x, const uint8_t* sc, const uint8_t* asc,
                                          int c, const u32x4_t (&q)[4 * NQ],
                                          floatx4_t (&acc)[MT][4]) const {
    uint32_t s[4];
    const uint32_t so = sro + 4 * (uint32_t)(c ^ swz);
#pragma unroll
    for (int t = 0; t < 4; ++t) s[t] = sc[so + 64 * t * Q];   // strip t: rows + 16 t
    if constexpr (kFP4A) {
      // all of the chunk's LDS reads first, then the MFMAs
      u32x4_t av[NMT];
      uint32_t sa[NMT];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) {
        const int r = 16 * mt + nl;
        av[mt] = *reinterpret_cast<const u32x4_t*>(x + r * 64 + 16 * (g ^ ((r >> 2) & 3)));
        sa[mt] = kAS ? asc[4 * r + g] : asc[scale_at<BM / 4>(r, c)];
      }
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          acc[mt][t] = mfma_fp4_16x16x128(q[t], s[t], av[mt], sa[mt], acc[mt][t]);
    } else {
      float scf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) scf[t] = e8m0_to_f32(s[t]);
      // Software pipeline over the chunk's four K-steps: step j + 1's A
      // fragments (LDS reads) and B fragments (dequantised weights) are
      // produced while step j's MFMAs run, interleaved MFMA by MFMA.
      bf16x8_t av[2][NMT], bv[2][4];
#pragma unroll
      for (int mt = 0; mt < NMT; ++mt) av[0][mt] = a_frag(x, mt, 0);
#pragma unroll
      for (int t = 0; t < 4; ++t) bv[0][t] = wfrag(q, t, 0, scf[t]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int cur = j & 1, nxt = cur ^ 1;
        if (j < 3) {
#pragma unroll
          for (int mt = 0; mt < NMT; ++mt) av[nxt][mt] = a_frag(x, mt, j + 1);
#pragma unroll
          for (int t = 0; t < 4; ++t) bv[nxt][t] = wfrag(q, t, j + 1, scf[t]);
        }
#pragma unroll
        for (int mt = 0; mt < NMT; ++mt)
#pragma unroll
          for (int t = 0; t < 4; ++t) acc[mt][t] = mfma_bf16_16x16x32(bv[cur][t], av[cur][mt], acc[mt][t]);
        if (j < 3) interleave<0, 4 * NMT, 16, NMT>();
        __builtin_amdgcn_sched_barrier(0);    // one scheduling region per K-step
      }
    }
  }

  // Scheduling groups for one K-step: after each of its NM MFMAs, a share of
  // the NV conversions that prepare the next step; the next step's ND LDS
  // reads all go right after the first MFMA, so their latency (bank
  // conflicts included) is covered by the step's remaining MFMAs (spread
  // evenly they left the last read a few MFMAs before its use: skewed
  // gate/up 1.401 -> 1.377 ms).
  template <int I, int NM, int NV, int ND>
  __device__ __forceinline__ static void interleave() {
    if constexpr (I < NM) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // MFMA
      constexpr int v = (I + 1) * NV / NM - I * NV / NM;
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x002, v, 0);   // VALU
      constexpr int d = I == 0 ? ND : 0;
      if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);   // DS read
      interleave<I + 1, NM, NV, ND>();
    }
  }

  // bf16 B operand of strip t, K-step j: the lane's 8 weights of the step
  // (MXFP4: dword j of its 16 bytes; MXFP8: bytes 8 j .. 8 j + 7 of its 32).
  __device__ __forceinline__ static bf16x8_t wfrag(const u32x4_t (&q)[4 * NQ], int t, int j,
                                                   float sc) {
    if constexpr (kW8) {
      const u32x4_t& d = q[2 * t + (j >> 1)];
      return dequant8_bf16_fp8(d[2 * (j & 1)], d[2 * (j & 1) + 1], sc);
    } else {
      return dequant8_bf16(q[t][j], sc);
    }
  }

  // bf16 A operand: rows 16 mt + (lane % 16), K-step j of the lane's K-group.
  __device__ __forceinline__ bf16x8_t a_frag(const uint8_t* x, int mt, int j) const {
    const int r = 16 * mt + nl;
    return *reinterpret_cast<const bf16x8_t*>(x + r * 256 + 16 * ((4 * g + j) ^ (r & 15)));
  }

  // stages[u]: one LDS array per stage (separate objects, so the compiler's
  // wait before reading stage u only covers the loads into stage u).  The
  // scale rows, issued first, are complete once the first stage is.
  // wrow(r): byte offset of weight scale row r; arow(r): of the tile's
  // activation scale row r (MXFP4) or kOOR.
  //
  // NSL = 2: the workgroup's two weight slices one after the other in one
  // pipeline (the second slice's first chunks load while the first's last
  // ones compute); both slices' scales are staged up front, the second's
  // 1 KiB * ceil(Q) further; after the first slice's last chunk
  // between(acc) stores its result and the accumulators restart at zero.
  // BP = (nch - 1) % NS: the stage of the first slice's last chunk, so that
  // one unrolled position holds the code between the slices.
  template <int NMT, int NSL = 1, int BP = 0, class WRow, class ARow, class Between>
  __device__ __forceinline__ void run(uint8_t* const (&stages)[NS], uint8_t* sc, uint8_t* asc,
                                      WRow wrow, ARow arow, floatx4_t (&acc)[MT][4],
                                      Between&& between) {
    u32x4_t q[NS][4 * NQ];
    const int scs = 1024 * ((64 * Q + 63) / 64);
    if (wave < 4) {
      stage_rows<64>(sc, ws, wrow);
      if constexpr (NSL > 1) stage_rows<64>(sc + scs, ws, [&](int r) { return wrow(r) + ssd; });
    }
    // kAS: slot u's activation scales at asc + 4 BM u (waves w < BM / 64
    // load rows 64 w + lane; the others write zeros past the slots)
    auto aslot = [&](int u) -> uint8_t* { return kAS ? asc + 4 * BM * u : asc; };
    auto adst = [&](int u) -> uint8_t* {
      return wave < BM / 64 ? asc + 4 * BM * u + 256 * wave : asc + 4 * BM * NS;
    };
    if constexpr (kAS) {
      aso = wave < BM / 64 ? arow(64 * wave + lane) : kOOR;
    } else if constexpr (kFP4A) {
      stage_rows<BM / 4>(asc, as, arow);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) {
      issue_w<NSL>(u, q[u]);
      issue_x<NSL>(stages[u], u, adst(u));
    }
    const int ntot = NSL * nch;
    for (int c0 = 0; c0 < ntot; c0 += NS) {
#pragma unroll
      for (int u = 0; u < NS; ++u) {
        const int c = c0 + u;
        wait_vmcnt<LPS * (NS - 2)>();
        // The weights of chunk c + NS - 1 go to registers this wave has
        // finished with (chunk c - 1's): they need not wait for the other
        // waves; the activations refill the stage chunk c - 1 was read
        // from, after the barrier that retires every read of it.
        issue_w<NSL>(c + NS - 1, q[(u + NS - 1) % NS]);
        stage_barrier();
        issue_x<NSL>(stages[(u + NS - 1) % NS], c + NS - 1, adst((u + NS - 1) % NS));
        if constexpr (NSL == 1) {
          if (c < nch) compute<NMT>(stages[u] + half * 64 * 256, sc, aslot(u), c, q[u], acc);
        } else if (c < ntot) {
          const bool hi = c >= nch;
          compute<NMT>(stages[u] + half * 64 * 256, hi ? sc + scs : sc, aslot(u),
                       hi ? c - nch : c, q[u], acc);
          if (u == BP && c == nch - 1) {
            between(acc);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
              for (int t = 0; t < 4; ++t) acc[mt][t] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
          }
        }
      }
    }
    wait_vmcnt<0>();
  }
  template <int NMT, class WRow, class ARow>
  __device__ __forceinline__ void run(uint8_t* const (&stages)[NS], uint8_t* sc, uint8_t* asc,
                                      WRow wrow, ARow arow, floatx4_t (&acc)[MT][4]) {
    run<NMT, 1>(stages, sc, asc, wrow, arow, acc, [](floatx4_t (&)[MT][4]) {});
  }
};

// The lane's activation source offsets for every stage: row r of the tile
// comes from source row src(r) (a token for gate/up, a sorted row for down).
template <int BM, bool kFP4A, bool kW8, int KV, bool kBlk, class SrcFn>
__device__ __forceinline__ void plan_x(TiledGemm<BM, kFP4A, kW8, KV, kBlk>& G, const TileT& ti, SrcFn src,
                                       uint32_t row_bytes) {
#pragma unroll
  for (int i = 0; i < G.XI; ++i) {
    const int k = G.wave * G.XI + i;
    int r, piece;
    if (kFP4A) {
      r = 16 * k + (G.lane >> 2);
      const int p = G.lane & 3;
      piece = p ^ ((r >> 2) & 3);
    } else {
      r = 4 * k + (G.lane >> 4);
      const int p = G.lane & 15;
      piece = p ^ (r & 15);
    }
    if constexpr (kBlk) {           // sorted row s = row0 + r, chunk 0 of its block
      const uint32_t s = (uint32_t)(ti.row0 + r);
      G.xo[i] = r < ti.rows ? (s >> 4) * (row_bytes / 64) * 1024u + (s & 15) * 64u + 16 * piece
                            : kOOR;
    } else {
      G.xo[i] = r < ti.rows ? src(r) * row_bytes + 16 * piece : kOOR;
    }
  }
}

// Common set-up of a workgroup's GEMM state (weights of one expert slice;
// K = reduction length; rs = K/32 scale bytes per weight row).
template <int BM, bool kFP4A, bool kW8, int KV, bool kBlk>
__device__ __forceinline__ void setup(TiledGemm<BM, kFP4A, kW8, KV, kBlk>& G, const TileT& ti, int K,
                                      const uint8_t* wq, const uint8_t* wsc, int wrows) {
  G.lane = threadIdx.x & 63;
  G.wave = threadIdx.x >> 6;
  G.wv = G.wave & 3;
  G.half = G.wave >> 2;                     // 0 unless kM2 (8 waves)
  G.nl = G.lane & 15;
  G.g = G.lane >> 4;
  G.nch = K / 128;
  G.Q = K / 128;
  G.swz = scale_swizzle(G.nl, G.Q);
  G.sro = 4 * (64 * G.wv + G.nl) * G.Q + G.g;
  const size_t wbytes = (size_t)wrows * (kW8 ? K : K / 2), sbytes = (size_t)wrows * (K / 32);
  G.w = make_rsrc(wq + ti.expert * wbytes, (uint32_t)wbytes);
  // The expert's only tile with bf16 activations streams its weights
  // non-temporally; with MXFP4 activations (or several tiles) an expert's
  // weight lines stay cacheable for the tiles that re-read them from L2.
  G.stream = !kFP4A && ti.single;
  G.ws = make_rsrc(wsc + ti.expert * sbytes, (uint32_t)sbytes);
}

template <int N>
struct IntC {
  static constexpr int value = N;
};

// Calls f(IntC<NMT>) with the number of 16-row sub-tiles the MFMAs cover:
// the live ones (ceil(rows / 16)), rounded up to an even count for 128-row
// tiles and to a multiple of four for 256-row tiles (four code variants per
// kernel).
template <int BM, class F>
__device__ __forceinline__ void with_nmt(int rows, F&& f) {
  const int need = (rows + 15) >> 4;
  if constexpr (BM == 256) {
    if (need > 12) f(IntC<16>());
    else if (need > 8) f(IntC<12>());
    else if (need > 4) f(IntC<8>());
    else f(IntC<4>());
  } else if constexpr (BM == 128) {
    if (need > 6) f(IntC<8>());
    else if (need > 4) f(IntC<6>());
    else if (need > 2) f(IntC<4>());
    else f(IntC<2>());
  } else {
    static_assert(BM == 64, "64- or 128-row tiles");
    if (need > 3) f(IntC<4>());
    else if (need > 2) f(IntC<3>());
    else if (need > 1) f(IntC<2>());
    else f(IntC<1>());
  }
}

// Static LDS of a kernel: NS stage arrays (separate objects), the weight
// scales, and for MXFP4 activations their scales and the tile's source
// rows; body(stages, scales, act_scales, src_rows) runs with them.
template <int BM, bool kFP4A, bool kW8, int KV, bool kBlk, class Body>
__device__ __forceinline__ void with_lds(Body&& body) {
  using Cfg = TileCfg<BM, kFP4A, kW8, KV, kBlk>;
  constexpr int XB = Cfg::XB, SCB = Cfg::SCB;
  __shared__ __align__(16) uint8_t sc[SCB];
  __shared__ __align__(16) uint8_t st0[XB];
  __shared__ __align__(16) uint8_t st1[XB];
  __shared__ __align__(16) uint8_t st2[XB];
  if constexpr (kFP4A && Cfg::NS == 4) {
    __shared__ __align__(16) uint8_t st3[XB];
    __shared__ __align__(16) uint8_t asc[Cfg::ASB];
    __shared__ int32_t srow[BM];
    uint8_t* const stages[4] = {st0, st1, st2, st3};
    body(stages, sc, asc, srow);
  } else if constexpr (kFP4A) {
    static_assert(Cfg::NS == 3, "three or four stages");
    __shared__ __align__(16) uint8_t asc[Cfg::ASB];
    __shared__ int32_t srow[BM];
    uint8_t* const stages[3] = {st0, st1, st2};
    body(stages, sc, asc, srow);
  } else if constexpr (Cfg::NS == 4) {
    __shared__ __align__(16) uint8_t st3[XB];
    uint8_t* const stages[4] = {st0, st1, st2, st3};
    body(stages, sc, (uint8_t*)nullptr, (int32_t*)nullptr);
  } else {
    static_assert(Cfg::NS == 3, "three or four stages");
    uint8_t* const stages[3] = {st0, st1, st2};
    body(stages, sc, (uint8_t*)nullptr, (int32_t*)nullptr);
  }
}

// The tile's K loop: source rows (MXFP4: tabled in LDS first, shared by the
// activation-code offsets and the activation-scale rows), then the pipeline.
// direct(r) = source row of tile row r < rows; wrow(r) = byte offset of
// weight scale row r; arow_bytes = activation scale bytes per source row.
// NSL, between: the weight slices per workgroup and what runs between them
// (bf16 activations, 64-row tiles).
struct NoBetween {
  template <class A>
  __device__ void operator()(A&) const {}
};

template <int BM, bool kFP4A, bool kW8, int KV, bool kBlk, int NSL = 1, class Direct, class WRow,
          class Between = NoBetween>
__device__ __forceinline__ void tile_loop(TiledGemm<BM, kFP4A, kW8, KV, kBlk>& G, const TileT& ti, Direct direct,
                                          WRow wrow, uint32_t row_bytes, uint32_t arow_bytes,
                                          floatx4_t (&acc)[TiledGemm<BM, kFP4A, kW8, KV, kBlk>::MT][4],
                                          Between&& between = {}) {
  static_assert(NSL == 1 || (BM == 64 && !kFP4A), "two slices: bf16 64-row tiles");
  with_lds<BM, kFP4A, kW8, KV, kBlk>([&](auto& stages, uint8_t* sc, uint8_t* asc, int32_t* srow) {
    if constexpr (kBlk) {
      plan_x<BM, kFP4A, kW8, KV, kBlk>(G, ti, direct, row_bytes);
      // scales of sorted row s, chunk 0: ((s / 16) * C) * 64 + (s % 16) * 4
      auto arow = [&](int r) -> uint32_t {
        const uint32_t s = (uint32_t)(ti.row0 + r);
        return r < ti.rows ? (s >> 4) * (arow_bytes / 4) * 64u + (s & 15) * 4u : kOOR;
      };
      with_nmt<BM>(ti.rows, [&](auto n) {
        G.template run<decltype(n)::value>(stages, sc, asc, wrow, arow, acc);
      });
    } else if constexpr (kFP4A) {
      const int t = threadIdx.x;
      if (t < BM) srow[t] = t < ti.rows ? (int32_t)direct(t) : 0;
      __syncthreads();
      plan_x<BM, kFP4A, kW8, KV, kBlk>(G, ti, [&](int r) { return (uint32_t)srow[r]; }, row_bytes);
      auto arow = [&](int r) -> uint32_t {
        return r < ti.rows ? (uint32_t)srow[r] * arow_bytes : kOOR;
      };
      with_nmt<BM>(ti.rows, [&](auto n) {
        G.template run<decltype(n)::value>(stages, sc, asc, wrow, arow, acc);
      });
    } else if constexpr (TiledGemm<BM, kFP4A, kW8, KV, kBlk>::kM2) {
      plan_x<BM, kFP4A, kW8, KV, kBlk>(G, ti, direct, row_bytes);
      auto arow = [](int) -> uint32_t { return kOOR; };
      // each half's live sub-tiles (a half with no rows runs one on zeros)
      with_nmt<64>(max(0, ti.rows - 64 * G.half), [&](auto n) {
        G.template run<decltype(n)::value>(stages, sc, asc, wrow, arow, acc);
      });
    } else {
      plan_x<BM, kFP4A, kW8, KV, kBlk>(G, ti, direct, row_bytes);
      auto arow = [](int) -> uint32_t { return kOOR; };
      with_nmt<BM>(ti.rows, [&](auto n) {
        constexpr int NMT = decltype(n)::value;
        if constexpr (NSL == 1) {
          G.template run<NMT>(stages, sc, asc, wrow, arow, acc);
        } else {
          static_assert(TiledGemm<BM, kFP4A, kW8, KV, kBlk>::NS == 3, "three stages");
          const int bp = (G.nch - 1) % 3;
          if (bp == 0) G.template run<NMT, NSL, 0>(stages, sc, asc, wrow, arow, acc, between);
          else if (bp == 1) G.template run<NMT, NSL, 1>(stages, sc, asc, wrow, arow, acc, between);
          else G.template run<NMT, NSL, 2>(stages, sc, asc, wrow, arow, acc, between);
        }
      });
    }
  });
}

// gate/up + SwiGLU: weight rows gate [i0, i0 + 128) and up [I + i0, I + i0 + 128),
// i0 = 128 s; wave w owns i in [i0 + 32 w, i0 + 32 w + 32): strips gate lo/hi, up lo/hi.
// kQH: h is written MXFP4-quantised in the blocked row order (hq, hs)
// instead of as bf16 h.
template <int BM, bool kFP4A, bool kW8, int KV = 0, bool kBlk = false, bool kQH = false>
__global__ __launch_bounds__((TileCfg<BM, kFP4A, kW8, KV, kBlk>::kThreads), KV ? 2 : 1) void gate_up_tiled_kernel(
    const void* __restrict__ act, const uint8_t* __restrict__ act_scale,
    const int32_t* __restrict__ sorted, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tiles, const int32_t* __restrict__ num_tiles,
    const uint8_t* __restrict__ w13, const uint8_t* __restrict__ w13s, int T, int H, int I, int Kp,
    uint16_t* __restrict__ h, uint8_t* __restrict__ hq, uint8_t* __restrict__ hs) {
  TileT ti;
  int s;
  if (!tile_slice<BM, kFP4A, kBlk ? 4 : 1>(blockIdx.x, tiles, offsets, *num_tiles, I / 128, &ti, &s))
    return;
  // (debug builds: a tile whose rows leave [0, A) stores nothing)
  if (!MOE_DOK(ti.row0 >= 0 && ti.rows > 0 && (int64_t)ti.row0 + ti.rows <= (int64_t)T * Kp,
               kDbgTiles))
    return;
  TiledGemm<BM, kFP4A, kW8, KV, kBlk> G;
  setup(G, ti, H, w13, w13s, 2 * I);
  const int nl = G.nl, g = G.g;
  const uint32_t rb = H / 2, rs = H / 32;
  const int i0 = s * 128 + G.wv * 32;
  const int rows4[4] = {i0 + nl, i0 + 16 + nl, I + i0 + nl, I + i0 + 16 + nl};
  // (a 128-row tile's upper half with no rows loads no weights)
  const bool idle = G.kM2 && ti.rows <= 64 * G.half;
#pragma unroll
  for (int st = 0; st < 4; ++st) G.wo[st] = idle ? kOOR : wnat_lane(rows4[st] >> 4, H, G.NQ, G.lane);
  if (kFP4A) {
    // per token, or (blocked) per sorted row in whole 16-row blocks
    const size_t nr = kBlk ? ((size_t)T * Kp + 15) / 16 * 16 : (size_t)T;
    G.a = make_rsrc(act, (uint32_t)(nr * rb));
    G.as = make_rsrc(act_scale, (uint32_t)(nr * rs));
  } else {
    G.a = make_rsrc(act, (uint32_t)((size_t)T * H * 2));
  }
  auto token = [&](int r) -> uint32_t {
    return min((unsigned)(sorted[ti.row0 + r] / Kp), (unsigned)(T - 1));
  };
  // workgroup row r (wave r/64, strip (r/16)%4, slot r%16) -> weight scale row
  auto wrow = [&](int r) -> uint32_t {
    const int t = (r >> 4) & 3;
    return rs * (uint32_t)((t < 2 ? 0 : I) + s * 128 + 32 * (r >> 6) + wnat_row(t & 1, r & 15));
  };

  constexpr int MT = TiledGemm<BM, kFP4A, kW8, KV, kBlk>::MT;
  floatx4_t acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[mt][st] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  tile_loop<BM, kFP4A, kW8, KV, kBlk>(G, ti, token, wrow, kFP4A ? rb : (uint32_t)H * 2, rs, acc);
  const int m0 = 64 * G.half;               // the wave's first tile row

  // h (bf16): lane 16 g + n holds tile row 16 mt + n at intermediate
  // columns i0 + 8 g .. i0 + 8 g + 7 (gate strips 0-1, up strips 2-3; strip
  // u, D row 4 g + r -> column i0 + 8 g + 4 u + r): one 16-byte store.
  if constexpr (kQH) {
    // MXFP4 h (the pages fuse the activation and its quantisation): the
    // wave's 32 columns are one scale block (K-group `wv` of chunk s), its
    // amax over the lanes n, n + 16, n + 32, n + 48 of the row; each lane
    // writes the four code bytes of its eight values, lane n the scale.
    const int C = I / 128;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      float v[8];
      uint32_t am = 0;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int u = k >> 2, r = k & 3;
        v[k] = __uint_as_float((uint32_t)f32_to_bf16_rne(swiglu(acc[mt][u][r], acc[mt][2 + u][r]))
                               << 16);
        am = max(am, __float_as_uint(v[k]) & 0x7FFFFFFFu);
      }
      const int X = mxfp4_block_exponent(__uint_as_float(xrow_max_u32(am)));
      const uint32_t codes = mxfp4_codes8(v, X);
      const int m = m0 + 16 * mt + nl;
      if (m < ti.rows) {
        const size_t p = (size_t)(ti.row0 + m);
        const size_t blk = (p >> 4) * C + s;
        *reinterpret_cast<uint32_t*>(hq + blk * 1024 + (p & 15) * 64 + 16 * G.wv + 4 * g) = codes;
        if (g == 0) hs[blk * 64 + (p & 15) * 4 + G.wv] = (uint8_t)(X + 127);
      }
    }
    return;
  }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int m = m0 + 16 * mt + nl;
    if (m < ti.rows) {
      u32x4_t v;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int u = k >> 1, r = 2 * (k & 1);
        v[k] = (uint32_t)f32_to_bf16_rne(swiglu(acc[mt][u][r], acc[mt][2 + u][r])) |
               (uint32_t)f32_to_bf16_rne(swiglu(acc[mt][u][r + 1], acc[mt][2 + u][r + 1])) << 16;
      }
      *reinterpret_cast<u32x4_t*>(h + (size_t)(ti.row0 + m) * I + i0 + 8 * g) = v;
    }
  }
}

// down: weight rows j in [256 s, 256 s + 256); wave w owns [256 s + 64 w, +64).
// NSL = 2 (bf16 64-row tiles): the workgroup takes slices 2 s and 2 s + 1 of
// its tile in one pipeline, the first slice's y stored between them.
template <int BM, bool kFP4A, bool kW8, int KV = 0, bool kBlk = false, int NSL = 1>
__global__ __launch_bounds__((TileCfg<BM, kFP4A, kW8, KV, kBlk>::kThreads), KV ? 2 : 1) void down_tiled_kernel(
    const void* __restrict__ hin, const uint8_t* __restrict__ hscale,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ tiles,
    const int32_t* __restrict__ num_tiles, const uint8_t* __restrict__ w2,
    const uint8_t* __restrict__ w2s, int A, int H, int I, uint16_t* __restrict__ y,
    uint8_t* __restrict__ ye) {
  TileT ti;
  int s;
  if (!tile_slice<BM, kFP4A, 4>(blockIdx.x, tiles, offsets, *num_tiles, H / 256 / NSL, &ti, &s))
    return;
  s *= NSL;
  // (debug builds: a tile whose rows leave [0, A) stores nothing)
  if (!MOE_DOK(ti.row0 >= 0 && ti.rows > 0 && (int64_t)ti.row0 + ti.rows <= (int64_t)A, kDbgTiles))
    return;
  TiledGemm<BM, kFP4A, kW8, KV, kBlk> G;
  setup(G, ti, I, w2, w2s, H);
  const int nl = G.nl, g = G.g;
  const uint32_t rb = I / 2, rs = I / 32;
  const int j0 = s * 256 + G.wv * 64;
  const bool idle = G.kM2 && ti.rows <= 64 * G.half;   // an upper half with no rows
#pragma unroll
  for (int st = 0; st < 4; ++st) G.wo[st] = idle ? kOOR : wnat_lane((j0 >> 4) + st, I, G.NQ, G.lane);
  G.wsd = wnat_lane(16, I, G.NQ, 0);                    // the next slice: 16 strips on
  G.ssd = 256 * rs;
  if (kFP4A) {
    const size_t nr = kBlk ? ((size_t)A + 15) / 16 * 16 : (size_t)A;
    G.a = make_rsrc(hin, (uint32_t)(nr * rb));
    G.as = make_rsrc(hscale, (uint32_t)(nr * rs));
  } else {
    G.a = make_rsrc(hin, (uint32_t)((size_t)A * I * 2));
  }
  auto srow = [&](int r) -> uint32_t { return (uint32_t)(ti.row0 + r); };
  // workgroup row r (wave r/64, strip (r/16)%4, slot r%16) -> weight scale row
  auto wrow = [&](int r) -> uint32_t {
    return rs * (uint32_t)(s * 256 + (r & ~31) + wnat_row((r >> 4) & 1, r & 15));
  };

  constexpr int MT = TiledGemm<BM, kFP4A, kW8, KV, kBlk>::MT;
  floatx4_t acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int st = 0; st < 4; ++st) acc[mt][st] = (floatx4_t){0.f, 0.f, 0.f, 0.f};
  const int m0 = 64 * G.half;               // the wave's first tile row

  // y in the staged fp16 format.  Lane 16 g + n holds tile row 16 mt + n at
  // columns j0 + 32 p + 8 g .. + 7 of strip pair p (strip 2 p + u, D row
  // 4 g + r -> column j0 + 32 p + 8 g + 4 u + r): one 16-byte store per
  // pair.  A pair's 32 columns are one exponent group, spread over lanes
  // n, n + 16, n + 32 and n + 48.
  auto store_y = [&](floatx4_t (&acc)[MT][4], int j0) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    uint32_t f = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 4; ++r) f = max_halves(f, pack_exponents(acc[mt][u][r], acc[mt][2 + u][r]));
    f = xrow_max_halves(f);
    const int e[2] = {y_exponent_of_field(f & 0xFFFFu), y_exponent_of_field(f >> 16)};
    const int m = m0 + 16 * mt + nl;
    if (m < ti.rows) {
      const size_t row = (size_t)(ti.row0 + m);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        u32x4_t v;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int u = k >> 1, r = 2 * (k & 1);
          v[k] = (uint32_t)y_encode(acc[mt][2 * p + u][r], e[p]) |
                 (uint32_t)y_encode(acc[mt][2 * p + u][r + 1], e[p]) << 16;
        }
        *reinterpret_cast<u32x4_t*>(y + row * H + j0 + 32 * p + 8 * g) = v;
      }
      if (g == 0)
        *reinterpret_cast<uint16_t*>(ye + row * (H / kYGroup) + j0 / kYGroup) =
            (uint16_t)((e[0] + 127) | (e[1] + 127) << 8);
    }
  }
  };
  if constexpr (NSL == 1) {
    tile_loop<BM, kFP4A, kW8, KV, kBlk>(G, ti, srow, wrow, kFP4A ? rb : (uint32_t)I * 2, rs, acc);
  } else {
    tile_loop<BM, kFP4A, kW8, KV, kBlk, NSL>(G, ti, srow, wrow, (uint32_t)I * 2, rs, acc,
                                             [&](floatx4_t (&a)[MT][4]) { store_y(a, j0); });
  }
  store_y(acc, j0 + 256 * (NSL - 1));
}

template <int BM, bool kFP4A, bool kW8 = false, int KV = 0, bool kBlk = false>
hipError_t launch_gate_up_bm(const void* act, const uint8_t* act_scale, const int32_t* sorted,
                             const int32_t* offsets, const int32_t* tiles,
                             const int32_t* num_tiles, int max_tiles, const uint8_t* w13,
                             const uint8_t* w13s, int T, int H, int I, int Kp, uint16_t* h,
                             hipStream_t stream, uint8_t* hq = nullptr, uint8_t* hs = nullptr) {
  const unsigned grid = tile_slice_grid<kFP4A>(max_tiles, I / 128);
  if constexpr (kFP4A) {
    if (hq) {
      hipLaunchKernelGGL((gate_up_tiled_kernel<BM, kFP4A, kW8, KV, kBlk, true>), dim3(grid),
                         dim3(TileCfg<BM, kFP4A, kW8, KV, kBlk>::kThreads),
                         0, stream, act, act_scale, sorted, offsets, tiles, num_tiles, w13, w13s, T,
                         H, I, Kp, h, hq, hs);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gate_up_tiled_kernel<BM, kFP4A, kW8, KV, kBlk>), dim3(grid),
                     dim3(TileCfg<BM, kFP4A, kW8, KV, kBlk>::kThreads), 0, stream, act,
                     act_scale, sorted, offsets, tiles, num_tiles, w13, w13s, T, H, I, Kp, h, hq, hs);
  return hipGetLastError();
}

template <int BM, bool kFP4A, bool kW8 = false, int KV = 0, bool kBlk = false, int NSL = 1>
hipError_t launch_down_bm(const void* h, const uint8_t* h_scale, const int32_t* offsets,
                          const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                          const uint8_t* w2, const uint8_t* w2s, int A, int H, int I, uint16_t* y,
                          hipStream_t stream) {
  const unsigned grid = tile_slice_grid<kFP4A>(max_tiles, H / 256 / NSL);
  uint8_t* ye = reinterpret_cast<uint8_t*>(y) + (size_t)A * H * 2;   // the group exponents
  hipLaunchKernelGGL((down_tiled_kernel<BM, kFP4A, kW8, KV, kBlk, NSL>), dim3(grid),
                     dim3(TileCfg<BM, kFP4A, kW8, KV, kBlk>::kThreads), 0, stream, h,
                     h_scale, offsets, tiles, num_tiles, w2, w2s, A, H, I, y, ye);
  return hipGetLastError();
}

template <int BM, bool kFP4A, bool kW8 = false>
bool fits(int H, int I) {
  return H <= TileCfg<BM, kFP4A, kW8>::KMAX && I <= TileCfg<BM, kFP4A, kW8>::KMAX;
}

// MXFP4 activations, per token (kBlk false) or in the blocked sorted-row
// order: 256-, 128- (variant by reduction length) or 64-row tiles.
template <bool kBlk>
hipError_t gate_up_fp4(int tile_m, const void* act, const uint8_t* act_scale,
                       const int32_t* sorted, const int32_t* offsets, const int32_t* tiles,
                       const int32_t* num_tiles, int max_tiles, const uint8_t* w13,
                       const uint8_t* w13s, int T, int H, int I, int Kp, uint16_t* h,
                       hipStream_t stream, uint8_t* hq, uint8_t* hs) {
#define MOE_GU_ARGS act, act_scale, sorted, offsets, tiles, num_tiles, max_tiles, w13, w13s, T, H, I, Kp, h, stream, hq, hs
  if (tile_m == 256) return launch_gate_up_bm<256, true, false, 0, kBlk>(MOE_GU_ARGS);
  if (tile_m == 128)
    return H <= 2048   ? launch_gate_up_bm<128, true, false, 1, kBlk>(MOE_GU_ARGS)
           : H <= 6144 ? launch_gate_up_bm<128, true, false, 2, kBlk>(MOE_GU_ARGS)
                       : launch_gate_up_bm<128, true, false, 0, kBlk>(MOE_GU_ARGS);
  return launch_gate_up_bm<64, true, false, 0, kBlk>(MOE_GU_ARGS);
#undef MOE_GU_ARGS
}

template <bool kBlk>
hipError_t down_fp4(int tile_m, const void* h, const uint8_t* h_scale, const int32_t* offsets,
                    const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                    const uint8_t* w2, const uint8_t* w2s, int A, int H, int I, uint16_t* y,
                    hipStream_t stream) {
#define MOE_DN_ARGS h, h_scale, offsets, tiles, num_tiles, max_tiles, w2, w2s, A, H, I, y, stream
  if (tile_m == 256) return launch_down_bm<256, true, false, 0, kBlk>(MOE_DN_ARGS);
  if (tile_m == 128)
    return I <= 2048   ? launch_down_bm<128, true, false, 1, kBlk>(MOE_DN_ARGS)
           : I <= 6144 ? launch_down_bm<128, true, false, 2, kBlk>(MOE_DN_ARGS)
                       : launch_down_bm<128, true, false, 0, kBlk>(MOE_DN_ARGS);
  return launch_down_bm<64, true, false, 0, kBlk>(MOE_DN_ARGS);
#undef MOE_DN_ARGS
}

}  // namespace

bool expert_gemm_tiled_supported(int tile_m, int act_fmt, int H, int I, int wfmt) {
  if (H % 256 || I % 128 || H <= 0 || I <= 0) return false;
  if (wfmt == 1) {                 // MXFP8 weights, bf16 activations: 64- and 128-row tiles
    if (act_fmt) return false;
    return tile_m == 64 ? fits<64, false, true>(H, I) : tile_m == 128 && fits<128, false, true>(H, I);
  }
  if (tile_m == 64) return act_fmt ? fits<64, true>(H, I) : fits<64, false>(H, I);
  if (tile_m == 128) return act_fmt ? fits<128, true>(H, I) : fits<128, false>(H, I);
  if (tile_m == 256) return act_fmt && fits<256, true>(H, I);
  return false;
}

// act_fmt: 0 bf16, 1 MXFP4 per token (gate/up) or per sorted row (down),
// 2 MXFP4 in the blocked sorted-row order.
hipError_t launch_gate_up_tiled(int tile_m, int act_fmt, int wfmt, const void* act,
                                const uint8_t* act_scale,
                                const int32_t* sorted, const int32_t* offsets,
                                const int32_t* tiles, const int32_t* num_tiles, int max_tiles,
                                const uint8_t* w13, const uint8_t* w13s, int T, int H, int I,
                                int Kp, uint16_t* h, hipStream_t stream, uint8_t* hq,
                                uint8_t* hs) {
  if (hq && !act_fmt) return hipErrorInvalidValue;
  if (wfmt == 1)
    return tile_m == 128 ? launch_gate_up_bm<128, false, true>(act, act_scale, sorted, offsets, tiles,
                                                               num_tiles, max_tiles, w13, w13s, T,
                                                               H, I, Kp, h, stream)
                         : launch_gate_up_bm<64, false, true>(act, act_scale, sorted, offsets, tiles,
                                                              num_tiles, max_tiles, w13, w13s, T, H,
                                                              I, Kp, h, stream);
  if (act_fmt == 2)
    return gate_up_fp4<true>(tile_m, act, act_scale, sorted, offsets, tiles, num_tiles, max_tiles,
                             w13, w13s, T, H, I, Kp, h, stream, hq, hs);
  if (act_fmt)
    return gate_up_fp4<false>(tile_m, act, act_scale, sorted, offsets, tiles, num_tiles, max_tiles,
                              w13, w13s, T, H, I, Kp, h, stream, hq, hs);
  return tile_m == 128 ? launch_gate_up_bm<128, false>(act, act_scale, sorted, offsets, tiles,
                                                       num_tiles, max_tiles, w13, w13s, T, H, I, Kp,
                                                       h, stream)
                       : launch_gate_up_bm<64, false>(act, act_scale, sorted, offsets, tiles,
                                                      num_tiles, max_tiles, w13, w13s, T, H, I, Kp,
                                                      h, stream);
}

hipError_t launch_down_tiled(int tile_m, int act_fmt, int wfmt, const void* h,
                             const uint8_t* h_scale,
                             const int32_t* offsets, const int32_t* tiles,
                             const int32_t* num_tiles, int max_tiles, const uint8_t* w2,
                             const uint8_t* w2s, int A, int H, int I, uint16_t* y,
                             hipStream_t stream) {
  if (wfmt == 1)
    return tile_m == 128 ? launch_down_bm<128, false, true>(h, h_scale, offsets, tiles, num_tiles,
                                                            max_tiles, w2, w2s, A, H, I, y, stream)
                         : launch_down_bm<64, false, true>(h, h_scale, offsets, tiles, num_tiles,
                                                           max_tiles, w2, w2s, A, H, I, y, stream);
  if (act_fmt == 2)
    return down_fp4<true>(tile_m, h, h_scale, offsets, tiles, num_tiles, max_tiles, w2, w2s, A, H,
                          I, y, stream);
  if (act_fmt)
    return down_fp4<false>(tile_m, h, h_scale, offsets, tiles, num_tiles, max_tiles, w2, w2s, A, H,
                           I, y, stream);
  if (tile_m == 128)
    return launch_down_bm<128, false>(h, h_scale, offsets, tiles, num_tiles, max_tiles, w2, w2s, A,
                                      H, I, y, stream);
  // two slices per workgroup where their scales fit beside each other
  if ((H / 256) % 2 == 0 && 2 * I <= TileCfg<64, false>::KMAX)
    return launch_down_bm<64, false, false, 0, false, 2>(h, h_scale, offsets, tiles, num_tiles,
                                                         max_tiles, w2, w2s, A, H, I, y, stream);
  return launch_down_bm<64, false>(h, h_scale, offsets, tiles, num_tiles, max_tiles, w2, w2s, A, H,
                                   I, y, stream);
}
