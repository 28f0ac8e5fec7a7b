// Device helpers of the grouping by expert (align_sort.hip, and the fused
// small-batch routing + grouping of route_align.hip): a stable histogram /
// prefix-scan permute of the flat assignments a = t*K' + k (ascending a
// inside each expert's group) and the table of tile_m-row tiles that drive
// the grouped GEMMs (VibeSys "Qwen3.5-397B on 4x MI300A" post, section
// "Prefill, cache and speculation": 32-row tiles in the MoE kernel).
//
// A file that includes this header first defines its debug flag word with
// MOE_DEBUG_FLAGS (the position checks below report into it).
#pragma once
#include "common.h"

namespace moe_grouping {

constexpr int kGroupThreads = 1024;           // one-workgroup grouping
constexpr int kGroupWaves = kGroupThreads / 64;

// Rank of this lane among the lanes of its wave holding the same expert e
// (lower lanes first) and the number of such lanes; e < 0 takes no part
// (rank = same = 0).  Experts are below 2^nbits (expert_bits).  One ballot
// per bit of the expert index: each lane keeps the lanes that agree with it
// on every bit, which are exactly the lanes holding its own expert.  A fixed
// cost, where one ballot round per distinct expert in the wave took ~60
// rounds under near-uniform routing.
__device__ __forceinline__ void wave_match_rank(int e, int nbits, int* rank, int* same) {
  const int lane = threadIdx.x & 63;
  uint64_t m = __ballot(e >= 0);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = (e >> b) & 1;
    const uint64_t ones = __ballot(bit);
    m &= bit ? ones : ~ones;
  }
  const bool ok = e >= 0;
  *rank = ok ? __popcll(m & ((1ull << lane) - 1ull)) : 0;
  *same = ok ? __popcll(m) : 0;
}

// Bits of an expert index below Ep.
__device__ __forceinline__ int expert_bits(int Ep) { return Ep <= 1 ? 0 : 32 - __clz(Ep - 1); }

// x plus the value DPP control CTRL moves into this lane (0 where it moves
// none: rows outside ROWMASK, or a row shift's first lanes)
template <int CTRL, int ROWMASK>
__device__ __forceinline__ int dpp_add(int x) {
  return x + __builtin_amdgcn_update_dpp(0, x, CTRL, ROWMASK, 0xF, false);
}

// Inclusive sum over the lanes of a wave, lane order, all in DPP lane moves
// (no LDS round trips, where a __shfl_up step is an LDS permute and a wait):
// shifts by 1, 2, 4 and 8 inside each 16-lane row, then row 0's total into
// row 1 and row 2's into row 3 (row_bcast:15), then lane 31's into rows 2
// and 3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_scan(int x) {
  x = dpp_add<0x111, 0xF>(x);                         // row_shr:1
  x = dpp_add<0x112, 0xF>(x);                         // row_shr:2
  x = dpp_add<0x114, 0xF>(x);                         // row_shr:4
  x = dpp_add<0x118, 0xF>(x);                         // row_shr:8
  x = dpp_add<0x142, 0xA>(x);                         // row_bcast:15 into rows 1, 3
  x = dpp_add<0x143, 0xC>(x);                         // row_bcast:31 into rows 2, 3
  return x;
}

// Exclusive scan of one value per thread over a 1024-thread block.
__device__ __forceinline__ int block_exclusive_scan(int v, int* tmp /* >= 17 ints */, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_scan(v);
  if (lane == 63) tmp[wave] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int w = 0; w < kGroupWaves; ++w) {
      int c = tmp[w];
      tmp[w] = run;
      run += c;
    }
    tmp[16] = run;
  }
  __syncthreads();
  int r = x - v + tmp[wave];
  *total = tmp[16];
  __syncthreads();
  return r;
}

// Counts [Ep] -> offsets [Ep + 1] (offsets[Ep] = A) and the tile table; each
// thread owns experts 2 tid and 2 tid + 1 (Ep <= 2048).  cnt_of(e) is the
// count of expert e; first(e, count, offset) is called for each owned expert.
// The table (expert-major, row start ascending) is written either by the
// owner of each expert, entry after entry, or (kByEntry) entry by entry,
// thread q taking entry q: its expert is the last one whose first entry
// tstart[e] is <= q, found by a binary search in LDS, so that a wave's stores
// are contiguous.  With many entries per expert the owners' stores touch 64
// cache lines each (3,060 entries: 11.3 us, by entry 5.1); with about one
// per expert (the decode batch) the search and its barrier cost more
// (6.95 -> 7.21 us).  kByEntry: tstart is LDS of Ep + 1 ints and roff LDS of
// Ep ints (the experts' row offsets); otherwise both unused.
template <bool kByEntry, class Cnt, class First>
__device__ __forceinline__ void group_offsets(Cnt&& cnt_of, int A, int Ep, int tile_m,
                                              int32_t* __restrict__ offsets,
                                              int32_t* __restrict__ tiles,
                                              int32_t* __restrict__ num_tiles, int* tmp,
                                              int* tstart, int* roff, First&& first) {
  int c[2] = {0, 0};
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * threadIdx.x + q;
    if (e < Ep) c[q] = cnt_of(e);
  }
  int total;
  const int base = block_exclusive_scan(c[0] + c[1], tmp, &total);
  const int off[2] = {base, base + c[0]};
  const int nt[2] = {(c[0] + tile_m - 1) / tile_m, (c[1] + tile_m - 1) / tile_m};
  int ttotal;
  const int tbase = block_exclusive_scan(nt[0] + nt[1], tmp, &ttotal);
  const int toff[2] = {tbase, tbase + nt[0]};
  [[maybe_unused]] const int max_tiles = (A + tile_m - 1) / tile_m + Ep;
  for (int q = 0; q < 2; ++q) {
    const int e = 2 * threadIdx.x + q;
    if (e < Ep) {
      offsets[e] = off[q];
      first(e, c[q], off[q]);
      if constexpr (kByEntry) {
        tstart[e] = toff[q];
        roff[e] = off[q];
      } else if (tiles) {
        for (int j = 0; j < nt[q]; ++j)
          if (MOE_DOK(toff[q] + j < max_tiles, kDbgAlign)) {
            tiles[2 * (toff[q] + j)] = e;
            tiles[2 * (toff[q] + j) + 1] = off[q] + j * tile_m;
          }
      }
    }
  }
  if (threadIdx.x == 0) {
    offsets[Ep] = A;
    *num_tiles = ttotal;
    if constexpr (kByEntry) tstart[Ep] = ttotal;
  }
  if (!kByEntry || !tiles) return;                    // (uniform in the block)
  __syncthreads();
  for (int q = threadIdx.x; q < ttotal; q += blockDim.x) {
    int lo = 0, hi = Ep;                              // tstart[lo] <= q < tstart[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tstart[mid] <= q) lo = mid;
      else hi = mid;
    }
    if (MOE_DOK(q < max_tiles, kDbgAlign)) {
      tiles[2 * q] = lo;
      tiles[2 * q + 1] = roff[lo] + (q - tstart[lo]) * tile_m;
    }
  }
}

// LDS bytes of group_small: cnt [Ep] and pos [Ep] ints, then a byte per
// (wave, expert).
__host__ __device__ constexpr size_t group_small_lds_bytes(int Ep) {
  return (size_t)2 * Ep * 4 + (((size_t)kGroupWaves * Ep + 3) & ~(size_t)3);
}

// Largest A of group_small: a thread keeps the ids of its assignments
// a = tid + 1024 i in registers (loaded once and used by both the histogram
// and the scatter).
constexpr int kGroupRounds = 5;
constexpr int kGroupMaxA = kGroupRounds * kGroupThreads;

// The whole grouping in one workgroup of kGroupThreads threads, A <=
// kGroupMaxA.  ids(a) is the expert of assignment a (ids outside [0, Ep)
// take no part).  kEarly: the ids are read on entry, so their loads overlap
// the clearing of the count table (ids in global memory); otherwise after
// the barrier that follows the clearing, which then also publishes ids that
// other threads of the workgroup have just written (the fused routing's
// LDS).  sh holds group_small_lds_bytes(Ep) bytes of LDS, tmp >= 17 ints.
//
// The scatter goes in rounds of 1024 assignments, one per thread.  A
// thread's position is its expert's running offset, plus the count of that
// expert in the round's earlier waves (a byte per (wave, expert), written by
// the first lane of each expert in each wave), plus its rank among the equal
// lanes of its own wave.  Between rounds each expert's offset advances by its
// count in the round.
template <bool kEarly, class Ids>
__device__ __forceinline__ void group_small(Ids&& ids, int A, int Ep, int tile_m,
                                            int32_t* __restrict__ counts,
                                            int32_t* __restrict__ offsets,
                                            int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
                                            int32_t* __restrict__ tiles,
                                            int32_t* __restrict__ num_tiles, int32_t* sh,
                                            int* tmp) {
  int32_t* cnt = sh;
  int32_t* pos = sh + Ep;
  uint8_t* tab = (uint8_t*)(sh + 2 * Ep);             // [kGroupWaves][Ep]
  const int tid = threadIdx.x;
  // the expert of assignment a, -1 for none or one outside [0, Ep)
  auto id_at = [&](int a) -> int {
    const int e = a < A ? ids(a) : -1;
    return (unsigned)e < (unsigned)Ep ? e : -1;
  };
  int ev[kEarly ? kGroupRounds : 1];                 // (kEarly) the thread's ids, round by round
  if constexpr (kEarly) {
#pragma unroll
    for (int i = 0; i < kGroupRounds; ++i) ev[i] = id_at(i * kGroupThreads + tid);
  }
  for (int e = tid; e < Ep; e += kGroupThreads) cnt[e] = 0;
  for (int i = tid; i < (kGroupWaves * Ep + 3) / 4; i += kGroupThreads) ((uint32_t*)tab)[i] = 0u;
  __syncthreads();
  if constexpr (kEarly) {
#pragma unroll
    for (int i = 0; i < kGroupRounds; ++i)
      if (ev[i] >= 0) atomicAdd(&cnt[ev[i]], 1);
  } else {
    for (int a = tid; a < A; a += kGroupThreads) {
      const int e = id_at(a);
      if (e >= 0) atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  group_offsets<false>([&](int e) { return cnt[e]; }, A, Ep, tile_m, offsets, tiles, num_tiles,
                       tmp, nullptr, nullptr, [&](int e, int c, int off) {
                         counts[e] = c;
                         pos[e] = off;
                       });
  // (pos is read only after the barrier that follows the table's writes)
  const int wave = tid >> 6;
  // one round: assignment a = r + tid of expert e (or -1)
  auto scatter = [&](int r, int e) {
    const int a = r + tid;
    int rank, same;
    wave_match_rank(e, expert_bits(Ep), &rank, &same);
    if (e >= 0 && rank == 0) tab[wave * Ep + e] = (uint8_t)same;
    __syncthreads();
    if (e >= 0) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += tab[w * Ep + e];
      const int p = pos[e] + before + rank;
      if (MOE_DOK(p >= 0 && p < A, kDbgAlign)) {
        sorted[p] = a;
        if (inv) inv[a] = p;
      }
    }
    if (r + kGroupThreads < A) {                     // another round (block-uniform)
      __syncthreads();
      for (int x = tid; x < Ep; x += kGroupThreads) {
        int s = 0;
        for (int w = 0; w < kGroupWaves; ++w) {
          s += tab[w * Ep + x];
          tab[w * Ep + x] = 0;
        }
        pos[x] += s;
      }
      __syncthreads();
    }
  };
  if constexpr (kEarly) {
#pragma unroll
    for (int i = 0; i < kGroupRounds; ++i) {
      if (i * kGroupThreads >= A) break;             // block-uniform
      scatter(i * kGroupThreads, ev[i]);
    }
  } else {
    for (int r = 0; r < A; r += kGroupThreads) scatter(r, id_at(r + tid));
  }
}

// The grouping of at most kWaveMaxA assignments by the first wave of a
// workgroup (the other waves, if any, only clear the count table and take
// the barriers): the same counts, offsets, sorted order, inverse map and tile
// table as group_small.  Lane a takes assignment a; the expert counts go
// through LDS atomics; lane l owns the experts [l * epl, l * epl + epl)
// (epl = ceil(Ep / 64) <= kWaveEPL) and wave scans of their counts and tile
// counts give the offsets and the tile table; each assignment lands at its
// expert's offset plus its rank among the lanes of the same expert.  ids(a)
// is read after the first barrier (which publishes ids that the workgroup
// has just written to LDS).  cnt: LDS of Ep ints.
constexpr int kWaveMaxA = 64;
constexpr int kWaveEPL = 17;                          // Ep <= 64 * 17

__device__ __forceinline__ int wave_exclusive_scan(int v) { return wave_inclusive_scan(v) - v; }

template <class Ids>
__device__ __forceinline__ void group_wave(Ids&& ids, int A, int Ep, int tile_m,
                                           int32_t* __restrict__ counts,
                                           int32_t* __restrict__ offsets,
                                           int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
                                           int32_t* __restrict__ tiles,
                                           int32_t* __restrict__ num_tiles, int32_t* cnt) {
  const int lane = threadIdx.x & 63;
  const bool first = threadIdx.x < 64;                // (a wave-uniform condition)
  for (int x = threadIdx.x; x < Ep; x += blockDim.x) cnt[x] = 0;
  __syncthreads();
  int e = first && lane < A ? ids(lane) : -1;
  if ((unsigned)e >= (unsigned)Ep) e = -1;
  if (e >= 0) atomicAdd(&cnt[e], 1);
  __syncthreads();
  if (first) {
    const int epl = (Ep + 63) / 64, e0 = lane * epl;
    int c[kWaveEPL];
    int sum = 0, tsum = 0;
#pragma unroll
    for (int j = 0; j < kWaveEPL; ++j) {
      c[j] = (j < epl && e0 + j < Ep) ? cnt[e0 + j] : 0;
      sum += c[j];
      tsum += (c[j] + tile_m - 1) / tile_m;
    }
    int off = wave_exclusive_scan(sum), toff = wave_exclusive_scan(tsum);
    const int ntiles = __builtin_amdgcn_readlane(toff + tsum, 63);
    [[maybe_unused]] const int max_tiles = (A + tile_m - 1) / tile_m + Ep;
#pragma unroll
    for (int j = 0; j < kWaveEPL; ++j) {
      const int x = e0 + j;
      if (j < epl && x < Ep) {
        counts[x] = c[j];
        offsets[x] = off;
        cnt[x] = off;                                 // (the scatter's positions)
        if (tiles)
          for (int q = 0; q * tile_m < c[j]; ++q)
            if (MOE_DOK(toff + q < max_tiles, kDbgAlign)) {
              tiles[2 * (toff + q)] = x;
              tiles[2 * (toff + q) + 1] = off + q * tile_m;
            }
        off += c[j];
        toff += (c[j] + tile_m - 1) / tile_m;
      }
    }
    if (lane == 0) {
      offsets[Ep] = A;
      *num_tiles = ntiles;
    }
  }
  __syncthreads();
  if (first) {
    int rank, same;
    wave_match_rank(e, expert_bits(Ep), &rank, &same);
    if (e >= 0) {
      const int p = cnt[e] + rank;
      if (MOE_DOK(p >= 0 && p < A, kDbgAlign)) {
        sorted[p] = lane;
        if (inv) inv[lane] = p;
      }
    }
  }
}

}  // namespace moe_grouping
