// Group the flat assignments a = t*K' + k by expert: a histogram / prefix-scan
// permute that is stable (ascending a inside each expert's group) with no
// atomic deciding any order, plus the table of tile_m-row tiles that drive
// the grouped GEMMs (VibeSys "Qwen3.5-397B on 4x MI300A" post, section
// "Prefill, cache and speculation": 32-row tiles in the MoE kernel; the
// InferenceX Qwen3.5 post's shared-expert bullet: one MoE dispatch covers
// the routed experts and the shared one).
//
// Up to kSmallA assignments: one workgroup does everything in LDS
// (grouping.h: group_small).  Beyond:
// four launches over chunks of kChunk assignments:
//   1. per-chunk histograms            hist[b][e]
//   2. column scans, one block per 64 experts, each of its 16 waves owning a
//      slice of the chunks (rows of 64 experts per load, up to twelve in
//      flight): counts[e] and, in place, hist[b][e] = the count of e in the
//      chunks before b
//   3. one block: the exclusive scan over experts (offsets) and the tile
//      table
//   4. per-chunk stable scatter from offsets[e] + hist[b][e]: inside a
//      chunk, wave by wave in order, each lane's rank among the earlier
//      lanes with the same expert
// A lane's rank among equal experts in its wave comes from ballots: one per
// bit of the expert index, no data exchange.
#include "common.h"
#include "kernels.h"

MOE_DEBUG_FLAGS(debug_flags_align)

#include "grouping.h"

namespace {

using namespace moe_grouping;

constexpr int kChunk = 512;       // assignments per block in passes 1 and 4
constexpr int kScanThreads = kGroupThreads;
// Single-workgroup path up to this many assignments.  Above it the chunked
// kernels take ~13-14.5 us whatever A (E = 512, kernel trace); the one
// workgroup takes 4.1 us at 704 assignments, 8.1 at 2,112, 8.6 at 2,816,
// 12.3 at 4,224, 14.6 at 5,632 and 19.2 at 8,184.
constexpr int kSmallA = 5120;
static_assert(kSmallA <= moe_grouping::kGroupMaxA, "group_small's register-held ids");
constexpr int kSlices = kScanThreads / 64;   // chunk slices of a column scan: one per wave
constexpr int kBatch = 12;        // histogram loads in flight per lane in a column scan

__global__ __launch_bounds__(256) void align_hist_kernel(const int32_t* __restrict__ ids, int A,
                                                         int Ep, int32_t* __restrict__ hist) {
  extern __shared__ int32_t sh[];
  for (int e = threadIdx.x; e < Ep; e += blockDim.x) sh[e] = 0;
  __syncthreads();
  const int a0 = blockIdx.x * kChunk;
  const int a1 = min(A, a0 + kChunk);
  for (int a = a0 + threadIdx.x; a < a1; a += blockDim.x) {
    const int e = ids[a];
    if ((unsigned)e < (unsigned)Ep) atomicAdd(&sh[e], 1);   // ids outside [0, Ep) are skipped
  }
  __syncthreads();
  for (int e = threadIdx.x; e < Ep; e += blockDim.x) hist[(size_t)blockIdx.x * Ep + e] = sh[e];
}

// Lane's expert e = 64 * block + lane; wave w's slice of the chunks,
// [b0, b0 + n): f(j, count of e in chunk b0 + j) for j ascending, loads
// kBatch at a time.
template <class F>
__device__ __forceinline__ void for_slice(const int32_t* hist, int Ep, int e, int b0, int n,
                                          F&& f) {
  for (int j0 = 0; j0 < n; j0 += kBatch) {
    int v[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      v[k] = j0 + k < n && e < Ep ? hist[(size_t)(b0 + j0 + k) * Ep + e] : 0;
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      if (j0 + k < n && e < Ep) f(j0 + k, v[k]);
  }
}

__global__ __launch_bounds__(kScanThreads) void align_colscan_kernel(
    int32_t* __restrict__ hist, int nb, int Ep, int32_t* __restrict__ counts) {
  __shared__ int part[kSlices][64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int e = 64 * blockIdx.x + lane;
  const int per = (nb + kSlices - 1) / kSlices;
  const int b0 = min(nb, w * per), n = min(nb, b0 + per) - b0;
  int sum = 0;
  for_slice(hist, Ep, e, b0, n, [&](int, int v) { sum += v; });
  part[w][lane] = sum;
  __syncthreads();
  int run = 0, total = 0;
  for (int s = 0; s < kSlices; ++s) {
    const int c = part[s][lane];
    run += s < w ? c : 0;
    total += c;
  }
  if (w == 0 && e < Ep) counts[e] = total;
  for_slice(hist, Ep, e, b0, n, [&](int j, int v) {
    hist[(size_t)(b0 + j) * Ep + e] = run;
    run += v;
  });
}

__global__ __launch_bounds__(kScanThreads) void align_offsets_kernel(
    const int32_t* __restrict__ counts, int A, int Ep, int tile_m, int32_t* __restrict__ offsets,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  __shared__ int tmp[17];
  __shared__ int tstart[2 * kScanThreads + 1], roff[2 * kScanThreads];
  group_offsets<true>([&](int e) { return counts[e]; }, A, Ep, tile_m, offsets, tiles, num_tiles,
                      tmp, tstart, roff, [](int, int, int) {});
}

__global__ __launch_bounds__(256) void align_scatter_kernel(
    const int32_t* __restrict__ ids, int A, int Ep, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ before, int32_t* __restrict__ sorted, int32_t* __restrict__ inv) {
  extern __shared__ int32_t pos[];
  for (int e = threadIdx.x; e < Ep; e += blockDim.x)
    pos[e] = offsets[e] + before[(size_t)blockIdx.x * Ep + e];
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int a0 = blockIdx.x * kChunk;
  const int a1 = min(A, a0 + kChunk);
  for (int r = a0; r < a1; r += 256) {
    const int a = r + threadIdx.x;
    int e = (a < A) ? ids[a] : -1;
    if ((unsigned)e >= (unsigned)Ep) e = -1;
    int rank, same;
    wave_match_rank(e, expert_bits(Ep), &rank, &same);
    for (int w = 0; w < 4; ++w) {
      if (w == wave && e >= 0) {
        int p = pos[e] + rank;
        if (MOE_DOK(p >= 0 && p < A, kDbgAlign)) {
          sorted[p] = a;
          if (inv) inv[a] = p;
        }
        if (rank == same - 1) pos[e] = p + 1;    // the last lane of this expert advances it
      }
      __syncthreads();
    }
  }
}


// Everything for A <= kSmallA in one workgroup of kScanThreads threads.
__global__ __launch_bounds__(kScanThreads) void align_small_kernel(
    const int32_t* __restrict__ ids, int A, int Ep, int tile_m, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ sorted, int32_t* __restrict__ inv,
    int32_t* __restrict__ tiles, int32_t* __restrict__ num_tiles) {
  extern __shared__ int32_t sh[];          // group_small_lds_bytes(Ep)
  __shared__ int tmp[17];
  group_small<true>([&](int a) { return ids[a]; }, A, Ep, tile_m, counts, offsets, sorted, inv, tiles,
              num_tiles, sh, tmp);
}

}  // namespace

size_t align_scratch_bytes(int A, int Ep) {
  const int nb = (A + kChunk - 1) / kChunk;
  return (size_t)(nb > 0 ? nb : 1) * Ep * sizeof(int32_t);
}

hipError_t launch_align_sort(const int32_t* ids, int A, int Ep, int tile_m, int32_t* counts,
                             int32_t* offsets, int32_t* sorted, int32_t* inv, int32_t* tiles,
                             int32_t* num_tiles, int32_t* scratch, hipStream_t stream) {
  if (A <= kSmallA) {
    hipLaunchKernelGGL(align_small_kernel, dim3(1), dim3(kScanThreads), group_small_lds_bytes(Ep),
                       stream, ids, A, Ep, tile_m, counts, offsets, sorted, inv, tiles, num_tiles);
    return hipGetLastError();
  }
  const int nb = (A + kChunk - 1) / kChunk;
  const size_t lds = (size_t)Ep * sizeof(int32_t);
  hipLaunchKernelGGL(align_hist_kernel, dim3(nb), dim3(256), lds, stream, ids, A, Ep, scratch);
  hipLaunchKernelGGL(align_colscan_kernel, dim3((Ep + 63) / 64), dim3(kScanThreads), 0, stream,
                     scratch, nb, Ep, counts);
  hipLaunchKernelGGL(align_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, counts, A, Ep,
                     tile_m, offsets, tiles, num_tiles);
  hipLaunchKernelGGL(align_scatter_kernel, dim3(nb), dim3(256), lds, stream, ids, A, Ep, offsets,
                     scratch, sorted, inv);
  return hipGetLastError();
}
