// Routing and grouping of a small batch in one workgroup: the softmax top-K
// of every token (routing.h) and then the stable grouping by expert with its
// tile table (grouping.h), the experts chosen handed over in LDS.  Same
// results as route_topk.hip followed by align_sort.hip, in one launch instead
// of two (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the
// specific optimisations: fused_topk at E = 512, K = 10, and the shared
// expert folded into the one MoE dispatch).
//
// Wave w of the 16 routes tokens w and w + 16 (NT of them, their dependency
// chains interleaved); after one barrier all 1024 threads group the T*K'
// assignments.  The smallest batches (at most 64 assignments) take a
// workgroup of one wave per token instead, whose first wave groups them.
// Used up to 128 / NPL tokens (32 at E <= 256, 16 at E <= 512, 8 at
// E <= 1024): there the one launch took 10-16 us against 16.5-18.5 us for
// the two.  Beyond, the routing of many tokens on one CU's four SIMDs (about
// 35 wave instructions per token and slot) costs more than the second
// launch, and the per-token route kernel spread over the chip wins.
#include "common.h"
#include "kernels.h"

MOE_DEBUG_FLAGS(debug_flags_route_align)

#include "grouping.h"
#include "routing.h"

namespace {

using namespace moe_grouping;
using namespace moe_routing;

constexpr int kMaxKeyTokens = 128;     // keys per lane x tokens of the one-launch path
constexpr size_t kMaxLds = 64 * 1024;

template <int NPL, int NT>
__global__ __launch_bounds__(kGroupThreads) void route_align_kernel(
    const float* __restrict__ logits, int ld, const float* __restrict__ gate, int gate_stride,
    int T, int E, int K, int shared, int renormalize, int tile_m, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ inv, int32_t* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  extern __shared__ int32_t sh[];      // group_small's LDS, then the chosen experts [T * K']
  __shared__ int tmp[17];
  const int Kp = K + shared, Ep = E + shared, A = T * Kp;
  int32_t* chosen = sh + group_small_lds_bytes(Ep) / 4;
  route_tokens<NPL, NT>(RowLogits{logits, ld}, GateLogit{gate, gate_stride}, threadIdx.x >> 6,
                        kGroupWaves, T, E, K, shared, renormalize,
                        [&](int t, int k, int e, float w) {
                          const int a = t * Kp + k;
                          ids[a] = e;
                          weights[a] = w;
                          chosen[a] = e;
                        });
  // (group_small's barrier after it clears its own LDS publishes chosen,
  // which it reads only then)
  group_small<false>([&](int a) { return chosen[a]; }, A, Ep, tile_m, counts, offsets, sorted, inv, tiles,
              num_tiles, sh, tmp);
}

int keys_per_lane(int E) { return E <= 256 ? 4 : E <= 512 ? 8 : 16; }

int tokens_per_wave(int T) { return T <= kGroupWaves ? 1 : 2; }

size_t lds_bytes(int T, int Kp, int Ep) { return group_small_lds_bytes(Ep) + (size_t)T * Kp * 4; }

// The smallest batches (T <= 16 tokens, T * K' <= 64 assignments): a
// workgroup of T waves, wave t routing token t, then the first wave groups
// the assignments (group_wave).  Dynamic LDS: the counts [Ep], then the
// chosen experts [64].  At T = 1 this took 6.7 us against 8.5 for the
// 1024-thread workgroup (E = 512, K' = 11) and 8.6 against 13.5 at E = 1024:
// the grouping's synchronisation of 16 waves over Ep experts is gone.
constexpr int kWaveMaxTokens = 16;
static_assert(64 * kMaxPerLane + 1 <= 64 * kWaveEPL, "group_wave's experts per lane");

template <int NPL>
__global__ __launch_bounds__(64 * kWaveMaxTokens) void route_align_wave_kernel(
    const float* __restrict__ logits, int ld, const float* __restrict__ gate, int gate_stride,
    int T, int E, int K, int shared, int renormalize, int tile_m, int32_t* __restrict__ ids,
    float* __restrict__ weights, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted, int32_t* __restrict__ inv, int32_t* __restrict__ tiles,
    int32_t* __restrict__ num_tiles) {
  extern __shared__ int32_t sh[];
  const int Kp = K + shared, Ep = E + shared, A = T * Kp;
  int32_t* chosen = sh + Ep;
  route_tokens<NPL, 1>(RowLogits{logits, ld}, GateLogit{gate, gate_stride}, threadIdx.x >> 6,
                       kWaveMaxTokens, T, E, K, shared, renormalize,
                       [&](int t, int k, int e, float w) {
                         const int a = t * Kp + k;
                         ids[a] = e;
                         weights[a] = w;
                         chosen[a] = e;
                       });
  // (group_wave's first barrier publishes chosen, which it reads only then)
  group_wave([&](int a) { return chosen[a]; }, A, Ep, tile_m, counts, offsets, sorted, inv, tiles,
             num_tiles, sh);
}

bool wave_fits(int T, int K, int shared) {
  return T >= 1 && T <= kWaveMaxTokens && (int64_t)T * (K + shared) <= kWaveMaxA;
}

template <int NPL>
void launch_wave(const float* logits, int ld, const float* gate, int gate_stride, int T, int E,
                 int K, int shared, int renormalize, int tile_m, int32_t* ids, float* weights,
                 int32_t* counts, int32_t* offsets, int32_t* sorted, int32_t* inv, int32_t* tiles,
                 int32_t* num_tiles, hipStream_t stream) {
  hipLaunchKernelGGL((route_align_wave_kernel<NPL>), dim3(1), dim3(64 * T),
                     (size_t)(E + shared + kWaveMaxA) * 4, stream, logits, ld, gate, gate_stride,
                     T, E, K, shared, renormalize, tile_m, ids, weights, counts, offsets, sorted,
                     inv, tiles, num_tiles);
}

template <int NPL, int NT>
void launch(const float* logits, int ld, const float* gate, int gate_stride, int T, int E, int K,
            int shared, int renormalize, int tile_m, int32_t* ids, float* weights, int32_t* counts,
            int32_t* offsets, int32_t* sorted, int32_t* inv, int32_t* tiles, int32_t* num_tiles,
            hipStream_t stream) {
  hipLaunchKernelGGL((route_align_kernel<NPL, NT>), dim3(1), dim3(kGroupThreads),
                     lds_bytes(T, K + shared, E + shared), stream, logits, ld, gate, gate_stride, T,
                     E, K, shared, renormalize, tile_m, ids, weights, counts, offsets, sorted, inv,
                     tiles, num_tiles);
}

}  // namespace

bool route_align_fits(int T, int E, int K, int shared) {
  if (T < 1 || E < 1 || E > 64 * kMaxPerLane) return false;
  if (keys_per_lane(E) * T > kMaxKeyTokens) return false;
  if ((int64_t)T * (K + shared) > moe_grouping::kGroupMaxA) return false;
  const int Kp = K + shared, Ep = E + shared;
  return Ep <= 2 * kGroupThreads && lds_bytes(T, Kp, Ep) <= kMaxLds;
}

hipError_t launch_route_align(const float* logits, int ld, const float* gate, int gate_stride,
                              int T, int E, int K, int shared, int renormalize, int tile_m,
                              int32_t* ids, float* weights, int32_t* counts, int32_t* offsets,
                              int32_t* sorted, int32_t* inv, int32_t* tiles, int32_t* num_tiles,
                              int32_t* scratch, hipStream_t stream) {
  if (!route_align_fits(T, E, K, shared)) {
    hipError_t e = launch_route_topk_rows(logits, ld, gate, gate_stride, T, E, K, shared,
                                          renormalize, ids, weights, stream);
    if (e != hipSuccess) return e;
    return launch_align_sort(ids, T * (K + shared), E + shared, tile_m, counts, offsets, sorted,
                             inv, tiles, num_tiles, scratch, stream);
  }
  if (wave_fits(T, K, shared)) {
#define MOE_RW_LAUNCH(P)                                                                         \
  launch_wave<P>(logits, ld, gate, gate_stride, T, E, K, shared, renormalize, tile_m, ids,        \
                 weights, counts, offsets, sorted, inv, tiles, num_tiles, stream)
    const int npl = keys_per_lane(E);
    if (npl == 4) MOE_RW_LAUNCH(4);
    else if (npl == 8) MOE_RW_LAUNCH(8);
    else MOE_RW_LAUNCH(kMaxPerLane);
#undef MOE_RW_LAUNCH
    return hipGetLastError();
  }
  const int npl = keys_per_lane(E), nt = tokens_per_wave(T);
#define MOE_RA_LAUNCH(P, N)                                                                      \
  launch<P, N>(logits, ld, gate, gate_stride, T, E, K, shared, renormalize, tile_m, ids, weights, \
               counts, offsets, sorted, inv, tiles, num_tiles, stream)
  // (NT = 2 only with 4 keys per lane: T <= 128 / NPL)
  if (npl == 4)
    nt == 1 ? MOE_RA_LAUNCH(4, 1) : MOE_RA_LAUNCH(4, 2);
  else if (npl == 8)
    MOE_RA_LAUNCH(8, 1);
  else
    MOE_RA_LAUNCH(kMaxPerLane, 1);
#undef MOE_RA_LAUNCH
  return hipGetLastError();
}
