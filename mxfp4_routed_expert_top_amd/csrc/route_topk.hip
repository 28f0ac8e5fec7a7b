// Softmax top-K routing: one wavefront per token (the per-token work is in
// routing.h).
//
// The experts are selected on the fp32 logits (softmax is monotone), ordered
// by (logit descending, expert index ascending), with -0.0 equal to +0.0
// (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the specific
// optimisations, fused_topk bullet: softmax-scored top-K at E = 512, K = 10).
// The weights are exp(l_k - l_0) / sum_k' exp(l_k' - l_0) over the K
// selected experts (renormalised) or over all E (not renormalised).  With a
// folded-in shared expert, slot K holds expert E with weight sigmoid(g)
// (same post, shared-expert fusion bullet: the shared expert becomes expert
// top-K+1 of the one MoE dispatch).  The logits come either from the caller
// or from the router GEMM (router_gemm.hip), whose split partial sums are
// first added in a fixed order.
#include "common.h"
#include "kernels.h"
#include "routing.h"

namespace {

using namespace moe_routing;

// logits fp32 rows of stride ld; the shared gate logit of token t at
// gate[t * gate_stride].  One token per wave, four waves per block.
template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int ld, const float* __restrict__ gate, int gate_stride,
    int T, int E, int K, int shared, int renormalize, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const size_t Kp = (size_t)(K + shared);
  route_tokens<NPL, 1>(RowLogits{logits, ld}, GateLogit{gate, gate_stride}, t, 0, T, E, K, shared,
                       renormalize, [&](int tt, int k, int e, float w) {
                         ids[tt * Kp + k] = e;
                         weights[tt * Kp + k] = w;
                       });
}

// The router GEMM's S partial sums P[s] (fp32 [S, n]) added in split order
// (a fixed order: equal inputs give equal logits): out[i] = sum_s P[s][i].
// All S loads of an element are issued before the adds.
constexpr int kMaxSplits = 32;

__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ partial, int S,
                                                         int64_t n, float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float v[kMaxSplits];
#pragma unroll
  for (int s = 0; s < kMaxSplits; ++s) v[s] = s < S ? partial[s * n + i] : 0.f;
  float acc = v[0];
#pragma unroll
  for (int s = 1; s < kMaxSplits; ++s)
    if (s < S) acc += v[s];
  out[i] = acc;
}

}  // namespace

// Keys per lane for E experts: 4, 8 or 16.
hipError_t launch_route_topk_rows(const float* logits, int ld, const float* gate,
                                  int gate_stride, int T, int E, int K, int shared,
                                  int renormalize, int32_t* ids, float* weights,
                                  hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
  if (E <= 256)
    hipLaunchKernelGGL(route_topk_kernel<4>, grid, block, 0, stream, logits, ld, gate,
                       gate_stride, T, E, K, shared, renormalize, ids, weights);
  else if (E <= 512)
    hipLaunchKernelGGL(route_topk_kernel<8>, grid, block, 0, stream, logits, ld, gate,
                       gate_stride, T, E, K, shared, renormalize, ids, weights);
  else
    hipLaunchKernelGGL(route_topk_kernel<kMaxPerLane>, grid, block, 0, stream, logits, ld, gate,
                       gate_stride, T, E, K, shared, renormalize, ids, weights);
  return hipGetLastError();
}

hipError_t launch_route_topk(const float* logits, const float* gate, int T, int E, int K,
                             int shared, int renormalize, int32_t* ids, float* weights,
                             hipStream_t stream) {
  return launch_route_topk_rows(logits, E, gate, 1, T, E, K, shared, renormalize, ids, weights,
                                stream);
}

int route_max_splits() { return kMaxSplits; }

hipError_t launch_sum_splits(const float* partial, int S, int T, int Ep, float* logits,
                             hipStream_t stream) {
  if (S <= 1) return hipSuccess;     // one split: the router GEMM wrote the logits itself
  const int64_t n = (int64_t)T * Ep;
  hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     partial, S, n, logits);
  return hipGetLastError();
}

hipError_t launch_route_topk_split(const float* partial, int S, int T, int E, int K, int shared,
                                   int renormalize, int32_t* ids, float* weights, float* logits,
                                   hipStream_t stream) {
  const int Ep = E + shared;
  hipError_t e = launch_sum_splits(partial, S, T, Ep, logits, stream);
  if (e != hipSuccess) return e;
  return launch_route_topk_rows(logits, Ep, logits + E, Ep, T, E, K, shared, renormalize, ids,
                                weights, stream);
}
