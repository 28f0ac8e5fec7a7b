// Softmax top-K routing: one wavefront per token.
//
// The experts are selected on the fp32 logits (softmax is monotone), ordered
// by (logit descending, expert index ascending), with -0.0 equal to +0.0
// (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the specific
// optimisations, fused_topk bullet: softmax-scored top-K at E = 512, K = 10).
// The weights are exp(l_k - l_0) / sum_k' exp(l_k' - l_0) over the K
// selected experts (renormalised) or over all E (not renormalised).  With a
// folded-in shared expert, slot K holds expert E with weight sigmoid(g)
// (same post, shared-expert fusion bullet: the shared expert becomes expert
// top-K+1 of the one MoE dispatch).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kMaxPerLane = 16;   // E <= 1024

// Orderable key: larger key = larger logit, ties -> smaller expert index.
__device__ __forceinline__ uint64_t route_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;                       // -0.0 == +0.0
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);     // monotone in v
  return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_value(uint64_t key) {
  uint32_t u = (uint32_t)(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    uint32_t lo = __shfl_xor((unsigned)(v & 0xFFFFFFFFu), m, MOE_WAVE);
    uint32_t hi = __shfl_xor((unsigned)(v >> 32), m, MOE_WAVE);
    uint64_t o = ((uint64_t)hi << 32) | lo;
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ gate, int T, int E, int K,
    int shared, int renormalize, int32_t* __restrict__ ids, float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;
  const int Kp = K + shared;

  uint64_t key[kMaxPerLane];
#pragma unroll
  for (int j = 0; j < kMaxPerLane; ++j) {
    int e = lane + 64 * j;
    key[j] = (e < E) ? route_key(row[e], e) : 0ull;    // 0 = never selected
  }

  float lmax = 0.f, sel_val = 0.f;
  int sel_e = 0;
  for (int k = 0; k < K; ++k) {
    uint64_t best = 0ull;
#pragma unroll
    for (int j = 0; j < kMaxPerLane; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    const float v = key_value(best);
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j < kMaxPerLane; ++j)
        if (j == (e >> 6)) key[j] = 0ull;
    }
    if (k == 0) lmax = v;
    if (lane == k) { sel_e = e; sel_val = v; }
  }

  // Denominator: over the K selected (renormalised) or over all E.
  float num = (lane < K) ? expf(sel_val - lmax) : 0.f;
  float den;
  if (renormalize) {
    den = wave_sum_f32(num);
  } else {
    float s = 0.f;
    for (int e = lane; e < E; e += 64) s += expf(row[e] - lmax);
    den = wave_sum_f32(s);
  }
  if (lane < K) {
    ids[(size_t)t * Kp + lane] = sel_e;
    weights[(size_t)t * Kp + lane] = num / den;
  }
  if (shared && lane == 0) {
    ids[(size_t)t * Kp + K] = E;
    weights[(size_t)t * Kp + K] = 1.0f / (1.0f + expf(-gate[t]));
  }
}

}  // namespace

hipError_t launch_route_topk(const float* logits, const float* gate, int T, int E, int K,
                             int shared, int renormalize, int32_t* ids, float* weights,
                             hipStream_t stream) {
  dim3 grid((T + 3) / 4), block(256);
  hipLaunchKernelGGL(route_topk_kernel, grid, block, 0, stream, logits, gate, T, E, K, shared,
                     renormalize, ids, weights);
  return hipGetLastError();
}
