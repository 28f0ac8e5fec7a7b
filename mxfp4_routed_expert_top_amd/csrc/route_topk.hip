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
// top-K+1 of the one MoE dispatch).  The logits come either from the caller
// or from the router GEMM (router_gemm.hip), whose split partial sums are
// first added in a fixed order.
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

// Wave-wide maximum of a 64-bit key held as (hi, lo), with DPP lane moves
// (no LDS round trip): quad swaps, half-row and row mirrors, then row
// broadcasts; lane 63 ends with the maximum, which is read back as a scalar.
template <int CTRL, int ROWMASK>
__device__ __forceinline__ void dpp_max_step(uint32_t& hi, uint32_t& lo) {
  const uint32_t h2 = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROWMASK, 0xF, false);
  const uint32_t l2 = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROWMASK, 0xF, false);
  const bool gt = (h2 > hi) || (h2 == hi && l2 > lo);
  hi = gt ? h2 : hi;
  lo = gt ? l2 : lo;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  dpp_max_step<0xB1, 0xF>(hi, lo);    // quad_perm [1,0,3,2]
  dpp_max_step<0x4E, 0xF>(hi, lo);    // quad_perm [2,3,0,1]
  dpp_max_step<0x141, 0xF>(hi, lo);   // row_half_mirror
  dpp_max_step<0x140, 0xF>(hi, lo);   // row_mirror
  dpp_max_step<0x142, 0xA>(hi, lo);   // row_bcast:15 into rows 1, 3
  dpp_max_step<0x143, 0xC>(hi, lo);   // row_bcast:31 into rows 2, 3
  hi = (uint32_t)__builtin_amdgcn_readlane((int)hi, 63);
  lo = (uint32_t)__builtin_amdgcn_readlane((int)lo, 63);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, MOE_WAVE);
  return v;
}

// Logits straight from an fp32 [T, ld] array.
struct RowLogits {
  const float* l;
  int ld;
  __device__ __forceinline__ float operator()(int t, int e) const { return l[(size_t)t * ld + e]; }
};

// One wave routes token t.  g = the shared expert's gate logit (used when
// shared = 1).  Lane l holds the keys of experts l, l + 64, ..., NPL of
// them (E <= 64 NPL), sorted descending once; each of the K rounds then
// takes the wave-wide maximum of the lanes' first keys (the next slot), and
// the lane that held it shifts its list by one.
template <int NPL>
__device__ __forceinline__ void route_token(const RowLogits& src, int t, int E, int K, int shared,
                                            int renormalize, float g, int32_t* __restrict__ ids,
                                            float* __restrict__ weights) {
  const int lane = threadIdx.x & 63;
  const int Kp = K + shared;

  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j) {
    int e = lane + 64 * j;
    key[j] = (e < E) ? route_key(src(t, e), e) : 0ull;    // 0 = never selected
  }
#pragma unroll
  for (int i = 1; i < NPL; ++i)                           // insertion network, descending
#pragma unroll
    for (int j = i; j > 0; --j) {
      const uint64_t a = key[j - 1], b = key[j];
      key[j - 1] = a > b ? a : b;
      key[j] = a > b ? b : a;
    }

  // Selected values are wave-uniform, so every lane accumulates the
  // renormalised denominator itself, in slot order.
  float lmax = 0.f, den = 0.f, num = 0.f;
  int sel_e = 0;
  for (int k = 0; k < K; ++k) {
    const uint64_t best = wave_max_u64(key[0]);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
    const float v = key_value(best);
    if ((e & 63) == lane) {
#pragma unroll
      for (int j = 0; j + 1 < NPL; ++j) key[j] = key[j + 1];
      key[NPL - 1] = 0ull;
    }
    if (k == 0) lmax = v;
    const float ek = expf(v - lmax);
    den += ek;
    if (lane == k) {
      sel_e = e;
      num = ek;
    }
  }

  if (!renormalize) {
    float s = 0.f;
    for (int e = lane; e < E; e += 64) s += expf(src(t, e) - lmax);
    den = wave_sum_f32(s);
  }
  if (lane < K) {
    ids[(size_t)t * Kp + lane] = sel_e;
    weights[(size_t)t * Kp + lane] = num / den;
  }
  if (shared && lane == 0) {
    ids[(size_t)t * Kp + K] = E;
    weights[(size_t)t * Kp + K] = 1.0f / (1.0f + expf(-g));
  }
}

// logits fp32 rows of stride ld; the shared gate logit of token t at
// gate[t * gate_stride].
template <int NPL>
__global__ __launch_bounds__(256) void route_topk_kernel(
    const float* __restrict__ logits, int ld, const float* __restrict__ gate, int gate_stride,
    int T, int E, int K, int shared, int renormalize, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  route_token<NPL>(RowLogits{logits, ld}, t, E, K, shared, renormalize,
                   shared ? gate[(size_t)t * gate_stride] : 0.f, ids, weights);
}

// Keys per lane for E experts: 4, 8 or 16.
hipError_t launch_route_kernel(const float* logits, int ld, const float* gate, int gate_stride,
                               int T, int E, int K, int shared, int renormalize, int32_t* ids,
                               float* weights, hipStream_t stream) {
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

hipError_t launch_route_topk(const float* logits, const float* gate, int T, int E, int K,
                             int shared, int renormalize, int32_t* ids, float* weights,
                             hipStream_t stream) {
  return launch_route_kernel(logits, E, gate, 1, T, E, K, shared, renormalize, ids, weights,
                             stream);
}

int route_max_splits() { return kMaxSplits; }

hipError_t launch_route_topk_split(const float* partial, int S, int T, int E, int K, int shared,
                                   int renormalize, int32_t* ids, float* weights, float* logits,
                                   hipStream_t stream) {
  const int Ep = E + shared;
  const int64_t n = (int64_t)T * Ep;
  if (S > 1) {                       // one split: the router GEMM wrote the logits itself
    hipLaunchKernelGGL(sum_splits_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       partial, S, n, logits);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return launch_route_kernel(logits, Ep, logits + E, Ep, T, E, K, shared, renormalize, ids,
                             weights, stream);
}
