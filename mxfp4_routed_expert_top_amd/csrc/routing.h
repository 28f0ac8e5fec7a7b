// Device helpers of the softmax top-K routing (route_topk.hip, and the
// fused small-batch routing + grouping of route_align.hip).
//
// The experts are selected on the fp32 logits (softmax is monotone), ordered
// by (logit descending, expert index ascending), with -0.0 equal to +0.0
// (InferenceX "MI355X Qwen3.5 SGLang v0.5.12" post, section on the specific
// optimisations, fused_topk bullet: softmax-scored top-K at E = 512, K = 10).
// The weights are exp(l_k - l_0) / sum_k' exp(l_k' - l_0) over the K
// selected experts (renormalised) or over all E (not renormalised).  With a
// folded-in shared expert, slot K holds expert E with weight sigmoid(g)
// (same post, shared-expert fusion bullet).
#pragma once
#include "common.h"

namespace moe_routing {

constexpr int kMaxPerLane = 16;   // E <= 1024

// Orderable 32-bit image of a logit: larger image = larger logit, -0.0 and
// +0.0 the same image; 0 (the image of no finite logit) marks an empty slot.
__device__ __forceinline__ uint32_t order_bits(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;                       // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // monotone in v
}

__device__ __forceinline__ float order_value(uint32_t u) {
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// Wave-wide maximum / minimum of a u32 with DPP lane moves (no LDS round
// trip): quad swaps, half-row and row mirrors, then row broadcasts; lane 63
// ends with the result, which is read back as a scalar.
// (lanes outside the row mask see the operation's identity, so each step can
// become one v_max_u32_dpp / v_min_u32_dpp)
template <int CTRL, int ROWMASK, bool MAX>
__device__ __forceinline__ uint32_t dpp_step(uint32_t v) {
  const uint32_t o =
      (uint32_t)__builtin_amdgcn_update_dpp(MAX ? 0 : -1, (int)v, CTRL, ROWMASK, 0xF, false);
  return MAX ? (o > v ? o : v) : (o < v ? o : v);
}

template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  v = dpp_step<0xB1, 0xF, MAX>(v);    // quad_perm [1,0,3,2]
  v = dpp_step<0x4E, 0xF, MAX>(v);    // quad_perm [2,3,0,1]
  v = dpp_step<0x141, 0xF, MAX>(v);   // row_half_mirror
  v = dpp_step<0x140, 0xF, MAX>(v);   // row_mirror
  v = dpp_step<0x142, 0xA, MAX>(v);   // row_bcast:15 into rows 1, 3
  v = dpp_step<0x143, 0xC, MAX>(v);   // row_bcast:31 into rows 2, 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
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

// The shared expert's gate logit of token t at g[t * stride] (read only when
// shared = 1).
struct GateLogit {
  const float* g;
  int stride;
  __device__ __forceinline__ float operator()(int t) const { return g[(size_t)t * stride]; }
};

// One wave routes the NT tokens t0 + j * dt (j < NT; those at or past T are
// skipped), their dependency chains interleaved.  Lane l holds the logits of
// experts l, l + 64, ..., NPL of them per token (E <= 64 NPL), as orderable
// images sorted descending once (stably: equal images keep ascending expert
// order).  Each of the K rounds takes the wave-wide maximum image of the
// lanes' heads; the lanes whose heads tie with it (usually one) give the
// smallest expert index among them, and that lane shifts its list by one.
// out(t, k, e, w) stores slot k of token t: expert e, weight w.
template <int NPL, int NT, class Src, class Out>
__device__ __forceinline__ void route_tokens(const Src& src, const GateLogit& gate, int t0, int dt,
                                             int T, int E, int K, int shared, int renormalize,
                                             Out&& out) {
  const int lane = threadIdx.x & 63;

  // (every load issued before the first use: clamped indices, then a select)
  uint32_t key[NT][NPL];
  int slot[NT][NPL];                                  // j of expert lane + 64 j
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + j * dt;
#pragma unroll
    for (int i = 0; i < NPL; ++i) key[j][i] = __float_as_uint(src(min(t, T - 1), min(lane + 64 * i, E - 1)));
  }
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + j * dt;
#pragma unroll
    for (int i = 0; i < NPL; ++i) {
      const int e = lane + 64 * i;
      key[j][i] = (t < T && e < E) ? order_bits(__uint_as_float(key[j][i])) : 0u;
      slot[j][i] = i;
    }
  }
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 1; i < NPL; ++i)                     // insertion network, descending, stable
#pragma unroll
      for (int m = i; m > 0; --m) {
        const bool sw = key[j][m] > key[j][m - 1];
        const uint32_t a = key[j][m - 1], b = key[j][m];
        const int sa = slot[j][m - 1], sb = slot[j][m];
        key[j][m - 1] = sw ? b : a;
        key[j][m] = sw ? a : b;
        slot[j][m - 1] = sw ? sb : sa;
        slot[j][m] = sw ? sa : sb;
      }

  // Lane k keeps slot k's expert and logit image; the weights come after
  // the K rounds: each lane its own exp(l_k - l_0), the renormalised
  // denominator summed over the slots in slot order.
  uint32_t lead[NT], sel_b[NT];
  int sel_e[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    lead[j] = sel_b[j] = 0u;
    sel_e[j] = 0;
  }
  for (int k = 0; k < K; ++k) {
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const uint32_t best = wave_reduce_u32<true>(key[j][0]);
      const int head_e = lane + 64 * slot[j][0];
      const uint64_t tied = __ballot(key[j][0] == best);
      int e;
      if (__popcll(tied) == 1)
        e = __builtin_amdgcn_readlane(head_e, __ffsll((unsigned long long)tied) - 1);
      else                                              // equal logits: the smallest index
        e = (int)wave_reduce_u32<false>(key[j][0] == best ? (uint32_t)head_e : 0xFFFFFFFFu);
      if (head_e == e) {
#pragma unroll
        for (int i = 0; i + 1 < NPL; ++i) {
          key[j][i] = key[j][i + 1];
          slot[j][i] = slot[j][i + 1];
        }
        key[j][NPL - 1] = 0u;
      }
      if (k == 0) lead[j] = best;
      if (lane == k) {
        sel_e[j] = e;
        sel_b[j] = best;
      }
    }
  }

#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int t = t0 + j * dt;
    if (t >= T) continue;                                  // wave-uniform
    const float lmax = order_value(lead[j]);
    const float ek = lane < K ? expf(order_value(sel_b[j]) - lmax) : 0.f;
    float den = 0.f;
    if (renormalize) {
      for (int k = 0; k < K; ++k) den += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(ek), k));
    } else {
      float l[NPL];
#pragma unroll
      for (int i = 0; i < NPL; ++i) l[i] = src(t, min(lane + 64 * i, E - 1));
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < NPL; ++i)
        if (lane + 64 * i < E) s += expf(l[i] - lmax);
      den = wave_sum_f32(s);
    }
    if (lane < K) out(t, lane, sel_e[j], ek / den);
    if (shared && lane == 0) out(t, K, E, 1.0f / (1.0f + expf(-gate(t))));
  }
}

}  // namespace moe_routing
