// The step after the MoE layer in a tensor-parallel decode: the ranks'
// partial outputs summed, the residual stream added, then RMSNorm, all in one
// pass over the rows.  The pages replace the per-layer all-reduce with a
// one-shot one fused with the residual add and RMSNorm (VibeSys
// "Qwen3.5-397B on 4x MI300A" post, section "Communication and
// concurrency"): each GPU reads every rank's partial output and produces
// the normalised rows itself.  This kernel is that epilogue over G partial
// buffers; on one GPU they are local (the shard layers of one GPU), across
// GPUs they would be the peers' buffers.  RMSNorm in its textbook form:
//   h[t, j] = bf16( residual[t, j] + sum_g partial[g][t, j] )   (new residual)
//   y[t, j] = bf16( h[t, j] * rstd_t * gamma[j] ),
//   rstd_t  = 1 / sqrt( mean_j h[t, j]^2 + eps ),
// the sum in fp32 in the order residual, partial 0, 1, ..., the mean of
// squares over h's bf16 values.
//
// One workgroup (4 waves) per row; a thread owns NG groups of 8 consecutive
// columns (16-byte loads and stores); up to H = 8192 every group's G + 1
// loads are issued before the first add.  Bound by HBM: (G + 1) * 2 H bytes
// read and 4 H written per row (gamma stays in the caches).
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kNormThreads = 256;

struct PartialPtrs {
  const uint16_t* p[kMaxNormRanks];
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Inputs larger than the memory-side cache (256 MiB) stream from HBM
// whatever the hint; they are read with non-temporal loads (kNT), which
// leave the caches to the rest (eight partials of 8,192 rows x 4,096:
// 139 -> 122 us).  Smaller ones may still sit in that cache, as when the
// kernels before have just written them, where the plain loads are faster
// (1,536 rows: 24.3 against 25.9 us).
constexpr size_t kStreamBytes = size_t(256) << 20;

template <bool kNT>
__device__ __forceinline__ u32x4_t load_in(const uint16_t* p) {
  if constexpr (kNT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else return load16(p);
}

// residual and residual_out may be the same buffer, and so may out and
// partial 0: every element is read before the thread that owns it writes.
template <int NG, bool kNT>
__global__ __launch_bounds__(kNormThreads) void residual_rmsnorm_kernel(
    PartialPtrs parts, int G, const uint16_t* residual, const uint16_t* __restrict__ gamma,
    float eps, int H, uint16_t* residual_out, uint16_t* out) {
  __shared__ float wsum[kNormThreads / MOE_WAVE];
  const size_t row = (size_t)blockIdx.x * H;
  const int tid = threadIdx.x;
  float h[NG][8];
  float ss = 0.f;
  // up to 4 groups (H <= 8192): every group's loads before the first add
  constexpr int NP = NG <= 4 ? NG : 1;
  u32x4_t pre[NP][kMaxNormRanks + 1];
  auto fetch = [&](int k, u32x4_t (&v)[kMaxNormRanks + 1]) {
    const int j = 8 * (tid + kNormThreads * k);
    if (j < H) {
      v[kMaxNormRanks] =
          residual ? load_in<kNT>(residual + row + j) : (u32x4_t){0u, 0u, 0u, 0u};
#pragma unroll
      for (int g = 0; g < kMaxNormRanks; ++g)
        if (g < G) v[g] = load_in<kNT>(parts.p[g] + row + j);
    }
  };
  if constexpr (NG <= 4) {
#pragma unroll
    for (int k = 0; k < NG; ++k) fetch(k, pre[k]);
  }
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int j = 8 * (tid + kNormThreads * k);
    if (j < H) {
      if constexpr (NG > 4) fetch(k, pre[0]);
      const u32x4_t(&v)[kMaxNormRanks + 1] = pre[NG <= 4 ? k : 0];
      const u32x4_t r = v[kMaxNormRanks];
      u32x4_t hb;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float lo = bf16_lo(r[q]), hi = bf16_hi(r[q]);
#pragma unroll
        for (int g = 0; g < kMaxNormRanks; ++g)
          if (g < G) {
            lo += bf16_lo(v[g][q]);
            hi += bf16_hi(v[g][q]);
          }
        const uint16_t blo = f32_to_bf16_rne(lo), bhi = f32_to_bf16_rne(hi);
        hb[q] = (uint32_t)blo | (uint32_t)bhi << 16;
        h[k][2 * q] = bf16_to_f32(blo);
        h[k][2 * q + 1] = bf16_to_f32(bhi);
        ss += h[k][2 * q] * h[k][2 * q] + h[k][2 * q + 1] * h[k][2 * q + 1];
      }
      if (residual_out) *reinterpret_cast<u32x4_t*>(residual_out + row + j) = hb;
    }
  }
  // the row's sum of squares: each wave's lanes, then the four waves in order
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, MOE_WAVE);
  if ((tid & (MOE_WAVE - 1)) == 0) wsum[tid / MOE_WAVE] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int w = 0; w < kNormThreads / MOE_WAVE; ++w) tot += wsum[w];
  const float rstd = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const int j = 8 * (tid + kNormThreads * k);
    if (j < H) {
      const u32x4_t gm = load16(gamma + j);
      u32x4_t o;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        o[q] = (uint32_t)f32_to_bf16_rne(h[k][2 * q] * rstd * bf16_lo(gm[q])) |
               (uint32_t)f32_to_bf16_rne(h[k][2 * q + 1] * rstd * bf16_hi(gm[q])) << 16;
      *reinterpret_cast<u32x4_t*>(out + row + j) = o;
    }
  }
}

template <int NG>
void launch_rn(bool nt, dim3 grid, const PartialPtrs& pp, int G, const uint16_t* residual,
               const uint16_t* gamma, float eps, int H, uint16_t* residual_out, uint16_t* out,
               hipStream_t stream) {
  if (nt)
    hipLaunchKernelGGL((residual_rmsnorm_kernel<NG, true>), grid, dim3(kNormThreads), 0, stream, pp,
                       G, residual, gamma, eps, H, residual_out, out);
  else
    hipLaunchKernelGGL((residual_rmsnorm_kernel<NG, false>), grid, dim3(kNormThreads), 0, stream,
                       pp, G, residual, gamma, eps, H, residual_out, out);
}

}  // namespace

int residual_rmsnorm_max_h() { return 8 * kNormThreads * 8; }

hipError_t launch_residual_rmsnorm(const uint16_t* const* partials, int G, const uint16_t* residual,
                                   const uint16_t* gamma, float eps, int T, int H,
                                   uint16_t* residual_out, uint16_t* out, hipStream_t stream) {
  PartialPtrs pp{};
  for (int g = 0; g < G; ++g) pp.p[g] = partials[g];
  const dim3 grid((unsigned)T);
  const int ng = (H + 8 * kNormThreads - 1) / (8 * kNormThreads);
  const bool nt = (size_t)(G + (residual ? 1 : 0)) * T * H * 2 > kStreamBytes;
  if (ng <= 1) launch_rn<1>(nt, grid, pp, G, residual, gamma, eps, H, residual_out, out, stream);
  else if (ng <= 2) launch_rn<2>(nt, grid, pp, G, residual, gamma, eps, H, residual_out, out, stream);
  else if (ng <= 3) launch_rn<3>(nt, grid, pp, G, residual, gamma, eps, H, residual_out, out, stream);
  else if (ng <= 4) launch_rn<4>(nt, grid, pp, G, residual, gamma, eps, H, residual_out, out, stream);
  else launch_rn<8>(nt, grid, pp, G, residual, gamma, eps, H, residual_out, out, stream);
  return hipGetLastError();
}
