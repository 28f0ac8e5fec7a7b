// MXFP4 quantisation of rows of bf16 or fp32 values (OCP MX v1.0 encoding:
// per block of 32 consecutive elements one E8M0 scale and 32 E2M1 codes).
// Used for the on-the-fly activation quantisation of the W4A4 path (OpenRelay
// "Gemma 4 31B on MI355X" post, sections "Optimisation 3" and
// "Optimisation 4": activation + MXFP4 quantisation in one kernel) and for
// packing float weights.
//
// Rule, per block: X = floor(log2 amax) - 2 clamped to [-127, 127] (an
// all-zero block gives -127); scale byte X + 127; each |v| / 2^X goes to the
// nearest E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code,
// saturating at 6; the sign bit of v is kept.  All steps are exact in fp32.
#include "common.h"
#include "kernels.h"

namespace {

// |v| / 2^X (exact) -> E2M1 magnitude code by the midpoints between grid
// values; at a midpoint the even code wins.
__device__ __forceinline__ uint32_t e2m1_code(float a) {
  uint32_t c = 7;
  c = (a <= 5.0f) ? 6 : c;
  c = (a < 3.5f) ? 5 : c;
  c = (a <= 2.5f) ? 4 : c;
  c = (a < 1.75f) ? 3 : c;
  c = (a <= 1.25f) ? 2 : c;
  c = (a < 0.75f) ? 1 : c;
  c = (a <= 0.25f) ? 0 : c;
  return c;
}

// Quantise 32 values held by one thread.
__device__ __forceinline__ void quant_block32(const float* v, u32x4_t* packed, uint8_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int X = max(ebits - 129, -127);                       // floor(log2 amax) - 2
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, a normal float
  uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    uint32_t c = e2m1_code(fabsf(v[i]) * inv) | ((__float_as_uint(v[i]) >> 31) << 3);
    w[i >> 3] |= c << (4 * (i & 7));
  }
  *packed = (u32x4_t){w[0], w[1], w[2], w[3]};
  *scale = (uint8_t)(X + 127);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void mxfp4_quant_kernel(const void* __restrict__ src,
                                                          int64_t nblocks,
                                                          uint8_t* __restrict__ packed,
                                                          uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if (kBf16) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(src) + b * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      u32x4_t d = p[q];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[8 * q + 2 * i] = __uint_as_float(d[i] << 16);
        v[8 * q + 2 * i + 1] = __uint_as_float(d[i] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(src) + b * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float4 d = p[q];
      v[4 * q] = d.x;
      v[4 * q + 1] = d.y;
      v[4 * q + 2] = d.z;
      v[4 * q + 3] = d.w;
    }
  }
  u32x4_t pk;
  uint8_t sc;
  quant_block32(v, &pk, &sc);
  reinterpret_cast<u32x4_t*>(packed)[b] = pk;
  scales[b] = sc;
}

}  // namespace

// rows x cols values (cols a multiple of 32) are one flat run of blocks: the
// packed output is [rows, cols/2] and the scales [rows, cols/32], row-major.
hipError_t launch_mxfp4_quant(const void* src, int src_is_bf16, int64_t rows, int64_t cols,
                              uint8_t* packed, uint8_t* scales, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks + 255) / 256;
  if (src_is_bf16)
    hipLaunchKernelGGL(mxfp4_quant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, src,
                       nblocks, packed, scales);
  else
    hipLaunchKernelGGL(mxfp4_quant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, src,
                       nblocks, packed, scales);
  return hipGetLastError();
}
