// MXFP8 quantisation of rows of bf16 or fp32 values (OCP MX v1.0 encoding:
// per block of 32 consecutive elements one E8M0 scale and 32 FP8 E4M3
// codes, one byte each).  Used to pack float expert weights into the MXFP8
// format the pages serve MoE models in next to MXFP4 (MiniMax M3 on MI355X
// post, section on its MI355X performance benchmarks: MXFP8 standard
// inference).
//
// Rule, per block: X = floor(log2 amax) - 8 clamped to [-127, 127] (an
// all-zero block gives -127); scale byte X + 127; each |v| / 2^X goes to the
// nearest E4M3 magnitude (3 mantissa bits, bias 7, subnormal quantum 2^-9,
// largest 448), ties to the even code, saturating at 448; the sign bit of v
// is kept.  All steps are exact in fp32.
#include "common.h"
#include "kernels.h"

namespace {

// |v| / 2^X (exact, below 512) -> E4M3 magnitude code.
__device__ __forceinline__ uint32_t e4m3_code(float a) {
  if (a >= 448.0f) return 0x7Eu;                     // nothing above 448 is nearer
  const uint32_t u = __float_as_uint(a);
  if (u < 0x3C800000u)                               // below 2^-6: multiples of 2^-9
    return (uint32_t)rintf(a * 512.0f);              // 0..8 (8 is the code of 2^-6)
  // Normal: round fp32's 23 mantissa bits to 3, nearest, ties to even; a
  // carry out of the mantissa moves into the exponent field as it should.
  const uint32_t r = u + 0x7FFFFu + ((u >> 20) & 1u);
  return (r >> 20) - (120u << 3);                    // fp32 exponent bias 127 -> E4M3 bias 7
}

template <bool kBf16>
__global__ __launch_bounds__(256) void mxfp8_quant_kernel(const void* __restrict__ src,
                                                          int64_t nblocks,
                                                          uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  float v[32];
  if (kBf16) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(src) + b * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t d = p[q];
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
      const float4 d = p[q];
      v[4 * q] = d.x;
      v[4 * q + 1] = d.y;
      v[4 * q + 2] = d.z;
      v[4 * q + 3] = d.w;
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int ebits = (int)((__float_as_uint(amax) >> 23) & 0xFF);
  const int X = max(ebits - 135, -127);                          // floor(log2 amax) - 8
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);  // 2^-X, a normal float
  uint32_t w[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const uint32_t c = e4m3_code(fabsf(v[i]) * inv) | ((__float_as_uint(v[i]) >> 31) << 7);
    w[i >> 2] |= c << (8 * (i & 3));
  }
  u32x4_t* out = reinterpret_cast<u32x4_t*>(codes) + 2 * b;
  out[0] = (u32x4_t){w[0], w[1], w[2], w[3]};
  out[1] = (u32x4_t){w[4], w[5], w[6], w[7]};
  scales[b] = (uint8_t)(X + 127);
}

}  // namespace

// rows x cols values (cols a multiple of 32) are one flat run of blocks: the
// codes are [rows, cols] and the scales [rows, cols/32], row-major.
hipError_t launch_mxfp8_quant(const void* src, int src_is_bf16, int64_t rows, int64_t cols,
                              uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t nblocks = rows * (cols / 32);
  if (nblocks == 0) return hipSuccess;
  const int64_t grid = (nblocks + 255) / 256;
  if (src_is_bf16)
    hipLaunchKernelGGL(mxfp8_quant_kernel<true>, dim3((unsigned)grid), dim3(256), 0, stream, src,
                       nblocks, codes, scales);
  else
    hipLaunchKernelGGL(mxfp8_quant_kernel<false>, dim3((unsigned)grid), dim3(256), 0, stream, src,
                       nblocks, codes, scales);
  return hipGetLastError();
}
