// MXFP4 quantisation of rows of bf16 or fp32 values (OCP MX v1.0 encoding:
// per block of 32 consecutive elements one E8M0 scale and 32 E2M1 codes).
// Used for the on-the-fly activation quantisation of the W4A4 path (OpenRelay
// "Gemma 4 31B on MI355X" post, sections "Optimisation 3" and
// "Optimisation 4": activation + MXFP4 quantisation in one kernel) and for
// packing float weights.
//
// Rule: mxfp4_block_exponent, e2m1_code and mxfp4_codes8 in common.h (the
// tiled gate/up GEMM's fused h quantisation uses the same ones).
#include "common.h"
#include "kernels.h"

namespace {

// Quantise 32 values held by one thread.
__device__ __forceinline__ void quant_block32(const float* v, u32x4_t* packed, uint8_t* scale) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const int X = mxfp4_block_exponent(amax);
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float e[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = v[8 * q + j];
    w[q] = mxfp4_codes8(e, X);
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

// The same rule, written in the blocked row order the tiled GEMMs read:
// output row p's chunk c (elements [128 c, 128 c + 128)) has its 64 code
// bytes at ((p / 16) * C + c) * 1024 + (p % 16) * 64 and its four scale
// bytes at ((p / 16) * C + c) * 64 + (p % 16) * 4 (C = cols / 128).
//
// Row p from source row p: a workgroup owns 16-row output block b and
// kChunksPerGroup chunks of it.  Lane L = 16 r + k takes elements
// [8 k, 8 k + 8) of row 16 b + r's chunk (one 16-byte bf16 load: each row's
// chunk is 256 contiguous bytes); the four lanes of a 32-block share its amax
// through two lane swaps, and lane L writes the four code bytes of its 8
// elements at byte 4 L of the block's KiB (the lane with k % 4 = 0 also the
// scale byte): each block's codes and scales are stored whole by one
// workgroup.
constexpr int kChunksPerGroup = 4;

// The 8 values at e quantised with the amax of the lane's aligned group of
// four lanes (one 32-block): the four code bytes and the scale byte.
template <bool kBf16>
__device__ __forceinline__ uint32_t quant8_in_block(const void* src, int64_t e, uint8_t* scale) {
  float v[8];
  if (kBf16) {
    const u32x4_t d = *reinterpret_cast<const u32x4_t*>(reinterpret_cast<const uint16_t*>(src) + e);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(d[j] << 16);
      v[2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
    }
  } else {
    const float4 d0 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + e);
    const float4 d1 = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(src) + e + 4);
    v[0] = d0.x; v[1] = d0.y; v[2] = d0.z; v[3] = d0.w;
    v[4] = d1.x; v[5] = d1.y; v[6] = d1.z; v[7] = d1.w;
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1, MOE_WAVE));
  amax = fmaxf(amax, __shfl_xor(amax, 2, MOE_WAVE));
  const int X = mxfp4_block_exponent(amax);
  const uint32_t w = mxfp4_codes8(v, X);
  *scale = (uint8_t)(X + 127);
  return w;
}

template <bool kBf16>
__global__ __launch_bounds__(256) void mxfp4_quant_blocked_kernel(
    const void* __restrict__ src, int64_t rows, int cols, int cgroups,
    uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t b = blockIdx.x / cgroups;
  const int cg = (int)(blockIdx.x - b * cgroups);
  const int L = threadIdx.x, r = L >> 4, k = L & 15;
  const int64_t t = 16 * b + r;
  const bool live = t < rows;
  const int C = cols / 128;
  for (int cc = 0; cc < kChunksPerGroup; ++cc) {
    const int c = cg * kChunksPerGroup + cc;
    if (c >= C) break;                                   // uniform in the workgroup
    uint8_t sc;
    const uint32_t w = quant8_in_block<kBf16>(src, live ? t * cols + 128 * c + 8 * k : 0, &sc);
    if (live) {
      const int64_t blk = b * C + c;
      *reinterpret_cast<uint32_t*>(packed + blk * 1024 + 4 * L) = w;
      if ((k & 3) == 0) scales[blk * 64 + 4 * r + (k >> 2)] = sc;
    }
  }
}

// Source row t to output rows map[t * Kp + k], k < Kp (a value outside
// [0, out_rows) writes nothing): thread i quantises 32-block i of the source
// (block i % (cols/32) of row i / (cols/32), loaded as in mxfp4_quant_kernel)
// and writes its 16 code bytes and its scale byte into every output row of
// its source row.  The four threads of a chunk are the lanes of one DPP
// quad (cols is a multiple of 128), so each output row's 64 code bytes of the
// chunk are written by adjacent lanes, one 16-byte store each, and the
// chunk's four scale bytes are gathered into the quad's first lane and
// written as one word.  (x of the W4A4 batch: 45 us; a lane per 8 elements
// with 4-byte code stores and byte-wide scale stores took 47: the 64-byte
// pieces of each slot's chunk, not the number of stores, bound it.)
template <bool kBf16>
__global__ __launch_bounds__(256) void mxfp4_quant_scatter_kernel(
    const void* __restrict__ src, int64_t nblocks, int cols, const int32_t* __restrict__ map,
    int Kp, int64_t out_rows, uint8_t* __restrict__ packed, uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= nblocks) return;
  const int nb = cols / 32;
  const int64_t t = i / nb;
  const int b = (int)(i - t * nb);
  float v[32];
  if (kBf16) {
    const u32x4_t* p = reinterpret_cast<const u32x4_t*>(src) + i * 4;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const u32x4_t d = p[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = __uint_as_float(d[j] << 16);
        v[8 * q + 2 * j + 1] = __uint_as_float(d[j] & 0xFFFF0000u);
      }
    }
  } else {
    const float4* p = reinterpret_cast<const float4*>(src) + i * 8;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4 d = p[q];
      v[4 * q] = d.x;
      v[4 * q + 1] = d.y;
      v[4 * q + 2] = d.z;
      v[4 * q + 3] = d.w;
    }
  }
  u32x4_t pk;
  uint8_t sc;
  quant_block32(v, &pk, &sc);
  // the quad's scale bytes, K-group order, in its first lane (quad_perm
  // [1,..], [2,..], [3,..] bring lanes 1, 2 and 3 to lane 0)
  const uint32_t s4 = (uint32_t)sc | dpp_move_u32<0x01>(sc) << 8 | dpp_move_u32<0x02>(sc) << 16 |
                      dpp_move_u32<0x03>(sc) << 24;
  const int64_t C = cols / 128;
  const int c = b >> 2, g = b & 3;
  for (int k = 0; k < Kp; ++k) {
    const int64_t p = map[t * Kp + k];
    if (p < 0 || p >= out_rows) continue;
    const int64_t blk = (p >> 4) * C + c;
    *reinterpret_cast<u32x4_t*>(packed + blk * 1024 + (p & 15) * 64 + 16 * g) = pk;
    if (g == 0) *reinterpret_cast<uint32_t*>(scales + blk * 64 + (p & 15) * 4) = s4;
  }
}

}  // namespace

hipError_t launch_mxfp4_quant_blocked(const void* src, int src_is_bf16, int64_t rows, int64_t cols,
                                      const int32_t* map, int Kp, int64_t out_rows,
                                      uint8_t* packed, uint8_t* scales, hipStream_t stream) {
  if (rows == 0 || cols == 0) return hipSuccess;
  if (map) {
    const int64_t nblocks = rows * (cols / 32);
    const unsigned grid = (unsigned)((nblocks + 255) / 256);
    if (src_is_bf16)
      hipLaunchKernelGGL(mxfp4_quant_scatter_kernel<true>, dim3(grid), dim3(256), 0, stream, src,
                         nblocks, (int)cols, map, Kp, out_rows, packed, scales);
    else
      hipLaunchKernelGGL(mxfp4_quant_scatter_kernel<false>, dim3(grid), dim3(256), 0, stream, src,
                         nblocks, (int)cols, map, Kp, out_rows, packed, scales);
    return hipGetLastError();
  }
  const int cgroups = (int)((cols / 128 + kChunksPerGroup - 1) / kChunksPerGroup);
  const unsigned grid = (unsigned)((rows + 15) / 16 * cgroups);
  if (src_is_bf16)
    hipLaunchKernelGGL(mxfp4_quant_blocked_kernel<true>, dim3(grid), dim3(256), 0, stream, src,
                       rows, (int)cols, cgroups, packed, scales);
  else
    hipLaunchKernelGGL(mxfp4_quant_blocked_kernel<false>, dim3(grid), dim3(256), 0, stream, src,
                       rows, (int)cols, cgroups, packed, scales);
  return hipGetLastError();
}

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
