// Expert weight codes: row-major -> the GEMM kernels' native order (see
// wnat_lane in common.h).  A one-time permutation at weight load, like the
// packing itself: every 16-byte piece moves, none changes.
#include "common.h"
#include "kernels.h"

namespace {

// One thread per destination piece p (16 bytes): p = ((s * nch + c) * NQ +
// hq) * 64 + l comes from row 32 (s / 2) + wnat_row(s % 2, l % 16), code
// bytes NQ * (64 c + 16 (l / 16)) + 16 hq of the row.
__global__ __launch_bounds__(256) void weights_native_kernel(const u32x4_t* __restrict__ src,
                                                             int64_t npieces, int nch, int nq,
                                                             int64_t row_bytes,
                                                             u32x4_t* __restrict__ dst) {
  for (int64_t p = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; p < npieces;
       p += (int64_t)gridDim.x * blockDim.x) {
    const int l = (int)(p & 63);
    const int64_t blk = p >> 6;
    const int hq = (int)(blk % nq);
    const int64_t sc = blk / nq;
    const int c = (int)(sc % nch);
    const int64_t s = sc / nch;
    const int64_t row = 32 * (s >> 1) + wnat_row((int)(s & 1), l & 15);
    const int64_t byte = (int64_t)nq * (64 * c + 16 * (l >> 4)) + 16 * hq;
    dst[p] = src[(row * row_bytes + byte) >> 4];
  }
}

}  // namespace

// rows x cols codes (rows a multiple of 32, cols of 128); nq = 1 for MXFP4
// (cols / 2 bytes per row), 2 for MXFP8 (cols bytes per row).
hipError_t launch_weights_native(const uint8_t* src, int nq, int64_t rows, int64_t cols,
                                 uint8_t* dst, hipStream_t stream) {
  const int64_t row_bytes = nq == 2 ? cols : cols / 2;
  const int64_t npieces = rows * row_bytes / 16;
  if (npieces == 0) return hipSuccess;
  const int64_t want = (npieces + 255) / 256;
  const unsigned grid = (unsigned)(want < 65536 ? want : 65536);
  hipLaunchKernelGGL(weights_native_kernel, dim3(grid), dim3(256), 0, stream,
                     reinterpret_cast<const u32x4_t*>(src), npieces, (int)(cols / 128), nq,
                     row_bytes, reinterpret_cast<u32x4_t*>(dst));
  return hipGetLastError();
}
