// Device helpers shared by the HIP kernels of the MXFP4 MoE layer (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef int int32x8_t __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

#define MOE_WAVE 64

// Debug builds (-DMOE_DEBUG): the kernels check every index that comes from a
// device table (the grouping's positions, a tile's rows, the combine's slot
// rows) against the sizes they were given.  A failed check skips the access
// and sets a bit in the source file's device flag word, which the host reads
// (and clears) through moe_debug_flags: a bad index is reported, not
// executed, and no check traps.  Release builds compile the checks away.
enum : uint32_t {
  kDbgAlign = 1u,     // a sorted / inv position or a tile-table entry out of range
  kDbgTiles = 2u,     // a GEMM tile's rows outside its expert's group or past A
  kDbgCombine = 4u,   // a slot row read by the combine at or past A
};
#ifdef MOE_DEBUG
// Defines the file's flag word and host_fn(reset), which returns it (ORed
// with 0x80000000 when the copy fails) and clears it when reset is set.
#define MOE_DEBUG_FLAGS(host_fn)                                                            \
  namespace {                                                                               \
  __device__ uint32_t g_moe_debug_flags;                                                    \
  }                                                                                         \
  uint32_t host_fn(bool reset) {                                                            \
    uint32_t v = 0;                                                                         \
    if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_moe_debug_flags), sizeof v) != hipSuccess)     \
      return 0x80000000u;                                                                   \
    const uint32_t zero = 0;                                                                \
    if (reset && hipMemcpyToSymbol(HIP_SYMBOL(g_moe_debug_flags), &zero, sizeof zero) !=   \
                     hipSuccess)                                                            \
      return v | 0x80000000u;                                                               \
    return v;                                                                               \
  }
#define MOE_DOK(cond, bit) moe_dok((cond), (bit), &g_moe_debug_flags)
__device__ __forceinline__ bool moe_dok(bool ok, uint32_t bit, uint32_t* flags) {
  if (!ok) atomicOr(flags, bit);
  return ok;
}
#else
#define MOE_DEBUG_FLAGS(host_fn) \
  uint32_t host_fn(bool) { return 0; }
#define MOE_DOK(cond, bit) true
#endif

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// E8M0 scale byte -> float 2^(b-127).  Bytes 1..254 are exact normals; byte 0
// gives 2^-127 (a float32 subnormal); byte 255 (NaN) is outside the contract.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Staged y (each sorted row's down-projection, between the down GEMM and the
// combine): fp16 values scaled by a power of two per row and 32-column
// group, the exponent e in a byte (e + 127) of its own; value = fp16 * 2^e.
// The group's largest magnitude lands in [2^14, 2^15): 11 significant bits
// for every element (bf16 has 8) at half the bytes of fp32.
constexpr int kYGroup = 32;

// Exponent fields (bits 23-30) of two fp32 values packed as two 16-bit
// halves, for max reductions of both at once.
__device__ __forceinline__ uint32_t pack_exponents(float a, float b) {
  return ((__float_as_uint(a) >> 23) & 0xFFu) | (((__float_as_uint(b) >> 23) & 0xFFu) << 16);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_move_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// Per-half maximum of packed 16-bit fields (one packed max).
__device__ __forceinline__ uint32_t max_halves(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}

// Maximum of each 16-bit half of v over the 16 lanes of each DPP row (lanes
// 16 i .. 16 i + 15): quad_perm [1,0,3,2] and [2,3,0,1] (each quad),
// row_half_mirror (each eight), row_mirror (the sixteen).  Every lane of the
// wave must take part.
__device__ __forceinline__ uint32_t row16_max_halves(uint32_t v) {
  v = max_halves(v, dpp_move_u32<0xB1>(v));
  v = max_halves(v, dpp_move_u32<0x4E>(v));
  v = max_halves(v, dpp_move_u32<0x141>(v));
  v = max_halves(v, dpp_move_u32<0x140>(v));
  return v;
}

// Maximum of each 16-bit half of v over lanes n, n ^ 16, n ^ 32, n ^ 48 (the
// same lane of the four DPP rows): each gfx950 permlane swap exchanges half
// of the wave between two copies of v, so every lane ends up with its own
// value and its partner's (at distance 32, then 16).
__device__ __forceinline__ uint32_t xrow_max_halves(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max_halves(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max_halves(b[0], b[1]);
}

// Maximum of v over lanes n, n ^ 16, n ^ 32, n ^ 48, as xrow_max_halves.
__device__ __forceinline__ uint32_t xrow_max_u32(uint32_t v) {
  const auto a = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  v = max(a[0], a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  return max(b[0], b[1]);
}

// MXFP4 quantisation (OCP MX v1.0 encoding), per block of 32 values: X =
// floor(log2 amax) - 2 clamped to [-127, 127] (an all-zero block gives
// -127); scale byte X + 127; each |v| / 2^X goes to the nearest E2M1
// magnitude {0, .5, 1, 1.5, 2, 3, 4, 6}, ties to the even code, saturating
// at 6; the sign bit of v is kept.  All steps are exact in fp32.
//
// |v| / 2^X -> E2M1 magnitude code by the midpoints between grid values; at
// a midpoint the even code wins.
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

// X of a block whose largest magnitude is amax.
__device__ __forceinline__ int mxfp4_block_exponent(float amax) {
  return max((int)((__float_as_uint(amax) >> 23) & 0xFF) - 129, -127);
}

// Eight values of a block with exponent X -> four code bytes (element j in
// nibble j, low nibble first).
__device__ __forceinline__ uint32_t mxfp4_codes8(const float (&v)[8], int X) {
  const float inv = __uint_as_float((uint32_t)(127 - X) << 23);   // 2^-X, a normal float
  uint32_t w = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w |= (e2m1_code(fabsf(v[j]) * inv) | ((__float_as_uint(v[j]) >> 31) << 3)) << (4 * j);
  return w;
}

// Exponent of a group whose largest biased fp32 exponent field is f:
// floor(log2 amax) - 14 = f - 141, clamped to [-127, 127] (an all-zero or
// all-subnormal group gets -127).
__device__ __forceinline__ int y_exponent_of_field(uint32_t f) {
  return min(127, max(-127, (int)f - 141));
}

__device__ __forceinline__ uint16_t y_encode(float v, int e) {
  return __builtin_bit_cast(uint16_t, (_Float16)__builtin_amdgcn_ldexpf(v, -e));
}

__device__ __forceinline__ float y_decode(uint16_t bits, int e) {
  return __builtin_amdgcn_ldexpf((float)__builtin_bit_cast(_Float16, bits), e);
}

// SiLU(g) * u in fp32.
__device__ __forceinline__ float swiglu(float g, float u) {
  return g / (1.0f + __expf(-g)) * u;
}

// Eight E2M1 codes (one dword, element 2j in the low nibble of byte j) times
// a power-of-two scale -> eight bf16 values, exact.  Uses the gfx950 scaled
// FP4 -> BF16 converter; op_sel picks the byte.
__device__ __forceinline__ bf16x8_t dequant8_bf16(uint32_t q, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 0);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 1);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 2);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(q, scale, 3);
  bf16x8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

// Eight E4M3 codes (two dwords, element i in byte i % 4 of dword i / 4)
// times a power-of-two scale -> eight bf16 values, exact (E4M3 keeps 4
// significant bits, bf16 8, with fp32's exponent range).  Uses the gfx950
// scaled FP8 -> BF16 converter; its word select picks bytes 0-1 or 2-3.
__device__ __forceinline__ bf16x8_t dequant8_bf16_fp8(uint32_t lo, uint32_t hi, float scale) {
  bf16x2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, false);
  bf16x2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, scale, true);
  bf16x2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, false);
  bf16x2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, scale, true);
  bf16x8_t r = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
  return r;
}

__device__ __forceinline__ floatx4_t mfma_bf16_16x16x32(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Scaled MFMA, both operands FP4 (E2M1): lane l supplies row (l % 16), K-block
// (l / 16) as 32 codes in four dwords plus that block's E8M0 byte.
__device__ __forceinline__ floatx4_t mfma_fp4_16x16x128(u32x4_t a, uint32_t sa, u32x4_t b,
                                                        uint32_t sb, floatx4_t c) {
  int32x8_t av = {(int)a[0], (int)a[1], (int)a[2], (int)a[3], 0, 0, 0, 0};
  int32x8_t bv = {(int)b[0], (int)b[1], (int)b[2], (int)b[3], 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 4, 4, 0, (int)sa, 0, (int)sb);
}

// Raw buffer loads: a wave-uniform resource (base, size in bytes) plus a
// per-lane byte offset and a wave-uniform byte offset.  Reads past the
// resource's size return zeros instead of touching memory.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#define MOE_BUFFER_FLAGS 0x00020000  // gfx9 raw buffer: 32-bit data format, no swizzle

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           MOE_BUFFER_FLAGS);
}

__device__ __forceinline__ u32x4_t bload16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}

// The same load marked non-temporal (cache policy NT: the lines are streamed
// through the caches rather than kept for reuse), for weight codes read once:
// an expert's only tile.  Streaming the decode step's expert weights this way
// raised its GEMMs from ~6.1 to ~6.8 TB/s; where other tiles of the expert
// re-read the weights from L2 it costs 7-26% instead.
constexpr int kCacheNT = 2;

__device__ __forceinline__ u32x4_t bload16_nt(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4_t,
                            __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, kCacheNT));
}

// Expert weight codes in the GEMM kernels' native order.  An expert's code
// matrix (rows a multiple of 32, reduction length K a multiple of 128; NQ =
// 1 byte per two MXFP4 codes -> 16 code bytes per lane and chunk, NQ = 2 for
// MXFP8's byte per code -> 32) is a sequence of 1 KiB blocks: block
// (s * (K / 128) + c) * NQ + hq holds, at byte 16 l, the 16 bytes lane
// l = 16 g + n loads for strip s, slot n, chunk c (elements [128 c,
// 128 c + 128)), K-group g, part hq: row-major code bytes [NQ (64 c + 16 g) +
// 16 hq, +16) of row 32 (s / 2) + wnat_row(s % 2, n).  A wave's load of one
// strip chunk is then one contiguous KiB, where the row-major layout touches
// 16 rows at half a 128-byte line each.
//
// The slots of a strip pair interleave the pair's 32 rows in runs of four:
// with the weights as the MFMA's A operand, lane 16 g + n holds D rows 4 g ..
// 4 g + 3 of each strip, which are then weight rows 8 g .. 8 g + 7 of the
// pair: eight consecutive output columns, one 16-byte store of fp16 / bf16.
__host__ __device__ constexpr int wnat_row(int u, int n) {
  return 8 * (n >> 2) + 4 * u + (n & 3);
}
__device__ __forceinline__ uint32_t wnat_lane(int strip, int K, int NQ, int lane) {
  return (uint32_t)strip * (uint32_t)(K / 128 * NQ) * 1024u + 16u * (uint32_t)lane;
}
__device__ __forceinline__ uint32_t wnat_chunk(int c, int NQ, int hq) {
  return (uint32_t)(NQ * c + hq) * 1024u;
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
// Vector memory operations complete in issue order, so it waits for all but
// the n most recent.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroup barrier without the release fence of __syncthreads: the fence
// would wait for every load still in flight, i.e. for the stages being
// prefetched.  Each wave waits for its own direct-to-LDS loads (wait_vmcnt)
// before the barrier, and every LDS read of a buffer has returned before the
// barrier that precedes its refill; the "memory" clobber keeps the compiler
// from moving memory accesses across.
__device__ __forceinline__ void stage_barrier() { asm volatile("s_barrier" ::: "memory"); }

typedef __attribute__((address_space(3))) void lds_void_t;

// Direct-to-LDS buffer loads: lane l's 16 (4) bytes land at lds + 16 l (4 l);
// lds is the same for the whole wave.
__device__ __forceinline__ void load_to_lds16(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 16, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ void load_to_lds4(rsrc_t r, uint32_t voff, uint32_t soff, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)lds, 4, (int)voff, (int)soff, 0, 0);
}

__device__ __forceinline__ uint32_t bload1(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, (int)voff, (int)soff, 0);
}

__device__ __forceinline__ u32x4_t load16(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ bf16x8_t load_bf16x8(const void* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}
