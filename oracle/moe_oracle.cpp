// CPU oracle of the MXFP4 routed-expert MoE layer: plain C++17, fp64.
//
// TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and bench.py's
// cpu_baseline leg may load this library or run its command-line tool; the
// product path never does, and nothing here includes or calls the HIP path.
// moe_oracle.h states what each function computes and the passage of the
// pages it follows; the comments below only say how.
//
// Parallelism is over independent outputs only (whole dot products, whole
// rows): every value is computed by the same arithmetic whatever the thread
// count, so results do not depend on it.

#include "moe_oracle.h"

#include <sched.h>

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <condition_variable>
#include <cstring>
#include <functional>
#include <limits>
#include <mutex>
#include <numeric>
#include <thread>
#include <vector>

namespace {

constexpr int kBlock = 32;        // elements per E8M0 scale block
constexpr int kE2M1Emax = 2;      // exponent of E2M1's largest value, 6 = 1.5 * 2^2
constexpr int kE4M3Emax = 8;      // exponent of E4M3's largest value, 448 = 1.75 * 2^8
constexpr int kE4M3Finite = 127;  // codes 0..126 are the finite non-negative E4M3 values

// ------------------------------------------------------------ thread pool --

// A fixed set of threads that runs body(i) for i in [0, n), handing out
// indices one at a time; the calling thread works too.
class Pool {
 public:
  explicit Pool(int threads) : n_threads_(std::max(1, threads)) {
    for (int i = 1; i < n_threads_; ++i) workers_.emplace_back([this] { worker(); });
  }
  ~Pool() {
    {
      std::lock_guard<std::mutex> g(m_);
      stop_ = true;
    }
    wake_.notify_all();
    for (auto &t : workers_) t.join();
  }
  Pool(const Pool &) = delete;
  Pool &operator=(const Pool &) = delete;

  int threads() const { return n_threads_; }

  void for_each(int64_t n, const std::function<void(int64_t)> &body) {
    if (n <= 0) return;
    if (n_threads_ == 1 || n == 1) {
      for (int64_t i = 0; i < n; ++i) body(i);
      return;
    }
    {
      std::lock_guard<std::mutex> g(m_);
      body_ = &body;
      count_ = n;
      next_.store(0);
      pending_ = n_threads_ - 1;
      ++generation_;
    }
    wake_.notify_all();
    drain(body, n);
    std::unique_lock<std::mutex> lk(m_);
    done_.wait(lk, [this] { return pending_ == 0; });
    body_ = nullptr;
  }

 private:
  void drain(const std::function<void(int64_t)> &body, int64_t n) {
    for (int64_t i = next_.fetch_add(1); i < n; i = next_.fetch_add(1)) body(i);
  }
  void worker() {
    uint64_t seen = 0;
    for (;;) {
      const std::function<void(int64_t)> *body;
      int64_t n;
      {
        std::unique_lock<std::mutex> lk(m_);
        wake_.wait(lk, [&] { return stop_ || generation_ != seen; });
        if (stop_) return;
        seen = generation_;
        body = body_;
        n = count_;
      }
      drain(*body, n);
      std::lock_guard<std::mutex> g(m_);
      if (--pending_ == 0) done_.notify_one();
    }
  }

  const int n_threads_;
  std::vector<std::thread> workers_;
  std::mutex m_;
  std::condition_variable wake_, done_;
  const std::function<void(int64_t)> *body_ = nullptr;
  int64_t count_ = 0;
  std::atomic<int64_t> next_{0};
  int pending_ = 0;
  uint64_t generation_ = 0;
  bool stop_ = false;
};

int resolve_threads(int threads) { return threads > 0 ? threads : oracle_default_threads(); }

// ---------------------------------------------------------- number formats --

double e2m1_value(int code) {
  const int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
  const double mag = e == 0 ? 0.5 * m : (1.0 + 0.5 * m) * std::ldexp(1.0, e - 1);
  return s ? -mag : mag;
}

double e4m3_value(int code) {
  const int s = (code >> 7) & 1, e = (code >> 3) & 15, m = code & 7;
  if (e == 15 && m == 7) return std::numeric_limits<double>::quiet_NaN();
  const double mag = e == 0 ? (m / 8.0) * std::ldexp(1.0, -6) : (1.0 + m / 8.0) * std::ldexp(1.0, e - 7);
  return s ? -mag : mag;
}

double e8m0_value(int b) {
  return b == 255 ? std::numeric_limits<double>::quiet_NaN() : std::ldexp(1.0, b - 127);
}

// Tables of the element values, built from the closed forms above.
struct Tables {
  double e2m1[16];
  double e4m3[256];
  Tables() {
    for (int c = 0; c < 16; ++c) e2m1[c] = e2m1_value(c);
    for (int c = 0; c < 256; ++c) e4m3[c] = e4m3_value(c);
  }
};
const Tables &tables() {
  static const Tables t;
  return t;
}

double round_bf16(double v) {
  if (v == 0.0 || !std::isfinite(v)) return v;
  int ex;
  std::frexp(v, &ex);                          // |v| in [2^(ex-1), 2^ex)
  const int q = std::max(ex - 8, -133);        // exponent of the bf16 quantum at |v|
  const double r = std::ldexp(std::nearbyint(std::ldexp(v, -q)), q);   // ties to even
  if (std::fabs(r) >= std::ldexp(1.0, 128)) return std::copysign(HUGE_VAL, v);
  return r;
}

uint16_t bf16_bits(double v) {
  const float f = static_cast<float>(round_bf16(v));   // exact: a bf16 value is a float
  uint32_t u;
  std::memcpy(&u, &f, 4);
  return static_cast<uint16_t>(u >> 16);
}

double bf16_value(uint16_t bits) {
  const uint32_t u = static_cast<uint32_t>(bits) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// Scale exponent X of one block: floor(log2 amax) - emax, clamped to
// [-127, 127]; -127 for an all-zero block.
int block_exponent(double amax, int emax) {
  if (!(amax > 0.0)) return -127;
  int ex;
  std::frexp(amax, &ex);                       // amax in [2^(ex-1), 2^ex)
  return std::min(127, std::max(-127, (ex - 1) - emax));
}

// Nearest E2M1 magnitude code (0..7) to mag >= 0: all eight candidates are
// tried in turn; a tie goes to the even code.  Above 6 the nearest is 6.
int nearest_e2m1(double mag) {
  const double *g = tables().e2m1;
  int best = 0;
  double best_d = std::fabs(mag - g[0]);
  for (int c = 1; c < 8; ++c) {
    const double d = std::fabs(mag - g[c]);
    if (d < best_d || (d == best_d && c % 2 == 0)) {
      best = c;
      best_d = d;
    }
  }
  return best;
}

// Nearest E4M3 magnitude code (0..126) to mag >= 0: the two grid neighbours
// of mag found by binary search over the ascending finite values; a tie
// goes to the even code; at or above 448 the code of 448.
int nearest_e4m3(double mag) {
  const double *g = tables().e4m3;
  if (mag >= g[kE4M3Finite - 1]) return kE4M3Finite - 1;
  int hi = static_cast<int>(std::lower_bound(g, g + kE4M3Finite, mag) - g);
  hi = std::min(std::max(hi, 1), kE4M3Finite - 1);
  const int lo = hi - 1;
  const double d_lo = mag - g[lo], d_hi = g[hi] - mag;
  return (d_hi < d_lo || (d_hi == d_lo && hi % 2 == 0)) ? hi : lo;
}

// One 32-element block -> its scale byte and 32 codes (sign in bit 3 for
// E2M1, bit 7 for E4M3).
template <bool kFp8>
uint8_t quantize_block(const double *v, uint8_t *codes) {
  double amax = 0.0;
  for (int i = 0; i < kBlock; ++i) amax = std::max(amax, std::fabs(v[i]));
  const int X = block_exponent(amax, kFp8 ? kE4M3Emax : kE2M1Emax);
  const double scale = std::ldexp(1.0, X);
  for (int i = 0; i < kBlock; ++i) {
    const double s = v[i] / scale;                       // exact: a power of two
    const int mag = kFp8 ? nearest_e4m3(std::fabs(s)) : nearest_e2m1(std::fabs(s));
    codes[i] = static_cast<uint8_t>(mag | (std::signbit(s) ? (kFp8 ? 0x80 : 0x8) : 0));
  }
  return static_cast<uint8_t>(X + 127);
}

// Rows of K values (fp64 or float32) -> codes and scales; MXFP4 packs two
// codes per byte, element 2j in the low nibble.
template <bool kFp8>
void quantize_rows(const void *src, bool f32, int64_t rows, int64_t K, uint8_t *out_codes,
                   uint8_t *out_scales, Pool &pool) {
  const int64_t nb = K / kBlock;
  pool.for_each(rows, [&](int64_t r) {
    double v[kBlock];
    uint8_t c[kBlock];
    for (int64_t b = 0; b < nb; ++b) {
      const int64_t k0 = r * K + b * kBlock;
      for (int i = 0; i < kBlock; ++i)
        v[i] = f32 ? static_cast<const float *>(src)[k0 + i] : static_cast<const double *>(src)[k0 + i];
      out_scales[r * nb + b] = quantize_block<kFp8>(v, c);
      if (kFp8) {
        std::memcpy(out_codes + k0, c, kBlock);
      } else {
        uint8_t *p = out_codes + k0 / 2;
        for (int i = 0; i < kBlock / 2; ++i) p[i] = static_cast<uint8_t>(c[2 * i] | (c[2 * i + 1] << 4));
      }
    }
  });
}

// One row of K weights -> fp64, exact: element value times 2^(scale - 127).
void decode_row(const uint8_t *codes, const uint8_t *scales, int64_t K, int wfmt, double *out) {
  const Tables &t = tables();
  for (int64_t b = 0; b < K / kBlock; ++b) {
    const double sc = e8m0_value(scales[b]);
    for (int64_t k = b * kBlock; k < (b + 1) * kBlock; ++k) {
      double v;
      if (wfmt == ORACLE_W_MXFP8) {
        v = t.e4m3[codes[k]];
      } else {
        const uint8_t byte = codes[k / 2];
        v = t.e2m1[(k % 2 == 0) ? (byte & 0xF) : (byte >> 4)];
      }
      out[k] = v * sc;
    }
  }
}

// Bytes of one weight row's codes.
int64_t row_bytes(int64_t K, int wfmt) { return wfmt == ORACLE_W_MXFP8 ? K : K / 2; }

// sum_{k < n} a[k] * b[k] in fp64, as 16 partial sums (element k goes to sum
// k mod 16) added at the end: the same fp64 additions in another order, whose
// effect is far below any tolerance here; independent sums let the CPU
// overlap them.  Every product on the path is exact in fp64 (bf16 or MXFP4
// activations times MXFP4/MXFP8 weights), so only the additions round.
double dot(const double *a, const double *b, int64_t n) {
  constexpr int kLanes = 16;
  double s[kLanes] = {};
  int64_t k = 0;
  for (; k + kLanes <= n; k += kLanes)
    for (int j = 0; j < kLanes; ++j) s[j] += a[k + j] * b[k + j];
  for (; k < n; ++k) s[k % kLanes] += a[k] * b[k];
  double total = 0.0;
  for (int j = 0; j < kLanes; ++j) total += s[j];
  return total;
}

double silu(double z) { return z / (1.0 + std::exp(-z)); }

// MXFP4 quantise-then-decode of one row of K values (W4A4 activations).
void mxfp4_roundtrip_row(double *v, int64_t K) {
  const Tables &t = tables();
  uint8_t c[kBlock];
  for (int64_t b = 0; b < K / kBlock; ++b) {
    const double sc = e8m0_value(quantize_block<false>(v + b * kBlock, c));
    for (int i = 0; i < kBlock; ++i) v[b * kBlock + i] = t.e2m1[c[i]] * sc;
  }
}

// Columns of one expert's gate/up GEMM handled by one work item.
constexpr int64_t kCols = 8;

// Gate/up GEMM + SwiGLU of one expert on n rows of a: h (n x I) gets the
// bf16-rounded values.
void expert_gate_up(const double *a, int64_t n, int64_t H, int64_t I, const uint8_t *w13,
                    const uint8_t *w13s, int wfmt, double *h, Pool &pool) {
  const int64_t rb13 = row_bytes(H, wfmt);
  // a work item owns intermediate columns [i0, i0 + kCols)
  pool.for_each((I + kCols - 1) / kCols, [&](int64_t item) {
    const int64_t i0 = item * kCols, ni = std::min(kCols, I - i0);
    std::vector<double> gate(ni * H), up(ni * H);
    for (int64_t i = 0; i < ni; ++i) {
      decode_row(w13 + (i0 + i) * rb13, w13s + (i0 + i) * (H / kBlock), H, wfmt, &gate[i * H]);
      decode_row(w13 + (I + i0 + i) * rb13, w13s + (I + i0 + i) * (H / kBlock), H, wfmt, &up[i * H]);
    }
    for (int64_t r = 0; r < n; ++r)
      for (int64_t i = 0; i < ni; ++i) {
        const double g = dot(a + r * H, &gate[i * H], H);
        const double u = dot(a + r * H, &up[i * H], H);
        h[r * I + i0 + i] = round_bf16(silu(g) * u);
      }
  });
}

// Down GEMM of one expert on n rows of bf16 h: y (n x H), fp64, unrounded.
// For W4A4 the rows of h are first quantised to MXFP4 (along I) and decoded.
void expert_down(const double *h, int64_t n, int64_t H, int64_t I, const uint8_t *w2,
                 const uint8_t *w2s, int act_fmt, int wfmt, double *y, Pool &pool) {
  const int64_t rb2 = row_bytes(I, wfmt);
  std::vector<double> hq;
  const double *hin = h;
  if (act_fmt == ORACLE_ACT_MXFP4) {
    hq.assign(h, h + n * I);
    pool.for_each(n, [&](int64_t r) { mxfp4_roundtrip_row(&hq[r * I], I); });
    hin = hq.data();
  }
  // a work item owns output columns [j0, j0 + kCols)
  pool.for_each((H + kCols - 1) / kCols, [&](int64_t item) {
    const int64_t j0 = item * kCols, nj = std::min(kCols, H - j0);
    std::vector<double> wrow(nj * I);
    for (int64_t j = 0; j < nj; ++j)
      decode_row(w2 + (j0 + j) * rb2, w2s + (j0 + j) * (I / kBlock), I, wfmt, &wrow[j * I]);
    for (int64_t r = 0; r < n; ++r)
      for (int64_t j = 0; j < nj; ++j) y[r * H + j0 + j] = dot(hin + r * I, &wrow[j * I], I);
  });
}

// One expert on n rows of a (see oracle_expert_mlp): h (n x I) always
// written, y (n x H) the fp64 down-projection.
void expert_mlp(const double *a, int64_t n, int64_t H, int64_t I, const uint8_t *w13,
                const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s, int act_fmt, int wfmt,
                double *y, double *h, Pool &pool) {
  expert_gate_up(a, n, H, I, w13, w13s, wfmt, h, pool);
  expert_down(h, n, H, I, w2, w2s, act_fmt, wfmt, y, pool);
}

void route(const float *logits, const float *gate, int64_t T, int32_t E, int32_t K, int32_t shared,
           int32_t renormalize, int32_t *ids, float *w) {
  const int32_t Kp = K + shared;
  std::vector<int32_t> order(E);
  for (int64_t t = 0; t < T; ++t) {
    const float *l = logits + t * E;
    std::iota(order.begin(), order.end(), 0);
    // larger logit first; equal logits (-0.0 == +0.0 included) keep index order
    std::stable_sort(order.begin(), order.end(), [l](int32_t a, int32_t b) { return l[a] > l[b]; });
    const double lmax = l[order[0]];
    double den = 0.0;
    if (renormalize) {
      for (int32_t k = 0; k < K; ++k) den += std::exp(static_cast<double>(l[order[k]]) - lmax);
    } else {
      for (int32_t e = 0; e < E; ++e) den += std::exp(static_cast<double>(l[e]) - lmax);
    }
    for (int32_t k = 0; k < K; ++k) {
      ids[t * Kp + k] = order[k];
      w[t * Kp + k] = static_cast<float>(std::exp(static_cast<double>(l[order[k]]) - lmax) / den);
    }
    if (shared) {
      ids[t * Kp + K] = E;
      w[t * Kp + K] = static_cast<float>(1.0 / (1.0 + std::exp(-static_cast<double>(gate[t]))));
    }
  }
}

void align(const int32_t *ids, int64_t A, int32_t Ep, int32_t tile_m, int32_t *counts,
           int32_t *offsets, int32_t *sorted_ids, int32_t *inv, std::vector<int32_t> *tiles) {
  std::fill(counts, counts + Ep, 0);
  for (int64_t a = 0; a < A; ++a) ++counts[ids[a]];
  offsets[0] = 0;
  for (int32_t e = 0; e < Ep; ++e) offsets[e + 1] = offsets[e] + counts[e];
  std::vector<int32_t> fill(offsets, offsets + Ep);
  for (int64_t a = 0; a < A; ++a) {           // ascending a: stable inside each group
    const int32_t p = fill[ids[a]]++;
    sorted_ids[p] = static_cast<int32_t>(a);
    inv[a] = p;
  }
  if (tiles) {
    tiles->clear();
    for (int32_t e = 0; e < Ep; ++e)
      for (int32_t s = 0; s < counts[e]; s += tile_m) {
        tiles->push_back(e);
        tiles->push_back(offsets[e] + s);
      }
  }
}

}  // namespace

// ================================================================ C API ==

extern "C" {

int oracle_default_threads(void) {
  cpu_set_t set;
  if (sched_getaffinity(0, sizeof(set), &set) == 0) {
    const int n = CPU_COUNT(&set);
    if (n > 0) return n;
  }
  const unsigned hw = std::thread::hardware_concurrency();
  return hw ? static_cast<int>(hw) : 1;
}

double oracle_e2m1_value(int code) { return e2m1_value(code & 15); }
double oracle_e4m3_value(int code) { return e4m3_value(code & 255); }
double oracle_e8m0_value(int b) { return e8m0_value(b & 255); }
double oracle_round_bf16(double v) { return round_bf16(v); }
uint16_t oracle_bf16_bits(double v) { return bf16_bits(v); }
double oracle_bf16_value(uint16_t bits) { return bf16_value(bits); }

void oracle_round_bf16_array(const double *v, int64_t n, double *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = round_bf16(v[i]);
}
void oracle_bf16_bits_array(const double *v, int64_t n, uint16_t *out) {
  for (int64_t i = 0; i < n; ++i) out[i] = bf16_bits(v[i]);
}

int oracle_mxfp4_quantize(const void *v, int src_f32, int64_t rows, int64_t K, uint8_t *packed,
                          uint8_t *scales, int threads) {
  if (!v || !packed || !scales || rows < 0 || K <= 0 || K % kBlock) return -1;
  Pool pool(resolve_threads(threads));
  quantize_rows<false>(v, src_f32 != 0, rows, K, packed, scales, pool);
  return 0;
}

int oracle_mxfp8_quantize(const void *v, int src_f32, int64_t rows, int64_t K, uint8_t *codes,
                          uint8_t *scales, int threads) {
  if (!v || !codes || !scales || rows < 0 || K <= 0 || K % kBlock) return -1;
  Pool pool(resolve_threads(threads));
  quantize_rows<true>(v, src_f32 != 0, rows, K, codes, scales, pool);
  return 0;
}

int oracle_mxfp4_decode(const uint8_t *packed, const uint8_t *scales, int64_t rows, int64_t K,
                        double *out) {
  if (!packed || !scales || !out || rows < 0 || K <= 0 || K % kBlock) return -1;
  for (int64_t r = 0; r < rows; ++r)
    decode_row(packed + r * (K / 2), scales + r * (K / kBlock), K, ORACLE_W_MXFP4, out + r * K);
  return 0;
}

int oracle_mxfp8_decode(const uint8_t *codes, const uint8_t *scales, int64_t rows, int64_t K,
                        double *out) {
  if (!codes || !scales || !out || rows < 0 || K <= 0 || K % kBlock) return -1;
  for (int64_t r = 0; r < rows; ++r)
    decode_row(codes + r * K, scales + r * (K / kBlock), K, ORACLE_W_MXFP8, out + r * K);
  return 0;
}

int oracle_route(const float *logits, const float *gate, int64_t T, int32_t E, int32_t K,
                 int32_t shared, int32_t renormalize, int32_t *ids, float *w) {
  if (T < 0 || E < 1 || K < 1 || K > E || (shared != 0 && shared != 1)) return -1;
  if (T > 0 && (!logits || !ids || !w || (shared && !gate))) return -1;
  route(logits, gate, T, E, K, shared, renormalize, ids, w);
  return 0;
}

int oracle_align(const int32_t *ids, int64_t A, int32_t Ep, int32_t tile_m, int32_t *counts,
                 int32_t *offsets, int32_t *sorted_ids, int32_t *inv, int32_t *tiles,
                 int64_t max_tiles, int64_t *n_tiles) {
  if (A < 0 || Ep < 1 || tile_m < 1 || !counts || !offsets || !n_tiles) return -1;
  if (A > 0 && (!ids || !sorted_ids || !inv)) return -1;
  for (int64_t a = 0; a < A; ++a)
    if (ids[a] < 0 || ids[a] >= Ep) return -1;
  std::vector<int32_t> list;
  align(ids, A, Ep, tile_m, counts, offsets, sorted_ids, inv, &list);
  const int64_t n = static_cast<int64_t>(list.size() / 2);
  *n_tiles = n;
  if (tiles) {
    if (n > max_tiles) return -1;
    std::copy(list.begin(), list.end(), tiles);
  }
  return 0;
}

int oracle_router_logits(const uint16_t *x_bits, const uint16_t *w_bits, int64_t T, int64_t R,
                         int64_t H, double *out, int threads) {
  if (T < 0 || R < 0 || H < 1 || (T > 0 && R > 0 && (!x_bits || !w_bits || !out))) return -1;
  std::vector<double> x(T * H), w(R * H);
  for (int64_t i = 0; i < T * H; ++i) x[i] = bf16_value(x_bits[i]);
  for (int64_t i = 0; i < R * H; ++i) w[i] = bf16_value(w_bits[i]);
  Pool pool(resolve_threads(threads));
  pool.for_each(T, [&](int64_t t) {
    for (int64_t r = 0; r < R; ++r) out[t * R + r] = dot(&x[t * H], &w[r * H], H);
  });
  return 0;
}

int oracle_expert_mlp(const double *a, int64_t n, int64_t H, int64_t I, const uint8_t *w13,
                      const uint8_t *w13s, const uint8_t *w2, const uint8_t *w2s, int act_fmt,
                      int wfmt, double *y, double *h, int threads) {
  if (n < 0 || H <= 0 || I <= 0 || H % kBlock || I % kBlock) return -1;
  if (!a || !w13 || !w13s || !w2 || !w2s || !y) return -1;
  if (wfmt == ORACLE_W_MXFP8 && act_fmt != ORACLE_ACT_BF16) return -1;
  std::vector<double> hbuf;
  if (!h) {
    hbuf.resize(n * I);
    h = hbuf.data();
  }
  Pool pool(resolve_threads(threads));
  expert_mlp(a, n, H, I, w13, w13s, w2, w2s, act_fmt, wfmt, y, h, pool);
  return 0;
}

int oracle_forward(const uint16_t *x_bits, const float *logits, const float *gate,
                   const uint8_t *const *w13, const uint8_t *const *w13s,
                   const uint8_t *const *w2, const uint8_t *const *w2s, int64_t T, int64_t H,
                   int64_t I, int32_t E, int32_t K, int32_t shared, int act_fmt, int wfmt,
                   int32_t renormalize, int32_t round_y, const int64_t *tokens,
                   int64_t n_tokens, int threads, int32_t *ids_out, float *w_out,
                   uint16_t *out_bits, double *out_f64, uint16_t *h_bits, double *seconds) {
  const auto t_start = std::chrono::steady_clock::now();
  if (T < 0 || H <= 0 || I <= 0 || H % kBlock || I % kBlock || E < 1 || K < 1 || K > E) return -1;
  if ((shared != 0 && shared != 1) || (shared && !gate)) return -1;
  if (wfmt == ORACLE_W_MXFP8 && act_fmt != ORACLE_ACT_BF16) return -1;
  if (T > 0 && (!x_bits || !logits || !w13 || !w13s || !w2 || !w2s)) return -1;
  if (tokens && h_bits) return -1;
  const int32_t Kp = K + shared, Ep = E + shared;
  const int64_t A = T * Kp;

  // 1. routing, 2. grouping (every token)
  std::vector<int32_t> ids(A), counts(Ep), offsets(Ep + 1), sorted_ids(A), inv(A);
  std::vector<float> w(A);
  route(logits, gate, T, E, K, shared, renormalize, ids.data(), w.data());
  align(ids.data(), A, Ep, 32, counts.data(), offsets.data(), sorted_ids.data(), inv.data(), nullptr);

  // the tokens whose outputs are computed; sel[t] = their position, or -1
  std::vector<int64_t> toks;
  if (tokens) {
    toks.assign(tokens, tokens + n_tokens);
  } else {
    toks.resize(T);
    std::iota(toks.begin(), toks.end(), 0);
  }
  const int64_t n = static_cast<int64_t>(toks.size());
  std::vector<int64_t> sel(T, -1);
  for (int64_t j = 0; j < n; ++j) {
    if (toks[j] < 0 || toks[j] >= T) return -1;
    sel[toks[j]] = j;
  }
  for (int32_t e = 0; e < Ep; ++e) {
    bool needed = false;
    for (int32_t p = offsets[e]; p < offsets[e + 1] && !needed; ++p) needed = sel[sorted_ids[p] / Kp] >= 0;
    if (needed && (!w13[e] || !w13s[e] || !w2[e] || !w2s[e])) return -2;
  }

  Pool pool(resolve_threads(threads));

  // 3. the activations each selected token feeds its experts: bf16 values,
  //    or (W4A4) their MXFP4 quantise-then-decode
  std::vector<double> act(n * H);
  pool.for_each(n, [&](int64_t j) {
    double *row = &act[j * H];
    for (int64_t k = 0; k < H; ++k) row[k] = bf16_value(x_bits[toks[j] * H + k]);
    if (act_fmt == ORACLE_ACT_MXFP4) mxfp4_roundtrip_row(row, H);
  });

  // 4. every expert on its selected rows; y per (token, slot), rounded to
  //    bf16 when round_y (where a path stores y in bf16 before the combine)
  std::vector<double> y(n * Kp * H);
  std::vector<double> a_e, y_e, h_e;
  for (int32_t e = 0; e < Ep; ++e) {
    std::vector<int32_t> rows;                 // sorted positions of the expert's selected rows
    for (int32_t p = offsets[e]; p < offsets[e + 1]; ++p)
      if (sel[sorted_ids[p] / Kp] >= 0) rows.push_back(p);
    const int64_t R = static_cast<int64_t>(rows.size());
    if (R == 0) continue;
    a_e.resize(R * H);
    y_e.resize(R * H);
    h_e.resize(R * I);
    for (int64_t r = 0; r < R; ++r) {
      const int64_t j = sel[sorted_ids[rows[r]] / Kp];
      std::copy(&act[j * H], &act[j * H] + H, &a_e[r * H]);
    }
    expert_mlp(a_e.data(), R, H, I, w13[e], w13s[e], w2[e], w2s[e], act_fmt, wfmt, y_e.data(),
               h_e.data(), pool);
    pool.for_each(R, [&](int64_t r) {
      const int32_t flat = sorted_ids[rows[r]];
      const int64_t j = sel[flat / Kp], k = flat % Kp;
      double *dst = &y[(j * Kp + k) * H];
      for (int64_t c = 0; c < H; ++c) dst[c] = round_y ? round_bf16(y_e[r * H + c]) : y_e[r * H + c];
      if (h_bits)
        for (int64_t i = 0; i < I; ++i) h_bits[static_cast<int64_t>(rows[r]) * I + i] = bf16_bits(h_e[r * I + i]);
    });
  }

  // 5. weighted combine, slots in order, fp64; one rounding to bf16
  pool.for_each(n, [&](int64_t j) {
    const int64_t t = toks[j];
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int32_t k = 0; k < Kp; ++k)
        acc += static_cast<double>(w[t * Kp + k]) * y[(j * Kp + k) * H + c];
      if (out_f64) out_f64[j * H + c] = acc;
      if (out_bits) out_bits[j * H + c] = bf16_bits(acc);
    }
  });

  if (ids_out) std::copy(ids.begin(), ids.end(), ids_out);
  if (w_out) std::copy(w.begin(), w.end(), w_out);
  if (seconds)
    *seconds = std::chrono::duration<double>(std::chrono::steady_clock::now() - t_start).count();
  return 0;
}

int oracle_forward_from_h(const uint16_t *h_bits, const float *logits, const float *gate,
                          const uint8_t *const *w2, const uint8_t *const *w2s, int64_t T,
                          int64_t H, int64_t I, int32_t E, int32_t K, int32_t shared, int act_fmt,
                          int wfmt, int32_t renormalize, int32_t round_y, int threads,
                          uint16_t *out_bits, double *out_f64) {
  if (T < 0 || H <= 0 || I <= 0 || H % kBlock || I % kBlock || E < 1 || K < 1 || K > E) return -1;
  if ((shared != 0 && shared != 1) || (shared && !gate)) return -1;
  if (wfmt == ORACLE_W_MXFP8 && act_fmt != ORACLE_ACT_BF16) return -1;
  if (T > 0 && (!h_bits || !logits || !w2 || !w2s)) return -1;
  const int32_t Kp = K + shared, Ep = E + shared;
  const int64_t A = T * Kp;
  std::vector<int32_t> ids(A), counts(Ep), offsets(Ep + 1), sorted_ids(A), inv(A);
  std::vector<float> w(A);
  route(logits, gate, T, E, K, shared, renormalize, ids.data(), w.data());
  align(ids.data(), A, Ep, 32, counts.data(), offsets.data(), sorted_ids.data(), inv.data(), nullptr);
  for (int32_t e = 0; e < Ep; ++e)
    if (counts[e] > 0 && (!w2[e] || !w2s[e])) return -2;
  Pool pool(resolve_threads(threads));
  std::vector<double> y(A * H);                // per flat assignment
  std::vector<double> h_e, y_e;
  for (int32_t e = 0; e < Ep; ++e) {
    const int64_t R = counts[e], p0 = offsets[e];
    if (R == 0) continue;
    h_e.resize(R * I);
    y_e.resize(R * H);
    for (int64_t i = 0; i < R * I; ++i) h_e[i] = bf16_value(h_bits[p0 * I + i]);
    expert_down(h_e.data(), R, H, I, w2[e], w2s[e], act_fmt, wfmt, y_e.data(), pool);
    pool.for_each(R, [&](int64_t r) {
      double *dst = &y[static_cast<int64_t>(sorted_ids[p0 + r]) * H];
      for (int64_t c = 0; c < H; ++c) dst[c] = round_y ? round_bf16(y_e[r * H + c]) : y_e[r * H + c];
    });
  }
  pool.for_each(T, [&](int64_t t) {
    for (int64_t c = 0; c < H; ++c) {
      double acc = 0.0;
      for (int32_t k = 0; k < Kp; ++k)
        acc += static_cast<double>(w[t * Kp + k]) * y[(t * Kp + k) * H + c];
      if (out_f64) out_f64[t * H + c] = acc;
      if (out_bits) out_bits[t * H + c] = bf16_bits(acc);
    }
  });
  return 0;
}

// The partial outputs of G ranks summed, the residual added, then RMSNorm
// (VibeSys post, section "Communication and concurrency": the all-reduce
// fused with the residual add and RMSNorm; RMSNorm in its textbook form).
// Each row: h = bf16(residual + sum of the partials), fp64 sums of exact
// bf16 values; then the mean of h^2 over the row, and y = bf16(h * rstd * gamma).
int oracle_residual_rmsnorm(const uint16_t *partials, int32_t G, const uint16_t *residual,
                            const uint16_t *gamma, double eps, int64_t T, int64_t H,
                            uint16_t *h_out, uint16_t *y_out, double *rstd_out) {
  if (!partials || !gamma || !h_out || !y_out || G < 1 || T < 0 || H < 1 || !(eps >= 0.0))
    return -1;
  std::vector<double> h(H);
  for (int64_t t = 0; t < T; ++t) {
    double ss = 0.0;
    for (int64_t j = 0; j < H; ++j) {
      double s = residual ? bf16_value(residual[t * H + j]) : 0.0;
      for (int32_t g = 0; g < G; ++g) s += bf16_value(partials[(g * T + t) * H + j]);
      h[j] = round_bf16(s);
      h_out[t * H + j] = bf16_bits(h[j]);
      ss += h[j] * h[j];
    }
    const double rstd = 1.0 / std::sqrt(ss / static_cast<double>(H) + eps);
    if (rstd_out) rstd_out[t] = rstd;
    for (int64_t j = 0; j < H; ++j) y_out[t * H + j] = bf16_bits(h[j] * rstd * bf16_value(gamma[j]));
  }
  return 0;
}

}  // extern "C"
