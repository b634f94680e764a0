// Host-side ternarizer and packers of the C ABI (include/tq.h).
//
// Definitions follow the project page "Scaling Laws and Efficient Inference
// for Ternary Language Models": "The model" (steps 1-2) for the ternarization,
// "Packing ternary weights" for both packings, "Fast inference on CPUs" for the
// 256-weight scale block.  Where the page leaves a choice open the library
// takes: an exactly rounded fp64 sum of |W| over the whole matrix, the decision
// on the fp64 quotient with ties to even, weight 4i+j in byte i bits 2j..2j+1,
// the first of five TQ1 weights as the most significant base-3 digit, and the
// last TQ1 group of a row padded with zero trits.

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

#include "tq.h"

namespace {

// ---------------------------------------------------------------- threading

template <class F>
void parallel_rows(int64_t N, int64_t work_per_row, F&& body) {
  int64_t total = N * std::max<int64_t>(work_per_row, 1);
  unsigned hw = std::thread::hardware_concurrency();
  int64_t threads = std::min<int64_t>(hw ? hw : 1, 64);
  if (total < (int64_t(1) << 20) || threads <= 1 || N < 2) {
    body(0, N, 0);
    return;
  }
  threads = std::min<int64_t>(threads, N);
  std::vector<std::thread> pool;
  int64_t per = (N + threads - 1) / threads;
  int tid = 0;
  for (int64_t r0 = 0; r0 < N; r0 += per, ++tid) {
    int64_t r1 = std::min(N, r0 + per);
    pool.emplace_back([&, r0, r1, tid] { body(r0, r1, tid); });
  }
  for (auto& t : pool) t.join();
}

int64_t thread_slots(int64_t N) {
  unsigned hw = std::thread::hardware_concurrency();
  return std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(hw ? hw : 1, 64), N));
}

// ---------------------------------------------------------------- exact sum of |W|
//
// Every finite fp32 value is m * 2^(e' - 150) with an integer m < 2^24 and
// e' = max(biased exponent, 1).  Summing the m of each exponent in a 64-bit
// integer is exact; the 255 bucket totals are then added into a wide integer
// and rounded once to fp64 (nearest, ties to even).  The result is the exactly
// rounded sum, independent of order and thread count.

struct BigSum {
  static constexpr int kLimbs = 12;  // 384 bits, enough for 2^64 * 2^253
  uint32_t limb[kLimbs] = {0};

  void add_shifted(uint64_t v, int shift) {  // += v << shift
    int li = shift / 32, bi = shift % 32;
    // spread v << bi over up to three limbs
    unsigned __int128 w = (unsigned __int128)v << bi;
    uint64_t carry = 0;
    for (int i = li; i < kLimbs; ++i) {
      uint64_t part = (uint64_t)(w & 0xFFFFFFFFu);
      w >>= 32;
      uint64_t s = (uint64_t)limb[i] + part + carry;
      limb[i] = (uint32_t)s;
      carry = s >> 32;
      if (w == 0 && carry == 0) break;
    }
  }
  int top_bit() const {
    for (int i = kLimbs - 1; i >= 0; --i)
      if (limb[i]) return i * 32 + 31 - __builtin_clz(limb[i]);
    return -1;
  }
  int bit(int b) const { return b < 0 ? 0 : (limb[b / 32] >> (b % 32)) & 1; }
  bool any_below(int b) const {  // any set bit strictly below position b
    if (b <= 0) return false;
    int full = b / 32;
    for (int i = 0; i < full; ++i)
      if (limb[i]) return true;
    int rem = b % 32;
    return rem && (limb[full] & ((1u << rem) - 1));
  }
  // Value * 2^scale_exp rounded to nearest even double.
  double to_double(int scale_exp) const {
    int h = top_bit();
    if (h < 0) return 0.0;
    uint64_t mant = 0;
    int lo = h - 52;  // lowest kept bit
    for (int b = h; b >= std::max(lo, 0); --b) mant = (mant << 1) | (uint64_t)bit(b);
    if (lo < 0) return std::ldexp((double)mant, scale_exp);  // fewer than 53 bits: exact
    int guard = bit(lo - 1);
    bool sticky = any_below(lo - 1);
    if (guard && (sticky || (mant & 1))) {
      ++mant;
      if (mant == (uint64_t(1) << 53)) { mant >>= 1; ++lo; }
    }
    return std::ldexp((double)mant, lo + scale_exp);
  }
};

// Returns TQ_OK and the exactly rounded sum, or TQ_ERR_VALUE on NaN/Inf.
int exact_abs_sum(const float* W, int64_t N, int64_t K, double* out) {
  int64_t slots = thread_slots(N);
  std::vector<uint64_t> buckets((size_t)slots * 256, 0);
  std::vector<int> bad((size_t)slots, 0);
  parallel_rows(N, K, [&](int64_t r0, int64_t r1, int tid) {
    uint64_t* bk = &buckets[(size_t)tid * 256];
    for (int64_t n = r0; n < r1; ++n) {
      const float* row = W + n * K;
      for (int64_t k = 0; k < K; ++k) {
        uint32_t u;
        std::memcpy(&u, &row[k], 4);
        uint32_t e = (u >> 23) & 0xFF;
        uint32_t m = u & 0x7FFFFF;
        if (e == 0xFF) { bad[tid] = 1; return; }
        if (e) m |= 0x800000;
        bk[e] += m;
      }
    }
  });
  for (int b : bad)
    if (b) return TQ_ERR_VALUE;
  BigSum s;
  for (int e = 0; e < 255; ++e) {
    uint64_t tot_hi = 0, tot = 0;  // sum over threads without overflow
    for (int64_t t = 0; t < slots; ++t) {
      uint64_t v = buckets[(size_t)t * 256 + e];
      uint64_t nt = tot + v;
      tot_hi += (nt < tot);
      tot = nt;
    }
    int shift = (e ? e : 1) - 1;  // value = m * 2^(e' - 150) = m * 2^(e'-1) * 2^-149
    if (tot) s.add_shifted(tot, shift);
    if (tot_hi) s.add_shifted(tot_hi, shift + 64);
  }
  *out = s.to_double(-149);
  return TQ_OK;
}

// ---------------------------------------------------------------- fp64 -> fp16

// One round-to-nearest-even step from binary64 to binary16.
uint16_t f64_to_f16_bits(double x) {
  uint64_t u;
  std::memcpy(&u, &x, 8);
  uint16_t sign = (uint16_t)((u >> 48) & 0x8000);
  int be = (int)((u >> 52) & 0x7FF);
  uint64_t mant = u & ((uint64_t(1) << 52) - 1);
  if (be == 0x7FF) return sign | (mant ? 0x7E00 : 0x7C00);
  if (be == 0) return sign;  // zero or fp64 subnormal (far below half's range)
  int E = be - 1023;
  uint64_t sig = mant | (uint64_t(1) << 52);
  int shift = (E >= -14) ? 42 : 42 + (-14 - E);
  if (shift >= 64) return sign;
  uint64_t r = sig >> shift;
  uint64_t rem = sig & ((uint64_t(1) << shift) - 1);
  uint64_t half = uint64_t(1) << (shift - 1);
  if (rem > half || (rem == half && (r & 1))) ++r;
  if (E >= -14) {
    if (r == (1u << 11)) { r >>= 1; ++E; }
    if (E > 15) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | (r & 0x3FF));
  }
  return sign | (uint16_t)r;  // subnormal; r == 0x400 is the smallest normal
}

// ---------------------------------------------------------------- ternarization

struct Gamma {
  double gamma;
  int status;
};

Gamma compute_gamma(const float* W, int64_t N, int64_t K, double eps) {
  double S = 0.0;
  int st = exact_abs_sum(W, N, K, &S);
  if (st != TQ_OK) return {0.0, st};
  double g = eps + S / (double)(N * K);
  if (!(std::isfinite(g) && g > 0.0)) return {0.0, TQ_ERR_VALUE};
  return {g, TQ_OK};
}

// round(clip(q, -1, 1)) with ties to even: only |q| > 1/2 leaves zero.
inline int8_t trit_of(float w, double gamma) {
  double q = (double)w / gamma;
  return (int8_t)((q > 0.5) - (q < -0.5));
}

inline bool valid_trit(int8_t t) { return t >= -1 && t <= 1; }

// Row producer: writes the K trits of row n into buf; returns false on a bad trit.
struct RowSource {
  int kind;
  const void* W;
  int64_t K;
  double gamma;
  bool row(int64_t n, int8_t* buf) const {
    if (kind == TQ_SRC_LATENT_F32) {
      const float* r = static_cast<const float*>(W) + n * K;
      for (int64_t k = 0; k < K; ++k) buf[k] = trit_of(r[k], gamma);
      return true;
    }
    const int8_t* r = static_cast<const int8_t*>(W) + n * K;
    for (int64_t k = 0; k < K; ++k) {
      if (!valid_trit(r[k])) return false;
      buf[k] = r[k];
    }
    return true;
  }
};

int prepare_source(int kind, const void* W, int64_t N, int64_t K, double eps,
                   uint16_t* scales, double* gamma_out, RowSource* src) {
  src->kind = kind;
  src->W = W;
  src->K = K;
  src->gamma = 0.0;
  if (kind == TQ_SRC_LATENT_F32) {
    Gamma g = compute_gamma(static_cast<const float*>(W), N, K, eps);
    if (g.status != TQ_OK) return g.status;
    src->gamma = g.gamma;
    uint16_t h = f64_to_f16_bits(g.gamma);
    int64_t ns = N * (K / 256);
    for (int64_t i = 0; i < ns; ++i) scales[i] = h;
    if (gamma_out) *gamma_out = g.gamma;
  }
  return TQ_OK;
}

int check_kind_args(int kind, const void* W, const void* qs, const uint16_t* scales) {
  if (!W || !qs) return TQ_ERR_NULL;
  if (kind != TQ_SRC_TERNARY_I8 && kind != TQ_SRC_LATENT_F32) return TQ_ERR_VALUE;
  if (kind == TQ_SRC_LATENT_F32 && !scales) return TQ_ERR_NULL;
  return TQ_OK;
}

// TQ1 code of five shifted digits, first digit most significant.
inline uint8_t tq1_code(const int8_t* t, int count) {
  unsigned n = 0;
  for (int j = 0; j < 5; ++j) n = 3 * n + (unsigned)((j < count ? t[j] : 0) + 1);
  return (uint8_t)((n * 256 + 242) / 243);
}

// Decode table for TQ1 by the multiply route: five times t = 3q, digit = t >> 8,
// q = t & 255.  An entry is valid when re-encoding gives the byte back.
struct Tq1Table {
  int8_t trit[256][5];
  bool valid[256];
  Tq1Table() {
    for (int b = 0; b < 256; ++b) {
      unsigned q = (unsigned)b;
      for (int j = 0; j < 5; ++j) {
        unsigned t = 3 * q;
        trit[b][j] = (int8_t)((int)(t >> 8) - 1);
        q = t & 0xFF;
      }
      valid[b] = tq1_code(trit[b], 5) == b;
    }
  }
};

const Tq1Table& tq1_table() {
  static const Tq1Table table;
  return table;
}

}  // namespace

// ====================================================================== ABI

extern "C" {

const char* tq_status_string(int status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_ERR_NULL: return "null pointer";
    case TQ_ERR_SHAPE: return "invalid shape";
    case TQ_ERR_VALUE: return "invalid value";
    case TQ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case TQ_ERR_DEVICE: return "HIP device error";
    case TQ_ERR_UNSUPPORTED: return "unsupported option";
    default: return "unknown status";
  }
}

int tq_abi_version(void) { return 1; }

int64_t tq_tq2_bytes(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % 4) return -1;
  return N * (K / 4);
}

int64_t tq_tq1_ldq(int64_t K) {
  if (K < 0) return -1;
  int64_t g = (K + 4) / 5;
  return (g + 15) / 16 * 16;
}

int64_t tq_num_scales(int64_t N, int64_t K) {
  if (N < 0 || K < 0 || K % 256) return -1;
  return N * (K / 256);
}

int tq_ternarize_f32(const float* W, int64_t N, int64_t K, double eps, int8_t* T,
                     double* gamma_out) {
  if (!W) return TQ_ERR_NULL;
  if (N < 1 || K < 1) return TQ_ERR_SHAPE;
  Gamma g = compute_gamma(W, N, K, eps);
  if (g.status != TQ_OK) return g.status;
  if (gamma_out) *gamma_out = g.gamma;
  if (T) {
    parallel_rows(N, K, [&](int64_t r0, int64_t r1, int) {
      for (int64_t n = r0; n < r1; ++n)
        for (int64_t k = 0; k < K; ++k) T[n * K + k] = trit_of(W[n * K + k], g.gamma);
    });
  }
  return TQ_OK;
}

int tq_pack_tq2(int kind, const void* W, int64_t N, int64_t K, double eps, uint8_t* qs,
                uint16_t* scales, double* gamma_out) {
  int st = check_kind_args(kind, W, qs, scales);
  if (st) return st;
  if (N < 1 || K < 256 || K % 256) return TQ_ERR_SHAPE;
  RowSource src;
  st = prepare_source(kind, W, N, K, eps, scales, gamma_out, &src);
  if (st) return st;
  std::vector<int> bad((size_t)thread_slots(N), 0);
  parallel_rows(N, K, [&](int64_t r0, int64_t r1, int tid) {
    std::vector<int8_t> t((size_t)K);
    for (int64_t n = r0; n < r1; ++n) {
      if (!src.row(n, t.data())) { bad[tid] = 1; return; }
      uint8_t* out = qs + n * (K / 4);
      for (int64_t i = 0; i < K / 4; ++i) {
        const int8_t* w = &t[(size_t)(4 * i)];
        out[i] = (uint8_t)((w[0] + 1) | ((w[1] + 1) << 2) | ((w[2] + 1) << 4) | ((w[3] + 1) << 6));
      }
    }
  });
  for (int b : bad)
    if (b) return TQ_ERR_VALUE;
  return TQ_OK;
}

int tq_pack_tq1(int kind, const void* W, int64_t N, int64_t K, double eps, int64_t ldq,
                uint8_t* qs, uint16_t* scales, double* gamma_out) {
  int st = check_kind_args(kind, W, qs, scales);
  if (st) return st;
  if (N < 1 || K < 256 || K % 256) return TQ_ERR_SHAPE;
  int64_t G = (K + 4) / 5;
  if (ldq < G) return TQ_ERR_SHAPE;
  RowSource src;
  st = prepare_source(kind, W, N, K, eps, scales, gamma_out, &src);
  if (st) return st;
  std::vector<int> bad((size_t)thread_slots(N), 0);
  parallel_rows(N, K, [&](int64_t r0, int64_t r1, int tid) {
    std::vector<int8_t> t((size_t)K);
    for (int64_t n = r0; n < r1; ++n) {
      if (!src.row(n, t.data())) { bad[tid] = 1; return; }
      uint8_t* out = qs + n * ldq;
      for (int64_t g = 0; g < G; ++g) {
        int64_t k0 = 5 * g;
        out[g] = tq1_code(&t[(size_t)k0], (int)std::min<int64_t>(5, K - k0));
      }
      for (int64_t g = G; g < ldq; ++g) out[g] = 0;
    }
  });
  for (int b : bad)
    if (b) return TQ_ERR_VALUE;
  return TQ_OK;
}

int tq_unpack_tq2(const uint8_t* qs, int64_t N, int64_t K, int8_t* T) {
  if (!qs || !T) return TQ_ERR_NULL;
  if (N < 1 || K < 1 || K % 4) return TQ_ERR_SHAPE;
  std::vector<int> bad((size_t)thread_slots(N), 0);
  parallel_rows(N, K, [&](int64_t r0, int64_t r1, int tid) {
    for (int64_t n = r0; n < r1; ++n) {
      const uint8_t* in = qs + n * (K / 4);
      int8_t* out = T + n * K;
      for (int64_t i = 0; i < K / 4; ++i) {
        unsigned b = in[i];
        for (int j = 0; j < 4; ++j) {
          unsigned d = (b >> (2 * j)) & 3u;
          if (d == 3) { bad[tid] = 1; return; }
          out[4 * i + j] = (int8_t)((int)d - 1);
        }
      }
    }
  });
  for (int b : bad)
    if (b) return TQ_ERR_VALUE;
  return TQ_OK;
}

int tq_unpack_tq1(const uint8_t* qs, int64_t N, int64_t K, int64_t ldq, int8_t* T) {
  if (!qs || !T) return TQ_ERR_NULL;
  int64_t G = (K + 4) / 5;
  if (N < 1 || K < 1 || ldq < G) return TQ_ERR_SHAPE;
  const Tq1Table& tab = tq1_table();
  std::vector<int> bad((size_t)thread_slots(N), 0);
  parallel_rows(N, K, [&](int64_t r0, int64_t r1, int tid) {
    for (int64_t n = r0; n < r1; ++n) {
      const uint8_t* in = qs + n * ldq;
      int8_t* out = T + n * K;
      for (int64_t g = 0; g < G; ++g) {
        unsigned b = in[g];
        if (!tab.valid[b]) { bad[tid] = 1; return; }
        for (int j = 0; j < 5; ++j) {
          int64_t k = 5 * g + j;
          if (k < K) {
            out[k] = tab.trit[b][j];
          } else if (tab.trit[b][j] != 0) {
            bad[tid] = 1;
            return;
          }
        }
      }
    }
  });
  for (int b : bad)
    if (b) return TQ_ERR_VALUE;
  return TQ_OK;
}

}  // extern "C"
