// MFMA kernel for 1.6-bit weights: Y = X (s . T)^T with T packed five trits
// per byte.
//
// Follows the project page "Scaling Laws and Efficient Inference for Ternary
// Language Models": "The model" (step 3) for the product; "1.6 bits per
// weight" for the code (byte b = floor((256 N + 242) / 243) of the base-3
// value N of five shifted digits, first weight most significant) and for the
// decoder that multiplies by 3 and splits high byte from low byte five times;
// "Fast inference on CPUs" for the 256-weight scale block; "TriRun: ternary
// inference on GPUs" for FP32 accumulation and FP16 output.  MI355X design:
//
//  * two weight bytes sit in the two 16-bit halves of a register, so each
//    step of the decoder (t = 3 q with v_lshl_add_u32, the digit field of t
//    kept by one v_and_b32, q = t & 0xff) serves two weights.  The kept field
//    d' 256 is an fp16 subnormal worth d' 2^-16, which the MFMA multiplies
//    exactly (it keeps subnormals); the shift d = d' - 1 is the sum of the
//    activations, taken in fp32 while staging them, seeding the accumulator;
//  * v_mfma_f32_16x16x32_f16 does the multiply-accumulate with 16 activation
//    rows per launch slice (grid.y walks M in slices of 16);
//  * the four lane groups of a wave cover one 32-byte span of a row (160
//    weights, 8 bytes per lane).  A span holds at most one 256-weight block
//    boundary and the MFMA sums over all four lane groups, so with C_a = the
//    span's MFMA sum and C_b = the same sum over the weights past the boundary
//    only, the span adds s_a C_a + (s_b - s_a) C_b: exact block scales
//    without per-weight work.  C_b comes from a masked copy of the
//    activations (zero before the boundary) kept next to the plain copy;
//  * both activation copies, with their sums, are staged in LDS in the
//    decoder's weight order; waves of a workgroup take spans round robin and
//    keep a ring of register buffers of weights in flight (the last ring group
//    issues no loads); per-wave set-up is kept to shifts and masks; partial
//    sums meet in LDS.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"
#include "tq_tq1.h"

namespace tq {
namespace {

template <int I, int N, class F>
__device__ __forceinline__ void sfor1(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor1<I + 1, N>(f);
  }
}

constexpr int kPad = 16;
constexpr int kXLds = 128 * 1024;   // activation window budget
constexpr int kScLds = 24 * 1024;   // staged scales budget (fp32)
constexpr int kLdsMax = 160 * 1024;
constexpr int kRowsMax = 32;        // activation rows of a workgroup (two 16-row slices)
constexpr int kSumBytes = 2 * kRowsMax * 4;  // per span: plain and masked row sums, fp32
constexpr int kTrash = (kUnitBytes + 4 * (kRowsMax + 1) + 15) & ~15;  // a unit's operands, sums
constexpr int kScaleRegs = 4;                // block scales per thread loaded ahead
// Activations in LDS, decoder order: for every (row m, span u, lane group g,
// operand o) 8 halves.  o < 5: plain X at the operand's weights (zero past K);
// o >= 5: the same masked to the weights at or past the span's block boundary.
// Next to them, per span, -2^-16 times the sum over the span of each row's
// plain and masked activations.  A window holds spans [u0, u0 + nu) of rows
// m_base .. m_base + mrows - 1; thread q stages unit q = (m, u, g) of every
// window (units <= threads): the 40 consecutive activations k0 = 160 (u0 + u)
// + 40 g .. k0 + 39, read with five coalesced 16-byte loads (K and k0 are
// multiples of 8, so a chunk is either wholly inside the row or wholly past
// K) one window ahead, then written with one v_perm_b32 per operand dword.
struct Tq1Unit {
  uint32_t e[20];
  int m, u;
  int k0;  // first activation of the unit
  bool ok;
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Position of unit q in a window of nuw spans: u + nuw m = q / 4 (float
// reciprocal: exact for q / 4 < 2^11), no integer division.
__device__ __forceinline__ void tq1_unit_at(Tq1Unit& un, int q, int nuw, int mrows) {
  const int r = q >> 2;
  const int m = (int)(((float)r + 0.5f) * (1.0f / (float)nuw));
  un.ok = m < mrows;
  un.m = un.ok ? m : 0;
  un.u = un.ok ? r - m * nuw : 0;
}

// Loads only (chunks past K re-read the row's first chunk; the store zeroes
// them), so that nothing waits for the loads before the store.
__device__ __forceinline__ void tq1_load_unit(Tq1Unit& un, const uint16_t* __restrict__ X,
                                              int m_base, int K, int u0, int g) {
  un.k0 = 160 * (u0 + un.u) + 40 * g;
  const uint16_t* xrow = X + (size_t)(m_base + un.m) * K;
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    const int k = un.k0 + 8 * c;
    const u32x4 v = *reinterpret_cast<const u32x4*>(xrow + (k + 8 <= K ? k : 0));
#pragma unroll
    for (int t = 0; t < 4; ++t) un.e[4 * c + t] = v[t];
  }
}

// Writes the unit's ten operands (tq1_store_operands' layout) and, after a
// sum over the four lane groups of its span, the span's row sums.
__device__ __forceinline__ void tq1_store_unit(const Tq1Unit& un, unsigned char* xs, float* sums,
                                               unsigned char* trash, int u0, int g, int xstride,
                                               int K) {
  const int k0 = un.k0;
  uint32_t e[20];
#pragma unroll
  for (int c = 0; c < 5; ++c)
#pragma unroll
    for (int t = 0; t < 4; ++t) e[4 * c + t] = k0 + 8 * c + 8 <= K ? un.e[4 * c + t] : 0u;
  const int kb = (((160 * (u0 + un.u)) >> 8) + 1) << 8;  // first block boundary of the span
  const int lim = kb - k0;
  unsigned char* dst = un.ok ? xs + un.m * xstride + un.u * kSpanBytes + g * kUnitBytes : trash;
  // Activation i of the unit is kept in the masked copy when i >= lim: bit i
  // of keep (all ones for lim <= 0, none for lim >= 40).
  const uint64_t keep = lim <= 0 ? ~uint64_t{0} : (lim >= 40 ? uint64_t{0} : ~uint64_t{0} << lim);
  const uint32_t keep_lo = (uint32_t)keep, keep_hi = (uint32_t)(keep >> 32);
  // Running sum of the activations in order; the masked sum is the total
  // minus the sum below lim (lim is a multiple of 8 when 0 < lim < 40: block
  // boundaries sit 32, 64, 96 or 128 weights into a span).
  const half2v ones = {(_Float16)1.0f, (_Float16)1.0f};
  float sa = 0.f, below = 0.f;
#pragma unroll
  for (int p = 0; p < 20; ++p) {
    sa = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, e[p]), ones, sa, false);
    if (p % 4 == 3) below = 2 * (p + 1) == lim ? sa : below;
  }
  float sb = lim <= 0 ? sa : (lim >= 40 ? 0.f : sa - below);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    u32x4 plain, masked;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // slot pair (2t, 2t + 1) holds activations a = 5 byte(2t) + j, b = 5 byte(2t+1) + j
      const int a = 5 * kByteOfSlot[2 * t] + j;
      const int b = 5 * kByteOfSlot[2 * t + 1] + j;
      const uint32_t sel = ((b & 1) ? 0x07060000u : 0x05040000u) | ((a & 1) ? 0x0302u : 0x0100u);
      plain[t] = perm(e[b >> 1], e[a >> 1], sel);
      // 0 or all ones from bit a / bit b of keep, merged into a half-word mask
      const uint32_t ka = (uint32_t)__builtin_amdgcn_sbfe(a < 32 ? keep_lo : keep_hi, a & 31, 1);
      const uint32_t kbm = (uint32_t)__builtin_amdgcn_sbfe(b < 32 ? keep_lo : keep_hi, b & 31, 1);
      masked[t] = plain[t] & ((ka & 0x0000FFFFu) | (kbm & 0xFFFF0000u));
    }
    *reinterpret_cast<u32x4*>(dst + 16 * j) = plain;
    *reinterpret_cast<u32x4*>(dst + 16 * (5 + j)) = masked;
  }
  sa += dpp_f32<0xB1>(sa);  // quad_perm [1, 0, 3, 2]: the span's four lane groups
  sb += dpp_f32<0xB1>(sb);
  sa += dpp_f32<0x4E>(sa);  // quad_perm [2, 3, 0, 1]
  sb += dpp_f32<0x4E>(sb);
  float* sd = un.ok ? sums + un.u * (2 * kRowsMax) + un.m : reinterpret_cast<float*>(trash + kUnitBytes);
  if (g == 0) {
    sd[0] = sa * -0x1p-16f;
    sd[kRowsMax] = sb * -0x1p-16f;
  }
}

// RF: each window's first ring loads go out before the window's activations
// are stored (else after: with one window, whose activations were loaded at
// the start, the weight stream then does not delay their copy).
template <int D, bool STAGE, int MS, bool RF>
__global__ __launch_bounds__(1024) void tq1_skinny_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs, int ldq,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K, int RG,
    int lwk, int nuw, int xregion) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int WK = 1 << lwk;
  const int W = RG << lwk;
  const int T = 64 * W;
  const int rg = wave >> lwk;
  const int wk = wave & (WK - 1);
  const int n_base = blockIdx.x * (16 * RG);
  const int rows = min(16 * RG, N - n_base);
  const int m_base = blockIdx.y * 16 * MS;  // MS slices of 16 activation rows
  const int mrows = min(16 * MS, M - m_base);
  const int groups = (K + 4) / 5;
  const int nu = (groups + 31) >> 5;  // 32-byte spans holding real bytes
  const int xstride = nuw * kSpanBytes + kPad;
  float* sums = reinterpret_cast<float*>(smem + mrows * xstride);
  unsigned char* trash = reinterpret_cast<unsigned char*>(sums + nuw * 2 * kRowsMax);
  float* sc_lds = reinterpret_cast<float*>(smem + xregion);

  const int nrow = 16 * rg + li < rows ? 16 * rg + li : 0;
  const uint16_t* srow_g = scales + (size_t)(n_base + nrow) * nb;
  const int ns = STAGE ? rows * nb : 0;
  // Staged scale rows sit nb + 1 floats apart: the 16 rows a wave reads at
  // once then fall in 16 different LDS banks.
  const int sc_row = nrow * (nb + 1);
  const float inv_nb = __builtin_amdgcn_rcpf((float)nb);  // within 1 ulp: ample for the row index
  const uint16_t* ssrc = scales + (size_t)n_base * nb;
  // Activation row of this lane in slice ms (rows past M repeat the last one;
  // their results are never written).
  const unsigned char* xa[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) {
    const int m = 16 * ms + li < mrows ? 16 * ms + li : mrows - 1;
    xa[ms] = smem + m * xstride + g * kUnitBytes;
  }

  float4v acc[MS];
#pragma unroll
  for (int ms = 0; ms < MS; ++ms) acc[ms] = float4v{0.f, 0.f, 0.f, 0.f};
  u32x2 wbuf[D];

  // Weights come through buffer loads: one resource per wave over its row
  // group (from a valid row: a group past N reads the tile's last row, and
  // rows past N in a group read its first), a lane offset fixed for the whole
  // kernel and the span's offset as a scalar, so a load costs no vector
  // instruction (a flat load's 64-bit address cost six; measured 3-5% faster
  // at N = 28672 and K = 28672).  The last span may reach past a row's ldq
  // bytes; such bytes stand for weights k >= K, whose activations are staged
  // as zero: they read the next row's first bytes, or zeros past the group's
  // last row (the resource's bounds check).
  const int rg0 = 16 * rg < rows ? 16 * rg : rows - 1;
  const int rin = rows - rg0 < 16 ? rows - rg0 : 16;  // rows of the group in the matrix
  const int lrow = 16 * rg + li < rows ? li : 0;
  const auto wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(qs) + (size_t)(n_base + rg0) * ldq, 0, rin * ldq, kBufferWord3);
  const int voff = lrow * ldq + 8 * g;  // < 16 ldq <= 2^28
  auto load = [&](int d, int u) {
    typedef int v2i __attribute__((ext_vector_type(2)));
    const v2i v = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, voff, 32 * u, 0);
    wbuf[d] = __builtin_bit_cast(u32x2, v);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto scale_at = [&](int b) -> float {
    if constexpr (STAGE) return sc_lds[sc_row + b];
    return h2f(srow_g[b]);
  };
  auto compute = [&](int d, int u, int uw) {
    const u32x2 w = wbuf[d];
    // bytes (0, 2), (1, 3), (4, 6), (5, 7) of the lane's 8 bytes, one per half
    uint32_t q[4] = {perm(0u, w[0], 0x0C020C00u), perm(0u, w[0], 0x0C030C01u),
                     perm(0u, w[1], 0x0C020C00u), perm(0u, w[1], 0x0C030C01u)};
    const int ba = (160 * u) >> 8;
    const float sa = scale_at(ba < nb ? ba : nb - 1);
    // A span holds a block boundary (and a second scale) only when the next
    // block starts before the span ends; otherwise the masked product is zero.
    const bool split = 256 * (ba + 1) < 160 * (u + 1) && ba + 1 < nb;  // wave-uniform
    const float* su = sums + uw * (2 * kRowsMax) + 4 * g;
    auto run = [&](auto with_b) {
      constexpr bool WB = decltype(with_b)::value;
      float4v Ca[MS], Cb[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) {
        Ca[ms] = *reinterpret_cast<const float4v*>(su + 16 * ms);  // -2^-16 (row sums)
        if constexpr (WB) Cb[ms] = *reinterpret_cast<const float4v*>(su + kRowsMax + 16 * ms);
      }
      sfor1<0, 5>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        u32x4 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const uint32_t t = (q[i] << 1) + q[i];  // no carry between halves: 3 * 255 < 2^16
          b[i] = t & 0x03000300u;                 // digit d' at bits 8..9: d' 2^-16
          q[i] = t & 0x00FF00FFu;
        }
        const half8 B = __builtin_bit_cast(half8, b);  // decoded once, used by every slice
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) {
          const unsigned char* xb = xa[ms] + uw * kSpanBytes;
          const half8 A = *reinterpret_cast<const half8*>(xb + 16 * j);
          Ca[ms] = mfma16(A, B, Ca[ms]);
          if constexpr (WB) {
            const half8 Am = *reinterpret_cast<const half8*>(xb + 16 * (5 + j));
            Cb[ms] = mfma16(Am, B, Cb[ms]);
          }
        }
      });
      if constexpr (WB) {
        const float sb = scale_at(ba + 1);
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) acc[ms] += sa * Ca[ms] + (sb - sa) * Cb[ms];
      } else {
#pragma unroll
        for (int ms = 0; ms < MS; ++ms) acc[ms] += sa * Ca[ms];
      }
    };
    if (split)
      run(std::true_type{});
    else
      run(std::false_type{});
  };

  // This thread's staging unit, loaded one window ahead (units <= threads).
  const int q = threadIdx.x;
  Tq1Unit un;
  tq1_unit_at(un, q, min(nuw, nu), mrows);
  tq1_load_unit(un, X, m_base, K, 0, q & 3);
  // block scales: read with the first window's activations, before the
  // weight prefetch
  uint16_t sreg[kScaleRegs];
  if constexpr (STAGE) {
#pragma unroll
    for (int r = 0; r < kScaleRegs; ++r) {
      const int e = threadIdx.x + r * T;
      sreg[r] = ssrc[e < ns ? e : 0];
    }
  }
  for (int u0 = 0; u0 < nu; u0 += nuw) {
    const int nuw_here = min(nuw, nu - u0);
    const int cnt = nuw_here > wk ? (nuw_here - wk + WK - 1) >> lwk : 0;
    auto span = [&](int i) { return cnt > 0 ? u0 + wk + WK * (i < cnt ? i : cnt - 1) : u0; };
    auto ring_start = [&] {
      sfor1<0, D>([&](auto dd) { load(decltype(dd)::value, span(decltype(dd)::value)); });
    };
    if constexpr (RF) ring_start();
    __syncthreads();  // the previous window is consumed
    // waves without a unit skip the store (their trash writes would all hit
    // the same LDS banks)
    if (__any(un.ok)) tq1_store_unit(un, smem, sums, trash, u0, q & 3, xstride, K);
    if constexpr (!RF) ring_start();
    if constexpr (STAGE) {
      if (u0 == 0) {
#pragma unroll
        for (int r = 0; r < kScaleRegs; ++r) {
          const int e = threadIdx.x + r * T;
          uint32_t v = sreg[r];
          asm volatile("" : "+v"(v));  // convert here, not ahead of the loop (no early wait)
          // row of scale e: exact in fp32 (e < 2^14, far below the margin)
          const int row = (int)(((float)e + 0.5f) * inv_nb);
          if (e < ns) sc_lds[e + row] = h2f((uint16_t)v);
        }
      }
    }
    __syncthreads();
    // First group.  The next window's activations are loaded after its first
    // step (after the last window a harmless re-read of this one), so they
    // are older than every weight load in flight in the loop below: the
    // compiler's wait before each step then covers exactly the oldest ring
    // buffer, on entry as on every later pass.
    sfor1<0, D>([&](auto dd) {
      constexpr int d = decltype(dd)::value;
      if (d < cnt) compute(d, span(d), wk + WK * d);
      if constexpr (d == 0) {
        const int u1 = u0 + nuw < nu ? u0 + nuw : u0;
        tq1_unit_at(un, q, min(nuw, nu - u1), mrows);
        tq1_load_unit(un, X, m_base, K, u1, q & 3);
      }
      load(d, span(d + D));
    });
    int i = D;
    for (; i + D < cnt; i += D) {
      sfor1<0, D>([&](auto dd) {
        constexpr int d = decltype(dd)::value;
        compute(d, span(i + d), wk + WK * (i + d));
        load(d, span(i + d + D));
      });
    }
    // last group: no loads past the wave's spans
    sfor1<0, D>([&](auto dd) {
      constexpr int d = decltype(dd)::value;
      if (i + d < cnt) compute(d, span(i + d), wk + WK * (i + d));
    });
  }

  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(ms * W + wave) * 256 + i * 64 + lane] = acc[ms][i];
  __syncthreads();
  for (int t = threadIdx.x; t < MS * RG * 256; t += T) {
    const int ms = MS == 1 ? 0 : t / (RG * 256);
    const int r = (t >> 8) - ms * RG;
    const int e = t & 255;
    const int l = e & 63;
    const int m = 16 * ms + 4 * (l >> 4) + (e >> 6);
    const int n = 16 * r + (l & 15);
    if (m < mrows && n < rows) {
      float sum = 0.f;
      for (int k = 0; k < WK; ++k) sum += red[(ms * W + r * WK + k) * 256 + e];
      Y[(size_t)(m_base + m) * N + n_base + n] = f2h_bits(sum * 0x1p16f);
    }
  }
}

constexpr int kDepth1 = 3;

template <bool STAGE, int MS, bool RF>
hipError_t launch_tq1_s(const GemmArgs& a, hipStream_t stream, dim3 grid, int W, int lds, int RG,
                        int lwk, int nuw, int xregion) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = lds_limit_once(
      reinterpret_cast<const void*>(tq1_skinny_kernel<kDepth1, STAGE, MS, RF>), kLdsMax, lds_set);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tq1_skinny_kernel<kDepth1, STAGE, MS, RF>), grid, dim3(64 * W), lds, stream,
                     static_cast<const uint16_t*>(a.X), static_cast<const uint8_t*>(a.qs),
                     (int)a.ldq, static_cast<const uint16_t*>(a.scales),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, RG, lwk, nuw,
                     xregion);
  return hipGetLastError();
}

template <bool STAGE, bool RF>
hipError_t launch_tq1_ms(int ms, const GemmArgs& a, hipStream_t stream, dim3 grid, int W, int lds,
                         int RG, int lwk, int nuw, int xregion) {
  if (ms == 2) return launch_tq1_s<STAGE, 2, RF>(a, stream, grid, W, lds, RG, lwk, nuw, xregion);
  return launch_tq1_s<STAGE, 1, RF>(a, stream, grid, W, lds, RG, lwk, nuw, xregion);
}

// Staged scales: 16 RG rows of K / 256 floats, rows padded by one float.
int64_t tq1_scale_bytes(int64_t RG, int64_t K) { return ((16 * RG * (K / 256 + 1) * 4) + 15) & ~15; }

}  // namespace

int tq1_depth() { return kDepth1; }

// Spans of 160 weights per activation window: as many as fit the LDS and
// one staging unit per thread (W waves), at most all of K.
int tq1_window_spans(int64_t M, int64_t K, int W) {
  const int64_t nu = (((K + 4) / 5) + 31) / 32;
  const int64_t ms = tq1_slices(M);
  const int64_t mrows = M < 16 * ms ? M : 16 * ms;
  int64_t nuw = (kXLds - mrows * kPad - kTrash) / (mrows * kSpanBytes + kSumBytes);
  if (nuw > nu) nuw = nu;
  if (nuw > 64 * W / (4 * mrows)) nuw = 64 * W / (4 * mrows);  // one staging unit per thread
  return (int)nuw;
}


int tq1_slices(int64_t M) { return M <= 16 ? 1 : 2; }

int tq1_lwk(int64_t N, int64_t K, int64_t M);

int tq1_stage(int64_t N, int64_t K, int64_t M) {
  const int64_t RG = skinny_rows(N);
  const int64_t threads = 64 * (RG << tq1_lwk(N, K, M));
  return tq1_scale_bytes(RG, K) <= kScLds && 16 * RG * (K / 256) <= kScaleRegs * threads ? 1 : 0;
}

// Waves per row group: 2^lwk, at most 16 waves per workgroup and no more than
// there are spans; from four activation rows on, with two or more row groups,
// at most four per row group (N = K = 8192: M = 4 11.6 us with 8 waves
// against 12.9 with 16, M = 16 20.3 against 22.3; at M = 1 16 waves stay
// ahead, 9.5 against 9.7).
int tq1_lwk(int64_t N, int64_t K, int64_t M) {
  const int RG = skinny_rows(N);
  const int64_t nu = ((K + 4) / 5 + 31) / 32;
  const int max_lwk = M >= 4 && RG >= 2 ? 2 : 4;
  int lwk = 0;
  while (lwk < max_lwk && (RG << (lwk + 1)) <= 16 && (int64_t{2} << lwk) <= nu) ++lwk;
  return lwk;
}

// The ring goes first only with several activation windows and fewer than 12
// waves: with one window (activations loaded at the start) the weight stream
// after the activation store measured faster (M = 1, N = 8192: 10.4 -> 10.0
// us; 3072 x 3072 6.25 -> 5.68), and so it did with 14-16 waves over several
// windows (M = 16, N = 28672: 38.7 -> 37.4; K = 28672, N = 8192, M = 1: 26.5
// -> 25.5), but with 8 waves over 7 windows each window's ring restart then
// waits for the barrier (M = 16, N = 8192: 21.5 -> 22.6).
bool tq1_ring_first_w(int64_t K, int64_t M, int W) {
  const int64_t nu = (((K + 4) / 5) + 31) / 32;
  return tq1_window_spans(M, K, W) < nu && W < 12;
}

bool tq1_ring_first(int64_t N, int64_t K, int64_t M) {
  return tq1_ring_first_w(K, M, skinny_rows(N) << tq1_lwk(N, K, M));
}

hipError_t launch_tq1_skinny_lwk(const GemmArgs& a, hipStream_t stream, int lwk) {
  const int M = (int)a.M, K = (int)a.K;
  const int RG = skinny_rows(a.N);
  const int W = RG << lwk;
  if (lwk < 0 || W > 16) return hipErrorInvalidValue;
  // Activation slices per workgroup: every weight is decoded once per
  // workgroup, so a workgroup takes up to 32 activation rows (more rows give
  // no gain: past that the activation reads from LDS, one per MFMA, bound it,
  // and the 1024-thread workgroup runs out of registers).
  const int ms = tq1_slices(M);
  const int mrows = M < 16 * ms ? M : 16 * ms;
  const int nuw = tq1_window_spans(M, K, W);
  if (nuw < 1) return hipErrorInvalidValue;
  const int xbytes = mrows * (nuw * kSpanBytes + kPad) + nuw * kSumBytes + kTrash;
  const int rbytes = ms * W * 1024;  // the partial sums reuse the window
  int xregion = xbytes > rbytes ? xbytes : rbytes;
  xregion = (xregion + 15) & ~15;
  const int64_t sbytes = tq1_scale_bytes(RG, K);
  // staged: every thread holds at most kScaleRegs of the workgroup's scales
  const bool stage = sbytes <= kScLds && int64_t{16} * RG * (K / 256) <= int64_t{kScaleRegs} * 64 * W;
  const int lds = xregion + (stage ? (int)sbytes : 0);
  if (lds > kLdsMax) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.N + 16 * RG - 1) / (16 * RG)), (unsigned)((a.M + 16 * ms - 1) / (16 * ms)));
  if (!tq1_ring_first_w(K, M, W))
    return stage ? launch_tq1_ms<true, false>(ms, a, stream, grid, W, lds, RG, lwk, nuw, xregion)
                 : launch_tq1_ms<false, false>(ms, a, stream, grid, W, lds, RG, lwk, nuw, xregion);
  return stage ? launch_tq1_ms<true, true>(ms, a, stream, grid, W, lds, RG, lwk, nuw, xregion)
               : launch_tq1_ms<false, true>(ms, a, stream, grid, W, lds, RG, lwk, nuw, xregion);
}

hipError_t launch_tq1_skinny(const GemmArgs& a, hipStream_t stream) {
  return launch_tq1_skinny_lwk(a, stream, tq1_lwk(a.N, a.K, a.M));
}

}  // namespace tq
