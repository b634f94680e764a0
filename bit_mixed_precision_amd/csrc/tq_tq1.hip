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
//    step of the decoder (t = 3 q with v_lshl_add_u32, digit = t >> 8 taken
//    straight into an fp16 mantissa with v_and_or_b32 against the exponent of
//    1024, one v_pk_fma_f16 to get the trit, q = t & 0xff) serves two weights;
//  * v_mfma_f32_16x16x32_f16 does the multiply-accumulate with 16 activation
//    rows per launch slice (grid.y walks M in slices of 16);
//  * the four lane groups of a wave cover one 32-byte span of a row (160
//    weights, 8 bytes per lane).  A span holds at most one 256-weight block
//    boundary and the MFMA sums over all four lane groups, so with C_a = the
//    span's MFMA sum and C_b = the same sum over the weights past the boundary
//    only, the span adds s_a C_a + (s_b - s_a) C_b: exact block scales
//    without per-weight work.  C_b comes from a masked copy of the
//    activations (zero before the boundary) kept next to the plain copy;
//  * both activation copies are staged in LDS in the decoder's weight order;
//    waves of a workgroup take spans round robin and keep a ring of register
//    buffers of weights in flight; partial sums meet in LDS.

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
constexpr int kScLds = 24 * 1024;   // staged scales budget
constexpr int kLdsMax = 160 * 1024;
// Activations in LDS, decoder order: for every (row m, span u, lane group g,
// operand o) 8 halves.  o < 5: plain X at the operand's weights (zero past K);
// o >= 5: the same masked to the weights at or past the span's block boundary.
// A window holds spans [u0, u0 + nu) of rows m_base .. m_base + mrows - 1;
// thread q stages unit q = (m, u, g) of every window (units <= threads): the
// 40 consecutive activations k0 = 160 (u0 + u) + 40 g .. k0 + 39, read with
// five coalesced 16-byte loads (K and k0 are multiples of 8, so a chunk is
// either wholly inside the row or wholly past K) one window ahead, then
// written with one v_perm_b32 per operand dword.
__device__ __forceinline__ void tq1_load_unit(uint32_t (&e)[20], const uint16_t* __restrict__ X,
                                              int m_base, int K, int u0, int nu, int q) {
  const int g = q & 3;
  const int u = (q >> 2) % nu;
  const int m = (q >> 2) / nu;
  const int k0 = 160 * (u0 + u) + 40 * g;
  const uint16_t* xrow = X + (size_t)(m_base + m) * K;
#pragma unroll
  for (int c = 0; c < 5; ++c) {
    u32x4 v = {0u, 0u, 0u, 0u};
    if (k0 + 8 * c + 8 <= K) v = *reinterpret_cast<const u32x4*>(xrow + k0 + 8 * c);
#pragma unroll
    for (int t = 0; t < 4; ++t) e[4 * c + t] = v[t];
  }
}

__device__ __forceinline__ void tq1_store_unit(unsigned char* xs, const uint32_t (&e)[20], int u0,
                                               int nu, int q, int xstride) {
  const int g = q & 3;
  const int u = (q >> 2) % nu;
  const int m = (q >> 2) / nu;
  const int k0 = 160 * (u0 + u) + 40 * g;
  const int kb = ((160 * (u0 + u)) / 256 + 1) * 256;  // first block boundary of the span
  tq1_store_operands(xs + m * xstride + u * kSpanBytes + g * kUnitBytes, e, kb - k0);
}

template <int D, bool STAGE, int MS>
__global__ __launch_bounds__(1024) void tq1_skinny_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs, int ldq,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K, int RG,
    int WK, int nuw, int xregion) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int rg = wave / WK;
  const int wk = wave % WK;
  const int n_base = blockIdx.x * (16 * RG);
  const int rows = min(16 * RG, N - n_base);
  const int m_base = blockIdx.y * 16 * MS;  // MS slices of 16 activation rows
  const int mrows = min(16 * MS, M - m_base);
  const int groups = (K + 4) / 5;
  const int nu = (groups + 31) / 32;  // 32-byte spans holding real bytes
  const int xstride = nuw * kSpanBytes + kPad;
  uint16_t* sc_lds = reinterpret_cast<uint16_t*>(smem + xregion);

  Tq1Decoder dc;
  dc.init();

  const int nrow = 16 * rg + li < rows ? 16 * rg + li : 0;
  const uint8_t* wrow = qs + (size_t)(n_base + nrow) * ldq + 8 * g;
  const uint16_t* srow_g = scales + (size_t)(n_base + nrow) * nb;
  if constexpr (STAGE) {
    const uint16_t* src = scales + (size_t)n_base * nb;
    for (int i = threadIdx.x; i < rows * nb; i += blockDim.x) sc_lds[i] = src[i];
  }
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

  // The last span may reach past the row's ldq bytes; such bytes only hold
  // weights k >= K, whose activations are staged as zero, so they re-read the
  // row's first span instead (a select, not a branch).
  auto load = [&](int d, int u) {
    const int off = (32 * u + 8 * g + 8 <= ldq) ? 32 * u : 0;
    wbuf[d] = *reinterpret_cast<const u32x2*>(wrow + off);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto scale_at = [&](int b) -> float {
    if constexpr (STAGE) return h2f(sc_lds[nrow * nb + b]);
    return h2f(srow_g[b]);
  };
  auto compute = [&](int d, int u, int uw) {
    const u32x2 w = wbuf[d];
    // bytes (0, 2), (1, 3), (4, 6), (5, 7) of the lane's 8 bytes, one per half
    uint32_t q[4] = {w[0] & 0x00FF00FFu, (w[0] >> 8) & 0x00FF00FFu, w[1] & 0x00FF00FFu,
                     (w[1] >> 8) & 0x00FF00FFu};
    const int ba = (160 * u) >> 8;
    const float sa = scale_at(ba < nb ? ba : nb - 1);
    // A span holds a block boundary (and a second scale) only when the next
    // block starts before the span ends; otherwise the masked product is zero.
    const bool split = 256 * (ba + 1) < 160 * (u + 1) && ba + 1 < nb;  // wave-uniform
    auto run = [&](auto with_b) {
      constexpr bool WB = decltype(with_b)::value;
      float4v Ca[MS], Cb[MS];
#pragma unroll
      for (int ms = 0; ms < MS; ++ms) Ca[ms] = Cb[ms] = float4v{0.f, 0.f, 0.f, 0.f};
      uint32_t qq[4] = {q[0], q[1], q[2], q[3]};
      sfor1<0, 5>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        u32x4 b;
#pragma unroll
        for (int i = 0; i < 4; ++i) b[i] = dc.step(qq[i]);
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

  // This thread's staging unit, one window ahead (units <= threads).
  const int q = threadIdx.x;
  uint32_t xe[20];
  if (q < mrows * min(nuw, nu) * 4) tq1_load_unit(xe, X, m_base, K, 0, min(nuw, nu), q);
  for (int u0 = 0; u0 < nu; u0 += nuw) {
    const int nuw_here = min(nuw, nu - u0);
    const int cnt = nuw_here > wk ? (nuw_here - wk + WK - 1) / WK : 0;
    auto span = [&](int i) { return u0 + wk + WK * (i < cnt ? i : cnt - 1); };
    if (cnt > 0) {
      sfor1<0, D>([&](auto dd) { load(decltype(dd)::value, span(decltype(dd)::value)); });
    }
    __syncthreads();  // the previous window is consumed
    if (q < mrows * nuw_here * 4) tq1_store_unit(smem, xe, u0, nuw_here, q, xstride);
    const int u1 = u0 + nuw;  // the next window's activations fly during this one
    if (u1 < nu && q < mrows * min(nuw, nu - u1) * 4)
      tq1_load_unit(xe, X, m_base, K, u1, min(nuw, nu - u1), q);
    __syncthreads();
    for (int i = 0; i < cnt; i += D) {
      sfor1<0, D>([&](auto dd) {
        constexpr int d = decltype(dd)::value;
        if (i + d < cnt) compute(d, span(i + d), wk + WK * (i + d));
        load(d, span(i + d + D));
      });
    }
  }

  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  const int nw = RG * WK;  // waves of the workgroup
#pragma unroll
  for (int ms = 0; ms < MS; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(ms * nw + wave) * 256 + i * 64 + lane] = acc[ms][i];
  __syncthreads();
  for (int t = threadIdx.x; t < MS * RG * 256; t += blockDim.x) {
    const int ms = t / (RG * 256);
    const int r = (t >> 8) % RG;
    const int e = t & 255;
    const int l = e & 63;
    const int m = 16 * ms + 4 * (l >> 4) + (e >> 6);
    const int n = 16 * r + (l & 15);
    if (m < mrows && n < rows) {
      float sum = 0.f;
      for (int k = 0; k < WK; ++k) sum += red[(ms * nw + r * WK + k) * 256 + e];
      Y[(size_t)(m_base + m) * N + n_base + n] = f2h_bits(sum);
    }
  }
}

constexpr int kDepth1 = 3;

template <bool STAGE, int MS>
hipError_t launch_tq1_s(const GemmArgs& a, hipStream_t stream, dim3 grid, int W, int lds, int RG,
                        int WK, int nuw, int xregion) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(tq1_skinny_kernel<kDepth1, STAGE, MS>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsMax);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL((tq1_skinny_kernel<kDepth1, STAGE, MS>), grid, dim3(64 * W), lds, stream,
                     static_cast<const uint16_t*>(a.X), static_cast<const uint8_t*>(a.qs),
                     (int)a.ldq, static_cast<const uint16_t*>(a.scales),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, RG, WK, nuw,
                     xregion);
  return hipGetLastError();
}

template <bool STAGE>
hipError_t launch_tq1_ms(int ms, const GemmArgs& a, hipStream_t stream, dim3 grid, int W, int lds,
                         int RG, int WK, int nuw, int xregion) {
  if (ms == 2) return launch_tq1_s<STAGE, 2>(a, stream, grid, W, lds, RG, WK, nuw, xregion);
  return launch_tq1_s<STAGE, 1>(a, stream, grid, W, lds, RG, WK, nuw, xregion);
}

}  // namespace

int tq1_depth() { return kDepth1; }

int tq1_slices(int64_t M) { return M <= 16 ? 1 : 2; }

int tq1_stage(int64_t N, int64_t K) {
  const int64_t RG = skinny_rows(N);
  const int64_t sbytes = ((16 * RG * (K / 256) * 2) + 15) & ~15;
  return sbytes <= kScLds ? 1 : 0;
}

hipError_t launch_tq1_skinny(const GemmArgs& a, hipStream_t stream) {
  const int M = (int)a.M, K = (int)a.K;
  const int nb = K / 256;
  const int groups = (K + 4) / 5;
  const int nu = (groups + 31) / 32;
  const int RG = skinny_rows(a.N);
  int WK = 16 / RG;
  if (WK > nu) WK = nu;
  if (WK < 1) WK = 1;
  const int W = RG * WK;
  // Activation slices per workgroup: every weight is decoded once per
  // workgroup, so a workgroup takes up to 32 activation rows (more rows give
  // no gain: past that the activation reads from LDS, one per MFMA, bound it,
  // and the 1024-thread workgroup runs out of registers).
  const int ms = tq1_slices(M);
  const int mrows = M < 16 * ms ? M : 16 * ms;
  int nuw = (kXLds / mrows - kPad) / kSpanBytes;
  if (nuw > nu) nuw = nu;
  if (nuw > 64 * W / (4 * mrows)) nuw = 64 * W / (4 * mrows);  // one staging unit per thread
  if (nuw < 1) return hipErrorInvalidValue;
  const int xbytes = mrows * (nuw * kSpanBytes + kPad);
  const int rbytes = ms * W * 1024;  // the partial sums reuse the window
  int xregion = xbytes > rbytes ? xbytes : rbytes;
  xregion = (xregion + 15) & ~15;
  const int sbytes = ((16 * RG * nb * 2) + 15) & ~15;
  const bool stage = sbytes <= kScLds;
  const int lds = xregion + (stage ? sbytes : 0);
  if (lds > kLdsMax) return hipErrorInvalidValue;
  dim3 grid((unsigned)((a.N + 16 * RG - 1) / (16 * RG)), (unsigned)((a.M + 16 * ms - 1) / (16 * ms)));
  return stage ? launch_tq1_ms<true>(ms, a, stream, grid, W, lds, RG, WK, nuw, xregion)
               : launch_tq1_ms<false>(ms, a, stream, grid, W, lds, RG, WK, nuw, xregion);
}

}  // namespace tq
