// Input gradient of the ternary product: dX = dY (s . T) for TQ2 weights.
//
// The forward product of the project page "Scaling Laws and Efficient
// Inference for Ternary Language Models" ("The model", step 3) is
// Y = X (s . T)^T; quantization-aware training backpropagates through it, and
// the gradient with respect to the activations is the same ternary matrix
// used the other way round: dX[m][k] = sum_n dY[m][n] s[n][k / 256] T[n][k],
// FP32 accumulation and one FP16 rounding as in "TriRun".  (The gradient
// with respect to the latent weights, dY^T X under the straight-through
// estimator, is a plain dense product and not part of this file.)
//
// MI355X design.  The reduction runs over n, the row index of the packed
// matrix, so every MFMA operand of weights (8 consecutive n of one column k)
// needs a transpose of the packed layout; the scale varies with n and stays
// inside the sum.  Decode cost per weight is amortized over the activation
// rows of a workgroup, LDS traffic over the columns of a wave:
//  * a workgroup of 8 waves owns 512 rows of dX x 128 columns k (one half of
//    a 256-column scale block); wave w owns rows 64 w .. 64 w + 63 and all 128
//    columns, 4 x 8 MFMA tiles (v_mfma_f32_16x16x32_f16) on 128 fp32
//    accumulators, and walks n in chunks of 32;
//  * dY goes from memory into the A operands without LDS: buffer loads (zero
//    outside the rows of the workgroup) give four consecutive lanes the four
//    16-byte pieces of one row's 64 bytes, the order the vector L1 serves at
//    full rate (in the MFMA order every lane of a quad is a different row and
//    the same load costs four times the cache accesses); one ds_bpermute per
//    dword, a chunk ahead of its use, then moves the piece of row r, n-group
//    g to lane 16 g + r;
//  * the weights of a chunk, 32 rows x 128 columns, are decoded once per
//    workgroup into LDS, k-major with pairs (n, n + 1) in one dword, which is
//    the B-operand order: every thread takes a 2-bit field position of one
//    dword of two adjacent rows (v_perm_b32 pairs their halves) and produces 4
//    dwords with one v_and_or_b32, one v_pk_add_f16 and one v_pk_mul_f16 each:
//    the field p = k % 4 stays in place, 1024 + d 4^p minus 1024 + 4^p is
//    (d - 1) 4^p exactly, times the scale pair (s_n, s_n+1) exactly, and the
//    4^p of column k leaves in the epilogue as an exact power-of-two factor;
//  * LDS rows of 20 dwords (16 pairs + 4) make both the decoded stores and
//    the 16-byte operand reads free of bank conflicts; two buffers, one
//    barrier per chunk, loads three chunks deep.
// Measured at 4096 x 8192 x 8192 the products alone run near the MFMA peak;
// what remains is LDS and barrier time around them (two 4-wave workgroups per
// CU, which decode every chunk twice, are slower).

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * kWave;
constexpr int kBM = kWaves * 64;   // activation rows per workgroup
constexpr int kBK = 128;           // columns k per workgroup
constexpr int kCN = 32;            // n per chunk
constexpr int kRowDw = 20;         // dwords per LDS row k: 16 pairs of n + 4
constexpr int kBufDw = kBK * kRowDw;
constexpr int kRing = 3;           // chunks of loads in flight
constexpr uint32_t kRsrcFlags = 0x00020000u;  // raw buffer, 32-bit data
constexpr uint32_t kOob = 0x80000000u;        // an offset past every range here

template <int I, int N, class F>
__device__ __forceinline__ void sfor_b(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor_b<I + 1, N>(f);
  }
}

// Buffer descriptor of a workgroup-uniform range (read through readfirstlane
// so that it lives in SGPRs and the loads need no per-lane loop).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, (int)n, (int)kRsrcFlags);
}

struct WRegs {     // one dword of 16 weights from each of rows n, n + 1, their scales
  uint32_t we, wo, se, so;
};
struct ARegs {     // A operands of the 4 row tiles of a wave for one chunk
  u32x4 a[4];
};

__global__ __launch_bounds__(kThreads) void tq2_bwd_x_kernel(const uint16_t* __restrict__ dY,
                                                             const uint8_t* __restrict__ qs,
                                                             const uint16_t* __restrict__ scales,
                                                             uint16_t* __restrict__ dX, int M,
                                                             int N, int K) {
  __shared__ __attribute__((aligned(16))) uint32_t lds[2 * kBufDw];
  const int k0 = blockIdx.x * kBK;
  const int m0 = blockIdx.y * kBM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nch = (N + kCN - 1) / kCN;
  const int rows = M - m0 < kBM ? M - m0 : kBM;
  const int qrow = K >> 2;  // bytes per packed row
  const int srow = K >> 8;  // scales per row

  // dY rows of this workgroup; lane l loads row 64 wave + 16 ms + l / 4,
  // n-group l % 4 (chunk 0 offsets), and takes from lane 4 li + g after the
  // permutation
  const __amdgpu_buffer_rsrc_t ry = rsrc(dY + (size_t)m0 * N, (uint32_t)rows * N * 2u);
  const int pq = lane & 3;
  uint32_t aoff[4];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms) aoff[ms] = ((64 * wave + 16 * ms + (lane >> 2)) * N + 8 * pq) * 2u;
  const int paddr = (4 * li + g) * 4;

  // decode role: row pair rp (rows 2 rp, 2 rp + 1 of the chunk), half h of
  // the dword (columns 16 wave + 8 h ..), field group q (fields 4 q .. 4 q + 3)
  const int rp = lane & 15;
  const int q = (lane >> 4) & 1;
  const int h = lane >> 5;
  const uint32_t wsel = h ? 0x07060302u : 0x05040100u;
  const uint32_t wsh = 8u * q;
  const uint32_t woff = (uint32_t)(2 * rp) * qrow + 4 * wave;
  const uint32_t soff = (uint32_t)(2 * rp) * srow * 2u;
  const int dcol = 16 * wave + 8 * h + 4 * q;  // first LDS row written

  auto ldW = [&](WRegs& r, int c) {
    // rows n0 .. n0 + 31 of columns k0 ..; rows past N are out of range (zero)
    const int n0 = c * kCN;
    const int nr = N - n0 < kCN ? (N - n0 > 0 ? N - n0 : 0) : kCN;
    const auto rq = rsrc(qs + (size_t)n0 * qrow + (k0 >> 2), (uint32_t)nr * qrow);
    const auto rs = rsrc(scales + (size_t)n0 * srow + (k0 >> 8), (uint32_t)nr * srow * 2u);
    r.we = __builtin_amdgcn_raw_buffer_load_b32(rq, woff, 0, 0);
    r.wo = __builtin_amdgcn_raw_buffer_load_b32(rq, woff + qrow, 0, 0);
    r.se = __builtin_amdgcn_raw_buffer_load_b16(rs, soff, 0, 0);
    r.so = __builtin_amdgcn_raw_buffer_load_b16(rs, soff + srow * 2u, 0, 0);
  };
  auto ldA = [&](ARegs& r, int c) {
    const int n0 = c * kCN;
    const bool ok = n0 + 8 * pq < N;  // N % 8 == 0: a piece is all in or all out
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
      r.a[ms] = __builtin_amdgcn_raw_buffer_load_b128(ry, ok ? aoff[ms] + 2u * n0 : kOob, 0, 0);
  };
  auto decode = [&](const WRegs& r, uint32_t* buf) {
    const uint32_t x = __builtin_amdgcn_perm(r.wo, r.we, wsel) >> wsh;
    const half2v s2 = __builtin_bit_cast(half2v, (r.se & 0xFFFFu) | (r.so << 16));
    uint32_t* dst = buf + dcol * kRowDw + rp;
    sfor_b<0, 4>([&](auto pp) {
      constexpr int p = decltype(pp)::value;
      constexpr _Float16 off = (_Float16)(-(1024.0f + float(1 << (2 * p))));
      const uint32_t v = (x & (0x00030003u << (2 * p))) | kMagic2;  // 1024 + d 4^p
      const half2v d = (__builtin_bit_cast(half2v, v) + half2v{off, off}) * s2;
      dst[p * kRowDw] = __builtin_bit_cast(uint32_t, d);
    });
  };

  auto permute = [&](ARegs& dst, const ARegs& src) {
#pragma unroll
    for (int ms = 0; ms < 4; ++ms)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dst.a[ms][e] = (uint32_t)__builtin_amdgcn_ds_bpermute(paddr, (int)src.a[ms][e]);
  };

  float4v acc[4][8];
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) acc[ms][kt] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const ARegs& r, const uint32_t* buf) {
    const uint32_t* bp = buf + li * kRowDw + 4 * g;
#pragma unroll
    for (int kt = 0; kt < 8; ++kt) {
      const half8 b = *reinterpret_cast<const half8*>(bp + 16 * kt * kRowDw);
#pragma unroll
      for (int ms = 0; ms < 4; ++ms)
        acc[ms][kt] = mfma16(__builtin_bit_cast(half8, r.a[ms]), b, acc[ms][kt]);
    }
  };

  // Ring of kRing chunks of raw loads (chunk c in slot c % kRing) and two of
  // permuted operands (chunk c in slot c % 2).  Step c issues the loads of
  // chunk c + 2 (past the end they are out of range and return zero),
  // permutes chunk c + 1, multiplies chunk c out of LDS buffer c & 1, decodes
  // chunk c + 1 into the other buffer and meets the barrier.  Loads are
  // unconditional and in program order, so each wait covers exactly the chunk
  // it needs.  The loop is unrolled by 6, a multiple of both ring sizes.
  WRegs wr[kRing];
  ARegs ar[kRing];
  ARegs ap[2];
  ldW(wr[0], 0);
  ldA(ar[0], 0);
  ldW(wr[1], 1);
  ldA(ar[1], 1);
  decode(wr[0], lds);
  permute(ap[0], ar[0]);
  __syncthreads();
  for (int c0 = 0; c0 < nch; c0 += 6) {
    sfor_b<0, 6>([&](auto pp) {
      constexpr int p = decltype(pp)::value;
      const int c = c0 + p;
      ldW(wr[(p + 2) % kRing], c + 2);
      ldA(ar[(p + 2) % kRing], c + 2);
      // keep the loads ahead of the products and the decode behind them, so
      // that no wait for chunk c + 1 is hoisted into the products of chunk c
      __builtin_amdgcn_sched_barrier(0);
      if (c < nch) {  // wave-uniform; no loads inside
        permute(ap[(p + 1) % 2], ar[(p + 1) % kRing]);
        compute(ap[p % 2], lds + (c & 1) * kBufDw);
        __builtin_amdgcn_sched_barrier(0);
        decode(wr[(p + 1) % kRing], lds + ((c + 1) & 1) * kBufDw);
        __syncthreads();
      }
    });
  }

  // column k0 + 16 kt + li carries the factor 4^(li % 4) of its field position
  const float unscale = 1.0f / float(1 << (2 * (li & 3)));
#pragma unroll
  for (int ms = 0; ms < 4; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 64 * wave + 16 * ms + 4 * g + i;
      if (m < M) {
        uint16_t* out = dX + (size_t)m * K + k0 + li;
#pragma unroll
        for (int kt = 0; kt < 8; ++kt) out[16 * kt] = f2h_bits(acc[ms][kt][i] * unscale);
      }
    }
}

}  // namespace

hipError_t launch_tq2_bwd_x(const void* dY, const void* qs, const void* scales, void* dX,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t mt = (M + kBM - 1) / kBM;
  // byte offsets inside one workgroup's rows of dY are 32-bit
  if (mt > 65535 || kBM * N * 2 >= (int64_t(1) << 31) || K / 4 * kCN >= (int64_t(1) << 31))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(tq2_bwd_x_kernel, dim3((unsigned)(K / kBK), (unsigned)mt), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(dY), static_cast<const uint8_t*>(qs),
                     static_cast<const uint16_t*>(scales), static_cast<uint16_t*>(dX), (int)M,
                     (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace tq
