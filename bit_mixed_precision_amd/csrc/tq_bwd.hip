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
// MI355X design:
//  * a workgroup of 4 waves owns a 128 x 128 tile of dX (128 activation rows,
//    128 columns k) and walks n in chunks of 32 (the MFMA reduction length);
//  * per chunk every thread loads one dword of packed weights (16 weights of
//    one row n, one block scale) and two 16-byte pieces of dY; it decodes the
//    dword into 16 fp16 values s d (v_and_or_b32 against the fp16 exponent of
//    1024, v_pk_add_f16, v_pk_mul_f16: exact) and writes them transposed into
//    LDS, k-major with n contiguous, which is the B-operand order of
//    v_mfma_f32_16x16x32_f16 for a reduction over n; dY goes to LDS m-major,
//    the A-operand order;
//  * wave w computes columns 32 w .. 32 w + 31 for all 128 rows: 16 MFMAs
//    per chunk on 16 fp32 accumulators, each decoded weight feeding 8 MFMAs;
//  * two LDS buffers and a ring of four chunks of loads in registers: a
//    chunk's loads go out three chunks before it is decoded into LDS, one
//    barrier per chunk.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

constexpr int kBM = 128;          // activation rows per workgroup
constexpr int kBK = 128;          // columns k per workgroup
constexpr int kCN = 32;           // n per chunk
constexpr int kStride = 40;       // halves per LDS row (32 + 8: spreads the banks)
constexpr int kBufHalves = (kBK + kBM) * kStride;  // one buffer: Wt then At
constexpr int kThreads = 256;
constexpr int kRing = 4;          // chunks of loads in flight per thread

template <int I, int N, class F>
__device__ __forceinline__ void sfor_b(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor_b<I + 1, N>(f);
  }
}

// Raw loads only (the zeroing of rows and columns past N happens in
// chunk_store), so nothing waits for them before the MFMAs of the chunk.
struct ChunkRegs {
  uint32_t w;      // 16 packed weights of row n, columns k0 + 16 j ..
  uint16_t s;      // their block scale
  bool nok;        // row n < N
  bool yok;        // dY columns < N
  u32x4 y[2];      // dY pieces (rows r0, r0 + 64; 8 values of n each)
};

__device__ __forceinline__ void chunk_load(ChunkRegs& r, const uint16_t* __restrict__ dY,
                                           const uint8_t* __restrict__ qs,
                                           const uint16_t* __restrict__ scales, int M, int N,
                                           int K, int m0, int k0, int n0) {
  const int t = threadIdx.x;
  // weights: row n0 + t / 8, dword t % 8 of the 32 bytes of columns k0 .. k0 + 127
  const int nn = n0 + (t >> 3);
  const int j = t & 7;
  const bool nok = nn < N;
  const int nr = nok ? nn : N - 1;
  r.w = *reinterpret_cast<const uint32_t*>(qs + (size_t)nr * (K >> 2) + (k0 >> 2) + 4 * j);
  r.s = scales[(size_t)nr * (K >> 8) + ((k0 + 16 * j) >> 8)];
  r.nok = nok;
  // dY: rows m0 + t / 4 and m0 + t / 4 + 64 (clamped: their results are not
  // stored), 8 values of n each; pieces past N are zero (N % 8 == 0)
  const int part = t & 3;
  const int n = n0 + 8 * part;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    int m = m0 + (t >> 2) + 64 * u;
    m = m < M ? m : M - 1;
    r.y[u] = *reinterpret_cast<const u32x4*>(dY + (size_t)m * N + (n < N ? n : 0));
  }
  r.yok = n < N;
}

__device__ __forceinline__ void chunk_store(const ChunkRegs& r, uint16_t* buf) {
  const int t = threadIdx.x;
  const int nn = t >> 3;
  const int j = t & 7;
  uint16_t* wt = buf;                   // [k][n], kStride halves per k
  uint16_t* at = buf + kBK * kStride;   // [m][n], kStride halves per m
  const half2v one = {(_Float16)-1025.0f, (_Float16)-1025.0f};
  const uint32_t su = r.nok ? r.s : 0u;  // rows past N contribute zero
  const uint32_t s2u = su | (su << 16);
  const half2v s2 = __builtin_bit_cast(half2v, s2u);
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    // fields c and c + 8 of the dword: columns 16 j + c and 16 j + c + 8
    const uint32_t v = ((r.w >> (2 * c)) & 0x00030003u) | kMagic2;  // 1024 + d'
    const half2v d = (__builtin_bit_cast(half2v, v) + one) * s2;    // (d' - 1) s, exact
    const uint32_t du = __builtin_bit_cast(uint32_t, d);
    wt[(16 * j + c) * kStride + nn] = (uint16_t)du;
    wt[(16 * j + c + 8) * kStride + nn] = (uint16_t)(du >> 16);
  }
  const int part = t & 3;
#pragma unroll
  for (int u = 0; u < 2; ++u)
    *reinterpret_cast<u32x4*>(at + ((t >> 2) + 64 * u) * kStride + 8 * part) =
        r.yok ? r.y[u] : u32x4{0u, 0u, 0u, 0u};
}

__global__ __launch_bounds__(kThreads) void tq2_bwd_x_kernel(const uint16_t* __restrict__ dY,
                                                             const uint8_t* __restrict__ qs,
                                                             const uint16_t* __restrict__ scales,
                                                             uint16_t* __restrict__ dX, int M,
                                                             int N, int K) {
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * kBufHalves];
  const int k0 = blockIdx.x * kBK;
  const int m0 = blockIdx.y * kBM;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nch = (N + kCN - 1) / kCN;

  float4v acc[8][2];
#pragma unroll
  for (int ms = 0; ms < 8; ++ms)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) acc[ms][ks] = float4v{0.f, 0.f, 0.f, 0.f};

  // Ring of kRing chunks in registers: at the start of step c the slots hold
  // chunks c .. c + kRing - 1 (chunk c already in LDS buffer c & 1).  Step c
  // computes chunk c, writes chunk c + 1 to the other buffer and refills the
  // freed slot with chunk c + kRing.  Loads are unconditional (chunks past
  // the end re-read the last one), so the compiler's wait before each store
  // covers exactly the oldest slot.
  ChunkRegs r[kRing];
  auto ld = [&](int slot, int c) {
    chunk_load(r[slot], dY, qs, scales, M, N, K, m0, k0, (c < nch ? c : nch - 1) * kCN);
  };
  sfor_b<0, kRing>([&](auto pp) { ld(decltype(pp)::value, decltype(pp)::value); });
  chunk_store(r[0], lds);
  __syncthreads();
  for (int c0 = 0; c0 < nch; c0 += kRing) {
    sfor_b<0, kRing>([&](auto pp) {
      constexpr int p = decltype(pp)::value;
      const int c = c0 + p;
      if (c < nch) {  // wave-uniform; no loads inside
        const uint16_t* buf = lds + (c & 1) * kBufHalves;
        const uint16_t* wt = buf + (32 * wave + li) * kStride + 8 * g;
        const uint16_t* at = buf + kBK * kStride + li * kStride + 8 * g;
        half8 B[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          B[ks] = *reinterpret_cast<const half8*>(wt + 16 * ks * kStride);
#pragma unroll
        for (int ms = 0; ms < 8; ++ms) {
          const half8 A = *reinterpret_cast<const half8*>(at + 16 * ms * kStride);
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) acc[ms][ks] = mfma16(A, B[ks], acc[ms][ks]);
        }
        chunk_store(r[(p + 1) % kRing], lds + ((c + 1) & 1) * kBufHalves);
        __syncthreads();
      }
      ld(p, c + kRing);
    });
  }

  const int kc = k0 + 32 * wave + li;
#pragma unroll
  for (int ms = 0; ms < 8; ++ms)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 16 * ms + 4 * g + i;
      if (m < M) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) dX[(size_t)m * K + kc + 16 * ks] = f2h_bits(acc[ms][ks][i]);
      }
    }
}

}  // namespace

hipError_t launch_tq2_bwd_x(const void* dY, const void* qs, const void* scales, void* dX,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  const int64_t mt = (M + kBM - 1) / kBM;
  if (mt > 65535) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(tq2_bwd_x_kernel, dim3((unsigned)(K / kBK), (unsigned)mt), dim3(kThreads), 0,
                     stream, static_cast<const uint16_t*>(dY), static_cast<const uint8_t*>(qs),
                     static_cast<const uint16_t*>(scales), static_cast<uint16_t*>(dX), (int)M,
                     (int)N, (int)K);
  return hipGetLastError();
}

}  // namespace tq
