// Plain GPU kernels: one wave per output feature n, VALU arithmetic only.
//
// They compute Y = X (s . T)^T exactly as the project page "Scaling Laws and
// Efficient Inference for Ternary Language Models" defines it ("The model",
// step 3), decoding TQ2 fields with a shift and a mask ("2 bits per weight")
// and TQ1 bytes with the multiply-by-3 route ("1.6 bits per weight").  They are
// the straightforward GPU path that the tuned kernels are checked against and
// the fallback for shapes the tuned kernels do not take.

#include "tq_common.h"
#include "tq_kernels.h"

namespace tq {
namespace {

constexpr int kMC = 4;  // output rows m handled per pass over a weight row

__global__ __launch_bounds__(256) void tq2_simple_kernel(const uint16_t* __restrict__ X,
                                                         const uint8_t* __restrict__ qs,
                                                         const uint16_t* __restrict__ scales,
                                                         uint16_t* __restrict__ Y, int M, int N,
                                                         int K) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const uint8_t* row = qs + (size_t)n * (K / 4);
  const uint16_t* srow = scales + (size_t)n * (K / kBlockK);
  const int chunks = K / 64;  // 16 bytes = 64 weights per chunk, inside one block
  for (int m0 = 0; m0 < M; m0 += kMC) {
    float acc[kMC] = {0.f, 0.f, 0.f, 0.f};
    for (int c = lane; c < chunks; c += kWave) {
      const uint4 w = *reinterpret_cast<const uint4*>(row + 16 * c);
      const uint32_t words[4] = {w.x, w.y, w.z, w.w};
      const float s = h2f(srow[c >> 2]);
      float part[kMC] = {0.f, 0.f, 0.f, 0.f};
      for (int i = 0; i < 4; ++i) {
        for (int j = 0; j < 16; ++j) {
          const int d = (int)((words[i] >> (2 * j)) & 3u) - 1;  // weight 64c + 16i + j
          const int k = 64 * c + 16 * i + j;
#pragma unroll
          for (int mm = 0; mm < kMC; ++mm)
            if (m0 + mm < M) part[mm] += (float)d * h2f(X[(size_t)(m0 + mm) * K + k]);
        }
      }
#pragma unroll
      for (int mm = 0; mm < kMC; ++mm) acc[mm] += s * part[mm];
    }
#pragma unroll
    for (int mm = 0; mm < kMC; ++mm) {
      const float tot = wave_sum(acc[mm]);
      if (lane == 0 && m0 + mm < M) Y[(size_t)(m0 + mm) * N + n] = f2h_bits(tot);
    }
  }
}

__global__ __launch_bounds__(256) void tq1_simple_kernel(const uint16_t* __restrict__ X,
                                                         const uint8_t* __restrict__ qs,
                                                         int ldq,
                                                         const uint16_t* __restrict__ scales,
                                                         uint16_t* __restrict__ Y, int M, int N,
                                                         int K) {
  const int lane = threadIdx.x & 63;
  const int n = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (n >= N) return;
  const uint8_t* row = qs + (size_t)n * ldq;
  const uint16_t* srow = scales + (size_t)n * (K / kBlockK);
  const int groups = (K + 4) / 5;
  for (int m0 = 0; m0 < M; m0 += kMC) {
    float acc[kMC] = {0.f, 0.f, 0.f, 0.f};
    for (int g = lane; g < groups; g += kWave) {
      unsigned q = row[g];
#pragma unroll
      for (int j = 0; j < 5; ++j) {
        const unsigned t = 3u * q;  // high byte: next digit, low byte: remainder
        const int d = (int)(t >> 8) - 1;
        q = t & 0xFFu;
        const int k = 5 * g + j;
        if (k < K) {
          const float w = (float)d * h2f(srow[k / kBlockK]);
#pragma unroll
          for (int mm = 0; mm < kMC; ++mm)
            if (m0 + mm < M) acc[mm] += w * h2f(X[(size_t)(m0 + mm) * K + k]);
        }
      }
    }
#pragma unroll
    for (int mm = 0; mm < kMC; ++mm) {
      const float tot = wave_sum(acc[mm]);
      if (lane == 0 && m0 + mm < M) Y[(size_t)(m0 + mm) * N + n] = f2h_bits(tot);
    }
  }
}

}  // namespace

hipError_t launch_tq2_simple(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.N + 3) / 4));
  hipLaunchKernelGGL(tq2_simple_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.X), static_cast<const uint8_t*>(a.qs),
                     static_cast<const uint16_t*>(a.scales), static_cast<uint16_t*>(a.Y),
                     (int)a.M, (int)a.N, (int)a.K);
  return hipGetLastError();
}

hipError_t launch_tq1_simple(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)((a.N + 3) / 4));
  hipLaunchKernelGGL(tq1_simple_kernel, grid, dim3(256), 0, stream,
                     static_cast<const uint16_t*>(a.X), static_cast<const uint8_t*>(a.qs),
                     (int)a.ldq, static_cast<const uint16_t*>(a.scales),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K);
  return hipGetLastError();
}

}  // namespace tq
