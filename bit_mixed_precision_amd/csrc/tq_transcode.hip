// TQ1 -> TQ2 transcoding on the device: the same trits, re-packed from five
// base-3 digits per byte into four 2-bit fields per byte.
//
// Both packings are those of the project page "Scaling Laws and Efficient
// Inference for Ternary Language Models": "1.6 bits per weight" (byte g of a
// row holds weights 5g..5g+4 as the digits, most significant first, of a
// base-3 number scaled by 256/243 and rounded up; the multiply-by-3 decoder
// reads them back) and "2 bits per weight" (field d' = d + 1 of weight k at
// bits 2 (k mod 4) of byte k / 4).  Both store d' = d + 1, so a TQ1 digit is
// a TQ2 field as it stands.
//
// Why: at large batch the product is MFMA-bound and the TQ1 kernels decode
// every weight once per activation tile (about two VALU ops per weight per
// 32 or 64 rows); decoding once per call into a 2-bit copy and running the
// TQ2 kernels, which decode with masks, is the cheaper way from about 48
// rows on.  The copy costs one read of the TQ1 matrix and one write and read
// of the TQ2 one.
//
// MI355X design: one thread per 16 TQ1 bytes (80 weights) of a row, one
// 16-byte load; each byte's five fields (10 bits) come from a 256-entry table
// that every workgroup builds in LDS with the multiply-by-3 decoder (t = 3 q,
// digit = t >> 8, q = t & 255, five times) and are OR-ed into the unit's
// 160-bit output (byte i at bit 10 i); the workgroup's contiguous output is
// staged in LDS and written with consecutive lanes on consecutive dwords.

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

constexpr int kTcThreads = 256;

__global__ __launch_bounds__(kTcThreads) void tq1_to_tq2_kernel(const uint8_t* __restrict__ qs1,
                                                               int ldq, int units, int64_t total,
                                                               int K, uint8_t* __restrict__ qs2) {
  __shared__ uint32_t table[256];
  __shared__ uint32_t stage[5 * kTcThreads];
  {
    // fields of byte value threadIdx.x: digits of the multiply-by-3 decoder
    uint32_t q = threadIdx.x, f = 0;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const uint32_t t = 3 * q;
      f |= (t >> 8) << (2 * j);
      q = t & 0xFFu;
    }
    table[threadIdx.x] = f;
  }
  __syncthreads();
  // The workgroup's units are consecutive, and so is their output: TQ2 dword
  // (n K / 16 + 5 u + w) for unit u of row n (a row's last unit may hold
  // fewer than five).  Stage it in LDS, then write it with consecutive lanes
  // on consecutive dwords.
  const int64_t t0 = (int64_t)blockIdx.x * kTcThreads;
  const int64_t t = t0 + threadIdx.x;
  const int64_t n0 = t0 / units;
  const int64_t base = n0 * (K >> 4) + 5 * (t0 - n0 * units);  // first dword of the workgroup
  if (t < total) {
    const int64_t n = t / units;
    const int u = (int)(t - n * units);
    const u32x4 raw = *reinterpret_cast<const u32x4*>(qs1 + n * ldq + 16 * u);
    uint32_t out[5] = {0u, 0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t f = table[(raw[i >> 2] >> (8 * (i & 3))) & 0xFFu];
      const int pos = 10 * i;
      out[pos >> 5] |= f << (pos & 31);
      if ((pos & 31) > 22) out[(pos >> 5) + 1] |= f >> (32 - (pos & 31));
    }
    const int local = (int)(n * (K >> 4) + 5 * u - base);
    const int k0 = 80 * u;
#pragma unroll
    for (int w = 0; w < 5; ++w)
      if (k0 + 16 * w < K) stage[local + w] = out[w];
  }
  __syncthreads();
  const int64_t tl = (t0 + kTcThreads < total ? t0 + kTcThreads : total) - 1;  // last unit
  const int64_t nl = tl / units;
  const int ul = (int)(tl - nl * units);
  const int rem = (K - 80 * ul) >> 4;  // dwords of the last unit
  const int count = (int)(nl * (K >> 4) + 5 * ul + (rem < 5 ? rem : 5) - base);
  uint32_t* dst = reinterpret_cast<uint32_t*>(qs2) + base;
  for (int i = threadIdx.x; i < count; i += kTcThreads) dst[i] = stage[i];
}

}  // namespace

hipError_t launch_tq1_to_tq2(const void* qs1, int64_t ldq, int64_t N, int64_t K, void* qs2,
                             hipStream_t stream) {
  const int64_t units = (K + 79) / 80;
  const int64_t total = N * units;
  const int64_t blocks = (total + kTcThreads - 1) / kTcThreads;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(tq1_to_tq2_kernel, dim3((unsigned)blocks), dim3(kTcThreads), 0, stream,
                     static_cast<const uint8_t*>(qs1), (int)ldq, (int)units, total, (int)K,
                     static_cast<uint8_t*>(qs2));
  return hipGetLastError();
}

}  // namespace tq
