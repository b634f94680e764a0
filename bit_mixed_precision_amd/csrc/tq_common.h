// Shared device helpers of the HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_fp16.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

constexpr int kWave = 64;
constexpr int kBlockK = 256;  // weights per fp16 scale along K

// Fourth word of a raw buffer resource on gfx9-family GPUs (gfx950
// included): 32-bit data format, no swizzle; loads past the resource's
// num_records bytes return zero.
constexpr int kBufferWord3 = 0x00020000;

// Sum over the 64 lanes of a wave; every lane gets the total.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

__device__ __forceinline__ float h2f(uint16_t bits) {
  return __half2float(__ushort_as_half(bits));
}

// fp32 -> fp16 bits, round to nearest even (overflow gives +-inf).
__device__ __forceinline__ uint16_t f2h_bits(float v) {
  return __half_as_ushort(__float2half_rn(v));
}

}  // namespace tq
