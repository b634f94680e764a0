// Shared pieces of the TQ1 kernels: the decoder-order activation layout and
// the multiply-by-3 digit decoder ("1.6 bits per weight" on the project page
// "Scaling Laws and Efficient Inference for Ternary Language Models").
#pragma once

#include "tq_common.h"
#include "tq_mfma.h"

namespace tq {

// Per (row m, span u, lane group g): 10 operands of 16 bytes (5 plain, 5 masked).
constexpr int kUnitBytes = 10 * 16;
constexpr int kSpanBytes = 4 * kUnitBytes;  // one 32-byte span of weights, 160 weights

// Slot s of operand j holds byte kByteOfSlot[s] of the lane's 8 bytes, digit j,
// i.e. weight 40 g + 5 kByteOfSlot[s] + j of the span.
__device__ constexpr int kByteOfSlot[8] = {0, 2, 1, 3, 4, 6, 5, 7};

// Writes the ten operands of one (row, span, lane group) unit to dst: e holds
// the 40 activations k0 .. k0 + 39 of the unit (two per dword, in order);
// operand j < 5 gathers, for every slot s, activation 5 kByteOfSlot[s] + j;
// operand 5 + j is the same with the activations below lim (relative to k0:
// those before the span's block boundary) zeroed.
__device__ __forceinline__ void tq1_store_operands(unsigned char* dst, const uint32_t (&e)[20],
                                                   int lim) {
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    uint32_t plain[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // slot pair (2t, 2t + 1) holds activations a = 5 byte(2t) + j, b = 5 byte(2t+1) + j
      const int a = 5 * kByteOfSlot[2 * t] + j;
      const int b = 5 * kByteOfSlot[2 * t + 1] + j;
      const uint32_t sel = ((b & 1) ? 0x07060000u : 0x05040000u) | ((a & 1) ? 0x0302u : 0x0100u);
      plain[t] = perm(e[b >> 1], e[a >> 1], sel);
    }
    *reinterpret_cast<u32x4*>(dst + 16 * j) = u32x4{plain[0], plain[1], plain[2], plain[3]};
    u32x4 masked;
    if (lim <= 0) {
      masked = u32x4{plain[0], plain[1], plain[2], plain[3]};
    } else if (lim >= 40) {
      masked = u32x4{0u, 0u, 0u, 0u};
    } else {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int a = 5 * kByteOfSlot[2 * t] + j;
        const int b = 5 * kByteOfSlot[2 * t + 1] + j;
        const uint32_t keep = (a >= lim ? 0x0000FFFFu : 0u) | (b >= lim ? 0xFFFF0000u : 0u);
        masked[t] = plain[t] & keep;
      }
    }
    *reinterpret_cast<u32x4*>(dst + 16 * (5 + j)) = masked;
  }
}

// The plain operands of one unit (tq1_store_operands' first half) at dst.
__device__ __forceinline__ void tq1_store_plain(unsigned char* dst, const uint32_t (&e)[20]) {
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    u32x4 plain;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int a = 5 * kByteOfSlot[2 * t] + j;
      const int b = 5 * kByteOfSlot[2 * t + 1] + j;
      const uint32_t sel = ((b & 1) ? 0x07060000u : 0x05040000u) | ((a & 1) ? 0x0302u : 0x0100u);
      plain[t] = perm(e[b >> 1], e[a >> 1], sel);
    }
    *reinterpret_cast<u32x4*>(dst + 16 * j) = plain;
  }
}

// The masked operands of one unit (tq1_store_operands' second half) at dst.
// lim must be the same in every active lane: the keep masks are then scalar.
__device__ __forceinline__ void tq1_store_masked_uniform(unsigned char* dst,
                                                         const uint32_t (&e)[20], int lim) {
  lim = __builtin_amdgcn_readfirstlane(lim);
#pragma unroll
  for (int j = 0; j < 5; ++j) {
    u32x4 masked;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int a = 5 * kByteOfSlot[2 * t] + j;
      const int b = 5 * kByteOfSlot[2 * t + 1] + j;
      const uint32_t sel = ((b & 1) ? 0x07060000u : 0x05040000u) | ((a & 1) ? 0x0302u : 0x0100u);
      const uint32_t keep = (a >= lim ? 0x0000FFFFu : 0u) | (b >= lim ? 0xFFFF0000u : 0u);
      masked[t] = perm(e[b >> 1], e[a >> 1], sel) & keep;
    }
    *reinterpret_cast<u32x4*>(dst + 16 * j) = masked;
  }
}

// Five digit steps of the multiply decoder on two bytes (one per 16-bit half).
struct Tq1Decoder {
  uint32_t magic, mul, add;
  __device__ __forceinline__ void init() {
    magic = in_vgpr(kMagic2);
    mul = in_vgpr(pack_half2(1.0f / 256.0f, 1.0f / 256.0f));
    add = in_vgpr(pack_half2(-5.0f, -5.0f));
  }
  // t = 3 q; returns the fp16 trit pair (digit - 1) of t's high byte; q <- t & 0xff.
  __device__ __forceinline__ uint32_t step(uint32_t& q) const {
    const uint32_t t = (q << 1) + q;  // no carry between halves: 3 * 255 < 2^16
    const uint32_t v = (t & 0x03000300u) | magic;  // 1024 + 256 * digit
    q = t & 0x00FF00FFu;
    const half2v d = __builtin_elementwise_fma(__builtin_bit_cast(half2v, v),
                                               __builtin_bit_cast(half2v, mul),
                                               __builtin_bit_cast(half2v, add));
    return __builtin_bit_cast(uint32_t, d);
  }
};

}  // namespace tq
