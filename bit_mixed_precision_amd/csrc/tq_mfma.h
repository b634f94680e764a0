// MFMA operand types and the fp16 "magic exponent" trit decoders (gfx950).
//
// v_mfma_f32_16x16x32_f16 operand layout (wave64, lane l):
//   A (16 x 32): row l % 16, k = 8 * (l / 16) + slot, slot = 0..7
//   B (32 x 16): column l % 16, k = 8 * (l / 16) + slot
//   D (16 x 16): column l % 16, rows 4 * (l / 16) + i, i = 0..3
// The k order inside an operand is free as long as A and B agree, so the
// kernels decode weights in whatever order is cheapest and arrange the
// activations to match.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float4v mfma16(half8 a, half8 b, float4v c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// 0x6400 is fp16 1024.0, whose ulp is 1: OR-ing a 2-bit field that sits at
// mantissa bits 2p..2p+1 gives the exact value 1024 + 4^p * d'.  One fused
// multiply-add by (4^-p, -(1024 / 4^p + 1)) then yields d = d' - 1 exactly.
constexpr uint32_t kMagic2 = 0x64006400u;

template <int P>
struct FieldConst {
  static constexpr float mul = 1.0f / float(1 << (2 * P));
  static constexpr float add = -(1024.0f / float(1 << (2 * P)) + 1.0f);
};

// Both halves take the field at bits 2P..2P+1 of their own 16 bits; returns
// the pair (d_lo, d_hi) as two fp16 in {-1, 0, 1}.
template <int P>
__device__ __forceinline__ uint32_t decode_pair_same(uint32_t x) {
  constexpr uint32_t mask = (3u << (2 * P)) | (3u << (16 + 2 * P));
  const uint32_t v = (x & mask) | kMagic2;
  const half2v h = __builtin_bit_cast(half2v, v);
  const half2v mul = {(_Float16)FieldConst<P>::mul, (_Float16)FieldConst<P>::mul};
  const half2v add = {(_Float16)FieldConst<P>::add, (_Float16)FieldConst<P>::add};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h, mul, add));
}

// Low half takes the field at bits 2PL.., high half the field at bits 2PH..
// of its own 16 bits.
template <int PL, int PH>
__device__ __forceinline__ uint32_t decode_pair_mixed(uint32_t x) {
  constexpr uint32_t mask = (3u << (2 * PL)) | (3u << (16 + 2 * PH));
  const uint32_t v = (x & mask) | kMagic2;
  const half2v h = __builtin_bit_cast(half2v, v);
  const half2v mul = {(_Float16)FieldConst<PL>::mul, (_Float16)FieldConst<PH>::mul};
  const half2v add = {(_Float16)FieldConst<PL>::add, (_Float16)FieldConst<PH>::add};
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(h, mul, add));
}

// Hides a constant from the optimizer so that it lives in a VGPR.  gfx9-class
// VOP3/VOP3P instructions take no literal and at most one SGPR, so keeping the
// decode constants in registers is what lets one v_and_or_b32 and one
// v_pk_fma_f16 do the work of each pair of weights.
__device__ __forceinline__ uint32_t in_vgpr(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ uint32_t pack_half2(float lo, float hi) {
  const half2v h = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, h);
}

// Decode constants for field positions 0..4 of a half (see decode_pair_same).
struct DecodeConsts {
  uint32_t magic;
  uint32_t mul[5];
  uint32_t add[5];
  __device__ __forceinline__ void init() {
    magic = in_vgpr(kMagic2);
#pragma unroll
    for (int p = 0; p < 5; ++p) {
      const float m = 1.0f / float(1 << (2 * p));
      const float a = -(1024.0f / float(1 << (2 * p)) + 1.0f);
      mul[p] = in_vgpr(pack_half2(m, m));
      add[p] = in_vgpr(pack_half2(a, a));
    }
  }
  // Same as decode_pair_same<P> with the constants held in VGPRs.
  template <int P>
  __device__ __forceinline__ uint32_t pair(uint32_t x) const {
    constexpr uint32_t mask = (3u << (2 * P)) | (3u << (16 + 2 * P));
    const uint32_t v = (x & mask) | magic;
    const half2v r = __builtin_elementwise_fma(__builtin_bit_cast(half2v, v),
                                               __builtin_bit_cast(half2v, mul[P]),
                                               __builtin_bit_cast(half2v, add[P]));
    return __builtin_bit_cast(uint32_t, r);
  }
};

// Byte select: result bytes from {lo (0..3), hi (4..7)} as v_perm_b32 does.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

// Natural-order decode constants: the low half takes field 2q of a byte, the
// high half field 2q + 1 (q = 0, 1).
struct NaturalConsts {
  uint32_t magic;
  uint32_t mul[2], add[2];
  __device__ __forceinline__ void init() {
    magic = in_vgpr(kMagic2);
    mul[0] = in_vgpr(pack_half2(1.0f, 0.25f));
    add[0] = in_vgpr(pack_half2(-1025.0f, -257.0f));
    mul[1] = in_vgpr(pack_half2(1.0f / 16.0f, 1.0f / 64.0f));
    add[1] = in_vgpr(pack_half2(-65.0f, -17.0f));
  }
  // z holds one weight byte in the low byte of both halves; returns the fp16
  // pair (s * d_{2q}, s * d_{2q+1}) for q = Q.
  template <int Q>
  __device__ __forceinline__ uint32_t pair(uint32_t z, uint32_t s2) const {
    constexpr uint32_t mask = Q == 0 ? 0x000C0003u : 0x00C00030u;
    const uint32_t v = (z & mask) | magic;
    const half2v d = __builtin_elementwise_fma(__builtin_bit_cast(half2v, v),
                                               __builtin_bit_cast(half2v, mul[Q]),
                                               __builtin_bit_cast(half2v, add[Q]));
    return __builtin_bit_cast(uint32_t, d * __builtin_bit_cast(half2v, s2));
  }
  // The trit pair (d_{2q}, d_{2q+1}) alone, exact in fp16.
  template <int Q>
  __device__ __forceinline__ uint32_t trits(uint32_t z) const {
    constexpr uint32_t mask = Q == 0 ? 0x000C0003u : 0x00C00030u;
    const uint32_t v = (z & mask) | magic;
    const half2v d = __builtin_elementwise_fma(__builtin_bit_cast(half2v, v),
                                               __builtin_bit_cast(half2v, mul[Q]),
                                               __builtin_bit_cast(half2v, add[Q]));
    return __builtin_bit_cast(uint32_t, d);
  }
  // B operand of 8 consecutive trits (no scale): the byte pair H of dword x.
  template <int H>
  __device__ __forceinline__ half8 trit_operand(uint32_t x) const {
    const uint32_t z = perm(x, x, H == 0 ? 0x01000100u : 0x03020302u);
    const uint32_t z2 = z >> 8;
    u32x4 r;
    r[0] = trits<0>(z);
    r[1] = trits<1>(z);
    r[2] = trits<0>(z2);
    r[3] = trits<1>(z2);
    return __builtin_bit_cast(half8, r);
  }
  // B operand of 8 consecutive weights: the byte pair H (0 or 1) of dword x,
  // times the scale pair s2.
  template <int H>
  __device__ __forceinline__ half8 operand(uint32_t x, uint32_t s2) const {
    return operand_sel(x, H == 0 ? 0x01000100u : 0x03020302u, s2);
  }
  // The same with the byte pair chosen by a v_perm_b32 selector (0x01000100
  // for bytes 0, 1; 0x03020302 for bytes 2, 3), which may differ per lane.
  __device__ __forceinline__ half8 operand_sel(uint32_t x, uint32_t sel, uint32_t s2) const {
    // both halves hold the selected bytes: [b, b', b, b']
    const uint32_t z = perm(x, x, sel);
    const uint32_t z2 = z >> 8;  // low byte of each half = b'
    u32x4 r;
    r[0] = pair<0>(z, s2);
    r[1] = pair<1>(z, s2);
    r[2] = pair<0>(z2, s2);
    r[3] = pair<1>(z2, s2);
    return __builtin_bit_cast(half8, r);
  }
};


}  // namespace tq
