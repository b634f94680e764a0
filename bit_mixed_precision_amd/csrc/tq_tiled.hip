// Tiled MFMA kernel (M > 16): Y = X (s . T)^T for TQ2 weights.
//
// Follows the project page "Scaling Laws and Efficient Inference for Ternary
// Language Models": "The model" (step 3), "2 bits per weight" (decoder),
// "Fast inference on CPUs" (256-weight scale block), "TriRun: ternary
// inference on GPUs" (FP32 accumulation, FP16 output).  MI355X design:
//
//  * a workgroup is 4 waves, NG weight-row groups x KG k-groups, and owns a
//    BM x BN output tile (BM = 16 MT activation rows, BN = 16 NR NG weight
//    rows); k-group c takes the 256-weight blocks c, c + KG, ...; the
//    k-groups' partial tiles meet in LDS at the end;
//  * activations reach LDS through the direct global -> LDS path
//    (global_load_lds_dwordx4): one instruction moves 8 rows x 128 B with 8
//    consecutive lanes per row, so every request is a whole cache line.  The
//    16-byte piece a lane fetches is XOR-swizzled on the global side, which
//    lets the MFMA-order ds_read_b128 of 16 rows hit 16 distinct bank groups.
//    A ring of kStages stages (64 k of every k-group's block each) keeps
//    kStages - 1 stages in flight behind one barrier per stage;
//  * weights and block scales take the same direct path a round ahead (16
//    rows x 64 B per weight instruction, 4 lanes per row), so the loop holds
//    no register loads and every wait is an explicit, exact vmcnt; a lane
//    reads 16 B of its row's 64-byte block back, and 4 v_perm_b32 and 4 lane
//    swaps (v_permlane32_swap / v_permlane16_swap) put them in MFMA B order;
//    one v_perm_b32 copies a byte pair into both halves, v_and_or_b32 against
//    the fp16 exponent of 1024 extracts two fields, v_pk_fma_f16 makes them
//    exact trits and v_pk_mul_f16 applies the block scale (+-s or 0, exact);
//  * v_mfma_f32_16x16x32_f16 with fp32 accumulators across all of K; one
//    fp32 -> fp16 rounding writes Y.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

template <int I, int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor<I + 1, N>(f);
  }
}

constexpr int kStages = 3;  // LDS ring depth (stages of 64 k)

// s_waitcnt immediate that waits for the vector-memory counter only.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

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
  // B operand of 8 consecutive weights: the byte pair H (0 or 1) of dword x,
  // times the scale pair s2.
  template <int H>
  __device__ __forceinline__ half8 operand(uint32_t x, uint32_t s2) const {
    // both halves hold bytes (2H, 2H + 1): [b, b', b, b']
    const uint32_t z = perm(x, x, H == 0 ? 0x01000100u : 0x03020302u);
    const uint32_t z2 = z >> 8;  // low byte of each half = b'
    u32x4 r;
    r[0] = pair<0>(z, s2);
    r[1] = pair<1>(z, s2);
    r[2] = pair<0>(z2, s2);
    r[3] = pair<1>(z2, s2);
    return __builtin_bit_cast(half8, r);
  }
};

// Lane (n, g) holds bytes 16 g .. 16 g + 15 of row n's 64-byte block.  In the
// MFMA B order lane (n, g) needs, for step j = 0..7 (32 weights each), the
// bytes 8 j + 2 g and 8 j + 2 g + 1 (weights 32 j + 8 g .. + 7).  Returns
// dword d = those byte pairs for steps 2 d and 2 d + 1: every lane first
// gathers, for each of the 4 lanes of its row, the dword that lane needs from
// it (4 v_perm_b32), then the 4 x 4 block of (register, 16-lane row) is
// transposed with two rounds of lane swaps.
__device__ __forceinline__ u32x4 to_b_order(u32x4 w) {
  const uint32_t e0 = perm(w[2], w[0], 0x05040100u);
  const uint32_t e1 = perm(w[2], w[0], 0x07060302u);
  const uint32_t e2 = perm(w[3], w[1], 0x05040100u);
  const uint32_t e3 = perm(w[3], w[1], 0x07060302u);
  // (rows 0, 1 of e0 | rows 0, 1 of e2) and (rows 2, 3 of e0 | rows 2, 3 of e2)
  const auto a = __builtin_amdgcn_permlane32_swap(e0, e2, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(e1, e3, false, false);
  // interleave 16-lane rows: (a0, b0, a2, b2) and (a1, b1, a3, b3)
  const auto c = __builtin_amdgcn_permlane16_swap(a[0], b[0], false, false);
  const auto d = __builtin_amdgcn_permlane16_swap(a[1], b[1], false, false);
  return u32x4{c[0], c[1], d[0], d[1]};
}

// Direct global -> LDS copies: each lane reads 16 (or 2) bytes at src; lane l
// writes LDS bytes dst + 16 l (dst + 4 l, zero-extended).  dst is the same for
// the whole wave.  Plain __device__ functions keep the gfx950-only 16-byte
// form out of the host compilation of the kernel templates.
__device__ __forceinline__ void dma16(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void dma2(const void* src, unsigned char* dst) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)dst, 2, 0, 0);
}

// Compiler-level memory fence: the barrier intrinsics alone do not keep LDS
// reads from moving across them, and the LDS writes of global_load_lds are
// not visible to the compiler.
__device__ __forceinline__ void mem_clobber() { asm volatile("" ::: "memory"); }

template <int MT, int NR, int NG, int KG>
struct TileGeom {
  static_assert(NG * KG == 4, "a workgroup is 4 waves");
  static constexpr int BM = 16 * MT;
  static constexpr int BNW = 16 * NR;  // weight rows per wave
  static constexpr int BN = NG * BNW;
  static constexpr int kChunk = BM * 128;  // one k-group's stage: BM rows x 64 k
  static constexpr int kStage = KG * kChunk;
  static constexpr int kRing = kStages * kStage;
  static constexpr int kXfer = KG * BM / 8;  // DMA instructions per stage
  static_assert(kXfer % 4 == 0, "DMA instructions split evenly over 4 waves");
  static constexpr int kPer = kXfer / 4;
  static constexpr int kWOff = kRing;             // weights: 1 KB per (wave, row group)
  static constexpr int kSOff = kWOff + 4 * NR * 1024;  // scales: one dword per wave lane
  static constexpr int kLoop = kSOff + 4 * 256;
  static constexpr int kRed = (KG - 1) * NG * MT * NR * 256 * 4;
  static constexpr int kLds = kLoop > kRed ? kLoop : kRed;
  static_assert(NR == 4, "one scale DMA covers the 64 weight rows of a wave");
};

// Workgroup L runs tile (n_tile, m_tile) with n_tile = 8 (L / 8 / m_tiles) +
// L % 8 and m_tile = (L / 8) % m_tiles: consecutive workgroups go to
// different XCDs, and the m tiles of one weight-row tile run back to back on
// the same XCD, so its weights are read from HBM once.
template <int MT, int NR, int NG, int KG>
__global__ __launch_bounds__(256) void tq2_tiled_kernel(const uint16_t* __restrict__ X,
                                                        const uint8_t* __restrict__ qs,
                                                        const uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ Y, int M, int N,
                                                        int K, int n_tiles, int m_tiles) {
  using G = TileGeom<MT, NR, NG, KG>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int L = blockIdx.x;
  const int m_tile = (L >> 3) % m_tiles;
  const int n_tile = ((L >> 3) / m_tiles) * 8 + (L & 7);
  if (n_tile >= n_tiles) return;  // whole workgroup
  const int n_base = n_tile * G::BN;
  const int m_base = m_tile * G::BM;

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % NG;
  const int wk = wave / NG;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int rounds = (nb + KG - 1) / KG;
  const int S = 4 * rounds;  // stages (>= 4 > kStages - 1)
  const size_t row_bytes = (size_t)(K >> 2);

  NaturalConsts dc;
  dc.init();

  // ---- activation DMA: instruction q = wave + 4 u moves rows 8 rg .. 8 rg + 7
  // of k-group c's chunk; lane i takes row 8 rg + i / 8, LDS piece i % 8, i.e.
  // global piece (i % 8) ^ swz(row), swz(row) = (row / 2) % 8.  Rows past M
  // read row m_base (valid data; never written).
  const uint16_t* xsrc[G::kPer];
  int xc[G::kPer];
  uint32_t xdst[G::kPer];
#pragma unroll
  for (int u = 0; u < G::kPer; ++u) {
    const int q = wave + 4 * u;
    const int c = q / (G::BM / 8);
    const int rg = q % (G::BM / 8);
    const int row = 8 * rg + (lane >> 3);
    const int gp = (lane & 7) ^ ((row >> 1) & 7);
    const int m = m_base + row < M ? m_base + row : m_base;
    xsrc[u] = X + (size_t)m * K + 8 * gp;
    xc[u] = c;
    xdst[u] = c * G::kChunk + rg * 1024;
  }
  auto issue = [&](int s) {
    const int r = s >> 2;
    const int ch = s & 3;
    const uint32_t slot = (uint32_t)(s % kStages) * G::kStage;
#pragma unroll
    for (int u = 0; u < G::kPer; ++u) {
      int b = r * KG + xc[u];
      b = b < nb ? b : nb - 1;
      dma16(xsrc[u] + 256 * (size_t)b + 64 * ch, smem + slot + xdst[u]);
    }
  };

  // ---- weights and scales of the wave's rows for round rd (block rd KG + wk),
  // one round ahead.  Weight instruction r moves rows 16 r .. 16 r + 15 of the
  // wave: lane i takes row i / 4, LDS piece i % 4, global piece
  // (i % 4) ^ ((row / 4) % 4).  The scale instruction gives lane i the scale of
  // the wave's row i (zero-extended into one LDS dword).  Rows past N read row
  // n_base (valid data; never written).
  const uint8_t* wsrc[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int row = 16 * r + (lane >> 2);
    const int n = n_base + wn * G::BNW + row;
    const int nn = n < N ? n : n_base;
    const int gp = (lane & 3) ^ ((row >> 2) & 3);
    wsrc[r] = qs + (size_t)nn * row_bytes + 16 * gp;
  }
  const uint16_t* ssrc;
  {
    const int n = n_base + wn * G::BNW + lane;
    ssrc = scales + (size_t)(n < N ? n : n_base) * nb;
  }
  const uint32_t wdst = G::kWOff + wave * NR * 1024;
  const uint32_t sdst = G::kSOff + wave * 256;
  auto issue_w = [&](int rd) {
    int b = rd * KG + wk;
    b = b < nb ? b : nb - 1;
#pragma unroll
    for (int r = 0; r < NR; ++r)
      dma16(wsrc[r] + 64 * (size_t)b, smem + wdst + r * 1024);
    dma2(ssrc + b, smem + sdst);
  };
  constexpr int kWIssue = NR + 1;  // DMA instructions of issue_w
  // Read-back offsets: lane (li, g) wants bytes 16 g .. 16 g + 15 of row
  // 16 r + li, and the scale of that row.
  const uint32_t w_rd = wdst + li * 64 + 16 * (g ^ ((li >> 2) & 3));
  const uint32_t s_rd = sdst + 4 * li;

  // ds_read_b128 offsets of the A operand (row li of m-tile i at +2048 i):
  // step H of a stage needs global piece 4 H + g of row li.
  uint32_t a_off[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) a_off[h] = li * 128 + 16 * ((4 * h + g) ^ ((li >> 1) & 7));

  float4v C[MT][NR];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < NR; ++r) C[i][r] = float4v{0.f, 0.f, 0.f, 0.f};

  u32x4 wb[NR];
  uint32_t s2[NR];

  issue_w(0);
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue(s);

  for (int rd = 0; rd < rounds; ++rd) {
    const bool active = rd * KG + wk < nb;  // wave-uniform
    sfor<0, 4>([&](auto cc) {
      constexpr int ch = decltype(cc)::value;
      const int s = 4 * rd + ch;
      // Stage s's DMA came kStages - 1 = 2 iterations ago; younger are the
      // next stage's DMA and, when ch = 1 fell in between (ch = 2, 3), the
      // weight/scale DMA issued after it.  The weight/scale DMA of round rd
      // is older than stage s's, so ch = 0 finds it complete as well.
      static_assert(kStages == 3, "the count below assumes a 3-stage ring");
      constexpr int younger = G::kPer + (ch >= 2 ? kWIssue : 0);
      mem_clobber();
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(younger));
      __builtin_amdgcn_s_barrier();
      mem_clobber();
      if constexpr (ch == 0) {
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          wb[r] = to_b_order(*reinterpret_cast<const u32x4*>(smem + w_rd + r * 1024));
          const uint32_t sc = *reinterpret_cast<const uint32_t*>(smem + s_rd + 64 * r);
          s2[r] = sc | (sc << 16);
        }
      }
      {
        const int sn = s + kStages - 1;
        issue(sn < S ? sn : S - 1);  // past the end: a harmless refill
      }
      if constexpr (ch == 1) issue_w(rd + 1 < rounds ? rd + 1 : rd);  // after this
      // wave's ch = 0 reads of the buffers, which the barrier above ordered
      if (active) {
        const unsigned char* base =
            smem + (uint32_t)(s % kStages) * G::kStage + wk * G::kChunk;
        sfor<0, 2>([&](auto hh) {
          constexpr int H = decltype(hh)::value;
          half8 B[NR];
#pragma unroll
          for (int r = 0; r < NR; ++r) B[r] = dc.operand<H>(wb[r][ch], s2[r]);
#pragma unroll
          for (int i = 0; i < MT; ++i) {
            const half8 A = *reinterpret_cast<const half8*>(base + a_off[H] + 2048 * i);
#pragma unroll
            for (int r = 0; r < NR; ++r) C[i][r] = mfma16(A, B[r], C[i][r]);
          }
        });
      }
    });
  }

  // Reduce the k-groups' partial tiles through LDS (the drain waits for the
  // trailing refills, and no wave reads the ring any more).
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
  constexpr int kTile = MT * NR * 256;  // floats per wave
  if (KG > 1 && wk > 0) {
    float* dst = red + ((wk - 1) * NG + wn) * kTile;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[((i * NR + r) * 4 + e) * 64 + lane] = C[i][r][e];
  }
  __syncthreads();
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        const int n = n_base + wn * G::BNW + 16 * r + li;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sum = C[i][r][e];
#pragma unroll
          for (int c = 1; c < KG; ++c)
            sum += red[((c - 1) * NG + wn) * kTile + ((i * NR + r) * 4 + e) * 64 + lane];
          const int m = m_base + 16 * i + 4 * g + e;
          if (m < M && n < N) Y[(size_t)m * N + n] = f2h_bits(sum);
        }
      }
    }
  }
}

template <int MT, int NR, int NG, int KG>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
  using G = TileGeom<MT, NR, NG, KG>;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(tq2_tiled_kernel<MT, NR, NG, KG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, G::kLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t n_tiles = (a.N + G::BN - 1) / G::BN;
  const int64_t m_tiles = (a.M + G::BM - 1) / G::BM;
  const int64_t groups = (n_tiles + 7) / 8;
  const int64_t wgs = groups * 8 * m_tiles;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((tq2_tiled_kernel<MT, NR, NG, KG>), dim3((unsigned)wgs), dim3(256), G::kLds,
                     stream, static_cast<const uint16_t*>(a.X),
                     static_cast<const uint8_t*>(a.qs), static_cast<const uint16_t*>(a.scales),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, (int)n_tiles,
                     (int)m_tiles);
  return hipGetLastError();
}

}  // namespace

// Tile choice: 32 activation rows per tile up to M = 32, else 64; two
// weight-row groups x two k-groups (BN = 128) when that still gives one
// workgroup per compute unit, else one weight-row group x four k-groups
// (BN = 64).
TiledShape tiled_shape(int64_t M, int64_t N) {
  const int64_t cus = device_cus();
  const int mt = M <= 32 ? 2 : 4;
  const int64_t m_tiles = (M + 16 * mt - 1) / (16 * mt);
  const int64_t wide = ((N + 127) / 128) * m_tiles;
  if (wide >= cus) return TiledShape{mt, 4, 2, 2};
  return TiledShape{mt, 4, 1, 4};
}

hipError_t launch_tq2_tiled(const GemmArgs& a, hipStream_t stream) {
  const TiledShape t = tiled_shape(a.M, a.N);
  if (t.mt == 2) {
    if (t.ng == 2) return launch_tiled<2, 4, 2, 2>(a, stream);
    return launch_tiled<2, 4, 1, 4>(a, stream);
  }
  if (t.ng == 2) return launch_tiled<4, 4, 2, 2>(a, stream);
  return launch_tiled<4, 4, 1, 4>(a, stream);
}

}  // namespace tq
