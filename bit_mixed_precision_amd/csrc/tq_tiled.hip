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
//    (buffer_load_dwordx4 ... lds): one instruction moves 8 rows x 128 B with 8
//    consecutive lanes per row, so every request is a whole cache line.  The
//    16-byte piece a lane fetches is XOR-swizzled on the global side, which
//    lets the MFMA-order ds_read_b128 of 16 rows hit 16 distinct bank groups.
//    A ring of XS stages (64 k of every k-group's block each) keeps XS - 1
//    stages in flight behind one barrier per stage; XS (3 to 6) and the
//    weight ring depth WD (1 or 2 rounds) are the deepest that fit the LDS
//    of one compute unit (8-wave workgroups) or half of it (4-wave ones);
//  * weights and block scales take the same direct path a round ahead (16
//    rows x 64 B per weight instruction, 4 lanes per row), so the loop holds
//    no register loads and every wait is an explicit, exact vmcnt; a lane
//    reads 16 B of its row's 64-byte block back, and 4 v_perm_b32 and 4 lane
//    swaps (v_permlane32_swap / v_permlane16_swap) put them in MFMA B order;
//    one v_perm_b32 copies a byte pair into both halves, v_and_or_b32 against
//    the fp16 exponent of 1024 extracts two fields and v_pk_fma_f16 makes
//    them exact trits;
//  * v_mfma_f32_16x16x32_f16 with fp32 accumulators: each round's block sums
//    in its own accumulators and its block scale is applied once per round
//    (one FMA per element); one fp32 -> fp16 rounding writes Y.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"
#include "tq_tiled_sched.h"

namespace tq {
namespace {

template <int I, int N, class F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor<I + 1, N>(f);
  }
}

// s_waitcnt immediate that waits for the vector-memory counter only.
constexpr int vmcnt_imm(int n) { return (n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14); }

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

// Direct global -> LDS copies through a buffer resource: each lane reads
// 16 (or 2) bytes at the resource's base + voff + soff (soff in a scalar
// register: the k offset, the same in every lane); lane l writes LDS bytes
// dst + 16 l (dst + 4 l, zero-extended).  dst is the same for the whole wave.
// The lane offsets are fixed for the whole kernel, so a copy costs no vector
// instruction (a flat copy's 64-bit address cost two; measured 1-4% faster).
// Plain __device__ functions keep the gfx950-only 16-byte form out of the
// host compilation of the kernel templates.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                      unsigned char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16,
                                           voff, soff, 0, 0);
}
__device__ __forceinline__ void dma2(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                     unsigned char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 2,
                                           voff, soff, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, int voff, int soff,
                                     unsigned char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 4,
                                           voff, soff, 0, 0);
}

// Compiler-level memory fence: the barrier intrinsics alone do not keep LDS
// reads from moving across them, and the LDS writes of the direct copies are
// not visible to the compiler.
__device__ __forceinline__ void mem_clobber() { asm volatile("" ::: "memory"); }

template <int MT, int NR, int NG, int KG, bool T1 = false>
struct TileGeom {
  static constexpr int WV = NG * KG;  // waves per workgroup
  static_assert(WV == 4 || WV == 8, "a workgroup is 4 or 8 waves");
  static constexpr int BM = 16 * MT;
  static constexpr int BNW = 16 * NR;  // weight rows per wave
  static constexpr int BN = NG * BNW;
  static constexpr int kChunk = BM * 128;  // one k-group's stage: BM rows x 64 k
  static constexpr int kStage = KG * kChunk;
  static constexpr int kWRound = WV * (NR * 1024 + 256);  // weights + scales of a round
  // Ring depths: the deepest (XS, WD) whose rings fit the LDS budget.
  static constexpr int kLut = T1 ? 1024 : 0;  // TQ1: byte -> five 2-bit fields
  static constexpr int kBudget = (WV == 8 ? 160 * 1024 : 80 * 1024) - kLut;
  // (A second weight slot in place of a fourth activation stage, which lets
  // the 1.6-bit decode spread over the whole round, measured slower for it:
  // M = 128, K = 8192, N = 28672 85.5 -> 90.5 us, N = 8192 36.6 -> 40.0 us.)
  static constexpr RingPlan kPlan = ring_plan(kStage, kWRound, kBudget);
  static constexpr int XS = kPlan.xs;
  static constexpr int WD = kPlan.wd;
  static constexpr int WCH = w_issue_ch(WD);  // stage of a round that issues weights
  static_assert(XS <= 4 * WD - WCH, "weights must arrive before the stage that reads them");
  static_assert(XS <= 6, "round 0 is the only round whose wait window reaches the prologue");
  // T1: row group r of the next round's weights is decoded at stage wch_of(r)
  // of the round, spread over the stages from the first at which they have
  // landed
  static constexpr int kWReady = w_ready_ch(XS, WD);
  static constexpr int wch_of(int r) { return kWReady + r * (4 - kWReady) / NR; }
  static constexpr int kRing = XS * kStage;
  static constexpr int RG8 = BM / 8;          // 8-row DMA groups per chunk
  static constexpr int kXfer = KG * RG8;      // DMA instructions per stage
  static_assert(kXfer % WV == 0, "DMA instructions split evenly over the waves");
  static_assert(RG8 % WV == 0 || WV % RG8 == 0, "row groups map evenly to waves");
  static constexpr int kPer = kXfer / WV;
  static constexpr int RP = RG8 >= WV ? RG8 / WV : 1;  // distinct row groups per wave
  static constexpr int kWOff = kRing;             // weights: 1 KB per (wave, row group)
  static constexpr int kSOff = kWOff + WD * WV * NR * 1024;  // scales: a dword per lane
  static constexpr int kLutOff = kSOff + WD * WV * 256;
  static constexpr int kLoop = kLutOff + kLut;
  static constexpr int kRed = (KG - 1) * NG * MT * NR * 256 * 4;
  static constexpr int kEpi = kRed + BM * (2 * BN + 16);  // partial tiles + fp16 tile
  static constexpr int kLds = kLoop > kEpi ? kLoop : kEpi;
  static_assert(NR <= 4, "one scale DMA (64 lanes) covers the weight rows of a wave");
  static_assert(kLds <= 160 * 1024, "the rings fit the LDS of a compute unit");
};

// Workgroup L runs on XCD L % 8; j = L / 8 orders the tiles an XCD runs.
// n-major (m_outer = 0): n_tile = 8 (j / m_tiles) + L % 8, m_tile = j % m_tiles:
// the m tiles of one weight-row tile run back to back on one XCD, so its
// weights are read from HBM once.  m-major (m_outer = 1, for many m tiles):
// m_tile = j / groups, n_tile = 8 (j % groups) + L % 8 with groups =
// ceil(n_tiles / 8): an XCD walks its weight tiles under one activation tile,
// which stays in its L2, instead of streaming all of X once per weight tile.
//
// T1: the weights are 1.6-bit rows (ldq bytes each, five trits per byte).  A
// round's block b of a row is the bytes floor(256 b / 5) .. floor((256 b +
// 255) / 5); the direct copy moves the 64 bytes from that first byte rounded
// down to 4 (16 lanes per row, one dword each), into the slot the 2-bit
// block would take.  On read-back a lane takes the 14 bytes that hold its 64
// weights, looks up each byte's five 2-bit fields (d' = d + 1, the 2-bit
// code's own fields) in a 256-entry LDS table that the workgroup fills with
// the pages' multiply-by-3 decoder, and shifts the 140-bit field string by
// the block's trit offset: the four dwords it gets are exactly the 2-bit
// block's, and the rest of the kernel is unchanged.
// SB: the block scale multiplies each decoded operand (one v_pk_mul_f16 per
// two weights, exact) instead of a second accumulator set, which frees the
// registers the table decode needs in the large wave tiles.
template <int MT, int NR, int NG, int KG, bool T1, bool SB>
__device__ __forceinline__ void tiled_body(const uint16_t* __restrict__ X,
                                           const uint8_t* __restrict__ qs, int ldq,
                                           const uint16_t* __restrict__ scales,
                                           uint16_t* __restrict__ Y, int M, int N, int K,
                                           int n_tiles, int m_tiles, int m_outer) {
  using G = TileGeom<MT, NR, NG, KG, T1>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int L = blockIdx.x;
  const int j = L >> 3;
  const int groups = (n_tiles + 7) >> 3;
  const int m_tile = m_outer ? j / groups : j % m_tiles;
  const int n_tile = (m_outer ? j % groups : j / m_tiles) * 8 + (L & 7);
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
  const int S = 4 * rounds;  // stages
  const size_t row_bytes = T1 ? (size_t)ldq : (size_t)(K >> 2);

  NaturalConsts dc;
  dc.init();

  // T1: entry v of the table holds the five 2-bit fields d' of byte value v,
  // weight j of the byte at bits 2 j .. 2 j + 1, by the multiply-by-3 decoder
  // (t = 3 q; d' = t >> 8; q = t & 255, most significant digit first).
  if constexpr (T1) {
    uint32_t* lut = reinterpret_cast<uint32_t*>(smem + G::kLutOff);
    for (int v = threadIdx.x; v < 256; v += 64 * G::WV) {
      uint32_t q = (uint32_t)v, code = 0u;
#pragma unroll
      for (int f = 0; f < 5; ++f) {
        const uint32_t t = 3u * q;
        code |= (t >> 8) << (2 * f);
        q = t & 255u;
      }
      lut[v] = code;
    }
    __syncthreads();
  }

  // ---- activation DMA: instruction q = wave + WV u moves rows 8 rg .. 8 rg + 7
  // (rg = q % RG8) of k-group c = q / RG8's chunk; lane i takes row
  // 8 rg + i / 8, LDS piece i % 8, i.e. global piece (i % 8) ^ swz(row),
  // swz(row) = (row / 2) % 8.  A wave touches only RP distinct row groups.
  // Rows past M read row m_base (valid data; never written).
  // Byte offsets from the tile's first activation row (< 64 rows x 2^21 B).
  const unsigned char* xbase = reinterpret_cast<const unsigned char*>(X + (size_t)m_base * K);
  const int xrows = M - m_base < G::BM ? M - m_base : G::BM;  // rows of the tile in X
  const auto xrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(xbase), 0,
                                                       xrows * K * 2, kBufferWord3);
  uint32_t xoff[G::RP];
#pragma unroll
  for (int p = 0; p < G::RP; ++p) {
    const int rg = G::RG8 >= G::WV ? wave + G::WV * p : wave % G::RG8;
    const int row = 8 * rg + (lane >> 3);
    const int gp = (lane & 7) ^ ((row >> 1) & 7);
    const int rel = m_base + row < M ? row : 0;
    xoff[p] = (uint32_t)rel * (uint32_t)K * 2u + 16u * gp;
  }
  auto issue = [&](int s) {
    const int r = s >> 2;
    const int ch = s & 3;
    const uint32_t slot = (uint32_t)(s % G::XS) * G::kStage;
#pragma unroll
    for (int u = 0; u < G::kPer; ++u) {
      const int p = u % G::RP;
      const int c = G::RG8 >= G::WV ? u / G::RP : wave / G::RG8 + u * (G::WV / G::RG8);
      const int rg = G::RG8 >= G::WV ? wave + G::WV * p : wave % G::RG8;
      int b = r * KG + c;
      b = b < nb ? b : nb - 1;
      dma16(xrsrc, (int)xoff[p], 512 * b + 128 * ch, smem + slot + c * G::kChunk + rg * 1024);
    }
  };

  // ---- weights and scales of the wave's rows for round rd (block rd KG + wk),
  // one round ahead.  Weight instruction r moves rows 16 r .. 16 r + 15 of the
  // wave: lane i takes row i / 4, LDS piece i % 4, global piece
  // (i % 4) ^ ((row / 4) % 4).  The scale instruction gives lane i the scale of
  // the wave's row i (zero-extended into one LDS dword).  Rows past N read row
  // n_base (valid data; never written).
  // 32-bit byte offsets from the workgroup's first row (the lowest row any
  // lane reads) keep the addresses in few registers: a tile spans at most 256
  // rows of K / 4 <= 2^18 bytes.
  const uint8_t* wbase = qs + (size_t)n_base * row_bytes;
  const uint16_t* sbase = scales + (size_t)n_base * nb;
  const int wrows = N - n_base < G::BN ? N - n_base : G::BN;  // rows of the tile in the matrix
  const auto wrsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(wbase), 0,
                                                       wrows * (int)row_bytes, kBufferWord3);
  const auto srsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(sbase), 0,
                                                       wrows * nb * 2, kBufferWord3);
  uint32_t woff[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    if constexpr (T1) {
      // 16 lanes per row, one dword each; instruction t of the 16-row group
      // adds 4 t rows through the scalar offset.  Rows past N lie past the
      // resource and read zeros (never written).
      const int row = 16 * r + (lane >> 4);
      const int rel = wn * G::BNW + row;
      woff[r] = (uint32_t)rel * (uint32_t)row_bytes + 4u * (uint32_t)(lane & 15);
    } else {
      const int row = 16 * r + (lane >> 2);
      const int n = n_base + wn * G::BNW + row;
      const int rel = n < N ? n - n_base : 0;
      const int gp = (lane & 3) ^ ((row >> 2) & 3);
      woff[r] = (uint32_t)rel * (uint32_t)row_bytes + 16u * gp;
    }
  }
  uint32_t soff;
  {
    const int n = n_base + wn * G::BNW + lane;
    soff = (uint32_t)(n < N ? n - n_base : 0) * (uint32_t)nb * 2u;
  }
  // Round rd's weights and scales sit in slot rd % WD of their rings.
  auto wdst = [&](int rd) { return G::kWOff + ((rd % G::WD) * G::WV + wave) * NR * 1024; };
  auto sdst = [&](int rd) { return G::kSOff + ((rd % G::WD) * G::WV + wave) * 256; };
  // The 256-weight block of round rd (past the end: a harmless refill of the
  // last round's block, which is also what read_w then decodes).
  auto block_of = [&](int rd) {
    const int rc = rd < rounds ? rd : rounds - 1;
    const int b = rc * KG + wk;
    return b < nb ? b : nb - 1;
  };
  auto issue_w = [&](int rd) {
    const int b = block_of(rd);
    if constexpr (T1) {
      const int ab = ((256 * b) / 5) & ~3;  // first byte of the block, rounded down to 4
#pragma unroll
      for (int r = 0; r < NR; ++r)
#pragma unroll
        for (int t = 0; t < 4; ++t)
          dma4(wrsrc, (int)woff[r], ab + 4 * t * ldq, smem + wdst(rd) + r * 1024 + t * 256);
    } else {
#pragma unroll
      for (int r = 0; r < NR; ++r) dma16(wrsrc, (int)woff[r], 64 * b, smem + wdst(rd) + r * 1024);
    }
    dma2(srsrc, (int)soff, 2 * b, smem + sdst(rd));
  };
  constexpr int kWIssue = (T1 ? 4 : 1) * NR + 1;  // DMA instructions of issue_w
  // Read-back offsets: lane (li, g) wants bytes 16 g .. 16 g + 15 of row
  // 16 r + li, and the scale of that row.
  const uint32_t w_rd = li * 64 + 16 * (g ^ ((li >> 2) & 3));
  const uint32_t s_rd = 4 * li;

  // ds_read_b128 offsets of the A operand (row li of m-tile i at +2048 i):
  // step H of a stage needs global piece 4 H + g of row li.
  // (4 + g) ^ swz = (g ^ swz) ^ 4 for g < 4, so step 1 is step 0's offset ^ 64.
  const uint32_t a_off0 = li * 128 + 16 * (g ^ ((li >> 1) & 7));

  float4v C[MT][NR];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < NR; ++r) C[i][r] = float4v{0.f, 0.f, 0.f, 0.f};
  // The B operands are the bare trits; a round's block (the k-group's one
  // 256-weight block) accumulates in Cb and its scale is applied once per
  // round, C += s * Cb: one FMA per accumulator element instead of a
  // v_pk_mul per two weights, whose VALU time bounded the loop of the small
  // wave tiles (4-8 VALU instructions per MFMA) and held back the larger
  // ones.  The products are exact either way; only the fp32 rounding order
  // differs.
  float4v Cb[MT][NR];
  // B operand of 8 weights from byte pair H of dword x: bare trits, or (SB)
  // trits times the round's scale pair
  auto operand = [&](auto hh, uint32_t x, uint32_t sc2) -> half8 {
    constexpr int H = decltype(hh)::value;
    if constexpr (SB)
      return dc.template operand<H>(x, sc2);
    else
      return dc.template trit_operand<H>(x);
  };
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;

  // Weights of round rd in B order and their scale pairs (read_w; read_w_row
  // for one row group of 1.6-bit rows, decoded from the copied TQ1 bytes); a
  // k-group without a block in the round (K / 256 not a multiple of KG) gets
  // scale 0, so its block sum adds nothing and every wave runs the same
  // straight-line code.
  auto read_w_row = [&](int rd, int r, u32x4* wbo, uint32_t* s2o) {
    const bool active = rd * KG + wk < nb;
    // Lane (li, g) wants weights 256 b + 64 g .. + 63 of its row: TQ1 bytes
    // i .. i + 13 (i = floor(x / 5), x = 256 b + 64 g), from trit ph = x - 5 i
    // of byte i on, i.e. byte o = i - ab of the copied row.
    const uint32_t b = (uint32_t)block_of(rd);
    const uint32_t x = 256u * b + 64u * (uint32_t)g;
    const uint32_t i5 = __umulhi(x, 0xCCCCCCCDu) >> 2;  // floor(x / 5), exact for 32 bits
    const uint32_t sh = 2u * (x - 5u * i5);               // field offset: 2 ph
    const uint32_t o = i5 - (((256u * b) / 5u) & ~3u);   // <= 42
    const uint32_t* lut = reinterpret_cast<const uint32_t*>(smem + G::kLutOff);
    const uint32_t* src = reinterpret_cast<const uint32_t*>(smem + wdst(rd) + r * 1024 +
                                                            (uint32_t)li * 64u + (o & ~3u));
    uint32_t D[5];
#pragma unroll
    for (int u = 0; u < 5; ++u) D[u] = src[u];
    uint32_t E[4];  // bytes o .. o + 15 of the row
#pragma unroll
    for (int t = 0; t < 4; ++t) E[t] = __builtin_amdgcn_alignbyte(D[t + 1], D[t], o & 3u);
    uint32_t c[14];
#pragma unroll
    for (int i = 0; i < 14; ++i) c[i] = lut[(E[i >> 2] >> (8 * (i & 3))) & 0xFFu];
    // the fields of byte i at bits 10 i .. 10 i + 9 of a 160-bit string
    uint32_t W[5];
    W[0] = c[0] | (c[1] << 10) | (c[2] << 20) | (c[3] << 30);
    W[1] = (c[3] >> 2) | (c[4] << 8) | (c[5] << 18) | (c[6] << 28);
    W[2] = (c[6] >> 4) | (c[7] << 6) | (c[8] << 16) | (c[9] << 26);
    W[3] = (c[9] >> 6) | (c[10] << 4) | (c[11] << 14) | (c[12] << 24);
    W[4] = (c[12] >> 8) | (c[13] << 2);
    u32x4 O;
#pragma unroll
    for (int t = 0; t < 4; ++t) O[t] = __builtin_amdgcn_alignbit(W[t + 1], W[t], sh);
    wbo[r] = to_b_order(O);
    const uint32_t sc = *reinterpret_cast<const uint32_t*>(smem + sdst(rd) + s_rd + 64 * r);
    s2o[r] = active ? (sc | (sc << 16)) : 0u;
  };
  auto read_w = [&](int rd, u32x4* wbo, uint32_t* s2o) {
    if constexpr (T1) {
#pragma unroll
      for (int r = 0; r < NR; ++r) read_w_row(rd, r, wbo, s2o);
    } else {
      const bool active = rd * KG + wk < nb;
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        wbo[r] = to_b_order(*reinterpret_cast<const u32x4*>(smem + wdst(rd) + w_rd + r * 1024));
        const uint32_t sc = *reinterpret_cast<const uint32_t*>(smem + sdst(rd) + s_rd + 64 * r);
        s2o[r] = active ? (sc | (sc << 16)) : 0u;
      }
    }
  };

  u32x4 wb[NR], wnx[NR];
  uint32_t s2[NR], s2n[NR];
  half8 Bc[NR];  // B operands of the coming stage's first step

#pragma unroll
  for (int rd = 0; rd < G::WD; ++rd) issue_w(rd);
#pragma unroll
  for (int s = 0; s < G::XS - 1; ++s) issue(s < S ? s : S - 1);
  // The wave's own round-0 weights (its oldest DMA) must have landed.
  mem_clobber();
  __builtin_amdgcn_s_waitcnt(vmcnt_imm((G::WD - 1) * kWIssue + (G::XS - 1) * G::kPer));
  mem_clobber();
  read_w(0, wb, s2);
#pragma unroll
  for (int r = 0; r < NR; ++r) Bc[r] = operand(H0{}, wb[r][0], s2[r]);

  for (int rd = 0; rd < rounds; ++rd) {
    sfor<0, 4>([&](auto cc) {
      constexpr int ch = decltype(cc)::value;
      const int s = 4 * rd + ch;
      // Stage s's DMA came XS - 1 iterations ago and is the last DMA of its
      // iteration; younger are the activation DMAs of the XS - 2 iterations
      // after it and the weight/scale DMA of those among them with ch = WCH
      // (issued first in its iteration).  Round rd + 1's weights, read at
      // ch = 3, are older than stage 4 rd + 3's DMA (XS <= 4 WD - WCH).
      mem_clobber();
      if (rd == 0)
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(vm_younger(G::XS, G::kPer, kWIssue, ch, true, G::WCH)));
      else
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(vm_younger(G::XS, G::kPer, kWIssue, ch, false, G::WCH)));
      __builtin_amdgcn_s_barrier();
      mem_clobber();
      const unsigned char* base = smem + (uint32_t)(s % G::XS) * G::kStage + wk * G::kChunk;
      half8 A[2][MT];
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < MT; ++i)
          A[h][i] = *reinterpret_cast<const half8*>(base + (a_off0 ^ (64u * h)) + 2048 * i);
      if constexpr (T1) {
        // the next round's row groups, each in its own stage of this round
        sfor<0, NR>([&](auto rr) {
          constexpr int r = decltype(rr)::value;
          if constexpr (G::wch_of(r) == ch) read_w_row(rd + 1, r, wnx, s2n);
        });
      } else if constexpr (ch == 3) {
        read_w(rd + 1, wnx, s2n);  // stale refill past the end
      }
      // all LDS reads of the stage are in flight before any of them is used
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (ch == G::WCH) issue_w(rd + G::WD);  // its slot held round rd, read
      // at ch = 3 of the round before
      {
        const int sn = s + G::XS - 1;
        issue(sn < S ? sn : S - 1);  // past the end: a harmless refill
      }
      __builtin_amdgcn_sched_barrier(0);
      // step 0 with the operands decoded one stage earlier, while step 1's
      // operands are decoded; then step 1 while the next stage's step 0 is
      half8 B1[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) B1[r] = operand(H1{}, wb[r][ch], s2[r]);
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          if constexpr (SB)
            C[i][r] = mfma16(A[0][i], Bc[r], C[i][r]);
          else if constexpr (ch == 0)  // a round's first product starts the block's sum
            Cb[i][r] = mfma16(A[0][i], Bc[r], float4v{0.f, 0.f, 0.f, 0.f});
          else
            Cb[i][r] = mfma16(A[0][i], Bc[r], Cb[i][r]);
        }
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if constexpr (ch < 3)
          Bc[r] = operand(H0{}, wb[r][ch + 1], s2[r]);
        else
          Bc[r] = operand(H0{}, wnx[r][0], s2n[r]);
      }
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          if constexpr (SB)
            C[i][r] = mfma16(A[1][i], B1[r], C[i][r]);
          else
            Cb[i][r] = mfma16(A[1][i], B1[r], Cb[i][r]);
        }
      if constexpr (ch == 3) {
        // the block's scale (0 for a k-group without a block this round)
        if constexpr (!SB) {
#pragma unroll
          for (int r = 0; r < NR; ++r) {
            const float sf = h2f((uint16_t)(s2[r] & 0xffffu));
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
              for (int e = 0; e < 4; ++e)
                C[i][r][e] = __builtin_fmaf(sf, Cb[i][r][e], C[i][r][e]);
          }
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          wb[r] = wnx[r];
          s2[r] = s2n[r];
        }
      }
      // Issue order: one MFMA, then up to four decode instructions, so the
      // matrix core and the vector ALU work side by side.
      sfor<0, 2 * MT * NR>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
      });
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
  // The k-group sums in fp16, row-major in LDS after the partial tiles (rows
  // BN + 8 halves apart, so the four rows of a store instruction fall in
  // different banks), then written out by every wave in 16-byte row chunks
  // (the MFMA layout would store 2 bytes per lane, 32 bytes per row).
  constexpr int kRowH = G::BN + 8;
  uint16_t* stg = reinterpret_cast<uint16_t*>(smem + G::kRed);
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int r = 0; r < NR; ++r) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float sum = C[i][r][e];
#pragma unroll
          for (int c = 1; c < KG; ++c)
            sum += red[((c - 1) * NG + wn) * kTile + ((i * NR + r) * 4 + e) * 64 + lane];
          stg[(16 * i + 4 * g + e) * kRowH + wn * G::BNW + 16 * r + li] = f2h_bits(sum);
        }
        __builtin_amdgcn_sched_barrier(0);  // one tile's partial sums at a time
      }
    }
  }
  __syncthreads();
  constexpr int kChunksRow = G::BN / 8;
  static_assert((kChunksRow & (kChunksRow - 1)) == 0, "row chunks: a power of two");
  const bool vec = (N & 7) == 0;  // rows start 16-byte aligned
  for (int c = threadIdx.x; c < G::BM * kChunksRow; c += 64 * G::WV) {
    const int row = c / kChunksRow;
    const int n0 = n_base + 8 * (c % kChunksRow);
    const int m = m_base + row;
    if (m >= M || n0 >= N) continue;
    const uint16_t* src = stg + row * kRowH + (n0 - n_base);
    uint16_t* dst = Y + (size_t)m * N + n0;
    if (vec) {
      *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
    } else {
      for (int j = 0; j < 8 && n0 + j < N; ++j) dst[j] = src[j];
    }
  }
}

// The 2-bit (TQ2) product.
template <int MT, int NR, int NG, int KG>
__global__ __launch_bounds__(64 * NG * KG, 8 / (NG * KG)) void tq2_tiled_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K,
    int n_tiles, int m_tiles, int m_outer) {
  tiled_body<MT, NR, NG, KG, false, false>(X, qs, 0, scales, Y, M, N, K, n_tiles, m_tiles,
                                           m_outer);
}

// The 1.6-bit (TQ1) product on the same tiles, the weights decoded from TQ1
// bytes through the LDS table (no 2-bit copy of the matrix anywhere).
template <int MT, int NR, int NG, int KG, bool SB>
__global__ __launch_bounds__(64 * NG * KG, 8 / (NG * KG)) void tq1_tab_tiled_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs, int ldq,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K,
    int n_tiles, int m_tiles, int m_outer) {
  tiled_body<MT, NR, NG, KG, true, SB>(X, qs, ldq, scales, Y, M, N, K, n_tiles, m_tiles,
                                       m_outer);
}

// From this many activation tiles on, the m-major order (see the kernel).
constexpr int64_t kMOuterTiles = 4;

// The scale goes into the operands where the wave tile is large (the second
// accumulator set would not fit beside the table decode).
constexpr bool t1_scale_in_b(int mt, int nr) { return mt * nr >= 16; }

template <int MT, int NR, int NG, int KG, bool T1 = false>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
  using G = TileGeom<MT, NR, NG, KG, T1>;
  constexpr bool SB = T1 && t1_scale_in_b(MT, NR);
  const void* fn;
  if constexpr (T1)
    fn = reinterpret_cast<const void*>(tq1_tab_tiled_kernel<MT, NR, NG, KG, SB>);
  else
    fn = reinterpret_cast<const void*>(tq2_tiled_kernel<MT, NR, NG, KG>);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = lds_limit_once(fn, G::kLds, lds_set);
  if (e != hipSuccess) return e;
  const int64_t n_tiles = (a.N + G::BN - 1) / G::BN;
  const int64_t m_tiles = (a.M + G::BM - 1) / G::BM;
  const int64_t groups = (n_tiles + 7) / 8;
  const int64_t wgs = groups * 8 * m_tiles;
  if (wgs > 0x7fffffff) return hipErrorInvalidConfiguration;
  const int m_outer = m_tiles >= kMOuterTiles ? 1 : 0;
  if constexpr (T1)
    hipLaunchKernelGGL((tq1_tab_tiled_kernel<MT, NR, NG, KG, SB>), dim3((unsigned)wgs),
                       dim3(64 * G::WV), G::kLds, stream, static_cast<const uint16_t*>(a.X),
                       static_cast<const uint8_t*>(a.qs), (int)a.ldq,
                       static_cast<const uint16_t*>(a.scales), static_cast<uint16_t*>(a.Y),
                       (int)a.M, (int)a.N, (int)a.K, (int)n_tiles, (int)m_tiles, m_outer);
  else
    hipLaunchKernelGGL((tq2_tiled_kernel<MT, NR, NG, KG>), dim3((unsigned)wgs), dim3(64 * G::WV),
                       G::kLds, stream, static_cast<const uint16_t*>(a.X),
                       static_cast<const uint8_t*>(a.qs), static_cast<const uint16_t*>(a.scales),
                       static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, (int)n_tiles,
                       (int)m_tiles, m_outer);
  return hipGetLastError();
}

}  // namespace

// Tile choice (measured at K = 8192, N = 8192 and 28672, M = 17..128).  A
// stage costs a wave about the same whatever the tile, so what counts is the
// number of stages a workgroup runs (fewer with more k-groups) and how many
// compute units have one.  The 8-wave tiles (one workgroup per compute unit,
// half the activation re-reads) win once they alone fill about 85% of the
// compute units: 128 x 128 (4 row groups of 32 x 2 k-groups: each decoded
// weight feeds 8 MFMAs, the weights are read once) past M = 64, 64 x 128
// (2 x 4) up to M = 64.  Below that 4-wave tiles of 1 row group x 4 k-groups,
// 64 weight rows wide, with 32 activation rows up to M = 64 so that the
// activation-row tiles spread over more compute units; 32 weight rows wide
// when 64 would leave compute units idle (M <= 32: 18.4 against 23.1 us at
// N = 8192); past M = 64 the 8-wave 64 x 64 tile (2 row groups of 32 x 4
// k-groups: 32.0 against 34.6 us at N = 8192, M = 128).  When the 32 x 32
// or 32 x 64 tiles number no more than the compute units (N <= 8192 on 256
// CUs), they run as 8 k-groups of one wave each instead of 4, twice the
// waves per SIMD on the same workgroups (M = 32, N = 8192: 16.6 against
// 18.4 us; M = 17: 15.7 against 18.0 us; M = 64: 22.8 against 23.9 us);
// with more tiles than compute units the 8-wave workgroup (one per CU)
// needs two passes and loses.
TiledShape tiled_shape(int64_t M, int64_t N) {
  const int64_t cus = device_cus();
  auto fills = [&](const TiledShape& t) {
    const int64_t bm = 16 * t.mt;
    const int64_t bn = 16 * t.nr * t.ng;
    const int64_t wgs = ((N + bn - 1) / bn) * ((M + bm - 1) / bm);
    return 20 * wgs >= 17 * cus;
  };
  if (M > 32) {
    const bool wide = M > 64;
    const TiledShape t8 = wide ? TiledShape{8, 2, 4, 2} : TiledShape{4, 4, 2, 4};
    if (fills(t8)) return t8;
    if (wide) return TiledShape{4, 2, 2, 4};
    // 32 x 64 tiles as 8 one-wave k-groups when they fit one per CU (M = 64,
    // N = 8192: 22.8 against 23.9 us; M = 33: 21.8 against 23.5 us)
    const int64_t wgs = ((N + 63) / 64) * ((M + 31) / 32);
    return wgs <= cus ? TiledShape{2, 4, 1, 8} : TiledShape{2, 4, 1, 4};
  }
  const TiledShape t{2, 4, 1, 4};
  if (fills(t)) return t;
  const int64_t narrow_wgs = ((N + 31) / 32) * ((M + 31) / 32);
  return narrow_wgs <= cus ? TiledShape{2, 2, 1, 8} : TiledShape{2, 2, 1, 4};
}

template <int MT, bool T1>
hipError_t launch_mt(const TiledShape& t, const GemmArgs& a, hipStream_t stream) {
  if constexpr (MT == 2) {
    if (t.kg == 8) return t.nr == 2 ? launch_tiled<2, 2, 1, 8, T1>(a, stream)
                                    : launch_tiled<2, 4, 1, 8, T1>(a, stream);
  }
  if (t.nr == 2) return t.ng == 2 ? launch_tiled<MT, 2, 2, 4, T1>(a, stream)
                                  : launch_tiled<MT, 2, 1, 4, T1>(a, stream);
  if (t.ng == 4) return launch_tiled<MT, 4, 4, 2, T1>(a, stream);
  if (t.kg == 4) return t.ng == 2 ? launch_tiled<MT, 4, 2, 4, T1>(a, stream)
                                  : launch_tiled<MT, 4, 1, 4, T1>(a, stream);
  return launch_tiled<MT, 4, 2, 2, T1>(a, stream);
}

bool tiled_compiled(const TiledShape& t) {
  if (t.mt == 8) return t.nr == 2 && t.ng == 4 && t.kg == 2;
  if (t.mt != 2 && t.mt != 4) return false;
  if (t.kg == 8) return t.mt == 2 && t.ng == 1 && (t.nr == 2 || t.nr == 4);
  if (t.nr == 2) return t.kg == 4 && (t.ng == 1 || t.ng == 2);
  if (t.nr != 4) return false;
  return (t.ng == 4 && t.kg == 2) || (t.ng == 2 && t.kg == 4) || (t.ng == 2 && t.kg == 2) ||
         (t.ng == 1 && t.kg == 4);
}

hipError_t launch_tq2_tiled_shape(const TiledShape& t, const GemmArgs& a, hipStream_t stream) {
  if (t.mt == 8) return launch_tiled<8, 2, 4, 2>(a, stream);
  return t.mt == 2 ? launch_mt<2, false>(t, a, stream) : launch_mt<4, false>(t, a, stream);
}

hipError_t launch_tq2_tiled(const GemmArgs& a, hipStream_t stream) {
  return launch_tq2_tiled_shape(tiled_shape(a.M, a.N), a, stream);
}

bool tq1_tab_scale_in_b(const TiledShape& t) { return t1_scale_in_b(t.mt, t.nr); }

// The 1.6-bit tiles: those of the 2-bit product, except that where that takes
// 32 activation rows x 64 weight rows past M = 32 (fewer compute units than
// its 64 x 128 tiles need) the table decode prefers 64 x 32 tiles, which
// decode each weight once per 64 activation rows (K = 8192, N = 8192, M = 64:
// 26.7 against 32.2 us).
TiledShape tq1_tab_shape(int64_t M, int64_t N) {
  const TiledShape t = tiled_shape(M, N);
  if (M > 32 && t.mt == 2 && t.nr == 4) return TiledShape{4, 2, 1, 4};
  return t;
}

hipError_t launch_tq1_tab_shape(const TiledShape& t, const GemmArgs& a, hipStream_t stream) {
  if (t.mt == 8) return launch_tiled<8, 2, 4, 2, true>(a, stream);
  return t.mt == 2 ? launch_mt<2, true>(t, a, stream) : launch_mt<4, true>(t, a, stream);
}

hipError_t launch_tq1_tab(const GemmArgs& a, hipStream_t stream) {
  // 32-bit row offsets within a tile: larger row strides take the skinny kernel
  if (a.ldq > kTq1TabMaxLdq) return launch_tq1_skinny(a, stream);
  return launch_tq1_tab_shape(tq1_tab_shape(a.M, a.N), a, stream);
}

}  // namespace tq
