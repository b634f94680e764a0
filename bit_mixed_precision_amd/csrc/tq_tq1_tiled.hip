// Tiled MFMA kernel for 1.6-bit weights and M > 16: Y = X (s . T)^T with T
// packed five trits per byte.
//
// Follows the project page "Scaling Laws and Efficient Inference for Ternary
// Language Models": "The model" (step 3) for the product, "1.6 bits per
// weight" for the code and its multiply-by-3 decoder, "Fast inference on
// CPUs" for the 256-weight scale block, "TriRun: ternary inference on GPUs"
// for FP32 accumulation and FP16 output.  MI355X design:
//
//  * a workgroup of NW x KG waves owns a tile of 16 MT activation rows x
//    16 NW weight rows; wave (wn, wk) decodes weight rows 16 wn .. 16 wn + 15
//    on the 32-byte spans (160 weights) u = wk, wk + KG, ... and feeds every
//    decoded operand to the MT MFMAs of its activation row tiles, so a weight
//    is decoded once per tile; the KG k-groups' partial tiles meet in LDS at
//    the end;
//  * a stage is one span per k-group.  Its activations are staged in LDS in
//    the decoder's weight order, one unit of 40 activations (a row's lane
//    group) per lane; stages flow through two LDS slots with one barrier per
//    stage: while stage s is multiplied, stage s + 1 is written from registers
//    and stage s + XP is loaded, so a load has XP - 1 stages of work to land;
//  * block scales: a span holds at most one 256-weight boundary; it adds
//    s_a C_a + (s_b - s_a) C_b, where C_b takes, per lane group, zeros (the
//    groups before the boundary), a masked copy of the one unit that holds
//    it, or the plain activations (the groups after it).  Only that unit is
//    stored twice, and only spans with a boundary run the C_b MFMAs;
//  * weights (8 bytes per lane per span) and the span's two block scales come
//    through a ring of D register buffers, D stages ahead; every load in the
//    loop is unconditional (past the end they re-read valid data), so the
//    compiler's count of loads in flight stays exact;
//  * fp32 accumulation across all of K; one fp32 -> fp16 rounding writes Y.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"
#include "tq_tq1.h"

namespace tq {
namespace {

template <int I, int N, class F>
__device__ __forceinline__ void tfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    tfor<I + 1, N>(f);
  }
}

__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes are done
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int MT, int NW, int KG>
struct T1Geom {
  static constexpr int BM = 16 * MT;
  static constexpr int BN = 16 * NW;
  static constexpr int WV = NW * KG;  // waves per workgroup
  // one activation row of one span: 4 plain units + the masked boundary unit,
  // 80 bytes each; 400 = 16 x 25 spreads 16 rows over distinct bank groups
  static constexpr int kRow = 5 * 80;
  static constexpr int kMasked = 4 * 80;
  static constexpr int kSpan = BM * kRow;
  static constexpr int kSlot = KG * kSpan;
  static constexpr int kZero = 2 * kSlot;  // 80 zero bytes
  static constexpr int kRing = kZero + 80;
  static constexpr int kRed = (KG - 1) * NW * MT * 1024;  // partial tiles of k-groups 1..KG-1
  static constexpr int kLds = kRing > kRed ? kRing : kRed;
  // staging units (span, activation row, lane group) per stage: 64 MT KG,
  // spread over the 64 WV lanes
  static constexpr int UX = MT > NW ? MT / NW : 1;
  static_assert(MT <= NW || MT % NW == 0, "staging units split evenly over the waves");
};

// Workgroup L runs tile (n_tile, m_tile) with n_tile = 8 (L / 8 / m_tiles) +
// L % 8 and m_tile = (L / 8) % m_tiles, as the TQ2 tiled kernel: the m tiles
// of one weight tile run back to back on one XCD, so its weights come from
// HBM once.
template <int MT, int NW, int KG, int D, int XP>
__global__ __launch_bounds__(64 * NW * KG) void tq1_tiled_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs, int ldq,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K,
    int n_tiles, int m_tiles) {
  using G = T1Geom<MT, NW, KG>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int L = blockIdx.x;
  const int m_tile = (L >> 3) % m_tiles;
  const int n_tile = ((L >> 3) / m_tiles) * 8 + (L & 7);
  if (n_tile >= n_tiles) return;  // whole workgroup
  const int n_base = n_tile * G::BN;
  const int m_base = m_tile * G::BM;
  const int mrows = min(G::BM, M - m_base);

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wn = wave % NW;
  const int wk = wave / NW;
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int groups = (K + 4) / 5;
  const int nu = (groups + 31) / 32;         // spans holding real bytes
  const int nst = (nu + KG - 1) / KG;        // stages
  const int nsteps = (nst + D - 1) / D * D;  // whole unrolled blocks

  Tq1Decoder dc;
  dc.init();

  if (threadIdx.x < 20) reinterpret_cast<uint32_t*>(smem + G::kZero)[threadIdx.x] = 0u;

  // This lane's weight row (rows past N read row n_base; never written).
  const int n = n_base + 16 * wn + li;
  const int nr = n < N ? n : n_base;
  const uint8_t* wrow = qs + (size_t)nr * ldq + 8 * g;
  const uint16_t* srow = scales + (size_t)nr * nb;

  // Staging unit q = threadIdx.x + 64 WV x (x < UX): span c = q / (4 BM) of
  // the stage, activation row m = q / 4 % BM, lane group q % 4.  Waves past
  // the units load a valid dummy unit and store nothing (wave-uniform).
  size_t xrow_off[G::UX];
  int xunit_c[G::UX], xunit_g[G::UX], xunit_dst[G::UX];
  bool xunit_on[G::UX];
#pragma unroll
  for (int x = 0; x < G::UX; ++x) {
    const int q = threadIdx.x + 64 * G::WV * x;
    xunit_on[x] = q < 64 * MT * KG;
    const int qq = xunit_on[x] ? q : 0;
    const int m = (qq >> 2) % G::BM;
    xunit_c[x] = qq / (4 * G::BM);
    xunit_g[x] = qq & 3;
    xunit_dst[x] = xunit_c[x] * G::kSpan + m * G::kRow;
    const int mr = m < mrows ? m : mrows - 1;
    xrow_off[x] = (size_t)(m_base + mr) * K;
  }
  // Loads the 40 activations of each unit of stage s; chunks past K read the
  // row start (valid data) and are zeroed when stored.
  auto xload = [&](uint32_t (&e)[G::UX][20], int s) {
#pragma unroll
    for (int x = 0; x < G::UX; ++x) {
      int u = KG * s + xunit_c[x];
      u = u < nu ? u : nu - 1;
      const int k0 = 160 * u + 40 * xunit_g[x];
#pragma unroll
      for (int c = 0; c < 5; ++c) {
        const int kk = k0 + 8 * c;
        const u32x4 v = *reinterpret_cast<const u32x4*>(X + xrow_off[x] + (kk + 8 <= K ? kk : 0));
#pragma unroll
        for (int t = 0; t < 4; ++t) e[x][4 * c + t] = v[t];
      }
    }
  };
  // lim: the span's next block boundary relative to its first weight; the
  // span holds it when lim < 160, in the unit of lane group lim / 40.
  auto span_lim = [&](int u) { return ((160 * u) / 256 + 1) * 256 - 160 * u; };
  auto xstore = [&](uint32_t (&e)[G::UX][20], int s, int slot) {
#pragma unroll
    for (int x = 0; x < G::UX; ++x) {
      if (xunit_on[x]) {  // wave-uniform
        int u = KG * s + xunit_c[x];
        u = u < nu ? u : nu - 1;  // the span is the same for the whole wave
        if (160 * u + 160 > K) {  // the last span: zero the chunks past K
          const int k0 = 160 * u + 40 * xunit_g[x];
#pragma unroll
          for (int c = 0; c < 5; ++c)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              if (k0 + 8 * c + 8 > K) e[x][4 * c + t] = 0u;
        }
        const int lim = span_lim(u);
        unsigned char* row = smem + slot * G::kSlot + xunit_dst[x];
        tq1_store_plain(row + 80 * xunit_g[x], e[x]);
        if (lim < 160 && xunit_g[x] == lim / 40)  // the unit that holds the boundary
          tq1_store_masked_uniform(row + G::kMasked, e[x], lim - 40 * xunit_g[x]);
      }
    }
  };

  // Row offset of activation tile i, lane (li, g): row 16 i + li of the
  // wave's span (rows past M read the last staged row; never written).
  uint32_t a_row[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    const int m = 16 * i + li < mrows ? 16 * i + li : mrows - 1;
    a_row[i] = (uint32_t)(wk * G::kSpan + m * G::kRow);
  }

  u32x2 wbuf[D];
  uint32_t sbuf[D];  // (s_a, s_b) of the span, fp16 bits
  auto wload = [&](int d, int s) {
    int u = KG * s + wk;
    u = u < nu ? u : nu - 1;
    // the last span may reach past the row's ldq bytes; those bytes only hold
    // weights k >= K, whose activations are zero, so read the row start instead
    const int off = (32 * u + 8 * g + 8 <= ldq) ? 32 * u : 0;
    wbuf[d] = *reinterpret_cast<const u32x2*>(wrow + off);
    const int ba = (160 * u) >> 8;
    const int bb = ba + 1 < nb ? ba + 1 : ba;
    sbuf[d] = (uint32_t)srow[ba] | ((uint32_t)srow[bb] << 16);
    __builtin_amdgcn_sched_barrier(0);
  };

  float4v acc[MT];
#pragma unroll
  for (int i = 0; i < MT; ++i) acc[i] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int d, int u, int slot) {
    const u32x2 w = wbuf[d];
    // bytes (0, 2), (1, 3), (4, 6), (5, 7) of the lane's 8 bytes, one per half
    uint32_t q[4] = {w[0] & 0x00FF00FFu, (w[0] >> 8) & 0x00FF00FFu, w[1] & 0x00FF00FFu,
                     (w[1] >> 8) & 0x00FF00FFu};
    const float sa = h2f((uint16_t)(sbuf[d] & 0xFFFFu));
    const int lim = span_lim(u);
    // A span holds a block boundary only when the next block starts before it ends.
    const bool split = lim < 160 && (160 * u) / 256 + 1 < nb;  // wave-uniform
    const uint32_t xs = (uint32_t)(slot * G::kSlot);
    const uint32_t plain = xs + 80 * g;
    // C_b operand source of this lane group: zeros (before the boundary), the
    // masked unit (holding it), or the plain activations (after it)
    const int gs = lim / 40;
    const bool zero_b = g < gs;
    const uint32_t bsrc = zero_b ? (uint32_t)G::kZero : (g == gs ? xs + G::kMasked : plain);
    uint32_t brow[MT];
#pragma unroll
    for (int i = 0; i < MT; ++i) brow[i] = zero_b ? 0u : a_row[i];
    auto run = [&](auto with_b) {
      constexpr bool WB = decltype(with_b)::value;
      float4v Ca[MT], Cb[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i) Ca[i] = Cb[i] = float4v{0.f, 0.f, 0.f, 0.f};
      tfor<0, 5>([&](auto jj) {
        constexpr int j = decltype(jj)::value;
        u32x4 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = dc.step(q[r]);
        const half8 B = __builtin_bit_cast(half8, b);
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const half8 A = *reinterpret_cast<const half8*>(smem + plain + a_row[i] + 16 * j);
          Ca[i] = mfma16(A, B, Ca[i]);
          if constexpr (WB) {
            const half8 Am = *reinterpret_cast<const half8*>(smem + bsrc + brow[i] + 16 * j);
            Cb[i] = mfma16(Am, B, Cb[i]);
          }
        }
      });
      if constexpr (WB) {
        const float sb = h2f((uint16_t)(sbuf[d] >> 16));
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] += sa * Ca[i] + (sb - sa) * Cb[i];
      } else {
#pragma unroll
        for (int i = 0; i < MT; ++i) acc[i] += sa * Ca[i];
      }
    };
    if (split)
      run(std::true_type{});
    else
      run(std::false_type{});
  };

  // Prologue: stage 0 staged, stages 1 .. XP - 1 loaded (register slot
  // (s - 1) % (XP - 1) holds stage s), weights of stages 0 .. D - 1 in flight.
  constexpr int XR = XP - 1;
  static_assert(XR >= 1 && D % XR == 0, "one unrolled step block covers both rings");
  uint32_t e[XR][G::UX][20];
  xload(e[0], 0);
  tfor<0, D>([&](auto dd) { wload(decltype(dd)::value, decltype(dd)::value); });
  xstore(e[0], 0, 0);
  tfor<0, XR>([&](auto rr) { xload(e[decltype(rr)::value], 1 + decltype(rr)::value); });
  bare_barrier();

  for (int s0 = 0; s0 < nsteps; s0 += D) {
    tfor<0, D>([&](auto dd) {
      constexpr int d = decltype(dd)::value;
      constexpr int r = d % XR;  // register slot of stage s + 1 (s0 is a multiple of XR)
      const int s = s0 + d;
      const int u = KG * s + wk;
      if (u < nu) compute(d, u, s & 1);  // wave-uniform
      // LDS slot (s + 1) & 1 held stage s - 1, which every wave finished before
      // the last barrier; past the end these refill with valid data
      xstore(e[r], s + 1, (s + 1) & 1);
      xload(e[r], s + XP);
      wload(d, s + D);
      bare_barrier();
    });
  }

  // Partial tiles of k-groups 1 .. KG - 1 meet k-group 0's through LDS (the
  // ring is free: every wave passed the last barrier).
  float* red = reinterpret_cast<float*>(smem);
  if constexpr (KG > 1) {
    if (wk > 0) {
#pragma unroll
      for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          red[(((wk - 1) * NW + wn) * MT + i) * 256 + r * 64 + lane] = acc[i][r];
    }
    __syncthreads();
  }
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float sum = acc[i][r];
#pragma unroll
        for (int c = 1; c < KG; ++c)
          sum += red[(((c - 1) * NW + wn) * MT + i) * 256 + r * 64 + lane];
        const int m = m_base + 16 * i + 4 * g + r;
        if (m < M && n < N) Y[(size_t)m * N + n] = f2h_bits(sum);
      }
    }
  }
}

constexpr int kDepthT1 = 4;  // weight ring: stages ahead

// Activations are loaded this many stages ahead; 16-wave workgroups keep one
// stage in registers (their register budget is 128 per lane).
constexpr int xahead(int nw, int kg) { return nw * kg >= 16 ? 2 : 3; }

template <int MT, int NW, int KG>
hipError_t launch_t1(const GemmArgs& a, hipStream_t stream) {
  using G = T1Geom<MT, NW, KG>;
  constexpr int D = kDepthT1;
  constexpr int XP = xahead(NW, KG);
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = lds_limit_once(
      reinterpret_cast<const void*>(tq1_tiled_kernel<MT, NW, KG, D, XP>), G::kLds, lds_set);
  if (e != hipSuccess) return e;
  const int64_t n_tiles = (a.N + G::BN - 1) / G::BN;
  const int64_t m_tiles = (a.M + G::BM - 1) / G::BM;
  // grid: n tiles rounded up to whole groups of 8 (one per XCD)
  const int64_t grid = (n_tiles + 7) / 8 * 8 * m_tiles;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((tq1_tiled_kernel<MT, NW, KG, D, XP>), dim3((unsigned)grid),
                     dim3(64 * G::WV), G::kLds, stream, static_cast<const uint16_t*>(a.X),
                     static_cast<const uint8_t*>(a.qs), (int)a.ldq,
                     static_cast<const uint16_t*>(a.scales), static_cast<uint16_t*>(a.Y),
                     (int)a.M, (int)a.N, (int)a.K, (int)n_tiles, (int)m_tiles);
  return hipGetLastError();
}

}  // namespace

int tq1_tiled_depth() { return kDepthT1; }

int tq1_tiled_xahead(const Tq1TiledShape& t) { return xahead(t.nw, t.kg); }

bool tq1_tiled_compiled(const Tq1TiledShape& t) {
  const int m = t.mt, w = t.nw, k = t.kg;
  return (m == 1 && w == 4 && k == 4) || (m == 2 && w == 4 && (k == 2 || k == 4)) ||
         (m == 4 && w == 4 && (k == 1 || k == 2)) || (m == 2 && w == 8 && k == 2);
}

// Measured at K = 8192: 32 activation rows per tile (each weight decoded
// twice at M = 64) beat 64-row tiles up to M = 64, whose 128 workgroups at
// N = 8192 leave half of the CUs idle.
Tq1TiledShape tq1_tiled_shape(int64_t M, int64_t N) {
  (void)N;
  if (M <= 64) return Tq1TiledShape{2, 4, 2};
  return Tq1TiledShape{4, 4, 2};
}

bool tq1_prefers_tiled(int64_t M, int64_t N) {
  // At K = 8192 the tiled kernel wins from M = 64 at N = 8192 (46 vs 68 us)
  // but loses at N = 28672 to the skinny kernel, whose 16-wave workgroups
  // stream more rows per CU.
  return M >= 48 && N <= 16384;
}

hipError_t launch_tq1_tiled_shape(const Tq1TiledShape& t, const GemmArgs& a, hipStream_t stream) {
  const int m = t.mt, w = t.nw, k = t.kg;
  if (m == 1 && w == 4 && k == 4) return launch_t1<1, 4, 4>(a, stream);
  if (m == 2 && w == 4 && k == 2) return launch_t1<2, 4, 2>(a, stream);
  if (m == 2 && w == 4 && k == 4) return launch_t1<2, 4, 4>(a, stream);
  if (m == 4 && w == 4 && k == 1) return launch_t1<4, 4, 1>(a, stream);
  if (m == 4 && w == 4 && k == 2) return launch_t1<4, 4, 2>(a, stream);
  if (m == 2 && w == 8 && k == 2) return launch_t1<2, 8, 2>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_tq1_tiled(const GemmArgs& a, hipStream_t stream) {
  return launch_tq1_tiled_shape(tq1_tiled_shape(a.M, a.N), a, stream);
}

}  // namespace tq
