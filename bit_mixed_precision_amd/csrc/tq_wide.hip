// Wide-tile MFMA kernel for batch sizes past the skinny kernel's range:
// Y = X (s . T)^T for TQ2 weights on v_mfma_f32_32x32x16_f16.
//
// Follows the project page "Scaling Laws and Efficient Inference for Ternary
// Language Models": "The model" (step 3), "2 bits per weight" (decoder),
// "Fast inference on CPUs" (256-weight scale block), "TriRun: ternary
// inference on GPUs" (FP32 accumulation, FP16 output).  MI355X design:
//
//  * a workgroup of 4 waves, NG weight-row groups x KG k-groups, owns a
//    BM x BN output tile (BM = 32 MT activation rows, BN = 32 NT NG weight
//    rows); wave (ng, kg) computes BM x 32 NT of it on MT x NT tiles of
//    v_mfma_f32_32x32x16_f16 over the k-group's quarter or half of every
//    stage, and the k-groups' partial tiles meet in LDS at the end.  A 32 x 32
//    MFMA reads 1 KB of A operands for 32 k of 32 weight rows where the
//    16 x 16 x 32 form needs 1 KB for 16 rows, so the activation reads from
//    LDS per weight are half as many;
//  * a stage is 64 KG consecutive k (inside one 256-weight block, so one scale
//    per row): the activation tile (BM x 64 KG, row-major, 16-byte pieces of
//    row r at slot piece ^ (r mod 16) so the 32 rows an A-operand read touches
//    fall in distinct banks), the packed weights (BN rows x 16 KG bytes) and
//    the rows' scales; staged by 16-byte buffer loads (rows past M or N read
//    as zero) two stages ahead in registers, two LDS buffers, one barrier per
//    stage;
//  * each lane reads its row's 16 packed bytes of the k-group chunk once per
//    stage and decodes a B operand (8 consecutive weights, 2 bytes) per 16-k
//    step with the natural-order decoder (v_perm_b32, v_and_or_b32 against the
//    fp16 exponent of 1024, v_pk_fma_f16, v_pk_mul_f16 by the block scale:
//    exact +-s or 0), which feeds MT MFMAs;
//  * workgroup ids are XCD-strided: XCD x runs a contiguous run of tiles
//    (weight-row tile major), so tiles sharing weight rows share that L2.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

typedef float float16v __attribute__((ext_vector_type(16)));

constexpr int kWideThreads = 256;
constexpr uint32_t kWRsrcFlags = 0x00020000u;  // raw buffer, 32-bit data
constexpr uint32_t kWOob = 0x80000000u;        // an offset past every range here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t wide_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, (int)n, (int)kWRsrcFlags);
}

template <int MT, int NT, int NG, int KG>
struct WideGeom {
  static_assert(NG * KG == 4, "a workgroup is 4 waves");
  static_assert(KG == 2 || KG == 4, "a stage of 64 KG k lies inside one 256-weight block");
  static constexpr int BM = 32 * MT;
  static constexpr int BN = 32 * NT * NG;
  static constexpr int SK = 64 * KG;                // k per stage
  static constexpr int XPitch = SK * 2;             // bytes per staged activation row
  static constexpr int XBytes = BM * XPitch;
  static constexpr int WPitch = SK / 4;             // packed bytes per staged weight row
  static constexpr int WBytes = BN * WPitch;
  static constexpr int SBytes = BN * 2;
  static constexpr int Stage = XBytes + WBytes + ((SBytes + 15) & ~15);
  static constexpr int XL = XBytes / 16 / kWideThreads;  // activation pieces per thread
  static constexpr int WPieces = WBytes / 16;            // weight pieces (<= threads)
  static_assert(XBytes % (16 * kWideThreads) == 0, "activation pieces split evenly");
  static_assert(WPieces <= kWideThreads && BN <= kWideThreads, "one weight piece per thread");
  static constexpr int Red = (KG - 1) * NG * MT * NT * 16 * 64 * 4;  // k-group partials
  static constexpr int Lds = 2 * Stage > Red ? 2 * Stage : Red;
  static_assert(Lds <= 160 * 1024, "fits the LDS of a compute unit");
};

template <int I, int N, class F>
__device__ __forceinline__ void wfor(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    wfor<I + 1, N>(f);
  }
}

template <int MT, int NT, int NG, int KG>
__global__ __launch_bounds__(kWideThreads) void tq2_wide_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K,
    int n_tiles, int tiles, int per_xcd) {
  using G = WideGeom<MT, NT, NG, KG>;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  const int tile = (b >> 3) + (b & 7) * per_xcd;
  if (tile >= tiles) return;  // workgroup-uniform: padding of the XCD-strided grid
  const int n0 = (tile % n_tiles) * G::BN;
  const int m0 = (tile / n_tiles) * G::BM;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int wn = wave % NG, wk = wave / NG;
  const int nb = K >> 8;
  const int steps = K / G::SK;

  const __amdgpu_buffer_rsrc_t rx = wide_rsrc(X, (uint32_t)((size_t)M * K * 2));
  const __amdgpu_buffer_rsrc_t rw = wide_rsrc(qs, (uint32_t)((size_t)N * (K >> 2)));
  const __amdgpu_buffer_rsrc_t rs = wide_rsrc(scales, (uint32_t)((size_t)N * nb * 2));

  // Staging roles.  Activation piece u = t + 256 j: row u / (8 KG), piece
  // u % (8 KG) of the stage's row chunk.  Weight piece t (t < WPieces): row
  // t / KG, 16-byte piece t % KG.  Scale: row t (t < BN).  Byte offsets of
  // stage 0; stage s adds 128 KG (activations), 16 KG (weights) or the block.
  uint32_t xoff[G::XL];
  int xslot[G::XL];
#pragma unroll
  for (int j = 0; j < G::XL; ++j) {
    const int u = t + kWideThreads * j;
    const int r = u / (8 * KG), c = u % (8 * KG);
    xoff[j] = m0 + r < M ? ((uint32_t)(m0 + r) * (uint32_t)K) * 2u + 16u * c : kWOob;
    xslot[j] = r * G::XPitch + ((c ^ (r & 15)) << 4);
  }
  const bool wl = t < G::WPieces;
  const int wr = t / KG, wc = t % KG;
  const uint32_t woff = wl && n0 + wr < N ? (uint32_t)(n0 + wr) * (uint32_t)(K >> 2) + 16u * wc
                                          : kWOob;
  const int wslot = G::XBytes + wr * G::WPitch + 16 * wc;
  const bool sl = t < G::BN;
  const uint32_t soff = sl && n0 + t < N ? (uint32_t)(n0 + t) * (uint32_t)nb * 2u : kWOob;
  const int sslot = G::XBytes + G::WBytes + 2 * t;

  struct Ring {
    u32x4 x[G::XL];
    u32x4 w;
    uint32_t s;
  };
  Ring ring[2];
  auto issue = [&](Ring& r, int s) {
#pragma unroll
    for (int j = 0; j < G::XL; ++j) {
      const uint32_t o = xoff[j] == kWOob ? kWOob : xoff[j] + (uint32_t)s * (2u * G::SK);
      r.x[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rx, o, 0, 0));
    }
    if (wl) {
      const uint32_t o = woff == kWOob ? kWOob : woff + (uint32_t)s * (uint32_t)(G::SK / 4);
      r.w = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rw, o, 0, 0));
    }
    if (sl) {
      const uint32_t o = soff == kWOob ? kWOob : soff + 2u * (uint32_t)((s * G::SK) >> 8);
      r.s = __builtin_amdgcn_raw_buffer_load_b16(rs, o, 0, 0);
    }
  };
  auto stage = [&](const Ring& r, int buf) {
    unsigned char* base = smem + buf * G::Stage;
#pragma unroll
    for (int j = 0; j < G::XL; ++j) *reinterpret_cast<u32x4*>(base + xslot[j]) = r.x[j];
    if (wl) *reinterpret_cast<u32x4*>(base + wslot) = r.w;
    if (sl) *reinterpret_cast<uint16_t*>(base + sslot) = (uint16_t)r.s;
  };

  // Operand roles.  A: m-tile i, 16-k step h, lane l reads row 32 i + l % 32,
  // piece 8 wk + 2 h + l / 32 of the stage row; (32 i + l % 32) % 16 = l % 16.
  int aoff[4];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    const int row = lane & 31;
    const int c = 8 * wk + 2 * h + (lane >> 5);
    aoff[h] = row * G::XPitch + ((c ^ (lane & 15)) << 4);
  }
  // B: n-tile j, lane l: weight row 32 (NT wn + j) + l % 32 of the tile, its
  // k-group's 16 bytes; step h takes dword h, byte pair l / 32.
  int boff[NT], scoff[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int row = 32 * (NT * wn + j) + (lane & 31);
    boff[j] = G::XBytes + row * G::WPitch + 16 * wk;
    scoff[j] = G::XBytes + G::WBytes + 2 * row;
  }
  const uint32_t bsel = (lane >> 5) ? 0x03020302u : 0x01000100u;
  NaturalConsts dc;
  dc.init();

  float16v acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[i][j] = float16v{};

  auto compute = [&](int buf) {
    const unsigned char* base = smem + buf * G::Stage;
    u32x4 wq[NT];
    uint32_t s2[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      wq[j] = *reinterpret_cast<const u32x4*>(base + boff[j]);
      const uint32_t sc = *reinterpret_cast<const uint16_t*>(base + scoff[j]);
      s2[j] = sc | (sc << 16);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      half8 A[MT];
#pragma unroll
      for (int i = 0; i < MT; ++i)
        A[i] = *reinterpret_cast<const half8*>(base + aoff[h] + i * 32 * G::XPitch);
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const half8 B = dc.operand_sel(wq[j][h], bsel, s2[j]);
#pragma unroll
        for (int i = 0; i < MT; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B, acc[i][j], 0, 0, 0);
      }
    }
  };

  // Stage s computes from LDS buffer s & 1, then stages step s + 1 (held in
  // ring slot (s + 1) & 1, loaded two stages earlier) into the other buffer,
  // whose reads (stage s - 1) ended before the previous barrier, and refills
  // that slot with stage s + 3.  Two stages per loop trip keep every slot and
  // buffer index a compile-time constant.
  auto step = [&](int s, auto parity) {
    constexpr int P = decltype(parity)::value;
    compute(P);
    if (s + 1 < steps) {
      stage(ring[P ^ 1], P ^ 1);
      if (s + 3 < steps) issue(ring[P ^ 1], s + 3);
    }
    __syncthreads();
  };
  issue(ring[0], 0);
  if (steps > 1) issue(ring[1], 1);
  stage(ring[0], 0);
  if (steps > 2) issue(ring[0], 2);
  __syncthreads();
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
  }
  if (s < steps) step(s, std::integral_constant<int, 0>{});

  // k-group partial tiles meet in LDS (the last barrier ended every read of
  // the stage buffers); k-group 0 adds them in k-group order and writes Y.
  float* red = reinterpret_cast<float*>(smem);
  constexpr int kPart = MT * NT * 16 * 64;  // floats per wave
  if (KG > 1 && wk > 0) {
    float* dst = red + ((wk - 1) * NG + wn) * kPart;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) dst[((i * NT + j) * 16 + e) * 64 + lane] = acc[i][j][e];
  }
  __syncthreads();
  if (wk == 0) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        const int n = n0 + 32 * (NT * wn + j) + (lane & 31);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float sum = acc[i][j][e];
#pragma unroll
          for (int c = 1; c < KG; ++c)
            sum += red[(((c - 1) * NG + wn) * MT * NT + i * NT + j) * 16 * 64 + e * 64 + lane];
          const int m = m0 + 32 * i + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (m < M && n < N) Y[(size_t)m * N + n] = f2h_bits(sum);
        }
      }
  }
}

template <int MT, int NT, int NG, int KG>
hipError_t launch_wide(const GemmArgs& a, hipStream_t stream) {
  using G = WideGeom<MT, NT, NG, KG>;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = lds_limit_once(reinterpret_cast<const void*>(tq2_wide_kernel<MT, NT, NG, KG>),
                                G::Lds, lds_set);
  if (e != hipSuccess) return e;
  const int64_t n_tiles = (a.N + G::BN - 1) / G::BN;
  const int64_t m_tiles = (a.M + G::BM - 1) / G::BM;
  const int64_t tiles = n_tiles * m_tiles;
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL((tq2_wide_kernel<MT, NT, NG, KG>), dim3((unsigned)(8 * per_xcd)),
                     dim3(kWideThreads), G::Lds, stream, static_cast<const uint16_t*>(a.X),
                     static_cast<const uint8_t*>(a.qs), static_cast<const uint16_t*>(a.scales),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, (int)n_tiles,
                     (int)tiles, (int)per_xcd);
  return hipGetLastError();
}

}  // namespace

bool wide_compiled(const WideShape& w) {
  if (w.ng * w.kg != 4 || (w.kg != 2 && w.kg != 4)) return false;
  if (w.mt != 1 && w.mt != 2 && w.mt != 4) return false;
  if (w.nt != 1 && w.nt != 2) return false;
  return !(w.mt == 4 && w.kg == 4);  // 16 activation pieces per thread: too many registers
}

// Whether the shape's buffers fit the kernel's 32-bit buffer offsets.
bool wide_fits(int64_t M, int64_t N, int64_t K) {
  return M * K * 2 < (int64_t(1) << 31) && N * (K / 4) < (int64_t(1) << 31);
}

hipError_t launch_tq2_wide_shape(const WideShape& w, const GemmArgs& a, hipStream_t stream) {
#define TQ_WIDE(MT_, NT_, NG_, KG_) \
  if (w.mt == MT_ && w.nt == NT_ && w.ng == NG_ && w.kg == KG_) return launch_wide<MT_, NT_, NG_, KG_>(a, stream);
  TQ_WIDE(4, 2, 2, 2)
  TQ_WIDE(4, 1, 2, 2)
  TQ_WIDE(2, 2, 2, 2)
  TQ_WIDE(2, 1, 2, 2)
  TQ_WIDE(1, 2, 2, 2)
  TQ_WIDE(1, 1, 2, 2)
  TQ_WIDE(2, 2, 1, 4)
  TQ_WIDE(2, 1, 1, 4)
  TQ_WIDE(1, 2, 1, 4)
  TQ_WIDE(1, 1, 1, 4)
#undef TQ_WIDE
  return hipErrorInvalidValue;
}

}  // namespace tq
