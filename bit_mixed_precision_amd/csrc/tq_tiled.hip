// Tiled MFMA kernel (M > 16): Y = X (s . T)^T for TQ2 weights.
//
// Follows the project page "Scaling Laws and Efficient Inference for Ternary
// Language Models": "The model" (step 3), "2 bits per weight" (decoder),
// "Fast inference on CPUs" (256-weight scale block), "TriRun: ternary
// inference on GPUs" (FP32 accumulation, FP16 output).  MI355X design:
//
//  * a workgroup (4 waves) owns a BM x BN output tile (BM = 16 MT activation
//    rows, BN = 16 NR weight rows) and all of K; the four waves split every
//    256-weight block into four 64-weight slices, so each weight is decoded
//    once per workgroup and each activation fragment read from LDS feeds NR
//    MFMAs;
//  * the activation block is staged in LDS (double-buffered, one block ahead);
//    weights are prefetched two blocks ahead in registers, issued after the
//    activation loads so that the in-order vector-memory counter never makes
//    the staging wait for the long-latency weight loads;
//  * weights are decoded in natural k order: one v_perm_b32 copies a byte
//    into both halves, one v_and_or_b32 against the fp16 exponent of 1024
//    extracts two fields, one v_pk_fma_f16 makes them exact trits and one
//    v_pk_mul_f16 applies the block scale (+-s or 0, exact), so every MFMA
//    accumulates across all of K;
//  * v_mfma_f32_16x16x32_f16 with fp32 accumulators; the four waves' partial
//    tiles meet in LDS at the end and one fp32 -> fp16 rounding writes Y.

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

constexpr int kStageRowBytes = 512 + 16;  // one 256-activation row of a stage + bank pad

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
  // B operand of 8 consecutive weights: bytes H (0 or 1) pair of dword x,
  // i.e. weights 8 H .. 8 H + 7 of the dword, times the scale pair s2.
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

// Lane (n = l % 16, g = l / 16) of wave w, block s: weight dword at byte
// 64 s + 16 w + 4 g of row n, i.e. weights k = 256 s + 64 w + 16 g + 0..15.
// k-step H (0, 1) of the wave uses k = 256 s + 64 w + 16 g + 8 H + 0..7 in both
// the B operand (from the dword) and the A operand (16 bytes of the staged row).
template <int MT, int NR>
__global__ __launch_bounds__(256) void tq2_tiled_kernel(const uint16_t* __restrict__ X,
                                                        const uint8_t* __restrict__ qs,
                                                        const uint16_t* __restrict__ scales,
                                                        uint16_t* __restrict__ Y, int M, int N,
                                                        int K) {
  constexpr int BM = 16 * MT;
  constexpr int BN = 16 * NR;
  constexpr int kStageBytes = BM * kStageRowBytes;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int n_base = blockIdx.x * BN;
  const int m_base = blockIdx.y * BM;
  const size_t row_bytes = (size_t)(K >> 2);

  NaturalConsts dc;
  dc.init();

  // weight rows of this lane (rows past N read row n_base; never written)
  const uint8_t* wrow[NR];
  const uint16_t* srow[NR];
#pragma unroll
  for (int r = 0; r < NR; ++r) {
    const int n = n_base + 16 * r + li;
    const int nn = n < N ? n : n_base;
    wrow[r] = qs + (size_t)nn * row_bytes + 16 * wave + 4 * g;
    srow[r] = scales + (size_t)nn * nb;
  }

  // Activation staging: thread t copies 16-byte chunks of the BM x 256 block
  // (rows past M read row m_base + 0 ... a valid row; their outputs are not
  // written).  Chunks per stage: BM * 32; per thread: BM / 8.
  constexpr int kChunks = BM * 32 / 256;
  u32x4 xr[kChunks];
  auto xload = [&](int s) {
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int q = threadIdx.x + 256 * c;
      const int row = q >> 5;
      const int col = q & 31;
      const int m = m_base + row < M ? m_base + row : m_base;
      xr[c] = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + 256 * s + 8 * col);
    }
  };
  auto xstore = [&](int buf) {
    unsigned char* base = smem + buf * kStageBytes;
#pragma unroll
    for (int c = 0; c < kChunks; ++c) {
      const int q = threadIdx.x + 256 * c;
      *reinterpret_cast<u32x4*>(base + (q >> 5) * kStageRowBytes + 16 * (q & 31)) = xr[c];
    }
  };

  uint32_t w0[NR], w1[NR], w2[NR];  // weight dwords for blocks s, s+1, s+2
  uint32_t s0[NR], s1[NR], s2[NR];  // scale pairs (fp16 x2) for the same blocks
  auto wload = [&](uint32_t(&w)[NR], uint32_t(&sp)[NR], int s) {
    const int ss = s < nb ? s : nb - 1;  // past the end: reload the last block
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      w[r] = *reinterpret_cast<const uint32_t*>(wrow[r] + 64 * ss);
      const uint32_t h = srow[r][ss];
      sp[r] = h | (h << 16);
    }
  };

  float4v C[MT][NR];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int r = 0; r < NR; ++r) C[i][r] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](int buf, const uint32_t(&w)[NR], const uint32_t(&sp)[NR]) {
    const unsigned char* xs = smem + buf * kStageBytes + li * kStageRowBytes + 128 * wave + 32 * g;
    sfor<0, 2>([&](auto hh) {
      constexpr int H = decltype(hh)::value;
      half8 B[NR];
#pragma unroll
      for (int r = 0; r < NR; ++r) B[r] = dc.operand<H>(w[r], sp[r]);
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const half8 A = *reinterpret_cast<const half8*>(xs + i * 16 * kStageRowBytes + 16 * H);
#pragma unroll
        for (int r = 0; r < NR; ++r) C[i][r] = mfma16(A, B[r], C[i][r]);
      }
    });
  };

  // Prologue: X(0) staged in LDS buffer 0, X(1) loads in registers, W(0..2)
  // in flight.  Issue order X(0), W(0), W(1), X(1), W(2): waiting for an
  // activation load never waits for a younger weight load.
  xload(0);
  wload(w0, s0, 0);
  wload(w1, s1, 1);
  __builtin_amdgcn_sched_barrier(0);
  xstore(0);
  xload(1 < nb ? 1 : nb - 1);
  wload(w2, s2, 2);
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();

  // Steady state, three blocks per trip so the weight buffers rotate in
  // place.  Entering block s: X(s) is in LDS buffer s % 2 (visible), X(s + 1)
  // is loading into registers, W(s), W(s + 1), W(s + 2) are loaded or in
  // flight.  Buffer (s + 1) % 2 was last read by block s - 1, which every wave
  // finished before the previous barrier, so it can be rewritten at once.
  auto step = [&](int s, const uint32_t(&w)[NR], const uint32_t(&sp)[NR], uint32_t(&wn)[NR],
                  uint32_t(&spn)[NR]) {
    compute(s & 1, w, sp);
    xstore((s + 1) & 1);  // X(s + 1) -> LDS
    xload(s + 2 < nb ? s + 2 : nb - 1);
    wload(wn, spn, s + 3);  // into the registers that held W(s)
    __builtin_amdgcn_sched_barrier(0);
    __syncthreads();  // X(s + 1) visible; block s done everywhere
  };
  for (int s = 0; s < nb; s += 3) {
    step(s, w0, s0, w0, s0);
    if (s + 1 >= nb) break;
    step(s + 1, w1, s1, w1, s1);
    if (s + 2 >= nb) break;
    step(s + 2, w2, s2, w2, s2);
  }

  // Reduce the four waves' partial tiles through LDS (reusing the stage
  // buffers), one 16 x 16 tile at a time per wave slot.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int r = 0; r < NR; ++r) {
#pragma unroll
      for (int e = 0; e < 4; ++e) red[((i * NR + r) * 4 + wave) * 256 + e * 64 + lane] = C[i][r][e];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < MT * NR * 256; t += 256) {
    const int tile = t >> 8;
    const int el = t & 255;
    const int i = tile / NR;
    const int r = tile % NR;
    const int l = el & 63;
    const int m = m_base + 16 * i + 4 * (l >> 4) + (el >> 6);
    const int n = n_base + 16 * r + (l & 15);
    if (m < M && n < N) {
      const float* p = red + tile * 4 * 256 + el;
      const float sum = (p[0] + p[256]) + (p[512] + p[768]);
      Y[(size_t)m * N + n] = f2h_bits(sum);
    }
  }
}

template <int MT, int NR>
hipError_t launch_tiled(const GemmArgs& a, hipStream_t stream) {
  constexpr int BM = 16 * MT, BN = 16 * NR;
  const int stage = BM * kStageRowBytes;
  int lds = 2 * stage;
  const int red = MT * NR * 4 * 1024;
  if (red > lds) lds = red;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(tq2_tiled_kernel<MT, NR>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  dim3 grid((unsigned)((a.N + BN - 1) / BN), (unsigned)((a.M + BM - 1) / BM));
  hipLaunchKernelGGL((tq2_tiled_kernel<MT, NR>), grid, dim3(256), lds, stream,
                     static_cast<const uint16_t*>(a.X), static_cast<const uint8_t*>(a.qs),
                     static_cast<const uint16_t*>(a.scales), static_cast<uint16_t*>(a.Y),
                     (int)a.M, (int)a.N, (int)a.K);
  return hipGetLastError();
}

}  // namespace

// Tile choice: the largest tile (most MFMA work per decoded weight and per
// staged activation) that still gives at least ~0.8 workgroups per CU, and no
// taller than the activation rows need.
TiledShape tiled_shape(int64_t M, int64_t N) {
  const int64_t cus = device_cus();
  const int64_t mt_cap = M > 64 ? 8 : (M > 32 ? 4 : 2);
  const TiledShape cands[5] = {{8, 2}, {4, 4}, {4, 2}, {2, 4}, {2, 2}};
  for (const TiledShape& t : cands) {
    if (t.mt > mt_cap) continue;
    const int64_t wgs = ((N + 16 * t.nr - 1) / (16 * t.nr)) * ((M + 16 * t.mt - 1) / (16 * t.mt));
    if (5 * wgs >= 4 * cus) return t;
  }
  return TiledShape{2, 2};
}

hipError_t launch_tq2_tiled(const GemmArgs& a, hipStream_t stream) {
  const TiledShape t = tiled_shape(a.M, a.N);
  if (t.mt == 2 && t.nr == 2) return launch_tiled<2, 2>(a, stream);
  if (t.mt == 2 && t.nr == 4) return launch_tiled<2, 4>(a, stream);
  if (t.mt == 4 && t.nr == 2) return launch_tiled<4, 2>(a, stream);
  if (t.mt == 4 && t.nr == 4) return launch_tiled<4, 4>(a, stream);
  return launch_tiled<8, 2>(a, stream);
}

}  // namespace tq
