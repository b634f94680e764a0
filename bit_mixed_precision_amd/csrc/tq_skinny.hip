// Skinny kernels (M <= 16): Y = X (s . T)^T with the weights streamed once.
//
// The work follows the project page "Scaling Laws and Efficient Inference for
// Ternary Language Models": "The model" (step 3) for the product, "2 bits per
// weight" for the decoder, "Fast inference on CPUs" for the 256-weight scale
// block, "TriRun: ternary inference on GPUs" for FP32 accumulation and FP16
// output.  The design is MI355X-specific:
//
//  * a workgroup owns R groups of 16 weight rows and all of K; one workgroup
//    per CU;
//  * its waves take the 256-weight blocks round robin, so at any time they read
//    neighbouring 64-byte pieces of the same rows; every lane streams 16-byte
//    loads through a ring of register buffers (inside the loop only weight
//    loads are in the vector-memory queue, so the prefetch overlaps the decode);
//  * the activations are staged in LDS once per window of K (the whole of K
//    when it fits) with coalesced loads, scattered into the order the decoder
//    produces weights; the block scales of the workgroup's rows are staged too;
//  * trits become fp16 with one v_and_or_b32 against the fp16 exponent of 1024
//    plus one v_pk_fma_f16 per pair of weights (exact -1 / 0 / +1);
//  * the multiply-accumulate runs on v_mfma_f32_16x16x32_f16 with the M <= 16
//    activation rows as the A operand, so the VALU only decodes;
//  * per block the MFMA partial sum is scaled once (4 FMAs per lane per 16
//    rows) into fp32 accumulators;
//  * partial sums of the waves meet in LDS and one fp32 -> fp16 rounding writes
//    Y.  No atomics: results are deterministic.

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// ----------------------------------------------------------------------------
// TQ2 weight order.  Lane (n = l % 16, g = l / 16) owns bytes [16 g, 16 g + 16)
// of each 64-byte block of weight row n: four dwords w0..w3 of sixteen 2-bit
// fields.  Decode class c (0..7) takes field c of the low and of the high half
// of every dword, so B-operand slot 2i / 2i+1 holds weight k = 64 g + 16 i + c /
// 64 g + 16 i + 8 + c of the block.  The matching A operand of class c is the
// lane's activations x[64 g + 8 s + c], s = 0..7, which the LDS copy stores as
// 16 contiguous bytes: Xt[m][block][g][c][s].
// ----------------------------------------------------------------------------

constexpr int kXRowPad = 16;          // bytes between LDS rows of Xt (bank spread)
constexpr int kXLdsMax = 132 * 1024;  // LDS budget of the activation window
constexpr int kScaleLdsMax = 24 * 1024;
constexpr int kLdsLimit = 160 * 1024;

template <int C>
__device__ __forceinline__ half8 tq2_class(const DecodeConsts& dc, const u32x4& w,
                                           const u32x4& ws) {
  u32x4 r;
  if constexpr (C < 5) {
    r[0] = dc.pair<C>(w[0]);
    r[1] = dc.pair<C>(w[1]);
    r[2] = dc.pair<C>(w[2]);
    r[3] = dc.pair<C>(w[3]);
  } else {
    r[0] = dc.pair<C - 5>(ws[0]);
    r[1] = dc.pair<C - 5>(ws[1]);
    r[2] = dc.pair<C - 5>(ws[2]);
    r[3] = dc.pair<C - 5>(ws[3]);
  }
  return __builtin_bit_cast(half8, r);
}

// Copies activations of blocks [wb0, wb0 + nbw) of rows m < M into LDS in
// decoder order.  Consecutive lanes read consecutive 16-byte pieces of a row,
// so each wave load covers whole cache lines; piece j of a row holds
// x[64 g + 8 s + c], c = 0..7 (block j / 32, g = j / 8 % 4, s = j % 8), and its
// eight activations go to their class slots Xt[m][block][g][c][s] with 2-byte
// LDS writes.  Four pieces per thread are in flight at a time.
__device__ __forceinline__ void stage_x(unsigned char* xs, const uint16_t* __restrict__ X, int M,
                                        int K, int wb0, int nbw, int xstride) {
  const int per_row = nbw * 32;
  const int total = M * per_row;
  const int T = blockDim.x;
  for (int p0 = threadIdx.x; p0 < total; p0 += 4 * T) {
    u32x4 v[4];
    int dst[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int p = p0 + u * T;
      const bool ok = p < total;
      p = ok ? p : 0;  // past the end: a valid dummy read, not stored
      const int m = p / per_row;
      const int j = p - m * per_row;
      v[u] = *reinterpret_cast<const u32x4*>(X + (size_t)m * K + 256 * wb0 + 8 * j);
      dst[u] = ok ? m * xstride + (j >> 5) * 512 + ((j >> 3) & 3) * 128 + (j & 7) * 2 : -1;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (dst[u] >= 0) {
        unsigned char* d = xs + dst[u];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          const uint32_t wv = v[u][c >> 1];
          *reinterpret_cast<uint16_t*>(d + 16 * c) = (uint16_t)((c & 1) ? (wv >> 16) : wv);
        }
      }
    }
  }
}

// A workgroup owns RG groups of 16 weight rows and all of K.  Its RG * WK
// waves are light: wave w works on row group w / WK and on the blocks
// b = w % WK + WK * i of K, so several waves per SIMD interleave decode, MFMA
// and memory waits.  Each wave keeps a ring of D register buffers of weights in
// flight (straight-line loop body; past its last block a wave re-reads its own
// previous block, a cache hit, so that no load sits under a branch and the
// wait before each decode covers exactly the oldest buffer).  STAGE: the block
// scales of the workgroup's rows are copied to LDS (else each block's scales
// come with its weights).  Rows past N and activation rows past M read valid
// dummy data whose results are never written (MFMA rows and columns do not mix).
template <int D, bool STAGE>
__global__ __launch_bounds__(1024) void tq2_skinny_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs,
    const uint16_t* __restrict__ scales, uint16_t* __restrict__ Y, int M, int N, int K, int RG,
    int WK, int nbw, int xregion) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int rg = wave / WK;  // row group of this wave
  const int wk = wave % WK;  // K slice of this wave
  const int n_base = blockIdx.x * (16 * RG);
  const int rows = min(16 * RG, N - n_base);
  const int xstride = nbw * 512 + kXRowPad;
  const size_t row_bytes = (size_t)(K >> 2);
  uint16_t* sc_lds = reinterpret_cast<uint16_t*>(smem + xregion);

  DecodeConsts dc;
  dc.init();

  const int nrow = 16 * rg + li < rows ? 16 * rg + li : 0;  // row of this lane in the tile
  const uint8_t* wrow = qs + (size_t)(n_base + nrow) * row_bytes + 16 * g;
  const uint16_t* srow = scales + (size_t)(n_base + nrow) * nb;
  if constexpr (STAGE) {
    const uint16_t* src = scales + (size_t)n_base * nb;
    for (int i = threadIdx.x; i < rows * nb; i += blockDim.x) sc_lds[i] = src[i];
  }
  const unsigned char* xa = smem + (li < M ? li : M - 1) * xstride + g * 128;

  float4v acc = {0.f, 0.f, 0.f, 0.f};
  u32x4 wbuf[D];
  uint16_t sbuf[D];

  auto load = [&](int d, int b) {
    wbuf[d] = *reinterpret_cast<const u32x4*>(wrow + 64 * b);
    if constexpr (!STAGE) sbuf[d] = srow[b];
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch where it is
  };
  auto compute = [&](int d, int b, int bw) {
    const u32x4 w = wbuf[d];
    u32x4 ws;
    ws[0] = w[0] >> 10;
    ws[1] = w[1] >> 10;
    ws[2] = w[2] >> 10;
    ws[3] = w[3] >> 10;
    const float sc = h2f(STAGE ? sc_lds[nrow * nb + b] : sbuf[d]);
    float4v C = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* xb = xa + bw * 512;
    static_for<0, 8>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      const half8 A = *reinterpret_cast<const half8*>(xb + 16 * c);
      C = mfma16(A, tq2_class<c>(dc, w, ws), C);
    });
    acc += sc * C;
  };

  for (int wb0 = 0; wb0 < nb; wb0 += nbw) {
    const int nbw_here = min(nbw, nb - wb0);
    const int cnt = nbw_here > wk ? (nbw_here - wk + WK - 1) / WK : 0;
    // block of step i; past the end, the wave's last real block (a cache hit);
    // a wave with no block in the window refetches block wb0
    auto blk = [&](int i) { return cnt > 0 ? wb0 + wk + WK * (i < cnt ? i : cnt - 1) : wb0; };
    __syncthreads();  // earlier window fully consumed
    stage_x(smem, X, M, K, wb0, nbw_here, xstride);
    // The first D weight loads go out after the activation loads, so waiting
    // for those does not wait for these; the prefetch is unconditional, which
    // keeps the compiler's count of loads in flight exact in the loop below.
    static_for<0, D>([&](auto dd) { load(decltype(dd)::value, blk(decltype(dd)::value)); });
    __syncthreads();
    for (int i = 0; i < cnt; i += D) {
      static_for<0, D>([&](auto dd) {
        constexpr int d = decltype(dd)::value;
        if (i + d < cnt) compute(d, blk(i + d), wk + WK * (i + d));
        load(d, blk(i + d + D));
      });
    }
  }

  // Partial sums: every wave writes its 16 x 16 tile to LDS (reusing the
  // activation window); each tile element sums the WK waves of its row group.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave * 256 + i * 64 + lane] = acc[i];
  __syncthreads();
  for (int t = threadIdx.x; t < RG * 256; t += blockDim.x) {
    const int r = t >> 8;
    const int e = t & 255;
    const int l = e & 63;
    const int m = 4 * (l >> 4) + (e >> 6);
    const int n = 16 * r + (l & 15);
    if (m < M && n < rows) {
      float sum = 0.f;
      for (int k = 0; k < WK; ++k) sum += red[(r * WK + k) * 256 + e];
      Y[(size_t)m * N + n_base + n] = f2h_bits(sum);
    }
  }
}

// Row groups per workgroup: enough to give one workgroup per CU (at most 16,
// one wave each).
int pick_rows(int64_t N, int cus) {
  const int64_t groups = (N + 15) / 16;
  int64_t r = (groups + cus - 1) / cus;
  if (r < 1) r = 1;
  if (r > 16) r = 16;
  return (int)r;
}

constexpr int kDepth = 4;

template <bool STAGE>
hipError_t launch_tq2_skinny_s(const GemmArgs& a, hipStream_t stream, int RG, int WK, int nbw,
                               int xregion, int lds) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e =
        hipFuncSetAttribute(reinterpret_cast<const void*>(tq2_skinny_kernel<kDepth, STAGE>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t groups = (a.N + 16 * RG - 1) / (16 * RG);
  hipLaunchKernelGGL((tq2_skinny_kernel<kDepth, STAGE>), dim3((unsigned)groups),
                     dim3(64 * RG * WK), lds, stream, static_cast<const uint16_t*>(a.X),
                     static_cast<const uint8_t*>(a.qs), static_cast<const uint16_t*>(a.scales),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, RG, WK, nbw,
                     xregion);
  return hipGetLastError();
}

}  // namespace

int skinny_rows(int64_t N) { return pick_rows(N, device_cus()); }

int skinny_depth() { return kDepth; }

int skinny_stage(int64_t N, int64_t K) {
  const int64_t RG = skinny_rows(N);
  const int64_t sbytes = ((16 * RG * (K / 256) * 2) + 15) & ~15;
  return sbytes <= kScaleLdsMax ? 1 : 0;
}

hipError_t launch_tq2_skinny(const GemmArgs& a, hipStream_t stream) {
  const int M = (int)a.M, K = (int)a.K;
  const int nb = K / 256;
  const int RG = skinny_rows(a.N);
  int WK = 16 / RG;  // waves per row group
  if (WK > nb) WK = nb;
  if (WK < 1) WK = 1;
  const int W = RG * WK;
  // activation window: as many blocks as fit the LDS budget
  int nbw = (kXLdsMax / M - kXRowPad) / 512;
  if (nbw > nb) nbw = nb;
  if (nbw < 1) nbw = 1;
  const int xbytes = M * (nbw * 512 + kXRowPad);
  int xregion = xbytes > W * 1024 ? xbytes : W * 1024;  // also holds the reduction
  xregion = (xregion + 15) & ~15;
  const int sbytes = ((16 * RG * nb * 2) + 15) & ~15;
  const bool stage = sbytes <= kScaleLdsMax;
  const int lds = xregion + (stage ? sbytes : 0);
  if (lds > kLdsLimit) return hipErrorInvalidValue;
  return stage ? launch_tq2_skinny_s<true>(a, stream, RG, WK, nbw, xregion, lds)
               : launch_tq2_skinny_s<false>(a, stream, RG, WK, nbw, xregion, lds);
}

}  // namespace tq
