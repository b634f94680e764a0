// Skinny kernel for 2-bit weights (M <= 16): Y = X (s . T)^T with the weights
// streamed once.
//
// The work follows the project page "Scaling Laws and Efficient Inference for
// Ternary Language Models": "The model" (step 3) for the product, "2 bits per
// weight" for the code (field value d' = d + 1, four fields per byte, first
// weight in the low bits), "Fast inference on CPUs" for the 256-weight scale
// block, "TriRun: ternary inference on GPUs" for FP32 accumulation and FP16
// output.  The design is MI355X-specific:
//
//  * a workgroup owns R groups of 16 weight rows and all of K; one workgroup
//    per CU;
//  * its waves take the 256-weight blocks round robin, so at any time they read
//    neighbouring 64-byte pieces of the same rows; every lane streams 16-byte
//    loads through a ring of register buffers;
//  * one v_and_b32 per pair of weights is the whole decode: masking a 2-bit
//    field that sits at mantissa bits 2p..2p+1 of an fp16 with a zero exponent
//    leaves the exact subnormal d' 4^p 2^-24, which the MFMA multiplies exactly
//    (it keeps fp16 subnormals).  Fields at p = 1 and p = 3 meet activations
//    pre-scaled by 1/4 in LDS, and the MFMAs of p = 0, 1 and of p = 2, 3 run in
//    two accumulator chains combined as C0 + C1 / 16, so every activation is
//    scaled by 1 or 1/4 only (exact above the fp16 subnormal range);
//  * the shift d = d' - 1 costs no per-weight work: the sum of the block's
//    activations, taken in fp32 while staging them, seeds the first chain;
//  * the multiply-accumulate runs on v_mfma_f32_16x16x32_f16 with the M <= 16
//    activation rows as the A operand; per block the two chains are combined
//    and scaled once (8 FMAs per lane per 16 rows);
//  * activations, their block sums and the block scales are staged once per
//    window of K (eight threads per 256 activations of a row, whose sum comes
//    from v_dot2_f32_f16 and three DPP adds), the window's last loads issued
//    before the first weight loads so that the wait for them does not wait for
//    the weights; per-wave set-up is kept to shifts and masks (it is a large
//    part of the time at one or two activation rows);
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
// Weight order.  Lane (n = l % 16, g = l / 16) owns bytes [16 g, 16 g + 16) of
// each 64-byte block of weight row n: four dwords w0..w3 of sixteen 2-bit
// fields, field j of dword i being weight k = 64 g + 16 i + j of the block.
// Class c (0..7) takes field c of the low and field c + 8 of the high half of
// every dword (classes 4..7 from the dwords shifted right by 8), so B-operand
// slot 2i / 2i+1 holds weight 64 g + 16 i + c / 64 g + 16 i + 8 + c, at field
// position p = c % 4 of its half.  The matching A operand of class c is the
// lane's activations x[64 g + 8 s + c], s = 0..7, times 1/4 for odd c, which
// the LDS copy stores as 16 contiguous bytes: Xt[m][block][g][c][s].
// Chain of class c: 0 for p in {0, 1}, 1 for p in {2, 3}; a chain-0 product
// is x d' 2^-24, a chain-1 product 16 x d' 2^-24.
// ----------------------------------------------------------------------------

constexpr int kXRowPad = 16;          // bytes between LDS rows of Xt (bank spread)
constexpr int kXLdsMax = 132 * 1024;  // LDS budget of the activation window and its sums
constexpr int kBiasBytes = 64;        // per block of the window: 16 fp32 row sums
constexpr int kScaleLdsMax = 24 * 1024;
constexpr int kLdsLimit = 160 * 1024;
constexpr int kScaleRegs = 4;         // block scales per thread loaded ahead
constexpr int kTrashX = 512;          // trash area: one unit's activations, then its sum
constexpr int kTrashBytes = kTrashX + 16;

template <int C>
__device__ __forceinline__ half8 tq2_class(const u32x4& w, const u32x4& w8) {
  constexpr uint32_t mask = 0x00030003u << (2 * (C & 3));
  u32x4 r;
  if constexpr (C < 4) {
    r = w & mask;
  } else {
    r = w8 & mask;
  }
  return __builtin_bit_cast(half8, r);
}

// Dwords shifted right by 8 bits, two at a time through 64-bit shifts (bits
// that move across a dword boundary land at 24..31, which no class reads).
__device__ __forceinline__ u32x4 shift8(const u32x4& w) {
  const uint64_t lo = ((uint64_t)w[1] << 32 | w[0]) >> 8;
  const uint64_t hi = ((uint64_t)w[3] << 32 | w[2]) >> 8;
  u32x4 r;
  r[0] = (uint32_t)lo;
  r[1] = (uint32_t)(lo >> 32);
  r[2] = (uint32_t)hi;
  r[3] = (uint32_t)(hi >> 32);
  return r;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}

// Staging unit = (activation row m, window block bw), taken by eight
// threads: thread s loads the four 16-byte pieces x[256 bw + 64 g + 8 s ..],
// g = 0..3 (eight threads read 128 contiguous bytes), so piece g holds the
// activations of lane group g, slot s, classes 0..7.  Thread t stages unit
// t / 8 of every batch of T / 8 units; its (m, bw) steps by (dm, dbw) per
// batch without divisions.  Units past the end read row 0 and store to a trash
// area of LDS.
struct PiecePos {
  int m, bw;
};

__device__ __forceinline__ void piece_load(u32x4 (&v)[4], const uint16_t* __restrict__ xw, PiecePos p,
                                           bool ok, int K) {
  const uint16_t* src = xw + (ok ? p.m * K + 256 * p.bw : 0);
#pragma unroll
  for (int g = 0; g < 4; ++g) v[g] = *reinterpret_cast<const u32x4*>(src + 64 * g);
}

// Writes a unit's activations to their class slots (odd classes times 1/4)
// and the block's negated row sum of the values the MFMAs see, times 2^-24.
__device__ __forceinline__ void piece_store(const u32x4 (&v)[4], bool ok, PiecePos p,
                                            unsigned char* xs, float* bias, unsigned char* trash,
                                            int xstride, int s) {
  const half2v quarter = {(_Float16)1.0f, (_Float16)0.25f};
  const half2v four = {(_Float16)1.0f, (_Float16)4.0f};
  float part = 0.f;
  unsigned char* d = (ok ? xs + p.m * xstride + p.bw * 512 : trash) + 2 * s;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // activations 8 s + 2 i, 8 s + 2 i + 1 of piece g: classes 2 i, 2 i + 1
      const uint32_t xv = v[g][i];  // (a bit cast of the vector element itself reads element 0)
      const half2v a = __builtin_bit_cast(half2v, xv) * quarter;
      part = __builtin_amdgcn_fdot2(a, four, part, false);
      const uint32_t ab = __builtin_bit_cast(uint32_t, a);
      *reinterpret_cast<uint16_t*>(d + g * 128 + (2 * i) * 16) = (uint16_t)ab;
      *reinterpret_cast<uint16_t*>(d + g * 128 + (2 * i + 1) * 16) = (uint16_t)(ab >> 16);
    }
  }
  part += dpp_f32<0xB1>(part);   // quad_perm [1, 0, 3, 2]
  part += dpp_f32<0x4E>(part);   // quad_perm [2, 3, 0, 1]
  part += dpp_f32<0x141>(part);  // row_half_mirror: the eight threads of the unit
  float* bd = ok ? bias + p.bw * 16 + p.m : reinterpret_cast<float*>(trash + kTrashX);
  if (s == 0) *bd = part * -0x1p-24f;
}

// A workgroup owns RG groups of 16 weight rows and all of K.  Its RG * WK
// waves (WK = 2^lwk) are light: wave w works on row group w / WK and on the
// blocks b = w % WK + WK * i of K, so several waves per SIMD interleave decode,
// MFMA and memory waits.  Each wave keeps a ring of D register buffers of weights
// in flight; the loop body is straight-line except for the last group of
// steps, which issues no loads, so the compiler's wait before each decode
// covers exactly the oldest buffer.  STAGE: the block scales of the
// workgroup's rows are copied to LDS as fp32 (else each block's scale comes
// with its weights).  Rows past N and activation rows past M read valid dummy
// data whose results are never written (MFMA rows and columns do not mix).
//
// GLU: the workgroup's first RG / 2 row groups read the gate matrix (qs,
// scales), the others the same rows of the up matrix (qs2, scales2), and the
// output is silu(g) u of the two products (SwiGLU of the decode step), one
// fp16 rounding.
template <int D, bool STAGE, bool GLU>
__global__ __launch_bounds__(1024) void tq2_skinny_kernel(
    const uint16_t* __restrict__ X, const uint8_t* __restrict__ qs,
    const uint16_t* __restrict__ scales, const uint8_t* __restrict__ qs2,
    const uint16_t* __restrict__ scales2, uint16_t* __restrict__ Y, int M, int N, int K, int RG,
    int lwk, int nbw, int xregion) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int lane = threadIdx.x & 63;
  const int li = lane & 15;
  const int g = lane >> 4;
  const int nb = K >> 8;
  const int WK = 1 << lwk;
  const int W = RG << lwk;
  const int T = 64 * W;        // threads
  const int rg = wave >> lwk;  // row group of this wave
  const int wk = wave & (WK - 1);  // K slice of this wave
  const int RGO = GLU ? RG >> 1 : RG;  // output row groups
  const bool up = GLU && rg >= RGO;    // wave-uniform: this wave reads the up matrix
  const int rgo = up ? rg - RGO : rg;
  const int n_base = blockIdx.x * (16 * RGO);
  const int rows = min(16 * RGO, N - n_base);
  const int xstride = nbw * 512 + kXRowPad;
  const size_t row_bytes = (size_t)(K >> 2);
  float* bias = reinterpret_cast<float*>(smem + M * xstride);
  unsigned char* trash = reinterpret_cast<unsigned char*>(bias + 16 * nbw);
  float* sc_lds = reinterpret_cast<float*>(smem + xregion);

  const int nrow = 16 * rgo + li < rows ? 16 * rgo + li : 0;  // row of this lane in the tile
  const uint8_t* wrow = (up ? qs2 : qs) + (size_t)(n_base + nrow) * row_bytes + 16 * g;
  const uint16_t* srow = (up ? scales2 : scales) + (size_t)(n_base + nrow) * nb;
  const unsigned char* xa = smem + (li < M ? li : M - 1) * xstride + g * 128;
  const float* ba = bias + 4 * g;

  // The workgroup's block scales (staged with the first window): ns of each
  // matrix, the up matrix's after the gate matrix's.
  const int ns = STAGE ? rows * nb : 0;
  const int ns_all = GLU ? 2 * ns : ns;
  const uint16_t* ssrc = scales + (size_t)n_base * nb;
  const uint16_t* ssrc2 = GLU ? scales2 + (size_t)n_base * nb : ssrc;
  // Staged scale rows sit nb + 1 floats apart, so the 16 rows a wave reads
  // at once fall in 16 different LDS banks (nb apart, with nb a multiple of
  // 32 or 64 as it usually is, they would all share one bank).
  const int sc_row = ((up ? rows : 0) + nrow) * (nb + 1);
  const float inv_nb = __builtin_amdgcn_rcpf((float)nb);  // within 1 ulp: ample for the row index

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
    const u32x4 w8 = shift8(w);
    const float sc = STAGE ? sc_lds[sc_row + b] : h2f(sbuf[d]);
    float4v c0 = *reinterpret_cast<const float4v*>(ba + 16 * bw);  // -2^-24 (row sums)
    float4v c1 = {0.f, 0.f, 0.f, 0.f};
    const unsigned char* xb = xa + bw * 512;
    auto A = [&](int c) { return *reinterpret_cast<const half8*>(xb + 16 * c); };
    c0 = mfma16(A(0), tq2_class<0>(w, w8), c0);
    c1 = mfma16(A(2), tq2_class<2>(w, w8), c1);
    c0 = mfma16(A(1), tq2_class<1>(w, w8), c0);
    c1 = mfma16(A(3), tq2_class<3>(w, w8), c1);
    c0 = mfma16(A(4), tq2_class<4>(w, w8), c0);
    c1 = mfma16(A(6), tq2_class<6>(w, w8), c1);
    c0 = mfma16(A(5), tq2_class<5>(w, w8), c0);
    c1 = mfma16(A(7), tq2_class<7>(w, w8), c1);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, __builtin_fmaf(c1[i], 0.0625f, c0[i]), acc[i]);
  };

  for (int wb0 = 0; wb0 < nb; wb0 += nbw) {
    const int nbw_here = min(nbw, nb - wb0);
    const int cnt = nbw_here > wk ? (nbw_here - wk + WK - 1) >> lwk : 0;
    // block of step i; past the end, the wave's last real block; a wave with
    // no block in the window refetches block wb0
    auto blk = [&](int i) { return cnt > 0 ? wb0 + wk + WK * (i < cnt ? i : cnt - 1) : wb0; };
    __syncthreads();  // earlier window fully consumed
    // Stage the window.  Every batch but the last is full and waits for its
    // own loads only; the last batch's loads (and the block scales) go out
    // before the weight prefetch, so its wait does not cover the weights.
    const int units = M * nbw_here;
    const uint16_t* xw = X + 256 * wb0 + 8 * (threadIdx.x & 7);
    const int per_batch = T >> 3;
    PiecePos pos{0, (int)(threadIdx.x >> 3)};
    while (pos.bw >= nbw_here) {
      pos.bw -= nbw_here;
      ++pos.m;
    }
    const int dm = per_batch / nbw_here;
    const int dbw = per_batch - dm * nbw_here;
    int q = 0;  // first unit of the batch
    for (; q + per_batch < units; q += per_batch) {
      u32x4 v[4];
      piece_load(v, xw, pos, true, K);
      piece_store(v, true, pos, smem, bias, trash, xstride, threadIdx.x & 7);
      pos.bw += dbw;
      pos.m += dm;
      if (pos.bw >= nbw_here) {
        pos.bw -= nbw_here;
        ++pos.m;
      }
    }
    {
      u32x4 v[4];
      const bool ok = pos.m < M;
      piece_load(v, xw, pos, ok, K);
      // block scales: read in every window (straight-line), stored in the first
      uint16_t sreg[kScaleRegs];
      if constexpr (STAGE) {
#pragma unroll
        for (int r = 0; r < kScaleRegs; ++r) {
          int e = threadIdx.x + r * T;
          e = e < ns_all ? e : 0;
          asm volatile("" : "+v"(e));  // keep the load in the window (not hoisted ahead of it)
          sreg[r] = e < ns ? ssrc[e] : ssrc2[e - ns];
        }
      }
      static_for<0, D>([&](auto dd) { load(decltype(dd)::value, blk(decltype(dd)::value)); });
      // waves without a unit skip the store (their trash writes would all
      // hit the same LDS banks)
      if (__any(ok)) piece_store(v, ok, pos, smem, bias, trash, xstride, threadIdx.x & 7);
      if constexpr (STAGE) {
        if (wb0 == 0) {
#pragma unroll
          for (int r = 0; r < kScaleRegs; ++r) {
            const int e = threadIdx.x + r * T;
            // row of scale e: exact in fp32, since e < 2^14 keeps the rounding
            // error far below the 0.5 / nb margin to the nearest integer
            const int row = (int)(((float)e + 0.5f) * inv_nb);
            if (e < ns_all) sc_lds[e + row] = h2f(sreg[r]);
          }
        }
      }
    }
    __syncthreads();
    int i = 0;
    for (; i + D < cnt; i += D) {
      static_for<0, D>([&](auto dd) {
        constexpr int d = decltype(dd)::value;
        compute(d, blk(i + d), wk + WK * (i + d));
        load(d, blk(i + d + D));
      });
    }
    // last group: no loads past the wave's blocks
    static_for<0, D>([&](auto dd) {
      constexpr int d = decltype(dd)::value;
      if (i + d < cnt) compute(d, blk(i + d), wk + WK * (i + d));
    });
  }

  // Partial sums: every wave writes its 16 x 16 tile to LDS (reusing the
  // activation window); each tile element sums the WK waves of its row group.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave * 256 + i * 64 + lane] = acc[i];
  __syncthreads();
  for (int t = threadIdx.x; t < RGO * 256; t += T) {
    const int r = t >> 8;
    const int e = t & 255;
    const int l = e & 63;
    const int m = 4 * (l >> 4) + (e >> 6);
    const int n = 16 * r + (l & 15);
    if (m < M && n < rows) {
      float sum = 0.f;
      for (int k = 0; k < WK; ++k) sum += red[(r * WK + k) * 256 + e];
      sum *= 0x1p24f;
      if constexpr (GLU) {
        float u = 0.f;
        for (int k = 0; k < WK; ++k) u += red[((RGO + r) * WK + k) * 256 + e];
        sum = sum / (1.0f + expf(-sum)) * (u * 0x1p24f);  // silu(g) u
      }
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

template <bool STAGE, bool GLU>
hipError_t launch_tq2_skinny_s(const GemmArgs& a, const void* qs2, const void* scales2,
                               hipStream_t stream, int RG, int lwk, int nbw, int xregion, int lds) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(tq2_skinny_kernel<kDepth, STAGE, GLU>),
        hipFuncAttributeMaxDynamicSharedMemorySize, kLdsLimit);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int RGO = GLU ? RG / 2 : RG;
  const int64_t groups = (a.N + 16 * RGO - 1) / (16 * RGO);
  hipLaunchKernelGGL((tq2_skinny_kernel<kDepth, STAGE, GLU>), dim3((unsigned)groups),
                     dim3(64 * (RG << lwk)), lds, stream, static_cast<const uint16_t*>(a.X),
                     static_cast<const uint8_t*>(a.qs), static_cast<const uint16_t*>(a.scales),
                     static_cast<const uint8_t*>(qs2), static_cast<const uint16_t*>(scales2),
                     static_cast<uint16_t*>(a.Y), (int)a.M, (int)a.N, (int)a.K, RG, lwk, nbw,
                     xregion);
  return hipGetLastError();
}

// Staged scales: 16 RG rows of K / 256 floats, rows padded by one float.
int64_t scale_lds_bytes(int64_t RG, int64_t K) { return ((16 * RG * (K / 256 + 1) * 4) + 15) & ~15; }

}  // namespace

int skinny_rows(int64_t N) { return pick_rows(N, device_cus()); }

int skinny_depth() { return kDepth; }

int skinny_lwk(int64_t N, int64_t K, int64_t M);

int skinny_stage(int64_t N, int64_t K, int64_t M) {
  const int64_t RG = skinny_rows(N);
  const int64_t threads = 64 * (RG << skinny_lwk(N, K, M));
  return scale_lds_bytes(RG, K) <= kScaleLdsMax && 16 * RG * (K / 256) <= kScaleRegs * threads
             ? 1
             : 0;
}

// Waves per row group: 2^lwk (a power of two, so the kernel's K slicing is
// shifts and masks), at most 16 waves per workgroup.  For one or two
// activation rows the per-wave set-up is a large part of the work, so waves
// then take at least 8 blocks each (measured: N = 8192, K = 8192, M = 1 runs
// 7.3 us with 8 waves against 8.3 us with 16).
int skinny_lwk(int64_t N, int64_t K, int64_t M) {
  const int RG = skinny_rows(N);
  const int64_t nb = K / 256;
  // At one or two activation rows, and at up to four with two or more row
  // groups per workgroup, fewer waves that each take at least 8 blocks beat
  // more waves (M = 4, N = K = 8192: 8 waves 8.6 us, 16 waves 9.4 us; with
  // one row group 8 waves of 4 blocks still win: N = 3072, 6.3 against 7.1).
  const int64_t min_blocks = (M <= 2 || (M <= 4 && RG >= 2)) ? 8 : 1;
  int lwk = 0;
  while ((RG << (lwk + 1)) <= 16 && (min_blocks << (lwk + 1)) <= nb) ++lwk;
  return lwk;
}

// Common launch: RG row groups in all (two matrices of RG / 2 each when
// glu), 2^lwk waves per row group.
hipError_t launch_skinny_rg(const GemmArgs& a, const void* qs2, const void* scales2, bool glu,
                            hipStream_t stream, int RG, int lwk) {
  const int M = (int)a.M, K = (int)a.K;
  const int nb = K / 256;
  const int W = RG << lwk;
  if (lwk < 0 || W > 16) return hipErrorInvalidValue;
  // activation window: as many blocks as fit the LDS budget with their sums
  int nbw = (kXLdsMax - M * kXRowPad - kTrashBytes) / (M * 512 + kBiasBytes);
  if (nbw > nb) nbw = nb;
  if (nbw < 1) nbw = 1;
  const int xbytes = M * (nbw * 512 + kXRowPad) + nbw * kBiasBytes + kTrashBytes;
  int xregion = xbytes > W * 1024 ? xbytes : W * 1024;  // also holds the reduction
  xregion = (xregion + 15) & ~15;
  const int64_t sbytes = scale_lds_bytes(RG, K);
  // staged: every thread holds at most kScaleRegs of the workgroup's scales
  const bool stage = sbytes <= kScaleLdsMax && int64_t{16} * RG * nb <= int64_t{kScaleRegs} * 64 * W;
  const int lds = xregion + (stage ? (int)sbytes : 0);
  if (lds > kLdsLimit) return hipErrorInvalidValue;
  if (glu)
    return stage ? launch_tq2_skinny_s<true, true>(a, qs2, scales2, stream, RG, lwk, nbw, xregion, lds)
                 : launch_tq2_skinny_s<false, true>(a, qs2, scales2, stream, RG, lwk, nbw, xregion, lds);
  return stage ? launch_tq2_skinny_s<true, false>(a, a.qs, a.scales, stream, RG, lwk, nbw, xregion, lds)
               : launch_tq2_skinny_s<false, false>(a, a.qs, a.scales, stream, RG, lwk, nbw, xregion, lds);
}

hipError_t launch_tq2_skinny_lwk(const GemmArgs& a, hipStream_t stream, int lwk) {
  return launch_skinny_rg(a, nullptr, nullptr, false, stream, skinny_rows(a.N), lwk);
}

hipError_t launch_tq2_skinny(const GemmArgs& a, hipStream_t stream) {
  return launch_tq2_skinny_lwk(a, stream, skinny_lwk(a.N, a.K, a.M));
}

// Waves per row group for the fused gate / up product: the same rule as
// skinny_lwk for 2 RGO row groups.
int glu_rows(int64_t N) {
  const int r = skinny_rows(N);
  return r > 8 ? 8 : r;
}

int glu_lwk(int64_t N, int64_t K, int64_t M) {
  const int RG = 2 * glu_rows(N);
  const int64_t nb = K / 256;
  const int64_t min_blocks = M <= 2 ? 8 : 1;
  int lwk = 0;
  while ((RG << (lwk + 1)) <= 16 && (min_blocks << (lwk + 1)) <= nb) ++lwk;
  return lwk;
}

hipError_t launch_tq2_swiglu(const GemmArgs& a, const void* qs_up, const void* scales_up,
                             hipStream_t stream) {
  return launch_skinny_rg(a, qs_up, scales_up, true, stream, 2 * glu_rows(a.N),
                          glu_lwk(a.N, a.K, a.M));
}

}  // namespace tq
