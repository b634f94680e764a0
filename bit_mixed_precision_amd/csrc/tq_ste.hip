// Gradient of a ternary linear with respect to its latent weights.
//
// "The model" (project page "Scaling Laws and Efficient Inference for Ternary
// Language Models") and "Architecture of TriLM and FloatLM" (Spectra page):
// the forward pass multiplies by the effective weights gamma * T, and a
// straight-through estimator hands the gradient back to the floating-point
// latent weights W.  With the quantizer W -> gamma * T taken as the identity
// in the backward pass, the latent weights receive the gradient with respect
// to the effective weights of Y = X (gamma T)^T:
//
//     dW[n][k] = sum_m dY[m][n] * X[m][k]        (dW = dY^T X, fp32)
//
// FP16 inputs, FP32 accumulation and FP32 output (the latent weights are
// kept in floating point); optionally added to an existing gradient.
//
// MI355X design.  The reduction runs over m, the row index of both inputs,
// so every MFMA operand (eight consecutive m of one column) is a column
// piece of a row-major matrix:
//  * a workgroup of 4 waves owns a 256 (n) x 256 (k) tile of dW; wave (wn, wk)
//    owns 128 x 128 of it as 4 x 4 tiles of v_mfma_f32_32x32x16_f16 (256 fp32
//    accumulators per lane), which reads each operand byte from LDS for 64
//    flops;
//  * per step of 32 rows m, the dY and X panels (32 x 256 each) are staged in
//    LDS in their memory order by 16-byte buffer loads (rows past M and
//    columns past N or K read as zero), two steps ahead in registers, two LDS
//    buffers, one barrier per step;
//  * operands come out of LDS with ds_read_b64_tr_b16, gfx950's transposing
//    read: each lane of a 16-lane group names one row and four columns, and
//    lane i receives column i of the four rows; two such reads give the eight
//    consecutive m of one MFMA operand;
//  * the 16-byte pieces of LDS row r sit at slot (piece ^ f(r % 4)) with
//    f = {0, 6, 10, 12}: the four rows of one transposing read then land in
//    distinct banks for both 32 and 64 banks;
//  * dW is written once, 32 consecutive k per half wave (128-byte rows).

#include <type_traits>

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

typedef float float16v __attribute__((ext_vector_type(16)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4v lds_short4;

constexpr int kSteWaves = 4;
constexpr int kSteThreads = kSteWaves * kWave;
constexpr int kTile = 256;           // n and k per workgroup
constexpr int kStepM = 32;           // rows m per step
constexpr int kRowBytes = kTile * 2;  // one LDS row: 256 halves
constexpr int kPanelBytes = kStepM * kRowBytes;  // 16 KB per operand per step
constexpr int kStageBytes = 2 * kPanelBytes;     // dY panel, then X panel
constexpr int kLoads = kStageBytes / 16 / kSteThreads;  // 16-byte pieces per thread per step (8)
constexpr uint32_t kRsrcFlags = 0x00020000u;  // raw buffer, 32-bit data
constexpr uint32_t kOob = 0x80000000u;        // an offset past every range here

__device__ __forceinline__ __amdgpu_buffer_rsrc_t ste_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(((uint64_t)hi << 32) | lo),
                                           (short)0, (int)n, (int)kRsrcFlags);
}

// Slot of 16-byte piece c in LDS row r.
__device__ __forceinline__ int swz(int r, int c) {
  const int f = (0xCA60 >> (4 * (r & 3))) & 15;  // {0, 6, 10, 12}
  return c ^ f;
}

template <int I, int N, class F>
__device__ __forceinline__ void sfor_s(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    sfor_s<I + 1, N>(f);
  }
}

// Grid: one workgroup per 256 x 256 tile; consecutive workgroup ids go to
// different XCDs, so the tile index is blockIdx.x / 8 + (blockIdx.x % 8) *
// per_xcd: each XCD walks a contiguous run of tiles (n-major), whose
// workgroups share dY panels in that XCD's L2.
__global__ __launch_bounds__(kSteThreads) void tq_ste_grad_w_kernel(
    const uint16_t* __restrict__ dY, const uint16_t* __restrict__ X, float* __restrict__ dW, int M,
    int N, int K, int tiles_k, int tiles, int per_xcd, int accumulate) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int b = blockIdx.x;
  const int tile = (b >> 3) + (b & 7) * per_xcd;
  if (tile >= tiles) return;  // workgroup-uniform: padding of the XCD-strided grid
  const int n0 = (tile / tiles_k) * kTile;
  const int k0 = (tile % tiles_k) * kTile;
  const int t = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int lane = t & 63;
  const int wn = wave >> 1, wk = wave & 1;

  const __amdgpu_buffer_rsrc_t ry = ste_rsrc(dY, (uint32_t)((size_t)M * N * 2));
  const __amdgpu_buffer_rsrc_t rx = ste_rsrc(X, (uint32_t)((size_t)M * K * 2));

  // Staging: loads j < kLoads / 2 take dY piece u = t + 256 j of a step, the
  // others X piece u = t + 256 (j - kLoads / 2) (row u / 32, piece u % 32);
  // which matrix is a compile-time fact of j, so every buffer descriptor stays
  // uniform.  Byte offsets of step 0; each step adds 32 rows.
  uint32_t goff[kLoads];
  int lslot[kLoads];
  int grow[kLoads];
  constexpr int kHalf = kLoads / 2;
#pragma unroll
  for (int j = 0; j < kLoads; ++j) {
    const bool xp = j >= kHalf;
    const int v = t + kSteThreads * (xp ? j - kHalf : j);
    const int r = v >> 5, c = v & 31;
    const int col = (xp ? k0 : n0) + 8 * c;
    const int ld = xp ? K : N;
    grow[j] = r;
    goff[j] = col < ld ? (uint32_t)(r * ld + col) * 2u : kOob;
    lslot[j] = (xp ? kPanelBytes : 0) + r * kRowBytes + (swz(r, c) << 4);
  }
  const uint32_t ystep = (uint32_t)kStepM * N * 2u, xstep = (uint32_t)kStepM * K * 2u;
  const int steps = (M + kStepM - 1) / kStepM;

  u32x4 ring[2][kLoads];
  auto issue = [&](int slot, int s) {
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const bool ok = s * kStepM + grow[j] < M && goff[j] != kOob;
      const uint32_t off = ok ? goff[j] + (uint32_t)s * (j >= kHalf ? xstep : ystep) : kOob;
      ring[slot][j] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(j >= kHalf ? rx : ry, off, 0, 0));
    }
  };
  auto stage = [&](int slot, int buf) {
    unsigned char* base = smem + buf * kStageBytes;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) *reinterpret_cast<u32x4*>(base + lslot[j]) = ring[slot][j];
  };

  // Transposing reads.  Lane group g16 = lane / 16 covers 16 columns
  // (16 (g16 & 1) ..) and rows 8 (g16 >> 1) .. + 7 of a 16-row k-step; source
  // lane s names row (s >> 2) (+ 4 for the second read), columns 4 (s & 3).
  // Every row it names has the same row % 4, so a tile's piece slot is one
  // value per lane; rows then add whole LDS rows (immediate offsets).
  const int g16 = lane >> 4;
  const int s16 = lane & 15;
  const int trow = 8 * (g16 >> 1) + (s16 >> 2);  // + 16 h for k-step h, + 4 for the second read
  const int tcol = 16 * (g16 & 1) + 4 * (s16 & 3);
  int abase[4], bbase[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int ca = 128 * wn + 32 * i + tcol, cb = 128 * wk + 32 * i + tcol;
    abase[i] = trow * kRowBytes + (swz(trow, ca >> 3) << 4) + ((ca & 7) << 1);
    bbase[i] = kPanelBytes + trow * kRowBytes + (swz(trow, cb >> 3) << 4) + ((cb & 7) << 1);
  }
  auto operand = [&](int buf, int base, int h) {
    const unsigned char* p = smem + buf * kStageBytes + base + 16 * h * kRowBytes;
    const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)p);
    const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(p + 4 * kRowBytes));
    const short4v v[2] = {lo, hi};
    return __builtin_bit_cast(half8, v);
  };

  float16v acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = float16v{};

  // Step s computes from LDS buffer s & 1, then stages step s + 1 (held in
  // ring slot (s + 1) & 1, loaded two steps earlier) into the other buffer,
  // whose reads (step s - 1) ended before the previous barrier, and refills
  // that slot with step s + 3.  Two steps per loop trip keep every slot and
  // buffer index a compile-time constant.
  auto step = [&](int s, auto parity) {
    constexpr int P = decltype(parity)::value;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      half8 A[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) A[i] = operand(P, abase[i], h);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const half8 B = operand(P, bbase[j], h);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[i], B, acc[i][j], 0, 0, 0);
      }
    }
    if (s + 1 < steps) {
      stage(P ^ 1, P ^ 1);
      if (s + 3 < steps) issue(P ^ 1, s + 3);
    }
    __syncthreads();
  };
  if (steps > 0) {
    issue(0, 0);
    if (steps > 1) issue(1, 1);
    stage(0, 0);
    if (steps > 2) issue(0, 2);
    __syncthreads();
  }
  int s = 0;
  for (; s + 1 < steps; s += 2) {
    step(s, std::integral_constant<int, 0>{});
    step(s + 1, std::integral_constant<int, 1>{});
  }
  if (s < steps) step(s, std::integral_constant<int, 0>{});

  // dW tile: register i of tile (a, c) is row 8 (i / 4) + 4 (lane / 32) + i % 4,
  // column lane % 32 of the 32 x 32 block.  With accumulate, a tile's 16
  // earlier values are loaded together before any is written back.
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int k = k0 + 128 * wk + 32 * c + (lane & 31);
      const int nb = n0 + 128 * wn + 32 * a + 4 * (lane >> 5);
      float* col = dW + k;
      float add[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int n = nb + 8 * (i >> 2) + (i & 3);
        add[i] = accumulate && n < N && k < K ? col[(size_t)n * K] : 0.f;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int n = nb + 8 * (i >> 2) + (i & 3);
        if (n < N && k < K) col[(size_t)n * K] = accumulate ? add[i] + acc[a][c][i] : acc[a][c][i];
      }
    }
}

}  // namespace

int64_t ste_tiles(int64_t N, int64_t K) {
  return ((N + kTile - 1) / kTile) * ((K + kTile - 1) / kTile);
}

hipError_t launch_ste_grad_w(const void* dY, const void* X, float* dW, int64_t M, int64_t N,
                             int64_t K, int accumulate, hipStream_t stream) {
  static std::atomic<uint64_t> lds_set{0};
  const int lds = 2 * kStageBytes;
  hipError_t e = lds_limit_once(reinterpret_cast<const void*>(tq_ste_grad_w_kernel), lds, lds_set);
  if (e != hipSuccess) return e;
  const int64_t tiles_k = (K + kTile - 1) / kTile;
  const int64_t tiles = ste_tiles(N, K);
  const int64_t per_xcd = (tiles + 7) / 8;
  hipLaunchKernelGGL(tq_ste_grad_w_kernel, dim3((unsigned)(8 * per_xcd)), dim3(kSteThreads), lds,
                     stream, static_cast<const uint16_t*>(dY), static_cast<const uint16_t*>(X), dW,
                     (int)M, (int)N, (int)K, (int)tiles_k, (int)tiles, (int)per_xcd, accumulate);
  return hipGetLastError();
}

}  // namespace tq
