// Skinny kernel for 2-bit weights (M <= 32): Y = X (s . T)^T with the weights
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
//  * its waves take pairs of 256-weight blocks round robin; a pair comes as
//    two loads of 8 rows x 128 contiguous bytes (whole cache lines) through
//    a ring of register buffers, and one DPP rotate per dword puts it in MFMA
//    operand order;
//  * one v_and_b32 per pair of weights is the whole decode: masking a 2-bit
//    field that sits at mantissa bits 2p..2p+1 of an fp16 with a zero exponent
//    leaves the exact subnormal d' 4^p 2^-24, which the MFMA multiplies exactly
//    (it keeps fp16 subnormals).  Fields at p = 1 and p = 3 meet activations
//    pre-scaled by 1/4 in LDS, and the MFMAs of p = 0, 1 and of p = 2, 3 run in
//    two accumulator chains combined as C0 + C1 / 16, so every activation is
//    scaled by 1 or 1/4 only (exact above the fp16 subnormal range);
//  * the shift d = d' - 1 costs no per-weight work: the sum of the block's
//    activations, taken in fp32 while staging them, seeds the first chain;
//  * the multiply-accumulate runs on v_mfma_f32_16x16x32_f16 with one or two
//    tiles of 16 activation rows as the A operand; per block the two chains
//    are combined and scaled once (8 FMAs per lane per 16 rows);
//  * activations, their block sums and the block scales are staged once per
//    window of K (eight threads per 256 activations of a row, whose sum comes
//    from v_dot2_f32_f16 and three DPP adds; neighbouring threads swap pairs so
//    that every LDS write is a dword), the first window's loads issued before
//    the first weight loads so that the wait for them does not wait for the
//    weights, later windows' loaded into registers a window ahead, with the
//    weight ring running on across window boundaries; per-wave set-up is kept
//    to shifts and masks (it is a large part of the time at one or two
//    activation rows);
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
// the LDS copy stores as 16 contiguous bytes: Xt[m][block][g][c][s], the
// blocks of a row kBlkStride bytes apart: the 512 bytes plus 32, so that the
// eight staging units of a wave (neighbouring blocks of one row) write to
// eight different groups of eight banks.
// Chain of class c: 0 for p in {0, 1}, 1 for p in {2, 3}; a chain-0 product
// is x d' 2^-24, a chain-1 product 16 x d' 2^-24.
// ----------------------------------------------------------------------------

constexpr int kXRowPad = 16;          // bytes between LDS rows of Xt (bank spread)
constexpr int kBlkStride = 512 + 32;  // bytes between the blocks of a row of Xt
constexpr int kBiasBytes = 64;        // per block of the window and 16 rows: fp32 row sums
constexpr int kScaleLdsMax = 24 * 1024;
constexpr int kScaleLdsMaxGlu = 32 * 1024;  // the gate / up kernel's 2 x RG / 2 rows
constexpr int kLdsLimit = 160 * 1024;
constexpr int kScaleRegs = 4;         // block scales per thread loaded ahead
constexpr int kScaleRegsGlu = 8;      // the same for the gate / up kernel
constexpr int kWavesMt2 = 16;        // waves per workgroup with two m tiles
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
// Threads s and s ^ 1 (all lanes active) swap their pairs with one DPP move,
// so that each writes a dword: the even one class 2 i at slots s, s + 1, the
// odd one class 2 i + 1 at slots s - 1, s.
__device__ __forceinline__ void piece_store(const u32x4 (&v)[4], bool ok, PiecePos p,
                                            unsigned char* xs, float* bias, unsigned char* trash,
                                            int xstride, int s, int bstride) {
  const half2v quarter = {(_Float16)1.0f, (_Float16)0.25f};
  const half2v four = {(_Float16)1.0f, (_Float16)4.0f};
  float part = 0.f;
  const int odd = s & 1;
  const uint32_t sel = odd ? 0x03020706u : 0x05040100u;  // (its hi, own hi) : (own lo, its lo)
  unsigned char* d = (ok ? xs + p.m * xstride + p.bw * kBlkStride : trash) + 16 * odd + 2 * (s & ~1);
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // activations 8 s + 2 i, 8 s + 2 i + 1 of piece g: classes 2 i, 2 i + 1
      const uint32_t xv = v[g][i];  // (a bit cast of the vector element itself reads element 0)
      const half2v a = __builtin_bit_cast(half2v, xv) * quarter;
      part = __builtin_amdgcn_fdot2(a, four, part, false);
      const uint32_t ab = __builtin_bit_cast(uint32_t, a);
      // quad_perm [1, 0, 3, 2]: the pair of thread s ^ 1
      const uint32_t other = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ab, 0xB1, 0xf, 0xf, false);
      *reinterpret_cast<uint32_t*>(d + g * 128 + (2 * i) * 16) = perm(other, ab, sel);
    }
  }
  part += dpp_f32<0xB1>(part);   // quad_perm [1, 0, 3, 2]
  part += dpp_f32<0x4E>(part);   // quad_perm [2, 3, 0, 1]
  part += dpp_f32<0x141>(part);  // row_half_mirror: the eight threads of the unit
  float* bd = ok ? bias + p.bw * bstride + p.m : reinterpret_cast<float*>(trash + kTrashX);
  if (s == 0) *bd = part * -0x1p-24f;
}

// A workgroup owns RG groups of 16 weight rows and all of K.  Its RG * WK
// waves (WK = 2^lwk) are light: wave w works on row group w / WK and on the
// pairs of blocks c = w % WK + WK * i of K, so several waves per SIMD
// interleave decode, MFMA and memory waits.  MT tiles of 16 activation rows
// share every decoded weight operand.  Each wave keeps D / 2 pairs of blocks
// in flight in a register ring; the loop body is straight-line except for
// the last group of steps, which issues no loads, so the compiler's wait
// before each decode covers exactly the oldest pair.  STAGE: the block scales of the
// workgroup's rows are copied to LDS as fp32 (else each block's scale comes
// with its weights).  Rows past N and activation rows past M read valid dummy
// data whose results are never written (MFMA rows and columns do not mix).
//
// RF: the first ring loads go out before the wait for the first window's
// activations (else after their LDS stores, so that they do not compete with
// a large activation copy).
//
// GLU: the workgroup's first RG / 2 row groups read the gate matrix (qs,
// scales), the others the same rows of the up matrix (qs2, scales2), and the
// output is silu(g) u of the two products (SwiGLU of the decode step), one
// fp16 rounding.
template <int D, bool STAGE, bool GLU, int MT, bool RF>
__global__ __launch_bounds__(MT == 1 ? 1024 : 64 * kWavesMt2) void tq2_skinny_kernel(
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
  const int xstride = nbw * kBlkStride + kXRowPad;
  const size_t row_bytes = (size_t)(K >> 2);
  constexpr int BS = 16 * MT;  // row sums per block
  float* bias = reinterpret_cast<float*>(smem + M * xstride);
  unsigned char* trash = reinterpret_cast<unsigned char*>(bias + BS * nbw);
  float* sc_lds = reinterpret_cast<float*>(smem + xregion);

  const int nrow = 16 * rgo + li < rows ? 16 * rgo + li : 0;  // row of this lane in the tile
  const uint16_t* srow = (up ? scales2 : scales) + (size_t)(n_base + nrow) * nb;
  // Weights come in pairs of blocks, each 16-row pair as two loads of 8 rows
  // x 128 contiguous bytes (whole cache lines; measured 15% faster to stream
  // than 16 rows x 64 bytes).  Load A: rows 0..7 of the group, lane (n, g)
  // taking piece g of block 0 for n < 8 and piece 4 + g (block 1) of row
  // n - 8 for n >= 8; load B the same for rows 8..15 with the halves swapped.
  // Block 0 in MFMA order is then A or B by lane, block 1 the other one
  // rotated by 8 lanes (one DPP move).  The loads are buffer loads: one
  // resource per wave over its row group (from a valid row: a group past N
  // reads the tile's last row, and rows past N in a group read its first),
  // lane offsets fixed for the whole kernel and the pair's offset in a scalar
  // register, so a load costs no vector instruction (measured 2% faster at
  // N = 28672, 4-5% for the gate / up product).  With an odd block count the
  // last pair's second half reads past the row (the next row's bytes, or
  // zeros past the group's last row) and is never used.
  const uint8_t* wq = up ? qs2 : qs;
  const int ra = 16 * rgo + (li & 7), rb = ra + 8;
  const int pa = li < 8 ? g : 4 + g, pb = li < 8 ? 4 + g : g;
  const int rg0 = 16 * rgo < rows ? 16 * rgo : rows - 1;
  const int rin = rows - rg0 < 16 ? rows - rg0 : 16;  // rows of the group in the matrix
  const auto wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(wq) + (size_t)(n_base + rg0) * row_bytes, 0, rin * (int)row_bytes,
      kBufferWord3);
  const int voffa = (ra < rows ? ra - rg0 : 0) * (int)row_bytes + 16 * pa;  // < 2^22
  const int voffb = (rb < rows ? rb - rg0 : 0) * (int)row_bytes + 16 * pb;
  const int npairs = (nb + 1) >> 1;
  // A operand rows of m tile t: activation rows 16 t + li (rows past M read
  // row M - 1; their results are never written)
  const unsigned char* xa[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t)
    xa[t] = smem + (16 * t + li < M ? 16 * t + li : M - 1) * xstride + g * 128;
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

  float4v acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = float4v{0.f, 0.f, 0.f, 0.f};
  constexpr int P = D / 2;  // pairs of blocks in flight
  u32x4 wa[P], wb[P];
  uint16_t sbuf[P][2];

  // Weights are read once: non-temporal loads (the nt bit of the cache
  // policy; measured 3-5% faster at M <= 8 on both layer shapes than plain
  // loads; the TQ1 kernel's 8-byte loads were slower with the hint, so it
  // keeps plain ones).  Pair c holds blocks 2c and 2c + 1.
  auto load = [&](int d, int c) {
    typedef int v4i __attribute__((ext_vector_type(4)));
    constexpr int kNt = 2;  // cache policy: non-temporal
    wa[d] = __builtin_bit_cast(u32x4, (v4i)__builtin_amdgcn_raw_buffer_load_b128(wrsrc, voffa, 128 * c, kNt));
    wb[d] = __builtin_bit_cast(u32x4, (v4i)__builtin_amdgcn_raw_buffer_load_b128(wrsrc, voffb, 128 * c, kNt));
    if constexpr (!STAGE) {
      sbuf[d][0] = srow[2 * c];
      sbuf[d][1] = srow[2 * c + 1 < nb ? 2 * c + 1 : 2 * c];
    }
    __builtin_amdgcn_sched_barrier(0);  // keep the prefetch where it is
  };
  auto compute = [&](const u32x4 w, uint16_t sb, int b, int bw) {
    const u32x4 w8 = shift8(w);
    const float sc = STAGE ? sc_lds[sc_row + b] : h2f(sb);
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      float4v c0 = *reinterpret_cast<const float4v*>(ba + BS * bw + 16 * t);  // -2^-24 (row sums)
      float4v c1 = {0.f, 0.f, 0.f, 0.f};
      const unsigned char* xb = xa[t] + bw * kBlkStride;
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
      for (int i = 0; i < 4; ++i)
        acc[t][i] = __builtin_fmaf(sc, __builtin_fmaf(c1[i], 0.0625f, c0[i]), acc[t][i]);
    }
  };
  auto compute_pair = [&](int d, int c, int bw0) {
    u32x4 w0, w1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w0[i] = li < 8 ? wa[d][i] : wb[d][i];
      const uint32_t t = li < 8 ? wb[d][i] : wa[d][i];
      w1[i] = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)t, 0x128, 0xf, 0xf, false);  // row_ror:8
    }
    compute(w0, sbuf[d][0], 2 * c, bw0);
    if (2 * c + 1 < nb) compute(w1, sbuf[d][1], 2 * c + 1, bw0 + 1);  // the same in every lane
  };

  // Windows of nbw blocks (the last may be shorter).  nbw is a multiple of
  // 2 WK unless one window holds all of K, so in every full window each wave
  // takes the same nbw / (2 WK) pairs: the waves walk one sequence of S steps,
  // step s being pair wk + WK s, in window s / spw, and meet at the same
  // window boundaries.  The weight ring runs on across the boundaries (the
  // next window's first blocks are in flight while it is staged), and the
  // first two staging batches of a window are loaded into registers one
  // window ahead, so a boundary costs two barriers and the LDS stores.
  const int per_batch = T >> 3;  // staging units per batch (eight threads each)
  const int nwin = (nb + nbw - 1) / nbw;
  const int spw = (nbw >> 1) >> lwk;            // steps (pairs) per full window
  const int S = (npairs + WK - 1) >> lwk;       // steps of every wave
  const int J = (npairs - wk + WK - 1) >> lwk;  // steps with a pair for this wave
  auto gpair = [&](int s) { return wk + WK * (s < J ? s : J - 1); };

  // Staging unit u of window w = (activation row u / nbw_w, window block
  // u % nbw_w); thread t takes units t / 8 + per_batch b, b = 0, 1, ..., whose
  // positions step by (dm, dbw) per batch without divisions.  Units past the
  // window read row 0 and are not stored (or go to the trash area).
  struct XBatch {
    u32x4 v[4];
    PiecePos pos;
    bool ok;
  };
  XBatch xr[2];
  auto x_step = [&](PiecePos& pos, int nbw_w, int dm, int dbw) {
    pos.bw += dbw;
    pos.m += dm;
    if (pos.bw >= nbw_w) {
      pos.bw -= nbw_w;
      ++pos.m;
    }
  };
  auto x_issue = [&](int w) {  // loads of the first two batches of window w
    const int nbw_w = min(nbw, nb - w * nbw);
    const uint16_t* xw = X + 256 * w * nbw + 8 * (threadIdx.x & 7);
    const int dm = per_batch / nbw_w;
    const int dbw = per_batch - dm * nbw_w;
    PiecePos pos{0, (int)(threadIdx.x >> 3)};
    while (pos.bw >= nbw_w) {
      pos.bw -= nbw_w;
      ++pos.m;
    }
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      xr[b].pos = pos;
      xr[b].ok = pos.m < M;
      piece_load(xr[b].v, xw, pos, xr[b].ok, K);
      x_step(pos, nbw_w, dm, dbw);
    }
  };
  auto x_store = [&](int w) {  // window w to LDS: the two batches held, then the rest
    const int nbw_w = min(nbw, nb - w * nbw);
    const uint16_t* xw = X + 256 * w * nbw + 8 * (threadIdx.x & 7);
    const int dm = per_batch / nbw_w;
    const int dbw = per_batch - dm * nbw_w;
    // waves without a unit skip the store (their trash writes would all hit
    // the same LDS banks)
#pragma unroll
    for (int b = 0; b < 2; ++b)
      if (__any(xr[b].ok)) piece_store(xr[b].v, xr[b].ok, xr[b].pos, smem, bias, trash, xstride, threadIdx.x & 7, BS);
    PiecePos pos = xr[1].pos;
    x_step(pos, nbw_w, dm, dbw);
    for (int q = 2 * per_batch; q < M * nbw_w; q += per_batch) {
      u32x4 v[4];
      const bool ok = pos.m < M;
      piece_load(v, xw, pos, ok, K);
      if (__any(ok)) piece_store(v, ok, pos, smem, bias, trash, xstride, threadIdx.x & 7, BS);
      x_step(pos, nbw_w, dm, dbw);
    }
  };

  // Window 0 and the block scales; the first ring loads go out after the
  // window's and the scales' loads, so the wait for those does not cover them.
  x_issue(0);
  constexpr int SR = GLU ? kScaleRegsGlu : kScaleRegs;
  uint16_t sreg[SR];
  if constexpr (STAGE) {
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      int e = threadIdx.x + r * T;
      e = e < ns_all ? e : 0;
      asm volatile("" : "+v"(e));  // keep the load here (not hoisted ahead of the window's)
      sreg[r] = e < ns ? ssrc[e] : ssrc2[e - ns];
    }
  }
  auto ring_start = [&] {
    static_for<0, P>([&](auto dd) { load(decltype(dd)::value, gpair(decltype(dd)::value)); });
  };
  if constexpr (RF) ring_start();
  x_store(0);
  if constexpr (!RF) ring_start();
  if constexpr (STAGE) {
#pragma unroll
    for (int r = 0; r < SR; ++r) {
      const int e = threadIdx.x + r * T;
      // row of scale e: exact in fp32, since e < 2^14 keeps the rounding
      // error far below the 0.5 / nb margin to the nearest integer
      const int row = (int)(((float)e + 0.5f) * inv_nb);
      if (e < ns_all) sc_lds[e + row] = h2f(sreg[r]);
    }
  }
  __syncthreads();
  if (nwin > 1) x_issue(1);

  int w = 0;                                // window being computed
  int next_b = nwin > 1 ? spw : S;          // first step of the next window
  auto step = [&](auto dd, int s, auto with_load) {
    constexpr int d = decltype(dd)::value;
    if (s == next_b) {  // the same step in every wave
      ++w;
      __syncthreads();  // window w - 1 consumed
      x_store(w);
      __syncthreads();
      if (w + 1 < nwin) x_issue(w + 1);
      next_b = w + 1 < nwin ? next_b + spw : S;
    }
    if (s < J) compute_pair(d, gpair(s), 2 * gpair(s) - w * nbw);
    if constexpr (decltype(with_load)::value) load(d, gpair(s + P));
  };
  int j = 0;
  for (; j + P < S; j += P)
    static_for<0, P>([&](auto dd) { step(dd, j + decltype(dd)::value, std::true_type{}); });
  // last group: no loads past the steps
  static_for<0, P>([&](auto dd) {
    if (j + decltype(dd)::value < S) step(dd, j + decltype(dd)::value, std::false_type{});
  });

  // Partial sums: every wave writes its MT tiles of 16 x 16 to LDS (reusing
  // the activation window); each tile element sums the WK waves of its row
  // group.
  __syncthreads();
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int t = 0; t < MT; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * MT + t) * 256 + i * 64 + lane] = acc[t][i];
  __syncthreads();
  for (int q = threadIdx.x; q < RGO * MT * 256; q += T) {
    const int r = q / (MT * 256);  // MT is 1 or 2: a shift
    const int t = (q >> 8) & (MT - 1);
    const int e = q & 255;
    const int l = e & 63;
    const int m = 16 * t + 4 * (l >> 4) + (e >> 6);
    const int n = 16 * r + (l & 15);
    if (m < M && n < rows) {
      float sum = 0.f;
      for (int k = 0; k < WK; ++k) sum += red[((r * WK + k) * MT + t) * 256 + e];
      sum *= 0x1p24f;
      if constexpr (GLU) {
        float u = 0.f;
        for (int k = 0; k < WK; ++k) u += red[(((RGO + r) * WK + k) * MT + t) * 256 + e];
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
constexpr int kDepthMt2 = 2;  // (two m tiles: one pair in flight, within 128 VGPRs)

template <bool STAGE, bool GLU, int MT, bool RF>
hipError_t launch_tq2_skinny_s(const GemmArgs& a, const void* qs2, const void* scales2,
                               hipStream_t stream, int RG, int lwk, int nbw, int xregion, int lds) {
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = lds_limit_once(
      reinterpret_cast<const void*>(tq2_skinny_kernel<MT == 1 ? kDepth : kDepthMt2, STAGE, GLU, MT, RF>),
      kLdsLimit, lds_set);
  if (e != hipSuccess) return e;
  const int RGO = GLU ? RG / 2 : RG;
  const int64_t groups = (a.N + 16 * RGO - 1) / (16 * RGO);
  hipLaunchKernelGGL((tq2_skinny_kernel<MT == 1 ? kDepth : kDepthMt2, STAGE, GLU, MT, RF>), dim3((unsigned)groups),
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

int skinny_depth(int64_t M) { return M > 16 ? kDepthMt2 : kDepth; }

// The first ring loads go out before the first window's activation wait when
// the copy is small (under 48 KB of activations), else after its LDS stores:
// a large copy then reaches LDS without the weight stream in its way.
// Measured (us, ring first / after): M = 8, N = K = 8192 9.0 / 7.8; M = 16,
// N = 28672 21.2 / 20.7; K = 28672, N = 8192, M = 1 16.2 / 15.6; the gate /
// up product at M = 16 35.2 / 34.2; and the other way round for small copies:
// 3072 x 3072 4.07 / 4.29, K = 8192 with N = 3072 5.42 / 5.61 (M = 1).
bool skinny_ring_first(int64_t M, int64_t K) { return M * K < 24576; }

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
  // On short rows (K < 8192) that leaves too few waves to cover the first
  // loads' latency; there 2 blocks per wave (M = 1: K = N = 3072 6.45 ->
  // 4.46 us, K = 3072, N = 8192 6.85 -> 5.09 us, K = N = 1024 3.47 -> 3.13 us;
  // one block per wave was slower at K = 3072, N = 8192: 6.03 us).
  const int64_t few = nb >= 32 ? 8 : 2;
  const int64_t min_blocks = (M <= 2 || (M <= 4 && RG >= 2)) ? few : 1;
  int lwk = 0;
  while ((RG << (lwk + 1)) <= 16 && (min_blocks << (lwk + 1)) <= nb) ++lwk;
  return lwk;
}

// Launch plan for RG row groups and at most 2^lwk waves per row group:
// every wave takes at least one pair of blocks, and when the activations
// need windows, a window holds whole steps (a pair of blocks for each wave of
// a row group, so that the waves meet at the same window boundaries); fewer
// waves per row group when it cannot.  Block scales are staged in LDS when
// every thread holds at most kScaleRegs (kScaleRegsGlu) of them.  The gate /
// up kernel stages up to 32 KB (14 row groups at N = 28672: 29.5 KB;
// measured 15-18% faster than loading each block's scales with its weights),
// the plain one up to 24 KB (eight registers, loaded only as far as needed,
// measured 3-6% slower for it at other shapes).
struct SkinnyPlan {
  int lwk, W, fit, unit;
  bool stage;
};

bool plan_skinny(int M, int K, int RG, int lwk, bool glu, SkinnyPlan* p) {
  const int nb = K / 256;
  const int mt = M > 16 ? 2 : 1;
  const int npairs = (nb + 1) / 2;
  if (lwk < 0) return false;
  while (lwk > 0 && (1 << lwk) > npairs) --lwk;
  const int64_t sbytes = scale_lds_bytes(RG, K);
  const int sregs = glu ? kScaleRegsGlu : kScaleRegs;
  const int64_t smax = glu ? kScaleLdsMaxGlu : kScaleLdsMax;
  const int wmax = mt == 1 ? 16 : kWavesMt2;
  while (lwk > 0 && (RG << lwk) > wmax) --lwk;
  for (;; --lwk) {
    p->lwk = lwk;
    p->W = RG << lwk;
    if (p->W > wmax) return false;
    p->stage = sbytes <= smax && int64_t{16} * RG * nb <= int64_t{sregs} * 64 * p->W;
    const int budget = kLdsLimit - (p->stage ? (int)sbytes : 0);
    p->fit = (budget - M * kXRowPad - kTrashBytes) / (M * kBlkStride + mt * kBiasBytes);
    p->unit = 2 << lwk;
    if (p->fit >= nb || p->fit >= p->unit || lwk == 0) return true;
  }
}

template <int MT, bool RF>
hipError_t launch_skinny_mt(const GemmArgs& a, const void* qs2, const void* scales2, bool glu,
                            bool stage, hipStream_t stream, int RG, int lwk, int nbw, int xregion,
                            int lds) {
  if constexpr (MT == 1) {  // the gate / up product serves M <= 16 only
    if (glu)
      return stage ? launch_tq2_skinny_s<true, true, MT, RF>(a, qs2, scales2, stream, RG, lwk, nbw, xregion, lds)
                   : launch_tq2_skinny_s<false, true, MT, RF>(a, qs2, scales2, stream, RG, lwk, nbw, xregion, lds);
  } else {
    if (glu) return hipErrorInvalidValue;
  }
  return stage ? launch_tq2_skinny_s<true, false, MT, RF>(a, a.qs, a.scales, stream, RG, lwk, nbw, xregion, lds)
               : launch_tq2_skinny_s<false, false, MT, RF>(a, a.qs, a.scales, stream, RG, lwk, nbw, xregion, lds);
}

// Common launch: RG row groups in all (two matrices of RG / 2 each when
// glu), 2^lwk waves per row group at most.
hipError_t launch_skinny_rg(const GemmArgs& a, const void* qs2, const void* scales2, bool glu,
                            hipStream_t stream, int RG, int lwk_max) {
  const int M = (int)a.M, K = (int)a.K;
  const int nb = K / 256;
  if (M > 32) return hipErrorInvalidValue;
  if (M > 16 && RG > kWavesMt2) RG = kWavesMt2;  // more, smaller workgroups (RG stays even)
  SkinnyPlan p;
  if (!plan_skinny(M, K, RG, lwk_max, glu, &p)) return hipErrorInvalidValue;
  const int lwk = p.lwk, W = p.W, fit = p.fit, unit = p.unit;
  const bool stage = p.stage;
  const int64_t sbytes = scale_lds_bytes(RG, K);
  // activation window: all of K when it fits the LDS left by the staged
  // scales; else the fewest windows that fit, each a multiple of a step
  int nbw = nb;
  if (fit < nb) {
    const int nwin = (nb + fit - 1) / fit;
    nbw = ((nb + nwin - 1) / nwin + unit - 1) / unit * unit;
    if (nbw > fit) nbw = fit / unit * unit;
    if (nbw < unit) return hipErrorInvalidValue;
  }
  const int mt = M > 16 ? 2 : 1;
  const int xbytes = M * (nbw * kBlkStride + kXRowPad) + nbw * mt * kBiasBytes + kTrashBytes;
  int xregion = xbytes > W * 1024 * mt ? xbytes : W * 1024 * mt;  // also holds the reduction
  xregion = (xregion + 15) & ~15;
  const int lds = xregion + (stage ? (int)sbytes : 0);
  if (lds > kLdsLimit) return hipErrorInvalidValue;
  const bool rf = skinny_ring_first(M, K);
  if (mt == 1)
    return rf ? launch_skinny_mt<1, true>(a, qs2, scales2, glu, stage, stream, RG, lwk, nbw, xregion, lds)
              : launch_skinny_mt<1, false>(a, qs2, scales2, glu, stage, stream, RG, lwk, nbw, xregion, lds);
  return rf ? launch_skinny_mt<2, true>(a, qs2, scales2, glu, stage, stream, RG, lwk, nbw, xregion, lds)
            : launch_skinny_mt<2, false>(a, qs2, scales2, glu, stage, stream, RG, lwk, nbw, xregion, lds);
}

int skinny_stage(int64_t N, int64_t K, int64_t M) {
  SkinnyPlan p;
  int RG = skinny_rows(N);
  if (M > 16 && RG > kWavesMt2) RG = kWavesMt2;
  return plan_skinny((int)M, (int)K, RG, skinny_lwk(N, K, M), false, &p) && p.stage
             ? 1
             : 0;
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
  const int64_t min_blocks = M <= 2 ? (nb >= 32 ? 8 : 2) : 1;  // as skinny_lwk
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
