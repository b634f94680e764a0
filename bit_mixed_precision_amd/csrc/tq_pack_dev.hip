// On-device ternarization and packing (the step before the product):
// gamma = eps + mean|W| over the whole matrix, T = round(clip(W / gamma, -1, 1)),
// then the TQ2 or TQ1 packing with fp16(gamma) in every block scale.
//
// Follows the project page "Scaling Laws and Efficient Inference for Ternary
// Language Models": "The model" (steps 1-2) for the ternarization, "Packing
// ternary weights" for both packings, "Fast inference on CPUs" for the
// 256-weight scale block.  The results are the host packer's bit for bit: the
// sum of |W| is exact (integer sums per fp32 exponent, rounded once to fp64),
// the quotient W / gamma is the same correctly rounded fp64 division, and the
// ties of round() go to even (only |q| > 1/2 leaves zero).
//
// Four kernels on one stream, no host round trip:
//  * tq_abs_sum_kernel: every workgroup adds the 24-bit significands of its
//    elements into 256 per-exponent 64-bit buckets in LDS (four copies per
//    wave, so that lanes sharing an exponent seldom share an address), then adds each
//    bucket into a 128-bit total in the workspace (64-bit integer atomics, the
//    carry counted in the high word); integer sums do not depend on the order,
//    so the total is the same on every run (a small kernel zeroes it first);
//  * tq_gamma_kernel: one workgroup adds the 32-bit pieces of the 255 shifted
//    totals into the 12 column sums of a 384-bit integer (LDS integer
//    atomics, order-free), one thread carries and rounds it to fp64 (nearest,
//    ties to even), forms gamma and its fp16 bits, and a status
//    (TQ_ERR_VALUE for a non-finite latent or gamma);
//  * tq_pack_tq2_dev_kernel: one output dword (16 weights) per thread,
//    grid-stride; tq_pack_tq1_dev_kernel: 1024 TQ1 bytes of a row per
//    workgroup, their latents staged in LDS by coalesced loads.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "tq.h"
#include "tq_common.h"

namespace {

constexpr int kSumThreads = 256;
constexpr int kSumWaves = kSumThreads / 64;
constexpr int64_t kElemsPerGroup = int64_t(1) << 16;  // target elements per sum workgroup
constexpr int64_t kMaxGroups = 2048;

// Workspace layout: [info: 64 B][lo: uint64 [256]][hi: uint64 [256]][bad: int32].
// info holds gamma (fp64), its fp16 bits and the status.
struct Info {
  double gamma;
  uint32_t h;
  int32_t status;
};

int64_t sum_groups(int64_t N, int64_t K) {
  const int64_t total = N * K;
  int64_t g = (total + kElemsPerGroup - 1) / kElemsPerGroup;
  if (g < 1) g = 1;
  if (g > kMaxGroups) g = kMaxGroups;
  return g;
}

constexpr int64_t kLoOff = 64;
constexpr int64_t kHiOff = kLoOff + 256 * 8;
constexpr int64_t kBadOff = kHiOff + 256 * 8;
constexpr int64_t kWorkspace = kBadOff + 64;

__global__ void tq_sum_init_kernel(unsigned long long* lo, unsigned long long* hi, int* bad) {
  const int e = threadIdx.x;
  lo[e] = 0ull;
  hi[e] = 0ull;
  if (e == 0) *bad = 0;
}

// Four copies of the 256 buckets per wave, picked by lane % 4: latents
// concentrate on a few exponents, and lanes adding to one LDS address in the
// same instruction are serialized.  A copy's stride of 260 entries puts the
// copies of a bucket in different banks.  Each thread keeps four 16-byte
// loads in flight.
constexpr int kCopies = 4;
constexpr int kCopyStride = 260;
constexpr int kSumUnroll = 4;

__global__ __launch_bounds__(kSumThreads) void tq_abs_sum_kernel(const float* __restrict__ W,
                                                                 int64_t total,
                                                                 unsigned long long* lo,
                                                                 unsigned long long* hi,
                                                                 int* bad_out) {
  __shared__ unsigned long long bk[kSumWaves * kCopies * kCopyStride];
  __shared__ int bad;
  for (int i = threadIdx.x; i < kSumWaves * kCopies * kCopyStride; i += blockDim.x) bk[i] = 0ull;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  unsigned long long* mine =
      bk + ((threadIdx.x >> 6) * kCopies + (threadIdx.x & (kCopies - 1))) * kCopyStride;
  int my_bad = 0;
  const int64_t q4 = total / 4;  // total is a multiple of 256
  const float4* W4 = reinterpret_cast<const float4*>(W);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < q4;
       i += kSumUnroll * stride) {
    float4 v[kSumUnroll];
#pragma unroll
    for (int r = 0; r < kSumUnroll; ++r)
      v[r] = i + r * stride < q4 ? W4[i + r * stride] : float4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < kSumUnroll; ++r) {
      const float vs[4] = {v[r].x, v[r].y, v[r].z, v[r].w};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t u = __float_as_uint(vs[t]);
        const uint32_t e = (u >> 23) & 0xFFu;
        uint32_t m = u & 0x7FFFFFu;
        if (e == 0xFFu) my_bad = 1;
        if (e) m |= 0x800000u;
        if (m) atomicAdd(&mine[e], (unsigned long long)m);
      }
    }
  }
  if (my_bad) atomicOr(&bad, 1);
  __syncthreads();
  for (int e = threadIdx.x; e < 256; e += blockDim.x) {
    unsigned long long s = 0;
    for (int c = 0; c < kSumWaves * kCopies; ++c) s += bk[c * kCopyStride + e];  // < 2^58
    if (s) {
      const unsigned long long old = atomicAdd(&lo[e], s);
      if (old + s < old) atomicAdd(&hi[e], 1ull);  // this add carried out of 64 bits
    }
  }
  if (threadIdx.x == 0 && bad) atomicOr(bad_out, 1);
}

// The exact total as a 384-bit integer: 12 column sums of 32-bit pieces
// (each column below 2^41, so 64-bit), then carries.  Every index is a
// compile-time constant so that the limbs stay in registers.
constexpr int kLimbs = 12;

// col[li..li+2] += the 32-bit pieces of v << shift (shift <= 317).
__device__ __forceinline__ void add_pieces(unsigned long long* col, unsigned long long v,
                                           int shift) {
  if (!v) return;
  const int li = shift >> 5;
  const int bi = shift & 31;
  const uint32_t p0 = (uint32_t)(v << bi);
  const uint32_t p1 = (uint32_t)(bi ? v >> (32 - bi) : v >> 32);
  const uint32_t p2 = (uint32_t)(bi ? v >> (64 - bi) : 0ull);
  if (p0) atomicAdd(&col[li], (unsigned long long)p0);
  if (p1) atomicAdd(&col[li + 1], (unsigned long long)p1);
  if (p2) atomicAdd(&col[li + 2], (unsigned long long)p2);
}

// L (little-endian 32-bit limbs) * 2^scale_exp, rounded to the nearest fp64,
// ties to even: a 64-bit window under the top bit gives the 53-bit
// significand, its next bit the guard, the rest of the window and every bit
// below it the sticky bit.
__device__ double limbs_to_double(const uint32_t (&L)[kLimbs], int scale_exp) {
  int h = -1;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i)
    if (L[i]) h = 32 * i + 31 - __clz(L[i]);
  if (h < 0) return 0.0;
  const int lo = h - 63;  // bit of the value at bit 0 of the window
  uint64_t W = 0;
  bool sticky = false;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    const int off = 32 * i - lo;  // window position of the limb's bit 0
    const uint64_t v = L[i];
    if (off >= 64) continue;
    if (off >= 0) {
      W |= v << off;
    } else if (off > -32) {
      W |= v >> (-off);
      sticky |= (v & ((uint64_t(1) << (-off)) - 1)) != 0;
    } else {
      sticky |= v != 0;
    }
  }
  uint64_t mant = W >> 11;
  const bool guard = (W >> 10) & 1;
  sticky |= (W & 0x3FFu) != 0;
  if (guard && (sticky || (mant & 1))) ++mant;  // 2^53 is exact in the ldexp below
  return ldexp((double)mant, h - 52 + scale_exp);
}

// One round-to-nearest-even step from binary64 to binary16.
__device__ uint16_t f64_to_f16_bits_dev(double x) {
  const uint64_t u = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((u >> 48) & 0x8000);
  const int be = (int)((u >> 52) & 0x7FF);
  const uint64_t mant = u & ((uint64_t(1) << 52) - 1);
  if (be == 0x7FF) return sign | (mant ? 0x7E00 : 0x7C00);
  if (be == 0) return sign;
  int E = be - 1023;
  const uint64_t sig = mant | (uint64_t(1) << 52);
  const int shift = (E >= -14) ? 42 : 42 + (-14 - E);
  if (shift >= 64) return sign;
  uint64_t r = sig >> shift;
  const uint64_t rem = sig & ((uint64_t(1) << shift) - 1);
  const uint64_t half = uint64_t(1) << (shift - 1);
  if (rem > half || (rem == half && (r & 1))) ++r;
  if (E >= -14) {
    if (r == (1u << 11)) {
      r >>= 1;
      ++E;
    }
    if (E > 15) return sign | 0x7C00;
    return sign | (uint16_t)(((E + 15) << 10) | (r & 0x3FF));
  }
  return sign | (uint16_t)r;
}

__global__ __launch_bounds__(256) void tq_gamma_kernel(const unsigned long long* lo,
                                                       const unsigned long long* hi,
                                                       const int* bad, int64_t total, double eps,
                                                       Info* info, double* gamma_out,
                                                       int* status_out) {
  __shared__ unsigned long long col[kLimbs];
  if (threadIdx.x < kLimbs) col[threadIdx.x] = 0;
  __syncthreads();
  const int e = threadIdx.x;
  if (e < 255) {
    const int shift = (e ? e : 1) - 1;  // m * 2^(e' - 150) = m * 2^(e' - 1) * 2^-149
    add_pieces(col, lo[e], shift);
    add_pieces(col, hi[e], shift + 64);
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  uint32_t L[kLimbs];
  unsigned long long carry = 0;
#pragma unroll
  for (int i = 0; i < kLimbs; ++i) {
    const unsigned long long t = col[i] + carry;
    L[i] = (uint32_t)t;
    carry = t >> 32;
  }
  const double S = limbs_to_double(L, -149);
  const double g = eps + S / (double)total;
  const bool ok = !*bad && isfinite(g) && g > 0.0;
  info->gamma = g;
  info->h = f64_to_f16_bits_dev(g);
  info->status = ok ? TQ_OK : TQ_ERR_VALUE;
  if (gamma_out) *gamma_out = g;
  if (status_out) *status_out = info->status;
}

// round(clip(w / gamma, -1, 1)) with ties to even, as the host decides it.
__device__ __forceinline__ int trit_of(float w, double gamma) {
  const double q = (double)w / gamma;
  return (q > 0.5) - (q < -0.5);
}

// One dword of qs (16 weights = 4 bytes of a row) per thread; the thread of a
// block's first dword writes the block's scale.
__global__ __launch_bounds__(256) void tq_pack_tq2_dev_kernel(const float* __restrict__ W,
                                                              int64_t N, int64_t K,
                                                              const Info* info,
                                                              uint32_t* __restrict__ qs,
                                                              uint16_t* __restrict__ scales) {
  const double gamma = info->gamma;
  const uint16_t h = (uint16_t)info->h;
  const int64_t words = N * (K / 16);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < words;
       i += (int64_t)gridDim.x * blockDim.x) {
    const float4* src = reinterpret_cast<const float4*>(W + 16 * i);
    uint32_t word = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 v = src[c];
      const float vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int t = 0; t < 4; ++t)
        word |= (uint32_t)(trit_of(vs[t], gamma) + 1) << (2 * (4 * c + t));
    }
    qs[i] = word;
    if ((i & 15) == 0) scales[i >> 4] = h;  // 16 dwords per 256-weight block
  }
}

// TQ1 bytes of one row, 1024 at a time per workgroup of 256 threads: the
// chunk's 5120 latents (weights 5 g .. 5 g + 4 of its groups g) come into LDS
// with coalesced 16-byte loads (zero past K), then thread t encodes groups
// t, t + 256, t + 512, t + 768 from LDS (a stride of 5 dwords, so the 64
// lanes hit 64 banks) and consecutive lanes write consecutive bytes.  Group g
// holds weights 5 g .. 5 g + 4, the first as the most significant base-3
// digit, weights past K as zero trits; bytes g >= ceil(K / 5) of the row are 0.
constexpr int kTq1Chunk = 1024;  // groups per workgroup
__global__ __launch_bounds__(256) void tq_pack_tq1_dev_kernel(const float* __restrict__ W,
                                                              int64_t N, int64_t K, int64_t ldq,
                                                              const Info* info,
                                                              uint8_t* __restrict__ qs,
                                                              uint16_t* __restrict__ scales) {
  __shared__ __attribute__((aligned(16))) float lat[5 * kTq1Chunk];
  const double gamma = info->gamma;
  const uint16_t h = (uint16_t)info->h;
  const int64_t G = (K + 4) / 5;
  const int64_t chunks = (ldq + kTq1Chunk - 1) / kTq1Chunk;
  for (int64_t wg = blockIdx.x; wg < N * chunks; wg += gridDim.x) {
    const int64_t n = wg / chunks;
    const int64_t g0 = (wg - n * chunks) * kTq1Chunk;
    const int64_t k0 = 5 * g0;
    __syncthreads();  // the previous chunk's reads are done
#pragma unroll
    for (int r = 0; r < 5; ++r) {
      const int q = threadIdx.x + 256 * r;  // float4 index in the chunk
      const int64_t k = k0 + 4 * q;        // K % 4 == 0: all in the row or all past it
      const float4 v = k < K ? *reinterpret_cast<const float4*>(W + n * K + k)
                             : float4{0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<float4*>(lat + 4 * q) = v;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = threadIdx.x + 256 * j;  // group in the chunk
      const int64_t g = g0 + c;
      if (g >= ldq) continue;
      uint32_t b = 0;
      if (g < G) {
        unsigned code = 0;
#pragma unroll
        for (int e = 0; e < 5; ++e) code = 3 * code + (unsigned)(trit_of(lat[5 * c + e], gamma) + 1);
        b = (code * 256 + 242) / 243;
      }
      qs[n * ldq + g] = (uint8_t)b;
    }
  }
  const int64_t ns = N * (K / 256);
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < ns;
       i += (int64_t)gridDim.x * blockDim.x)
    scales[i] = h;
}

int check_dev(const float* W, int64_t N, int64_t K, const void* qs, const uint16_t* scales,
              void* workspace, int64_t workspace_bytes_given) {
  if (!W || !qs || !scales || !workspace) return TQ_ERR_NULL;
  if (N < 1 || K < 256 || K % 256 || N > (int64_t(1) << 24) || K > (int64_t(1) << 20))
    return TQ_ERR_SHAPE;
  if (workspace_bytes_given < kWorkspace) return TQ_ERR_SHAPE;
  if (((uintptr_t)W | (uintptr_t)qs | (uintptr_t)scales | (uintptr_t)workspace) & 15)
    return TQ_ERR_ALIGN;
  return TQ_OK;
}

int have_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    return TQ_ERR_DEVICE;
  }
  return TQ_OK;
}

int launch_gamma(const float* W, int64_t N, int64_t K, double eps, double* gamma,
                 int* status, unsigned char* ws, hipStream_t stream) {
  if (have_device() != TQ_OK) return TQ_ERR_DEVICE;
  auto* lo = reinterpret_cast<unsigned long long*>(ws + kLoOff);
  auto* hi = reinterpret_cast<unsigned long long*>(ws + kHiOff);
  int* bad = reinterpret_cast<int*>(ws + kBadOff);
  Info* info = reinterpret_cast<Info*>(ws);
  hipLaunchKernelGGL(tq_sum_init_kernel, dim3(1), dim3(256), 0, stream, lo, hi, bad);
  hipLaunchKernelGGL(tq_abs_sum_kernel, dim3((unsigned)sum_groups(N, K)), dim3(kSumThreads), 0,
                     stream, W, N * K, lo, hi, bad);
  hipLaunchKernelGGL(tq_gamma_kernel, dim3(1), dim3(256), 0, stream, lo, hi, bad, N * K, eps,
                     info, gamma, status);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

int pack_grid(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 8192) g = 8192;
  return (int)(g < 1 ? 1 : g);
}

// The workspace of tq_pack_tq2_dev_noalloc: one fixed array per device,
// reserved when the library is loaded and held until the process ends.  Host
// code never uses the array's name as an address (on the host it is only a
// stand-in for the symbol); the device address comes from
// hipGetSymbolAddress, once per device, kept in scratch_addr.
constexpr int64_t kScratchBytes = kWorkspace;
static_assert(kScratchBytes % 16 == 0, "scratch keeps the workspace's 16-byte alignment");
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<unsigned char*> scratch_addr[kMaxDevices];

// Device address of the current device's scratch array (looked up on the
// first call on each device; concurrent first calls store the same value).
int scratch_on_current_device(unsigned char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return TQ_ERR_DEVICE;
  }
  unsigned char* p = scratch_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    void* a = nullptr;
    if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) {
      (void)hipGetLastError();
      return TQ_ERR_DEVICE;
    }
    p = static_cast<unsigned char*>(a);
    scratch_addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return TQ_OK;
}

}  // namespace

extern "C" {

int tq_pack_tq2_dev_noalloc(const float* W, int64_t N, int64_t K, double eps, uint8_t* qs,
                            uint16_t* scales, double* gamma, int* status, void* stream) {
  // same checks as tq_pack_tq2_dev, with the fixed scratch as the workspace
  if (!W || !qs || !scales) return TQ_ERR_NULL;
  if (N < 1 || K < 256 || K % 256 || N > (int64_t(1) << 24) || K > (int64_t(1) << 20))
    return TQ_ERR_SHAPE;
  if (tq_pack_dev_workspace_bytes(N, K) > kScratchBytes) return TQ_ERR_SHAPE;
  if (((uintptr_t)W | (uintptr_t)qs | (uintptr_t)scales) & 15) return TQ_ERR_ALIGN;
  if (have_device() != TQ_OK) return TQ_ERR_DEVICE;
  unsigned char* ws = nullptr;
  const int st = scratch_on_current_device(&ws);
  if (st != TQ_OK) return st;
  return tq_pack_tq2_dev(W, N, K, eps, qs, scales, gamma, status, ws, kScratchBytes, stream);
}

int64_t tq_pack_dev_workspace_bytes(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256) return -1;
  return kWorkspace;
}

int tq_pack_tq2_dev(const float* W, int64_t N, int64_t K, double eps, uint8_t* qs,
                    uint16_t* scales, double* gamma, int* status, void* workspace,
                    int64_t workspace_bytes_given, void* stream) {
  int st = check_dev(W, N, K, qs, scales, workspace, workspace_bytes_given);
  if (st != TQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  st = launch_gamma(W, N, K, eps, gamma, status, ws, s);
  if (st != TQ_OK) return st;
  hipLaunchKernelGGL(tq_pack_tq2_dev_kernel, dim3(pack_grid(N * (K / 16))), dim3(256), 0, s, W,
                     N, K, reinterpret_cast<const Info*>(ws), reinterpret_cast<uint32_t*>(qs),
                     scales);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

int tq_pack_tq1_dev(const float* W, int64_t N, int64_t K, double eps, int64_t ldq, uint8_t* qs,
                    uint16_t* scales, double* gamma, int* status, void* workspace,
                    int64_t workspace_bytes_given, void* stream) {
  int st = check_dev(W, N, K, qs, scales, workspace, workspace_bytes_given);
  if (st != TQ_OK) return st;
  if (ldq < (K + 4) / 5) return TQ_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  unsigned char* ws = static_cast<unsigned char*>(workspace);
  st = launch_gamma(W, N, K, eps, gamma, status, ws, s);
  if (st != TQ_OK) return st;
  const int64_t chunks = N * ((ldq + kTq1Chunk - 1) / kTq1Chunk);
  hipLaunchKernelGGL(tq_pack_tq1_dev_kernel, dim3((unsigned)(chunks < 65536 ? chunks : 65536)),
                     dim3(256), 0, s, W, N, K, ldq, reinterpret_cast<const Info*>(ws), qs, scales);
  return hipGetLastError() == hipSuccess ? TQ_OK : TQ_ERR_DEVICE;
}

}  // extern "C"
