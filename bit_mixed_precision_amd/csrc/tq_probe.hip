// Plain streaming read: the practical ceiling the weight-streaming kernels are
// measured against.  The project page "Scaling Laws and Efficient Inference
// for Ternary Language Models" ("TriRun: ternary inference on GPUs") states
// that small-batch ternary inference is bound by reading the packed weights;
// on a real GPU the attainable read rate at a given size is below the HBM peak
// (launch cost, first-load latency), and this kernel measures it: it reads
// every byte once with the same 16-byte non-temporal loads and writes nothing
// (unless the folded data equals one fixed value, which keeps the loads alive).
//
// MI355X shape: workgroups of 1024 threads, each streaming a contiguous slice
// two 16-byte loads deep per thread; 256 workgroups (one per CU) up to 32 MiB,
// 2048 above.  A sweep of grids (256 .. 4096), block sizes (256 .. 1024) and
// depths (2 .. 8), timed as back-to-back launches over >= 1 GiB of rotating
// buffers, put these among the fastest for both sizes of an M = 1 call:
// 17.3 MB in 4.34 us and 60.6 MB in 10.33 us (the earlier 256 x 512 x 4 shape:
// 4.91 and 12.80 us).

#include "tq_common.h"
#include "tq_kernels.h"
#include "tq_mfma.h"

namespace tq {
namespace {

constexpr int kReadThreads = 1024;
constexpr int kReadDepth = 2;
constexpr int64_t kSmallReadBytes = int64_t(32) << 20;
constexpr uint32_t kSinkMagic = 0x9E3779B9u;

__global__ __launch_bounds__(kReadThreads) void tq_stream_read_kernel(const u32x4* __restrict__ p,
                                                                     int64_t n16,
                                                                     uint32_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t b = per * blockIdx.x;
  const int64_t e = b + per < n16 ? b + per : n16;
  uint32_t acc = 0;
  int64_t i = b + threadIdx.x;
  for (; i + (kReadDepth - 1) * kReadThreads < e; i += kReadDepth * kReadThreads) {
    u32x4 v[kReadDepth];
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) v[d] = __builtin_nontemporal_load(p + i + d * kReadThreads);
#pragma unroll
    for (int d = 0; d < kReadDepth; ++d) acc ^= v[d][0] ^ v[d][1] ^ v[d][2] ^ v[d][3];
  }
  for (; i < e; i += kReadThreads) {
    const u32x4 v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == kSinkMagic) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream) {
  const unsigned grid = bytes <= kSmallReadBytes ? 256u : 2048u;
  hipLaunchKernelGGL(tq_stream_read_kernel, dim3(grid), dim3(kReadThreads), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<uint32_t*>(sink));
  return hipGetLastError();
}

}  // namespace tq
