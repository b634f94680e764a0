// C ABI of the device GEMMs (include/tq.h): argument checks and kernel choice.

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include <atomic>

#include "tq.h"
#include "tq_kernels.h"

namespace {

constexpr int64_t kMaxMN = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxBwdN = int64_t(1) << 20;  // 32-bit offsets in 512 rows of dY
// Largest TQ1 row stride: the kernels take it as a 32-bit int and form byte
// offsets such as 16 rows * ldq inside a workgroup in 32 bits.
constexpr int64_t kMaxLdq = int64_t(1) << 24;
// Largest dY and X of the weight gradient, in elements: 2 GiB of fp16 each,
// so that every byte offset fits the kernel's 32-bit buffer offsets.
constexpr int64_t kMaxSteElems = int64_t(1) << 30;
// Activation rows from which a TQ1 product with a workspace transcodes the
// weights once and runs the TQ2 kernels, instead of the table-decode tiled
// kernel (which reads the TQ1 bytes once and needs no workspace; its LDS
// table lookups cost it 25-55% over the TQ2 kernel on the same tile, the
// transcoding a read and a write of the matrix).  Measured at K = 8192 (us,
// table kernel / transcode + TQ2): N = 8192 M = 32 19.8 / 22.6, M = 64
// 27.8 / 28.6, M = 128 36.6 / 35.4; N = 28672 M = 32 47.0 / 47.4, M = 48
// 66.6 / 59.1, M = 64 67.2 / 62.4, M = 128 85.5 / 84.8.
int64_t tq1_transcode_min_m(int64_t N) { return N <= 16384 ? 96 : 33; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Null -> shape -> alignment, in that order.  Returns TQ_OK or an error code;
// *noop is set when M or N is zero (nothing to do, no pointer is touched).
int check_gemm(const void* X, const void* qs, const void* scales, const void* Y, int64_t M,
               int64_t N, int64_t K, bool tq1, int64_t ldq, bool* noop) {
  *noop = false;
  if (M < 0 || N < 0) return TQ_ERR_SHAPE;
  if (M == 0 || N == 0) {
    *noop = true;
    return TQ_OK;
  }
  if (!X || !qs || !scales || !Y) return TQ_ERR_NULL;
  if (M > kMaxMN || N > kMaxMN || K < 256 || K % 256 || K > kMaxK) return TQ_ERR_SHAPE;
  if (tq1 && (ldq < (K + 4) / 5 || ldq % 16 || ldq > kMaxLdq)) return TQ_ERR_SHAPE;
  if (!aligned16(X) || !aligned16(qs) || !aligned16(scales) || !aligned16(Y)) return TQ_ERR_ALIGN;
  return TQ_OK;
}

int device_ready() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return TQ_ERR_DEVICE;
  }
  return TQ_OK;
}

int finish(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return TQ_ERR_DEVICE;
  }
  return TQ_OK;
}

using Launcher = hipError_t (*)(const tq::GemmArgs&, hipStream_t);

struct Choice {
  Launcher launch;   // nullptr when the path is not available
  const char* name;  // kernel template, as profilers list it
  int variant;       // first template argument, or -1 for none
  int variant2;      // second template argument, or -1 for none
  int variant3 = -1;  // third to fifth template arguments, or -1 for none
  int variant4 = -1;
  int variant5 = -1;
};

constexpr int64_t kSkinnyMaxM = 16;     // one m tile of the TQ2 skinny kernel
constexpr int64_t kSkinnyLimitM = 32;   // the TQ2 skinny kernel's limit (two m tiles)

// TQ2 at 17..32 activation rows: the skinny kernel (every workgroup stages
// all M x K activations, the weights stream once) beats the tiled one where
// the weight rows per CU are many against the activation rows.  Measured
// (K = 8192, us skinny / tiled): N = 28672 M = 17 28.3 / 33.5, M = 32
// 35.0 / 35.3; N = 16384 M = 17 18.1 / 23.6, M = 32 23.3 / 23.9; N = 8192
// M = 17 12.6 / 13.4, M = 20 15.7 / 13.7, M = 32 20.3 / 14.2; N = 4096
// M = 20 17.0 / 15.1; K = 28672, N = 8192, M = 17 50.2 / 49.0.
bool tq2_skinny_two_tiles(int64_t M, int64_t N, int64_t K) {
  return M <= kSkinnyLimitM && K <= 16384 && N >= 480 * M;
}

// The kernel each (format, shape, path) runs.  Shapes are already validated.
Choice choose(bool tq1, int64_t M, int64_t N, int64_t K, int path) {
  if (path == TQ_PATH_AUTO) {
    if (tq1)
      path = M > kSkinnyMaxM ? TQ_PATH_TILED : TQ_PATH_SKINNY;
    else
      path = M <= kSkinnyMaxM || tq2_skinny_two_tiles(M, N, K) ? TQ_PATH_SKINNY : TQ_PATH_TILED;
  }
  switch (path) {
    case TQ_PATH_SIMPLE:
      return tq1 ? Choice{tq::launch_tq1_simple, "tq1_simple_kernel", -1, -1}
                 : Choice{tq::launch_tq2_simple, "tq2_simple_kernel", -1, -1};
    case TQ_PATH_SKINNY:
      if (tq1)
        return Choice{tq::launch_tq1_skinny, "tq1_skinny_kernel", tq::tq1_depth(),
                      tq::tq1_stage(N, K, M), tq::tq1_slices(M),
                      tq::tq1_ring_first(N, K, M) ? 1 : 0};
      if (M > kSkinnyLimitM) return Choice{nullptr, "", -1, -1};
      return Choice{tq::launch_tq2_skinny, "tq2_skinny_kernel", tq::skinny_depth(M),
                    tq::skinny_stage(N, K, M), M > 16 ? 2 : 1,
                    tq::skinny_ring_first(M, K) ? 1 : 0};
    case TQ_PATH_TILED: {
      if (tq1) {
        const tq::TiledShape t = tq::tq1_tab_shape(M, N);
        return Choice{tq::launch_tq1_tab, "tq1_tab_tiled_kernel", t.mt, t.nr, t.ng, t.kg,
                      tq::tq1_tab_scale_in_b(t) ? 1 : 0};
      }
      const tq::TiledShape t = tq::tiled_shape(M, N);
      return Choice{tq::launch_tq2_tiled, "tq2_tiled_kernel", t.mt, t.nr, t.ng, t.kg};
    }
    default:
      return Choice{nullptr, "", -1, -1};
  }
}

int run(bool tq1, const tq::GemmArgs& a, int path, hipStream_t s) {
  Choice c = choose(tq1, a.M, a.N, a.K, path);
  if (!c.launch) return TQ_ERR_UNSUPPORTED;
  return finish(c.launch(a, s));
}

}  // namespace

namespace tq {

// Compute units of the current device, cached per device; 256 (MI355X) when no
// device can be queried, so that host-only callers see the MI355X choice.
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
    (void)hipGetLastError();
    return 256;
  }
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0) {
    (void)hipGetLastError();
    cus = 256;
  }
  cache[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

hipError_t lds_limit_once(const void* fn, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t{1} << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

}  // namespace tq

extern "C" {

int tq_gemm_tq2_ex(const void* X, const void* qs, const void* scales, void* Y, int64_t M,
                   int64_t N, int64_t K, int path, void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, false, 0, &noop);
  if (st != TQ_OK || noop) return st;
  if (path < TQ_PATH_AUTO || path > TQ_PATH_SIMPLE) return TQ_ERR_VALUE;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs, scales, Y, M, N, K, 0};
  return run(false, a, path, static_cast<hipStream_t>(stream));
}

int tq_gemm_tq1_ex(const void* X, const void* qs, int64_t ldq, const void* scales, void* Y,
                   int64_t M, int64_t N, int64_t K, int path, void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, true, ldq, &noop);
  if (st != TQ_OK || noop) return st;
  if (path < TQ_PATH_AUTO || path > TQ_PATH_SIMPLE) return TQ_ERR_VALUE;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs, scales, Y, M, N, K, ldq};
  return run(true, a, path, static_cast<hipStream_t>(stream));
}

int tq_kernel_name(int format, int64_t M, int64_t N, int64_t K, int path, char* name,
                   int64_t cap) {
  if (!name) return TQ_ERR_NULL;
  if (M < 1 || N < 1 || M > kMaxMN || N > kMaxMN || K < 256 || K % 256 || K > kMaxK || cap < 1)
    return TQ_ERR_SHAPE;
  if ((format != 1 && format != 2) || path < TQ_PATH_AUTO || path > TQ_PATH_SIMPLE)
    return TQ_ERR_VALUE;
  Choice c = choose(format == 1, M, N, K, path);
  if (!c.launch) return TQ_ERR_UNSUPPORTED;
  char buf[160];
  if (c.launch == tq::launch_tq1_skinny)
    snprintf(buf, sizeof buf, "%s<%d, %s, %d, %s>", c.name, c.variant,
             c.variant2 ? "true" : "false", c.variant3, c.variant4 ? "true" : "false");
  else if (c.variant2 >= 0 && c.launch == tq::launch_tq2_skinny)  // plain product: GLU = false
    snprintf(buf, sizeof buf, "%s<%d, %s, false, %d, %s>", c.name, c.variant,
             c.variant2 ? "true" : "false", c.variant3, c.variant4 ? "true" : "false");
  else if (c.launch == tq::launch_tq1_tab)  // last argument: scale in the operands
    snprintf(buf, sizeof buf, "%s<%d, %d, %d, %d, %s>", c.name, c.variant, c.variant2,
             c.variant3, c.variant4, c.variant5 ? "true" : "false");
  else if (c.variant5 >= 0)
    snprintf(buf, sizeof buf, "%s<%d, %d, %d, %d, %d>", c.name, c.variant, c.variant2,
             c.variant3, c.variant4, c.variant5);
  else if (c.variant4 >= 0)
    snprintf(buf, sizeof buf, "%s<%d, %d, %d, %d>", c.name, c.variant, c.variant2, c.variant3,
             c.variant4);
  else if (c.variant2 >= 0)
    snprintf(buf, sizeof buf, "%s<%d, %d>", c.name, c.variant, c.variant2);
  else if (c.variant >= 0)
    snprintf(buf, sizeof buf, "%s<%d>", c.name, c.variant);
  else
    snprintf(buf, sizeof buf, "%s", c.name);
  int64_t i = 0;
  for (; buf[i] && i + 1 < cap; ++i) name[i] = buf[i];
  name[i] = '\0';
  return TQ_OK;
}

int tq_gemm_tq2_tiled(const void* X, const void* qs, const void* scales, void* Y, int64_t M,
                      int64_t N, int64_t K, int mt, int ng, int kg, void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, false, 0, &noop);
  if (st != TQ_OK || noop) return st;
  const tq::TiledShape t{mt, mt == 8 ? 2 : 4, ng, kg};
  if (!tq::tiled_compiled(t)) return TQ_ERR_UNSUPPORTED;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs, scales, Y, M, N, K, 0};
  return finish(tq::launch_tq2_tiled_shape(t, a, static_cast<hipStream_t>(stream)));
}

int tq_gemm_tq2_swiglu(const void* X, const void* qs_gate, const void* scales_gate,
                       const void* qs_up, const void* scales_up, void* Y, int64_t M, int64_t N,
                       int64_t K, void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs_gate, scales_gate, Y, M, N, K, false, 0, &noop);
  if (st != TQ_OK || noop) return st;
  if (!qs_up || !scales_up) return TQ_ERR_NULL;
  if (!aligned16(qs_up) || !aligned16(scales_up)) return TQ_ERR_ALIGN;
  if (M > kSkinnyMaxM) return TQ_ERR_UNSUPPORTED;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs_gate, scales_gate, Y, M, N, K, 0};
  return finish(tq::launch_tq2_swiglu(a, qs_up, scales_up, static_cast<hipStream_t>(stream)));
}

int tq_gemm_tq2_bwd_x(const void* dY, const void* qs, const void* scales, void* dX, int64_t M,
                      int64_t N, int64_t K, void* stream) {
  if (M < 0 || N < 0) return TQ_ERR_SHAPE;
  if (M == 0) return TQ_OK;
  if (!dY || !qs || !scales || !dX) return TQ_ERR_NULL;
  if (N == 0 || N % 8 || M > kMaxMN || N > kMaxBwdN || K < 256 || K % 256 || K > kMaxK)
    return TQ_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(qs) || !aligned16(scales) || !aligned16(dX)) return TQ_ERR_ALIGN;
  int st = device_ready();
  if (st != TQ_OK) return st;
  return finish(tq::launch_tq2_bwd_x(dY, qs, scales, dX, M, N, K, static_cast<hipStream_t>(stream)));
}

int tq_ste_grad_w(const void* dY, const void* X, float* dW, int64_t M, int64_t N, int64_t K,
                  int accumulate, void* stream) {
  if (M < 0 || N < 0 || K < 0) return TQ_ERR_SHAPE;
  if (N == 0 || K == 0 || (M == 0 && accumulate == 1)) return TQ_OK;
  if (!dW || (M > 0 && (!dY || !X))) return TQ_ERR_NULL;  // M = 0 reads neither input
  if (N % 8 || K % 8 || N > kMaxMN || K > kMaxMN || M * N > kMaxSteElems ||
      M * K > kMaxSteElems)
    return TQ_ERR_SHAPE;
  if (!aligned16(dY) || !aligned16(X) || !aligned16(dW)) return TQ_ERR_ALIGN;
  if (accumulate != 0 && accumulate != 1) return TQ_ERR_VALUE;
  int st = device_ready();
  if (st != TQ_OK) return st;
  return finish(tq::launch_ste_grad_w(dY, X, dW, M, N, K, accumulate,
                                      static_cast<hipStream_t>(stream)));
}

int tq_stream_read(const void* src, int64_t bytes, void* sink, void* stream) {
  if (bytes < 0 || bytes % 16) return TQ_ERR_SHAPE;
  if (bytes == 0) return TQ_OK;
  if (!src || !sink) return TQ_ERR_NULL;
  if (!aligned16(src) || !aligned16(sink)) return TQ_ERR_ALIGN;
  int st = device_ready();
  if (st != TQ_OK) return st;
  return finish(tq::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

int tq_gemm_tq2_tile(const void* X, const void* qs, const void* scales, void* Y, int64_t M,
                     int64_t N, int64_t K, int mt, int nr, int ng, int kg, void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, false, 0, &noop);
  if (st != TQ_OK || noop) return st;
  const tq::TiledShape t{mt, nr, ng, kg};
  if (!tq::tiled_compiled(t)) return TQ_ERR_UNSUPPORTED;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs, scales, Y, M, N, K, 0};
  return finish(tq::launch_tq2_tiled_shape(t, a, static_cast<hipStream_t>(stream)));
}

int tq_gemm_tq2_wide(const void* X, const void* qs, const void* scales, void* Y, int64_t M,
                     int64_t N, int64_t K, int mt, int nt, int ng, int kg, void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, false, 0, &noop);
  if (st != TQ_OK || noop) return st;
  const tq::WideShape w{mt, nt, ng, kg};
  if (!tq::wide_compiled(w)) return TQ_ERR_UNSUPPORTED;
  if (!tq::wide_fits(M, N, K)) return TQ_ERR_SHAPE;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs, scales, Y, M, N, K, 0};
  return finish(tq::launch_tq2_wide_shape(w, a, static_cast<hipStream_t>(stream)));
}

int tq_gemm_tq1_tile(const void* X, const void* qs, int64_t ldq, const void* scales, void* Y,
                     int64_t M, int64_t N, int64_t K, int mt, int nr, int ng, int kg,
                     void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, true, ldq, &noop);
  if (st != TQ_OK || noop) return st;
  const tq::TiledShape t{mt, nr, ng, kg};
  if (!tq::tiled_compiled(t) || ldq > tq::kTq1TabMaxLdq) return TQ_ERR_UNSUPPORTED;
  st = device_ready();
  if (st != TQ_OK) return st;
  tq::GemmArgs a{X, qs, scales, Y, M, N, K, ldq};
  return finish(tq::launch_tq1_tab_shape(t, a, static_cast<hipStream_t>(stream)));
}

int tq_gemm_tq2(const void* X, const void* qs, const void* scales, void* Y, int64_t M, int64_t N,
                int64_t K, void* stream) {
  return tq_gemm_tq2_ex(X, qs, scales, Y, M, N, K, TQ_PATH_AUTO, stream);
}

int tq_gemm_tq1(const void* X, const void* qs, int64_t ldq, const void* scales, void* Y,
                int64_t M, int64_t N, int64_t K, void* stream) {
  return tq_gemm_tq1_ex(X, qs, ldq, scales, Y, M, N, K, TQ_PATH_AUTO, stream);
}

int tq_transcode_tq1_tq2(const void* qs1, int64_t ldq, int64_t N, int64_t K, void* qs2,
                         void* stream) {
  if (N < 0) return TQ_ERR_SHAPE;
  if (N == 0) return TQ_OK;
  if (!qs1 || !qs2) return TQ_ERR_NULL;
  if (N > kMaxMN || K < 256 || K % 256 || K > kMaxK || ldq < (K + 4) / 5 || ldq % 16 ||
      ldq > kMaxLdq)
    return TQ_ERR_SHAPE;
  if (!aligned16(qs1) || !aligned16(qs2)) return TQ_ERR_ALIGN;
  int st = device_ready();
  if (st != TQ_OK) return st;
  return finish(tq::launch_tq1_to_tq2(qs1, ldq, N, K, qs2, static_cast<hipStream_t>(stream)));
}

int64_t tq_tq1_transcode_min_m(int64_t N, int64_t K) {
  if (N < 1 || K < 256 || K % 256) return TQ_ERR_SHAPE;
  return tq1_transcode_min_m(N);
}

int tq_gemm_tq1_ws(const void* X, const void* qs, int64_t ldq, const void* scales, void* Y,
                   int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                   void* stream) {
  bool noop = false;
  int st = check_gemm(X, qs, scales, Y, M, N, K, true, ldq, &noop);
  if (st != TQ_OK || noop) return st;
  if (workspace_bytes < 0) return TQ_ERR_SHAPE;
  if (workspace && !aligned16(workspace)) return TQ_ERR_ALIGN;
  const bool transcode =
      M >= tq1_transcode_min_m(N) && workspace && workspace_bytes >= N * (K / 4);
  if (!transcode) return tq_gemm_tq1_ex(X, qs, ldq, scales, Y, M, N, K, TQ_PATH_AUTO, stream);
  st = device_ready();
  if (st != TQ_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = finish(tq::launch_tq1_to_tq2(qs, ldq, N, K, workspace, s));
  if (st != TQ_OK) return st;
  return run(false, tq::GemmArgs{X, workspace, scales, Y, M, N, K, 0}, TQ_PATH_AUTO, s);
}

}  // extern "C"
