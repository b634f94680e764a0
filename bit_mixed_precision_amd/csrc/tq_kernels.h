// Internal launchers of the GEMM kernels.  Callers (tq_api.hip) have already
// validated every argument: shapes, alignment and sizes are as include/tq.h
// states, and M, N >= 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace tq {

struct GemmArgs {
  const void* X;       // fp16 [M][K]
  const void* qs;      // TQ2: uint8 [N][K/4]; TQ1: uint8 [N][ldq]
  const void* scales;  // fp16 [N][K/256]
  void* Y;             // fp16 [M][N]
  int64_t M, N, K;
  int64_t ldq;  // TQ1 row stride in bytes (unused for TQ2)
};

// Number of compute units of the current device (cached per device).
int device_cus();

// Raises the dynamic-LDS limit of kernel `fn` to `bytes` on the current device
// the first time a launcher needs it there.  `done` holds one bit per device
// (devices 0..63) and is shared by every call for that kernel, so concurrent
// first calls from several host threads are safe: each sets the attribute (an
// idempotent call) before it launches, and no device inherits another's bit.
hipError_t lds_limit_once(const void* fn, int bytes, std::atomic<uint64_t>& done);

hipError_t launch_tq2_simple(const GemmArgs& a, hipStream_t stream);
hipError_t launch_tq1_simple(const GemmArgs& a, hipStream_t stream);

// Skinny MFMA kernels for M <= 16; skinny_rows(N) is the number of 16-row
// groups one workgroup owns (the template argument of the kernel).
int skinny_rows(int64_t N);
int skinny_depth(int64_t M);             // register ring depth (template argument)
bool skinny_ring_first(int64_t M, int64_t K);  // ring loads before the activation wait
int skinny_stage(int64_t N, int64_t K, int64_t M);  // 1 when block scales are staged in LDS
hipError_t launch_tq2_skinny(const GemmArgs& a, hipStream_t stream);
// Fused decode-step gate / up product: a.qs / a.scales the gate matrix, Y =
// silu(X G^T) * (X U^T), M <= 16.
hipError_t launch_tq2_swiglu(const GemmArgs& a, const void* qs_up, const void* scales_up,
                             hipStream_t stream);
int glu_rows(int64_t N);
// Input gradient dX [M][K] = dY [M][N] (s . T) of a TQ2 matrix (N % 8 == 0).
hipError_t launch_tq2_bwd_x(const void* dY, const void* qs, const void* scales, void* dX,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Latent-weight gradient under the straight-through estimator:
// dW [N][K] (fp32) = dY^T X (+ dW when accumulate), dY [M][N], X [M][K] fp16,
// N and K multiples of 8, M N and M K at most 2^30.
hipError_t launch_ste_grad_w(const void* dY, const void* X, float* dW, int64_t M, int64_t N,
                             int64_t K, int accumulate, hipStream_t stream);

// TQ1 MFMA kernel: any M, in slices of 16 activation rows.
hipError_t launch_tq1_skinny(const GemmArgs& a, hipStream_t stream);
int tq1_depth();
int tq1_stage(int64_t N, int64_t K, int64_t M);
int tq1_slices(int64_t M);  // 16-row activation slices per workgroup (template argument)
int tq1_window_spans(int64_t M, int64_t K, int W);  // spans per activation window
bool tq1_ring_first(int64_t N, int64_t K, int64_t M);  // ring loads before the activation store

// Tiled MFMA kernels for M > 16: a workgroup of 4 waves (ng weight-row
// groups x kg k-groups) owns 16 mt activation rows x 16 nr ng weight rows.
struct TiledShape {
  int mt, nr, ng, kg;
};
TiledShape tiled_shape(int64_t M, int64_t N);
bool tiled_compiled(const TiledShape& t);  // one of the instantiated tiles
hipError_t launch_tq2_tiled(const GemmArgs& a, hipStream_t stream);
hipError_t launch_tq2_tiled_shape(const TiledShape& t, const GemmArgs& a, hipStream_t stream);
// The same tiles on 1.6-bit rows (a.ldq bytes each), decoded through an LDS
// table of byte -> five 2-bit fields; a.ldq <= kTq1TabMaxLdq.
constexpr int64_t kTq1TabMaxLdq = int64_t(1) << 22;
bool tq1_tab_scale_in_b(const TiledShape& t);  // block scale folded into the operands
TiledShape tq1_tab_shape(int64_t M, int64_t N);  // the automatic tile
hipError_t launch_tq1_tab(const GemmArgs& a, hipStream_t stream);
hipError_t launch_tq1_tab_shape(const TiledShape& t, const GemmArgs& a, hipStream_t stream);

// Wide-tile MFMA kernel (v_mfma_f32_32x32x16_f16): a workgroup of 4 waves
// (ng weight-row groups x kg k-groups) owns 32 mt activation rows x 32 nt ng
// weight rows.
struct WideShape {
  int mt, nt, ng, kg;
};
bool wide_compiled(const WideShape& w);
bool wide_fits(int64_t M, int64_t N, int64_t K);  // 32-bit buffer offsets suffice
hipError_t launch_tq2_wide_shape(const WideShape& w, const GemmArgs& a, hipStream_t stream);

// Plain streaming read of `bytes` (a multiple of 16) at src; sink gets a
// write only if the folded data equals one fixed value.
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream);

// TQ1 rows (ldq bytes each) -> TQ2 rows (K / 4 bytes each), the same trits.
hipError_t launch_tq1_to_tq2(const void* qs1, int64_t ldq, int64_t N, int64_t K, void* qs2,
                             hipStream_t stream);

}  // namespace tq
