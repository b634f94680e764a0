// Internal launchers of the GEMM kernels.  Callers (tq_api.hip) have already
// validated every argument: shapes, alignment and sizes are as include/tq.h
// states, and M, N >= 1.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

hipError_t launch_tq2_simple(const GemmArgs& a, hipStream_t stream);
hipError_t launch_tq1_simple(const GemmArgs& a, hipStream_t stream);

// Skinny MFMA kernels for M <= 16; skinny_rows(N) is the number of 16-row
// groups one workgroup owns (the template argument of the kernel).
int skinny_rows(int64_t N);
int skinny_depth();                      // register ring depth (template argument)
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

// TQ1 MFMA kernel: any M, in slices of 16 activation rows.
hipError_t launch_tq1_skinny(const GemmArgs& a, hipStream_t stream);
int tq1_depth();
int tq1_stage(int64_t N, int64_t K, int64_t M);
int tq1_slices(int64_t M);  // 16-row activation slices per workgroup (template argument)

// Tiled MFMA kernels for M > 16: a workgroup of 4 waves (ng weight-row
// groups x kg k-groups) owns 16 mt activation rows x 16 nr ng weight rows.
struct TiledShape {
  int mt, nr, ng, kg;
};
TiledShape tiled_shape(int64_t M, int64_t N);
bool tiled_compiled(const TiledShape& t);  // one of the instantiated tiles
hipError_t launch_tq2_tiled(const GemmArgs& a, hipStream_t stream);
hipError_t launch_tq2_tiled_shape(const TiledShape& t, const GemmArgs& a, hipStream_t stream);

// Tiled MFMA kernel for TQ1 and M > 16: a workgroup of nw x kg waves (kg of
// them split K) owns 16 mt activation rows x 16 nw weight rows.
struct Tq1TiledShape {
  int mt, nw, kg;
};
Tq1TiledShape tq1_tiled_shape(int64_t M, int64_t N);
bool tq1_prefers_tiled(int64_t M, int64_t N);  // the automatic choice for M > 16
bool tq1_tiled_compiled(const Tq1TiledShape& t);
int tq1_tiled_depth();                           // weight ring depth in stages
int tq1_tiled_xahead(const Tq1TiledShape& t);    // stages the activations are loaded ahead
hipError_t launch_tq1_tiled(const GemmArgs& a, hipStream_t stream);
hipError_t launch_tq1_tiled_shape(const Tq1TiledShape& t, const GemmArgs& a, hipStream_t stream);

// Plain streaming read of `bytes` (a multiple of 16) at src; sink gets a
// write only if the folded data equals one fixed value.
hipError_t launch_stream_read(const void* src, int64_t bytes, void* sink, hipStream_t stream);

// TQ1 rows (ldq bytes each) -> TQ2 rows (K / 4 bytes each), the same trits.
hipError_t launch_tq1_to_tq2(const void* qs1, int64_t ldq, int64_t N, int64_t K, void* qs2,
                             hipStream_t stream);

}  // namespace tq
