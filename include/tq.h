/*
 * tq.h -- C ABI of the ternary-weight FP16 GEMM library (libtq.so), gfx950.
 *
 * The library computes Y = X (gamma T)^T, with FP16 activations X and ternary
 * weights T in {-1, 0, 1} stored in one of two lossless packings, as defined on
 * the project page "Scaling Laws and Efficient Inference for Ternary Language
 * Models":
 *   - "The model", steps 1-3: gamma = eps + mean|W| over the whole matrix,
 *     T = round(clip(W / gamma, -1, 1)), Y = X (gamma T)^T;
 *   - "Packing ternary weights" / "2 bits per weight" (TQ2): d' = d + 1 in a
 *     2-bit field, d' = (b >> 2j) & 3, four weights per byte;
 *   - "Packing ternary weights" / "1.6 bits per weight" (TQ1): five shifted
 *     digits read as a base-3 number N in [0, 242], stored as
 *     b = floor((256 N + 242) / 243);
 *   - "Fast inference on CPUs": one 16-bit scale per block of 256 weights;
 *   - "TriRun: ternary inference on GPUs": FP32 accumulation, FP16 output.
 *
 * Layouts (all row-major, no padding unless stated):
 *   X       fp16 [M][K]
 *   Y       fp16 [M][N]            Y[m][n] = sum_k X[m][k] * s[n][k/256] * T[n][k]
 *   T       int8 [N][K]            row n is output feature n (as nn.Linear)
 *   scales  fp16 [N][K/256]        s[n][b] scales weights k in [256 b, 256 b + 256)
 *   TQ2 qs  uint8 [N][K/4]         weight k = 4 i + j of a row: byte i, bits 2j..2j+1
 *   TQ1 qs  uint8 [N][ldq]         byte g of a row: weights 5 g .. 5 g + 4, the first
 *                                  one most significant; the last group of a row is
 *                                  padded with zero trits; bytes ceil(K/5) .. ldq-1
 *                                  are written as 0 and never read for values.
 *
 * Every function returns an int status (TQ_OK = 0, errors < 0).  No function
 * throws, aborts or prints.  Arguments are checked in this order: null
 * pointers, shapes, alignment, values; argument errors are reported before any
 * output is written or any kernel launched.  The caller owns every buffer.
 */
#ifndef TQ_H_
#define TQ_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum tq_status {
  TQ_OK = 0,
  TQ_ERR_NULL = -1,        /* a required pointer is NULL                         */
  TQ_ERR_SHAPE = -2,       /* negative or unsupported M, N, K, ldq               */
  TQ_ERR_VALUE = -3,       /* trit outside {-1,0,1}, NaN/Inf latent, gamma <= 0,  */
                           /* invalid packed byte                                 */
  TQ_ERR_ALIGN = -4,       /* a device pointer is not 16-byte aligned            */
  TQ_ERR_DEVICE = -5,      /* no usable HIP device, or a launch failed           */
  TQ_ERR_UNSUPPORTED = -6  /* an option this build does not provide              */
};

/* Source of the weights handed to the packers. */
typedef enum {
  TQ_SRC_TERNARY_I8 = 0, /* int8 [N][K] trits in {-1, 0, 1}                        */
  TQ_SRC_LATENT_F32 = 1  /* float [N][K] latent weights, ternarized with eps        */
} tq_src;

/* Kernel family for tq_gemm_*_ex.  AUTO picks, for TQ2, the skinny kernel for
 * M <= 16, and for M <= 32 when K <= 16384 and N >= 480 M, the tiled MFMA
 * kernel otherwise; for TQ1, the skinny kernel for M <= 16 and the tiled
 * (table-decode) kernel above (measured at K = 8192).  The others force one
 * family (used by the tests to cover both sides of the switch); the TQ2
 * skinny family serves M <= 32 and returns TQ_ERR_UNSUPPORTED above.  The
 * TQ1 tiled family takes ldq <= 2^22; a larger row stride runs the skinny
 * kernel instead. */
typedef enum {
  TQ_PATH_AUTO = 0,
  TQ_PATH_SKINNY = 1,
  TQ_PATH_TILED = 2,
  TQ_PATH_SIMPLE = 3 /* one wave per output row, VALU only: the plain GPU kernel */
} tq_path;

/* Human-readable name of a status code (static storage; never NULL). */
const char* tq_status_string(int status);

/* Version of this ABI; bumped on any incompatible change. */
int tq_abi_version(void);

/* Buffer sizes, in elements (bytes for qs).  Return -1 for invalid shapes. */
int64_t tq_tq2_bytes(int64_t N, int64_t K);  /* N * K / 4                           */
int64_t tq_tq1_ldq(int64_t K);               /* ceil(K / 5) rounded up to 16         */
int64_t tq_num_scales(int64_t N, int64_t K); /* N * K / 256                          */

/* ---------------------------------------------------------------------------
 * Host side (offline).  Thread-safe and stateless; uses several host threads
 * for large matrices.  All pointers are host memory.
 * ------------------------------------------------------------------------- */

/* "The model", steps 1-2.  W float [N][K], N, K >= 1.  gamma = eps + S / (N K),
 * where S is the exactly rounded fp64 sum of |W|; each trit is the fp64
 * quotient W / gamma clipped to [-1, 1] and rounded half to even.
 * T (int8 [N][K]) may be NULL to obtain gamma only; gamma_out may be NULL.
 * Errors: TQ_ERR_VALUE for a NaN/Inf weight, or a gamma that is not finite and
 * positive (e.g. eps = 0 and W = 0). */
int tq_ternarize_f32(const float* W, int64_t N, int64_t K, double eps,
                     int8_t* T, double* gamma_out);

/* TQ2 packing ("2 bits per weight").  K must be a positive multiple of 256.
 *   kind = TQ_SRC_LATENT_F32: W is float [N][K]; ternarize as tq_ternarize_f32,
 *     write qs, fill every entry of scales (fp16 bits [N][K/256]) with fp16(gamma)
 *     rounded to nearest even in one step from fp64, and store gamma in
 *     *gamma_out when non-NULL.  scales must not be NULL.
 *   kind = TQ_SRC_TERNARY_I8: W is int8 [N][K]; only qs is written; scales,
 *     gamma_out and eps are ignored (scales may be NULL).
 * qs is uint8 [N][K/4]. */
int tq_pack_tq2(int kind, const void* W, int64_t N, int64_t K, double eps,
                uint8_t* qs, uint16_t* scales_f16, double* gamma_out);

/* TQ1 packing ("1.6 bits per weight").  Same kinds and scales as tq_pack_tq2;
 * qs is uint8 [N][ldq] with ldq >= ceil(K/5).  K must be a positive multiple
 * of 256 (the scale block); the rows' last group is padded with zero trits. */
int tq_pack_tq1(int kind, const void* W, int64_t N, int64_t K, double eps, int64_t ldq,
                uint8_t* qs, uint16_t* scales_f16, double* gamma_out);

/* Inverse of the packers: T int8 [N][K].  K >= 1 (a multiple of 4 for TQ2).
 * TQ_ERR_VALUE for a 2-bit field equal to 3 (TQ2), for one of the 13 byte values
 * that no pattern produces, or for a non-zero padding trit (TQ1). */
int tq_unpack_tq2(const uint8_t* qs, int64_t N, int64_t K, int8_t* T);
int tq_unpack_tq1(const uint8_t* qs, int64_t N, int64_t K, int64_t ldq, int8_t* T);

/* ---------------------------------------------------------------------------
 * Device side.  Every pointer is device memory on the current HIP device.
 * The call only enqueues work on `stream` (a hipStream_t; NULL = the default
 * stream) and returns; it allocates nothing, never synchronizes and uses no
 * atomics, so Y is the same bit for bit on every run with the same inputs.
 *
 *   Y = X (s . T)^T :  X fp16 [M][K], Y fp16 [M][N], scales fp16 [N][K/256].
 *
 * Shapes: M, N >= 0 (M == 0 or N == 0 is a no-op that touches no pointer);
 * K a positive multiple of 256; M, N <= 2^24, K <= 2^20.  For TQ1,
 * ceil(K/5) <= ldq <= 2^24 and ldq % 16 == 0.  X, qs, scales and Y must be
 * 16-byte aligned.
 * Accumulation is fp32; Y is rounded to fp16 (nearest even) once, overflow
 * gives +-inf.  Trits are not validated on the device: a TQ2 field equal to 3
 * or an unused TQ1 byte gives unspecified (finite) values for that row.
 * Errors: TQ_ERR_DEVICE when no HIP device is usable or the launch fails.
 * ------------------------------------------------------------------------- */
int tq_gemm_tq2(const void* X, const void* qs, const void* scales_f16, void* Y,
                int64_t M, int64_t N, int64_t K, void* stream);
int tq_gemm_tq1(const void* X, const void* qs, int64_t ldq, const void* scales_f16, void* Y,
                int64_t M, int64_t N, int64_t K, void* stream);

/* Name of the kernel that tq_gemm_tq2_ex (format = 2) or tq_gemm_tq1_ex
 * (format = 1, with ldq <= 2^22) launches for this shape and path, as
 * profilers show it, copied NUL-terminated into name[cap].  TQ_ERR_SHAPE for an invalid shape,
 * TQ_ERR_VALUE for an unknown format or path, TQ_ERR_NULL for a NULL name,
 * TQ_ERR_UNSUPPORTED when the path is not available for the format.  Host
 * only; touches no device. */
int tq_kernel_name(int format, int64_t M, int64_t N, int64_t K, int path, char* name,
                   int64_t cap);

/* Same as above with an explicit kernel family (tq_path). */
int tq_gemm_tq2_ex(const void* X, const void* qs, const void* scales_f16, void* Y,
                   int64_t M, int64_t N, int64_t K, int path, void* stream);
int tq_gemm_tq1_ex(const void* X, const void* qs, int64_t ldq, const void* scales_f16, void* Y,
                   int64_t M, int64_t N, int64_t K, int path, void* stream);

/* ---------------------------------------------------------------------------
 * On-device ternarization and packing (the step before the product; project
 * page "The model" steps 1-2 and "Packing ternary weights").  The same
 * results as tq_pack_tq2 / tq_pack_tq1 with TQ_SRC_LATENT_F32, bit for bit:
 * gamma = eps + mean|W| with an exactly rounded fp64 sum of |W|, trits from
 * the fp64 quotient W / gamma with ties to even, fp16(gamma) in every scale.
 *
 * W float [N][K], qs, scales, gamma (one double), status (one int) and the
 * workspace are device memory on the current device; the call enqueues four
 * kernels on `stream` and returns (no host round trip, no allocation).
 * gamma and status may be NULL.  The workspace holds at least
 * tq_pack_dev_workspace_bytes(N, K) bytes (a few KB); its contents need no
 * initialization and are overwritten, so calls that may overlap need
 * separate workspaces.  The exact sum uses 64-bit integer atomics, whose
 * result does not depend on their order: every run gives the same bits.  W, qs, scales and the workspace must be
 * 16-byte aligned.  Shapes: N >= 1, 256 <= K <= 2^20, K % 256 == 0, N <=
 * 2^24; TQ1 ldq >= ceil(K/5).  Synchronous errors: TQ_ERR_NULL, TQ_ERR_SHAPE
 * (also a workspace that is too small), TQ_ERR_ALIGN, TQ_ERR_DEVICE.  A
 * non-finite latent or gamma is reported through *status (TQ_ERR_VALUE, else
 * TQ_OK) once the stream reaches it; qs and scales are then unspecified. */
int64_t tq_pack_dev_workspace_bytes(int64_t N, int64_t K); /* -1 for a bad shape */
int tq_pack_tq2_dev(const float* W, int64_t N, int64_t K, double eps, uint8_t* qs,
                    uint16_t* scales_f16, double* gamma, int* status, void* workspace,
                    int64_t workspace_bytes, void* stream);
int tq_pack_tq1_dev(const float* W, int64_t N, int64_t K, double eps, int64_t ldq, uint8_t* qs,
                    uint16_t* scales_f16, double* gamma, int* status, void* workspace,
                    int64_t workspace_bytes, void* stream);

/* tq_pack_tq2_dev without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops,
 * harnesses that forbid hipMalloc).  It runs the same four kernels with the
 * workspace in a fixed array of the library, tq_pack_dev_workspace_bytes()
 * bytes (4224) per device, reserved when the library is loaded and held until
 * the process ends; no call allocates or frees anything.  Every call on a
 * device uses that device's one array, so calls that overlap in time on one
 * device (other streams, other host threads) race and give unspecified qs,
 * scales and gamma; calls in one stream's order do not (each clears the
 * totals it needs at its start).  Arguments, results, status and errors as
 * tq_pack_tq2_dev (the same shape limits: N <= 2^24, K <= 2^20; a shape whose
 * workspace would exceed the array gives TQ_ERR_SHAPE); TQ_ERR_DEVICE also
 * when the array's device address cannot be obtained. */
int tq_pack_tq2_dev_noalloc(const float* W, int64_t N, int64_t K, double eps, uint8_t* qs,
                            uint16_t* scales_f16, double* gamma, int* status, void* stream);

/* TQ2 product on the tiled kernel with an explicit tile, for tuning and for
 * tests of every tile: 16 mt activation rows x 64 ng weight rows (32 ng when
 * mt = 8) per workgroup of ng x kg waves (kg of them split K).  Compiled
 * tiles: mt in {2, 4} with (ng, kg) in {(4, 2), (2, 4), (2, 2), (1, 4)},
 * mt = 2 with (1, 8), and mt = 8 with (4, 2); any other tile gives
 * TQ_ERR_UNSUPPORTED.  Everything
 * else is as tq_gemm_tq2. */
int tq_gemm_tq2_tiled(const void* X, const void* qs, const void* scales_f16, void* Y,
                      int64_t M, int64_t N, int64_t K, int mt, int ng, int kg, void* stream);

/* Fused gate / up product of the decode step's gated MLP (SwiGLU, named in
 * the architecture section of the project page "Scaling Laws and Efficient
 * Inference for Ternary Language Models"; each product as in "The model"):
 *   Y[m][n] = silu(g) * u,  g = sum_k X[m][k] s_g[n][k/256] T_g[n][k],
 *                           u = sum_k X[m][k] s_u[n][k/256] T_u[n][k],
 * silu(g) = g / (1 + exp(-g)), g, u and the product in fp32, one fp16
 * rounding.  Gate and up matrices are TQ2 packed as for tq_gemm_tq2 (qs
 * [N][K/4], scales [N][K/256] fp16), both N x K; X [M][K] and Y [M][N] fp16,
 * all device pointers, 16-byte aligned, owned by the caller.  For decode
 * sizes: 1 <= M <= 16 (larger M gives TQ_ERR_UNSUPPORTED); one launch streams
 * both matrices, the skinny kernel's offset rounding applies to g and u.
 * Errors as tq_gemm_tq2 (M = 0 or N = 0 is a no-op returning TQ_OK). */
int tq_gemm_tq2_swiglu(const void* X, const void* qs_gate, const void* scales_gate_f16,
                       const void* qs_up, const void* scales_up_f16, void* Y, int64_t M,
                       int64_t N, int64_t K, void* stream);

/* Input gradient of the ternary product for quantization-aware training
 * (the backward pass through "The model", step 3, on the project page
 * "Scaling Laws and Efficient Inference for Ternary Language Models"):
 *   dX[m][k] = sum_n dY[m][n] * scales[n][k/256] * T[n][k],
 * i.e. dY (s . T) with the TQ2 matrix of tq_gemm_tq2 (qs [N][K/4], scales
 * [N][K/256] fp16) read the other way round; dY [M][N] and dX [M][K] fp16,
 * device pointers, 16-byte aligned, owned by the caller; FP32 accumulation,
 * one fp16 rounding.  N must be a positive multiple of 8 and at most 2^20, K
 * a multiple of 256 (TQ_ERR_SHAPE otherwise); M = 0 is a no-op returning
 * TQ_OK.  Block scales must satisfy |s| < 1024: the kernel carries a column's
 * field position as an exact factor of up to 64 on the decoded s.  The weight
 * gradient under the straight-through estimator is tq_ste_grad_w. */
int tq_gemm_tq2_bwd_x(const void* dY, const void* qs, const void* scales_f16, void* dX,
                      int64_t M, int64_t N, int64_t K, void* stream);

/* Gradient that reaches the latent weights of a ternary linear under the
 * straight-through estimator (project page "Scaling Laws and Efficient
 * Inference for Ternary Language Models", "The model": gradients pass to the
 * latent weights with a straight-through estimator; Spectra page,
 * "Architecture of TriLM and FloatLM").  The quantizer W -> gamma T is taken
 * as the identity in the backward pass, so the latent weights receive the
 * gradient with respect to the effective weights of Y = X (gamma T)^T:
 *   dW[n][k] = sum_m dY[m][n] * X[m][k]            (accumulate = 0)
 *   dW[n][k] = dW[n][k] + sum_m dY[m][n] X[m][k]   (accumulate = 1)
 * gamma is not differentiated and no weight is masked (e.g. outside the clip
 * window |W / gamma| <= 1); the result does not depend on W, gamma or T.
 * dY fp16 [M][N] (the output gradient), X fp16 [M][K] (the layer input), dW
 * fp32 [N][K] (the latent weights' layout), all row-major device pointers,
 * 16-byte aligned, owned by the caller; FP32 accumulation, FP32 output, the
 * same bits on every run.  Shapes: M >= 0 (M = 0 writes zeros and reads
 * neither input, which may then be NULL, or is a no-op with accumulate = 1);
 * N = 0 or K = 0 is a no-op; N and K multiples of 8 and
 * at most 2^24; M N and M K at most 2^30 (split larger batches and
 * accumulate).  Errors: TQ_ERR_SHAPE, TQ_ERR_NULL, TQ_ERR_ALIGN,
 * TQ_ERR_VALUE (accumulate not 0 or 1), TQ_ERR_DEVICE. */
int tq_ste_grad_w(const void* dY, const void* X, float* dW, int64_t M, int64_t N, int64_t K,
                  int accumulate, void* stream);

/* Re-pack TQ1 weights as TQ2 on the device: the trits of qs1 ([N][ldq],
 * "1.6 bits per weight" on the project page "Scaling Laws and Efficient
 * Inference for Ternary Language Models") written as the 2-bit fields of qs2
 * ([N][K/4], "2 bits per weight"), bit for bit what tq_pack_tq2 writes for
 * the same trits; the block scales are shared unchanged.  Device pointers,
 * 16-byte aligned, owned by the caller; qs2 holds tq_tq2_bytes(N, K) bytes.
 * K a multiple of 256, ceil(K/5) <= ldq <= 2^24 and ldq a multiple of 16
 * (TQ_ERR_SHAPE otherwise); N = 0 is a no-op.  Byte values that no trit group encodes are
 * not detected. */
int tq_transcode_tq1_tq2(const void* qs1, int64_t ldq, int64_t N, int64_t K, void* qs2,
                         void* stream);

/* Activation rows from which tq_gemm_tq1_ws transcodes for an N x K matrix
 * (the measured crossover against the table-decode tiled kernel: 96 for
 * N <= 16384, else 33); TQ_ERR_SHAPE for
 * N < 1 or K not a positive multiple of 256. */
int64_t tq_tq1_transcode_min_m(int64_t N, int64_t K);

/* TQ1 product with a caller workspace, for batch and prefill sizes: with
 * M >= tq_tq1_transcode_min_m(N, K) and workspace_bytes >= tq_tq2_bytes(N, K),
 * the weights are first re-packed into the workspace as by
 * tq_transcode_tq1_tq2 and the TQ2 kernels of tq_gemm_tq2 run on it (the
 * TQ1 tiled kernel decodes every weight through LDS table lookups once per
 * activation tile; this decodes it once per call, at the cost of writing and
 * reading a 2-bit copy), so Y equals tq_gemm_tq2's on the same trits bit for
 * bit.
 * Otherwise (smaller M, no or too small a workspace) it is tq_gemm_tq1.
 * The workspace is device memory owned by the caller, 16-byte aligned when
 * given (TQ_ERR_ALIGN otherwise), overwritten by the call, and must not
 * overlap X, qs, scales or Y; calls that overlap on one workspace race.
 * Everything else is as tq_gemm_tq1. */
int tq_gemm_tq1_ws(const void* X, const void* qs, int64_t ldq, const void* scales_f16, void* Y,
                   int64_t M, int64_t N, int64_t K, void* workspace, int64_t workspace_bytes,
                   void* stream);

/* Measurement aid: the practical read ceiling for the weight-streaming
 * kernels.  Small-batch ternary inference is bound by reading the packed
 * weights ("TriRun: ternary inference on GPUs" on the project page "Scaling
 * Laws and Efficient Inference for Ternary Language Models"); this reads
 * `bytes` bytes at `src` once, with the loads the GEMV kernels use, and
 * computes nothing, so its time at a given size is what a launch that only
 * streams those bytes costs on this GPU.  src and sink are device pointers,
 * 16-byte aligned, owned by the caller; sink (4 bytes) is written only when
 * the XOR of the data equals one fixed 32-bit value.  bytes must be a
 * non-negative multiple of 16 (TQ_ERR_SHAPE otherwise); 0 is a no-op. */
int tq_stream_read(const void* src, int64_t bytes, void* sink, void* stream);

/* As tq_gemm_tq2_tiled with the weight rows per wave explicit: 16 mt
 * activation rows x 16 nr ng weight rows per workgroup of ng x kg waves.
 * Compiled tiles (mt, nr, ng, kg): mt in {2, 4} with (4, 4, 2), (4, 2, 4),
 * (4, 2, 2), (4, 1, 4), (2, 1, 4), (2, 2, 4), and (2, 2, 1, 8), (2, 4, 1, 8),
 * (8, 2, 4, 2);
 * any other gives TQ_ERR_UNSUPPORTED.  Everything else is as tq_gemm_tq2. */
int tq_gemm_tq2_tile(const void* X, const void* qs, const void* scales_f16, void* Y, int64_t M,
                     int64_t N, int64_t K, int mt, int nr, int ng, int kg, void* stream);

/* TQ2 product on the wide-tile kernel (v_mfma_f32_32x32x16_f16) with an
 * explicit tile, for tuning and for tests of every tile: 32 mt activation rows
 * x 32 nt ng weight rows per workgroup of ng x kg = 4 waves (kg of them split
 * K).  Compiled tiles: mt in {1, 2, 4}, nt in {1, 2}, (ng, kg) in {(2, 2),
 * (1, 4)}, except mt = 4 with kg = 4; any other gives TQ_ERR_UNSUPPORTED.
 * M K and N K / 4 must stay below 2^31 bytes (TQ_ERR_SHAPE otherwise).
 * Everything else is as tq_gemm_tq2. */
int tq_gemm_tq2_wide(const void* X, const void* qs, const void* scales_f16, void* Y, int64_t M,
                     int64_t N, int64_t K, int mt, int nt, int ng, int kg, void* stream);

/* TQ1 product on the table-decode tiled kernel with an explicit tile, for
 * tuning and for tests of every tile.  The tiles and their meaning are
 * tq_gemm_tq2_tile's; the weights are the 1.6-bit rows of tq_gemm_tq1 ("1.6
 * bits per weight" on the project page "Scaling Laws and Efficient Inference
 * for Ternary Language Models"), read once from HBM with no 2-bit copy:
 * each block's bytes are copied to LDS and every byte's five trits come from
 * a 256-entry table built with the pages' multiply-by-3 decoder.  ldq above
 * 2^22 or a tile not compiled gives TQ_ERR_UNSUPPORTED.  Everything else is as
 * tq_gemm_tq1. */
int tq_gemm_tq1_tile(const void* X, const void* qs, int64_t ldq, const void* scales_f16, void* Y,
                     int64_t M, int64_t N, int64_t K, int mt, int nr, int ng, int kg,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TQ_H_ */
