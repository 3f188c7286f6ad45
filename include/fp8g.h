/*
 * fp8g.h -- C ABI of the MI355X (gfx950) scaled FP8 GEMM library (libfp8g.so).
 *
 * The operation (one definition, used by every entry point):
 *
 *     y[m,n] = bf16_rne( (sum_{k<K} x[m,k] * w[n,k]) * scale[n] )
 *
 *   x     [M,K]  FP8 E4M3 (OCP, no infinities; torch.float8_e4m3fn) codes,
 *                row-major, row stride K bytes ("activation")
 *   w     [N,K]  FP8 E4M3 codes, row-major, row stride K bytes ("weight":
 *                one row per output channel n)
 *   scale [N]    fp32, per-output-channel dequantisation factor
 *   y     [M,N]  bf16 bit patterns, row-major, row stride N elements
 *
 * The products are summed by the gfx950 f8f6f4 matrix cores into fp32
 * accumulators; the scale multiplies the finished fp32 sum once, and the result
 * is rounded to bf16, to nearest, ties to even.  Sources on the pages
 * (kernelbench.com model pages, cells named by the kernel they audit):
 *   - fp8 x fp8 products, fp32 accumulation, bf16 output:
 *     "DeepSeek V4 Flash (0731)", CUTLASS 3.x SM90 fp8 GEMM cell.
 *   - the live per-output-channel scale is applied in the epilogue, before the
 *     bf16 store: "Kimi K3 (256k)", SM120 warp-specialised FP8 GEMM cell.
 *   - every call reads the live operands and writes a fresh output; nothing is
 *     cached between calls: "Claude Fable 5", Triton split-K cell;
 *     "Qwen 3.8 Max", stale odd-K pad-cache cell (what goes wrong otherwise).
 *   - skinny M runs as split-K with fp32 partials and a reduce/scale/cast
 *     step: "Claude Fable 5", Triton split-K cell; "Kimi K3 (256k)", SM120
 *     cell (skinny path with a scaled finalize kernel).  Here the step runs in
 *     the same launch, by the last workgroup to finish each column tile.
 *   - K need not be a multiple of any tile size.  The pages zero-pad copies of
 *     the operands ("Kimi K3 (256k)", SM100 persistent-TMA Triton cell: zero
 *     bytes add nothing to the dot); this library reads the operand rows where
 *     they lie, at any byte alignment, and masks the last K step inside the
 *     kernel (bytes past K enter as zeros).  No operand is copied or padded.
 *
 * Ownership and threading: the caller owns every buffer.  The library keeps no
 * data between calls; its only globals are a thread-local copy of the last
 * error message, an atomic call counter (ids for split-K tickets) and one
 * memory pool per device for call workspaces (created on first use, under a
 * lock; it keeps up to 64 MiB of freed workspace for reuse and returns the
 * rest).  Calls are asynchronous: they enqueue kernels on `stream` (a
 * hipStream_t; NULL is the default stream) and return without synchronising.
 * Buffers must stay valid until that work has finished.
 */
#ifndef FP8G_H
#define FP8G_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
#define FP8G_OK 0
#define FP8G_ERR_INVALID_ARG 1 /* rejected before any HIP call; nothing enqueued */
#define FP8G_ERR_UNSUPPORTED 2 /* valid arguments outside what this build handles */
#define FP8G_ERR_HIP 3         /* a HIP call failed (no device, launch, allocation) */

/* Largest supported K (bytes per operand row).  Kernels address a tile of up
 * to 256 rows through 32-bit buffer offsets. */
#define FP8G_MAX_K ((int64_t)16777215)
/* Largest supported M and N: 2^30 - 1, so that a byte range of N fp32 scales
 * or biases (4 N bytes) fits a 32-bit buffer range.  Shapes whose launch grid
 * would exceed the device's limits are rejected with FP8G_ERR_UNSUPPORTED. */
#define FP8G_MAX_MN ((int64_t)1073741823)

/* Execution paths a plan can choose. */
#define FP8G_PATH_NONE 0   /* M == 0 or N == 0: nothing to do */
#define FP8G_PATH_ZERO 1   /* K == 0: y is filled with +0 (the empty sum) */
#define FP8G_PATH_MAIN 2   /* tiled MFMA kernel, fused scale/bf16 epilogue */
#define FP8G_PATH_SPLITK 3 /* skinny M: one split-K launch; with split_k > 1
                              the last slice of each column tile to finish
                              adds the fp32 partials, scales and casts */

/* A launch plan.  Pure host integer arithmetic; computing one makes no HIP call. */
typedef struct fp8g_plan {
    int32_t path;           /* FP8G_PATH_* */
    int32_t variant;        /* kernel configuration id within the path */
    int32_t tile_m;         /* rows of y per workgroup tile */
    int32_t tile_n;         /* columns of y per workgroup tile */
    int32_t tile_k;         /* K bytes per pipeline step */
    int32_t split_k;        /* K slices (splitk path); 1 otherwise */
    int64_t k_slice;        /* K bytes per slice (splitk path); K otherwise */
    int32_t group_m;        /* tile-raster group height (main path) */
    int32_t k_tail;         /* 1 if K is not a multiple of the K step */
    int64_t grid;           /* workgroups of the first kernel */
    int64_t workspace_bytes;/* per-tile tickets + fp32 partials the call
                               allocates (split-K with split_k > 1, or
                               stream-K) */
    int32_t dp_tiles;       /* main path: tiles computed whole, one workgroup
                               each (all tiles unless stream-K) */
    int32_t sk_groups;      /* main path variant 16: stream-K workgroups that
                               share the remaining tiles; 0 otherwise */
} fp8g_plan;

/* y = bf16_rne((x . w^T) * scale), as defined above.
 *   x, w, scale, y : device pointers.  x and w need no alignment.  scale must
 *                    be 4-byte aligned, y 2-byte aligned.  y must not overlap
 *                    x, w or scale.  y is fully overwritten.
 *   M, N, K        : 0 <= M, N <= FP8G_MAX_MN, 0 <= K <= FP8G_MAX_K.
 *                    M == 0 or N == 0 enqueues nothing; K == 0 writes +0.
 *   stream         : hipStream_t, or NULL for the default stream of the current
 *                    device; the buffers must be on the stream's device.
 * Returns FP8G_OK, FP8G_ERR_INVALID_ARG (bad sizes, null pointers with non-zero
 * extent, misaligned scale/y, overlapping output), or FP8G_ERR_HIP (no device,
 * launch failure, or failure to allocate the call's workspace; that is
 * allocated stream-ordered from the library's pool and freed with hipFreeAsync
 * on `stream` inside the call, so calls on different streams never share it). */
int fp8_gemm_scaled(const void *x, const void *w, const float *scale, void *y,
                    int64_t M, int64_t N, int64_t K, void *stream);

/* Same operation with parts of the plan forced, for tests and tuning.  Each
 * override is 0 for "let the planner choose":
 *   path    : FP8G_PATH_MAIN or FP8G_PATH_SPLITK (SPLITK needs M <= 128)
 *   variant : a configuration id valid for the path (fp8_gemm_plan_ex reports
 *             the tile it implies).  Main path: 10 = 256x256 tiles, eight
 *             waves, five LDS slots, any K (the default for 256x256 tiles
 *             with a K tail); 19 = 256x256 tiles on four waves of 128x128
 *             (the default for 256x256 tiles when K % 128 == 0; needs it);
 *             17 = 128x256 and 18 = 128x128 (mid M); 3 = 64x64 (small
 *             problems); 16 = variant 10 with stream-K (opt-in); 20 = variant
 *             19's tiles on rows fetched as whole 128-byte cache lines and
 *             realigned in registers (the default for odd K above 128;
 *             needs odd K > 128, M*K and N*K multiples of 16 and x, w
 *             128-byte aligned, else FP8G_ERR_INVALID_ARG); 27 = one wave
 *             per 16x16 block of y with the operands loaded straight into
 *             the MFMA registers, no LDS (the default for tiny problems: at
 *             most 256 such blocks and K <= 256; needs K % 16 == 0).  Split-K
 *             path: 1-5 = 16*v w rows per workgroup through per-wave LDS
 *             rings, 4 waves (the default for M > 32); 21-24 = 16*(v-20)
 *             rows with 8 waves (the default for M <= 32).  Row counts are
 *             limited by M (the staged x rows share the LDS): 1-5 up to
 *             5/4/2 blocks for M <= 16/32/128, 21-24 up to 4/3/1 blocks for
 *             M <= 16/32/64.
 *   split_k : splitk path: 1..64 K slices; main path variant 16: 1..2048
 *             stream-K workgroups; must be 0 for the other main variants.
 * Invalid overrides give FP8G_ERR_INVALID_ARG.  The result is the same
 * operation to within fp32 summation order. */
int fp8_gemm_scaled_ex(const void *x, const void *w, const float *scale, void *y,
                       int64_t M, int64_t N, int64_t K, int32_t path, int32_t variant,
                       int32_t split_k, void *stream);

/* The plan fp8_gemm_scaled would use for (M, N, K).  Host-only, no HIP call.
 * Returns FP8G_OK or FP8G_ERR_INVALID_ARG. */
int fp8_gemm_plan(int64_t M, int64_t N, int64_t K, fp8g_plan *out);

/* The plan fp8_gemm_scaled_ex would use with the same overrides. */
int fp8_gemm_plan_ex(int64_t M, int64_t N, int64_t K, int32_t path, int32_t variant,
                     int32_t split_k, fp8g_plan *out);

/* ------------------------------------------------- epilogue and formats ----
 * The same operation with a per-column bias, an elementwise activation and a
 * choice of FP8 format for each operand:
 *
 *     y[m,n] = bf16_rne( act( (sum_k dec_x(x[m,k]) * dec_w(w[n,k])) * scale[n]
 *                             + bias[n] ) )
 *
 * Sources on the pages: the per-output-channel scale is applied by the
 * per-column linear-combination + per-column bias + elementwise-activation
 * epilogue kind ("DeepSeek V4 Flash (0731)", CUTLASS 3.x SM90 fp8 GEMM cell);
 * the f8f6f4 matrix-core kind takes either FP8 format ("Claude Fable 5",
 * tcgen05 fp8 GEMM cell).  Formats: E4M3 as above; E5M2 is the OCP FP8 E5M2
 * format (bias 15, largest finite 57344, with infinities and NaN).  The sum
 * is accumulated in fp32 by the matrix cores; scale, bias and activation are
 * applied in fp32 in that order.  Activations: ReLU max(z, 0); SiLU
 * z / (1 + e^-z); GELU in its tanh form 0.5 z (1 + tanh(sqrt(2/pi) (z +
 * 0.044715 z^3))); each takes its limit at +-inf and keeps NaN. */
#define FP8G_FMT_E4M3 0
#define FP8G_FMT_E5M2 1

#define FP8G_ACT_NONE 0
#define FP8G_ACT_RELU 1
#define FP8G_ACT_SILU 2
#define FP8G_ACT_GELU_TANH 3

/*   bias     : device pointer to N fp32 values, 4-byte aligned, or NULL (no
 *              bias); must not overlap y.
 *   x_format, w_format : FP8G_FMT_E4M3 or FP8G_FMT_E5M2.
 *   activation         : FP8G_ACT_*.
 * Other arguments, ownership, errors and threading as fp8_gemm_scaled.  With
 * K == 0 the sum is +0 and y = bf16(act(bias)) (+0 without a bias). */
int fp8_gemm_scaled_act(const void *x, const void *w, const float *scale, const float *bias, void *y,
                        int64_t M, int64_t N, int64_t K, int32_t x_format, int32_t w_format,
                        int32_t activation, void *stream);

/* With forced plan parts as fp8_gemm_scaled_ex.  Operands other than E4M3 x
 * E4M3 are built for every variant except stream-K (main variant 16), which
 * gives FP8G_ERR_INVALID_ARG for them.  Bias and activation work with every
 * variant. */
int fp8_gemm_scaled_act_ex(const void *x, const void *w, const float *scale, const float *bias, void *y,
                           int64_t M, int64_t N, int64_t K, int32_t x_format, int32_t w_format,
                           int32_t activation, int32_t path, int32_t variant, int32_t split_k,
                           void *stream);

/* ------------------------------------------------------------- timing -----
 * fp8_gemm_scaled_act_ex with two HIP events attached to the call's own
 * kernels (hipExtLaunchKernel): start_event is recorded when the call's first
 * kernel begins and stop_event when its last kernel has ended, so
 * hipEventElapsedTime(start, stop) is the GPU time of the call's kernel
 * without the marker packets
 * that hipEventRecord adds around it.  The stream-ordered workspace allocation
 * and release are not kernels and fall outside that window.
 *   start_event, stop_event : hipEvent_t handles created by the caller (with
 *              timing enabled) on the device of the call, or NULL (not
 *              recorded).  Borrowed: the library records them, nothing more.
 * With M == 0 or N == 0 no kernel runs and both events are recorded with
 * hipEventRecord on the stream.  The events are recorded only on success;
 * after an error their state is unspecified.  Everything else as
 * fp8_gemm_scaled_act_ex. */
int fp8_gemm_scaled_act_timed(const void *x, const void *w, const float *scale, const float *bias, void *y,
                              int64_t M, int64_t N, int64_t K, int32_t x_format, int32_t w_format,
                              int32_t activation, int32_t path, int32_t variant, int32_t split_k,
                              void *stream, void *start_event, void *stop_event);

/* ---------------------------------------------------- allocation-free -----
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.  The same
 * operation and arguments as fp8_gemm_scaled_ex (path, variant, split_k: 0 =
 * the planner's choice), but the call allocates nothing: where its plan needs
 * a workspace (split-K with split_k > 1: fp32 partials and tickets; stream-K:
 * partial tiles and tickets) it uses a device array inside the library of
 * FP8G_NOALLOC_SCRATCH_BYTES, one per GPU, held until the process ends.
 *   Plans that need more workspace than that (fp8_gemm_plan_ex reports
 *   workspace_bytes) give FP8G_ERR_UNSUPPORTED before anything is enqueued.
 *   Nothing in the array has to be cleared between calls (tickets carry the
 *   id of their call; partials are written before they are read).
 *   All calls on one GPU share its array: calls whose kernels may overlap on
 *   one GPU (different streams with no ordering between them) race on it and
 *   must not be issued; calls ordered on one stream are safe.
 * Errors as fp8_gemm_scaled; FP8G_ERR_HIP also if the array's device address
 * cannot be obtained (looked up on the first call on each device). */
#define FP8G_NOALLOC_SCRATCH_BYTES ((int64_t)32 << 20)
int fp8_gemm_scaled_noalloc(const void *x, const void *w, const float *scale, void *y,
                            int64_t M, int64_t N, int64_t K, int32_t path, int32_t variant,
                            int32_t split_k, void *stream);

/* Static description of a status code. */
const char *fp8_gemm_strerror(int status);

/* Detail of the last failure on the calling thread (argument name, HIP error
 * string); "" if none.  Valid until the next call on the same thread. */
const char *fp8_gemm_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8G_H */
