/*
 * sq.h - C ABI of the SmoothQuant W8A8 linear layer for AMD Instinct MI355X (gfx950).
 *
 * The library implements, as HIP kernels, the run-time and load-time steps of
 * a W8A8 int8 linear layer with SmoothQuant smoothing, and the LLM.int8()
 * vectorwise decomposition. The pages defining the operations:
 *
 *   [W8A8]  "Half the Size, Better Performance, Same Accuracy: Understanding
 *           W8A8 INT8 LLM Quantization"
 *   [CALIB] "How does SmoothQuant int8 LLM calibration work and what steps do
 *           technicians need to follow for accurate deployment?"
 *   [INT8]  the LLM.int8() page (aicassindra.com, "quant_llm_int8")
 *
 * Conventions shared by every entry point:
 *
 *  - Pointers to tensors are DEVICE pointers, allocated and owned by the
 *    caller. The library never allocates, frees or keeps device memory; where
 *    an entry point needs scratch memory the caller passes a workspace of at
 *    least the size the matching *_workspace_size() returns (NULL is allowed
 *    when that size is 0).
 *  - Matrices are row-major with an explicit leading dimension in elements.
 *    W is [K x N] (rows are input channels, columns output channels) as on
 *    the pages; the int8 weight Wq is stored transposed, [N x K], so both
 *    GEMM operands are contiguous along K.
 *  - Every call is asynchronous on the given stream (NULL = the default
 *    stream): it returns once the work is enqueued. Results are visible after
 *    the stream is synchronised. Calls are stateless and may be made from any
 *    host thread.
 *  - All arguments are validated before anything is enqueued, so a call that
 *    returns an error has done no work. SQ_ERR_HIP reports a failed launch;
 *    sq_last_hip_error() returns the HIP error code of the latest such
 *    failure on the calling thread.
 *  - Shape rules: M, N, T >= 0 (a zero size is a valid no-op); K >= 64 and
 *    K % 64 == 0. Tensor pointers must be 16-byte aligned and leading
 *    dimensions must keep every row 16-byte aligned.
 *  - Inputs containing NaN or infinity are outside the contract (no check is
 *    made, to keep the kernels at memory speed).
 */
#ifndef SQ_H_
#define SQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipStream_t without pulling in the HIP headers. */
typedef struct ihipStream_t* sq_stream_t;

typedef enum sq_status {
  SQ_OK = 0,
  SQ_ERR_NULL = 1,      /* a required pointer is NULL */
  SQ_ERR_DTYPE = 2,     /* element type not supported by this entry point */
  SQ_ERR_SHAPE = 3,     /* negative size, K not a positive multiple of 64, ld < row length */
  SQ_ERR_ALIGN = 4,     /* pointer or row not 16-byte aligned */
  SQ_ERR_RANGE = 5,     /* value out of range: alpha outside [0,1], K beyond int32 headroom, bad flags */
  SQ_ERR_WORKSPACE = 6, /* workspace missing or smaller than *_workspace_size() */
  SQ_ERR_HIP = 7        /* a HIP launch failed; see sq_last_hip_error() */
} sq_status;

typedef enum sq_dtype {
  SQ_F32 = 0,  /* IEEE binary32 */
  SQ_BF16 = 1, /* bfloat16 */
  SQ_F16 = 2,  /* IEEE binary16 */
  SQ_I32 = 3,  /* int32 (raw GEMM accumulator output) */
  SQ_I8 = 4
} sq_dtype;

/* Largest K for which the int32 accumulator cannot overflow:
 * 127 * 127 * K < 2^31  <=>  K <= 133144. */
#define SQ_MAX_K_INT32 133144
/* Longest row sq_rmsnorm_quant accepts (its exact sum of squares is sized for it). */
#define SQ_MAX_K_NORM 32768
/* Longest row sq_silu_mul_quant accepts (its rows stay in registers). */
#define SQ_MAX_K_SILU 32768
/* Longest K of the FP8 entry points (their quantiser keeps rows in registers). */
#define SQ_MAX_K_FP8 32768
/* Largest K of the GPTQ calls (the K x K binary64 Hessian and its factor). */
#define SQ_MAX_K_GPTQ 32768

/* Flags of sq_smooth_fold_weights. */
#define SQ_SMOOTH_COMPUTE 0u /* compute s from absmax and W, write it to `smooth` */
#define SQ_SMOOTH_GIVEN 1u   /* read s from `smooth` (not written) */
#define SQ_SMOOTH_NONE 2u    /* s = 1 (plain per-channel weight quantisation); `smooth` and `absmax` may be NULL */

const char* sq_status_string(sq_status status);
int sq_last_hip_error(void);
/* Library version as 10000*major + 100*minor + patch. */
int sq_version(void);

/*
 * Calibration: per-input-channel activation absmax, as a running maximum.
 * [W8A8] "How the smoothing factor is computed" (A_j is the largest activation
 * seen in channel j over the calibration samples); [CALIB] "The Technical
 * Workflow for Int8 Quantization Deployment" (maximum absolute value per
 * channel).
 *
 *   absmax[j] = max(absmax[j], max_{0<=t<T} |x[t*ldx + j]|)   for 0 <= j < K
 *
 * x:      [T x ldx] of type xt (SQ_F32, SQ_BF16 or SQ_F16), read only.
 * absmax: [K] binary32, read and written. The caller zero-fills it once before
 *         the first calibration batch and then calls once per batch. Entries
 *         stay non-negative.
 * The result is exact (a maximum), independent of launch order.
 */
sq_status sq_calibrate_absmax(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx,
                              float* absmax, sq_stream_t stream);

/*
 * Load-time weight preparation: smoothing factor, fold, per-output-channel
 * symmetric int8 quantisation.
 * [W8A8] "How the smoothing factor is computed" (s_j from the activation
 * absmax A_j, the largest weight magnitude W_j of row j and alpha; row j of W
 * is multiplied by s_j); "How the Model Was Compressed" and "Why Naive Weight
 * Quantization Doesn't Work" (scale = max|column| / 127, q = round(w/scale),
 * one scale per output channel).
 *
 *   W_j   = max_n |w[j][n]|
 *   s_j   = fl32( A_j^alpha / W_j^(1-alpha) )   powers and quotient in binary64;
 *           s_j = 1 when A_j == 0 or W_j == 0              (SQ_SMOOTH_COMPUTE)
 *   W'_jn = fl32(s_j * w[j][n])
 *   sw_n  = fl32(max_j |W'_jn| / 127)
 *   wq[n][j] = clamp(round_half_even(fl32(W'_jn / sw_n)), -127, 127); 0 when sw_n == 0
 *
 * absmax:  [K] binary32 (from sq_calibrate_absmax); unused with SQ_SMOOTH_GIVEN/NONE.
 * w:       [K x ldw] of type wt (SQ_F32, SQ_BF16 or SQ_F16). Unlike the other
 *          inputs, W may have any leading dimension >= N (16-byte aligned rows
 *          are read with vector loads, others element by element); the
 *          pointer must be aligned to the element size.
 * alpha:   migration strength in [0, 1] ([CALIB]); unused unless SQ_SMOOTH_COMPUTE.
 * flags:   one of SQ_SMOOTH_COMPUTE, SQ_SMOOTH_GIVEN, SQ_SMOOTH_NONE.
 * smooth:  [K] binary32; written (COMPUTE), read (GIVEN) or unused (NONE, may be NULL).
 * wq:      [N x K] int8 output (K-contiguous).
 * w_scale: [N] binary32 output.
 * ws:      workspace of sq_smooth_fold_workspace_size(k, n) bytes.
 */
size_t sq_smooth_fold_workspace_size(int64_t k, int64_t n);
sq_status sq_smooth_fold_weights(const float* absmax, const void* w, sq_dtype wt, int64_t k, int64_t n,
                                 int64_t ldw, double alpha, uint32_t flags, float* smooth, int8_t* wq,
                                 float* w_scale, void* ws, size_t ws_bytes, sq_stream_t stream);

/*
 * Run-time per-token dynamic int8 activation quantisation with the
 * smoothing divide fused in.
 * [W8A8] "How the Model Was Compressed" (one scale per token over all its
 * channels, computed at run time); "Why Activation Quantization Is Hard"
 * (scale = max|x| / 127, q = round(x/scale)); "How the smoothing factor is
 * computed" (the activation side is divided by s).
 *
 *   xh_ij = fl32(x_ij / s_j)          (x_ij itself when smooth == NULL)
 *   d_i   = fl32(max_j |xh_ij| / 127)
 *   xq_ij = clamp(round_half_even(fl32(xh_ij / d_i)), -127, 127); 0 when d_i == 0
 *
 * Every division is correctly rounded binary32, as in IEEE-754.
 * x: [M x ldx] of type xt (SQ_F32, SQ_BF16 or SQ_F16). smooth: [K] or NULL.
 * xq: [M x K] int8 output. x_scale: [M] binary32 output.
 */
sq_status sq_quant_act_per_token(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx,
                                 const float* smooth, int8_t* xq, float* x_scale, sq_stream_t stream);

/*
 * int8 x int8 -> int32 GEMM with the fused per-token x per-output-channel
 * dequantisation epilogue, on the gfx950 int8 matrix cores.
 * [INT8] "The architecture: every piece explained" (int32 accumulation; the
 * accumulator is scaled by the product of its row and column scales);
 * [W8A8] "Performance After Quantization", Inter-Token Latency (the int8
 * matmul output is converted back to bf16).
 *
 *   acc_in = sum_k xq[i][k] * wq[n][k]                       exact int32
 *   y[i][n] = out( fl32( fl32( fl32(acc_in) * x_scale_i ) * w_scale_n ) )
 *
 * out() is round-to-nearest-even to yt = SQ_BF16, SQ_F16 or SQ_F32; yt =
 * SQ_I32 writes acc itself (scales unused, may be NULL).
 * xq: [M x K], wq: [N x K] (K-contiguous, rows 16-byte aligned), y: [M x ldy].
 * K must not exceed SQ_MAX_K_INT32.
 * ws: workspace of sq_w8a8_linear_workspace_size(m, n, k) bytes, 16-byte
 *     aligned; NULL when that size is 0. The size is non-zero where K is
 *     split over several workgroups: decode shapes (K % 128 == 0 and
 *     M <= 64, or M <= 255 where no tiled kernel would cover the compute
 *     units; one ticket counter per 64 output columns and 64 tokens) and
 *     shapes of the 256-row prefill kernel (M >= 256, or M >= 129 over
 *     layers at least 4096 wide with K >= 2560) whose tiles number fewer
 *     than 128 (up to 8 slices of at least 1024 K each; one ticket counter
 *     per output tile). The size depends on (m, n, k) only.
 *     The workspace then holds the ticket counters, in a fixed region of
 *     the first 1 KiB, and the int32 partial tiles after it. Contract: the
 *     counter region reads zero when a call starts. The caller zero-fills
 *     the workspace once, before its first use; every call leaves its
 *     counters at zero again, and no call writes partial tiles into the
 *     counter region, so one zero-filled workspace of the largest size
 *     needed serves any later sequence of calls, at any shapes, without
 *     clearing. Failure mode: non-zero counters at the start of a call (a
 *     workspace never zero-filled, or one shared by calls in flight at the
 *     same time) let the tile reduction run before every slice has
 *     published, or never, so Y is wrong or left unwritten; nothing
 *     detects this. One workspace serves one call at a time (calls in
 *     flight together on different streams need their own). The one-call
 *     entry points (sq_w8a8_linear_dyn and the fused norm / gated-MLP
 *     calls) clear the counters themselves. The split changes only how the
 *     exact int32 sum is formed, never its value.
 */
size_t sq_w8a8_linear_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_w8a8_linear(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                         int64_t m, int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy,
                         void* ws, size_t ws_bytes, sq_stream_t stream);

/*
 * The whole run-time path in one call: sq_quant_act_per_token followed by
 * sq_w8a8_linear on the same stream, with Xq, the row scales and the GEMM's
 * workspace held in the workspace. The results equal those of the two calls
 * made separately.
 * ws: workspace of sq_w8a8_linear_dyn_workspace_size(m, n, k) bytes, 16-byte
 *     aligned. Its contents need no initialisation: the quantisation launch
 *     clears the GEMM's split-K counters.
 */
size_t sq_w8a8_linear_dyn_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_w8a8_linear_dyn(const void* x, sq_dtype xt, int64_t ldx, const float* smooth,
                             const int8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k,
                             void* y, sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes,
                             sq_stream_t stream);

/*
 * sq_w8a8_linear_dyn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops and
 * harnesses that forbid allocation). It allocates nothing: its scratch (Xq,
 * the row scales, the split-K counters and partial tiles) is a static device
 * array of SQ_STATIC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on until the process ends. Same arguments and results as
 * sq_w8a8_linear_dyn, without ws / ws_bytes.
 * Errors: those of sq_w8a8_linear_dyn; SQ_ERR_WORKSPACE when
 * sq_w8a8_linear_dyn_workspace_size(m, n, k) exceeds SQ_STATIC_SCRATCH_BYTES
 * (nothing is enqueued); SQ_ERR_HIP when the array's device address cannot be
 * looked up on the first call on a device (current device >= 64: SQ_ERR_RANGE).
 * All calls on one GPU share its array: calls that overlap in time on one GPU
 * (other streams, other host threads) race and give wrong results, so the
 * caller serialises them. Contents left by an earlier call do not matter (the
 * call's quantisation launch clears the counters).
 */
#define SQ_STATIC_SCRATCH_BYTES (32u << 20)
sq_status sq_w8a8_linear_dyn_static(const void* x, sq_dtype xt, int64_t ldx, const float* smooth,
                                    const int8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k,
                                    void* y, sq_dtype yt, int64_t ldy, sq_stream_t stream);

/*
 * The smoothing factor moved into RMSNorm's gain, once at load time.
 * [W8A8] "How the smoothing factor is computed" (SmoothQuant divides the
 * norm's gamma by s and multiplies the matching weight rows by s, which
 * sq_smooth_fold_weights does) and the smoothed example of "Where the outlier
 * actually comes from".
 *
 *   gain_j = fl32(gamma_j / s_j)          (gamma_j itself when smooth == NULL)
 *
 * gamma: [K] of type gt (SQ_F32, SQ_BF16 or SQ_F16), element-aligned.
 * smooth: [K] binary32 or NULL. gain: [K] binary32 output. Any K >= 0.
 */
sq_status sq_fold_norm_gain(const void* gamma, sq_dtype gt, const float* smooth, int64_t k, float* gain,
                            sq_stream_t stream);

/*
 * RMSNorm with the folded gain, fused with the per-token int8 quantisation of
 * its output: the activation never goes to memory in floating point.
 * [W8A8] "Where the outlier actually comes from" (divide by the vector's
 * root-mean-square, then scale channel j by the gain), "How the smoothing
 * factor is computed" (the gain carries 1/s, so no division by s is left),
 * "How the Model Was Compressed" and "Why Activation Quantization Is Hard"
 * (one scale per token, max|a| / 127).
 *
 *   S_i    = sum_j x_ij^2, summed exactly and rounded once to binary64
 *   inv_i  = RN32(1 / sqrt(S_i / K + eps)), each binary64 operation
 *            (divide, add, square root, reciprocal) correctly rounded
 *   a_ij   = fl32(fl32(x_ij * inv_i) * gain_j)
 *   d_i    = fl32(max_j |a_ij| / 127)
 *   xq_ij  = clamp(round_half_even(fl32(a_ij / d_i)), -127, 127); 0 when d_i == 0
 *
 * A row whose S_i / K + eps is 0, or whose inv_i overflows binary32 (only
 * possible with eps == 0 and every |x| below about 2^-124), normalises to 0.
 * x: [M x ldx] of type xt (SQ_F32, SQ_BF16 or SQ_F16). gain: [K] binary32
 * (from sq_fold_norm_gain), 16-byte aligned. eps: finite, >= 0 (SQ_ERR_RANGE
 * otherwise). K <= SQ_MAX_K_NORM (SQ_ERR_RANGE otherwise).
 * xq: [M x K] int8 output. x_scale: [M] binary32 output.
 */
sq_status sq_rmsnorm_quant(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* gain,
                           float eps, int8_t* xq, float* x_scale, sq_stream_t stream);

/*
 * sq_rmsnorm_quant followed by sq_w8a8_linear on the same stream, with Xq,
 * the row scales and the GEMM's workspace held in ws (the same layout and
 * size as sq_w8a8_linear_dyn; its contents need no initialisation). The
 * results equal those of the two calls made separately.
 */
size_t sq_rmsnorm_w8a8_linear_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_rmsnorm_w8a8_linear(const void* x, sq_dtype xt, int64_t ldx, const float* gain, float eps,
                                 const int8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                                 sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes, sq_stream_t stream);

/*
 * The down projection's input of a gated MLP, h = SiLU(gate) * up, fused with
 * the smoothing divide and the per-token int8 quantisation of h.
 * [W8A8] "How the Model Was Compressed" and "Why Activation Quantization Is
 * Hard" (one scale per token, max / 127), "How the smoothing factor is
 * computed" (the activation is divided by s), "Performance After
 * Quantization" (the per-token quantisation steps are memory-bound and cost
 * inter-token latency: here h never goes to memory in floating point).
 *
 *   e      = exp(-gate_ij) by a fixed binary32 algorithm (argument reduction
 *            k = rint(t * RN32(1/ln2)), r = (t - k*L1) - k*L2, degree-7 Taylor
 *            polynomial with coefficients RN32(1/n!) in Horner form, ldexp;
 *            t > 100 -> +inf, t < -110 -> 0), no fused multiply-add
 *   h_ij   = bf16(fl32(fl32(gate_ij * fl32(1 / fl32(1 + e))) * up_ij))
 *   xh_ij  = fl32(h_ij / s_j)                (h_ij itself when smooth == NULL)
 *   d_i    = fl32(max_j |xh_ij| / 127)
 *   xq_ij  = clamp(round_half_even(fl32(xh_ij / d_i)), -127, 127); 0 when d_i == 0
 *
 * gate, up: [M x ldg], [M x ldu] bf16 (t must be SQ_BF16), e.g. the two
 * halves of one [M x 2K] gate/up output with ldg = ldu = 2K. smooth: [K] or
 * NULL. K <= SQ_MAX_K_SILU (SQ_ERR_RANGE otherwise). xq: [M x K] int8 output.
 * x_scale: [M] binary32 output.
 */
sq_status sq_silu_mul_quant(const void* gate, const void* up, sq_dtype t, int64_t m, int64_t k, int64_t ldg,
                            int64_t ldu, const float* smooth, int8_t* xq, float* x_scale, sq_stream_t stream);

/*
 * sq_silu_mul_quant followed by sq_w8a8_linear (the down projection) on the
 * same stream; Xq, the row scales and the GEMM's workspace live in ws (the
 * layout and size of sq_w8a8_linear_dyn; no initialisation needed). The
 * results equal those of the two calls made separately.
 */
size_t sq_silu_mul_w8a8_linear_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_silu_mul_w8a8_linear(const void* gate, const void* up, sq_dtype t, int64_t ldg, int64_t ldu,
                                  const float* smooth, const int8_t* wq, const float* w_scale, int64_t m, int64_t n,
                                  int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes,
                                  sq_stream_t stream);

/*
 * FP8 (E4M3) W8A8 variant.
 * [W8A8] "Conclusion": FP8 quantisation skips the calibration algorithms
 * (SmoothQuant, GPTQ) and needs newer hardware; the pages give no format or
 * scaling details. E4M3 here is the OCP encoding (1 sign, 4 exponent bits
 * with bias 7, 3 mantissa bits, largest finite 448, no infinities), stored
 * one code per byte; scales are the int8 path's with 448 for 127; no
 * smoothing.
 *
 * sq_quant_act_fp8 (per token):
 *   d_i = fl32(max_j |x_ij| / 448);  xq_ij = E4M3(fl32(x_ij / d_i)), nearest
 *   value, ties to even; 0 when d_i == 0.
 *   x: [M x ldx] of type xt (SQ_F32, SQ_BF16, SQ_F16). xq: [M x K] codes.
 *   K <= SQ_MAX_K_FP8.
 * sq_quant_weights_fp8 (per output channel, load time):
 *   sw_n = fl32(max_k |W_kn| / 448);  wq[n][k] = E4M3(fl32(W_kn / sw_n))
 *   w: [K x ldw] of type wt, 16-byte aligned rows, N % 64 == 0. wq: [N x K]
 *   codes (transposed like the int8 weights). ws: at least
 *   sq_quant_weights_fp8_workspace_size(k, n) bytes (column maxima).
 * sq_fp8_linear:
 *   acc_in = sum_k E4M3(xq_ik) * E4M3(wq_nk) on the matrix cores (binary32
 *            sums that are not rounded to nearest: within ~2^-12 of the sum
 *            of |products| per 64-term instruction, measured)
 *   y[i][n] = out(fl32(fl32(acc_in * x_scale_i) * w_scale_n)), yt = SQ_F32,
 *   SQ_BF16 or SQ_F16. K % 128 == 0, K <= SQ_MAX_K_FP8.
 *   ws: sq_fp8_linear_workspace_size(m, n, k) bytes, 16-byte aligned (NULL
 *   when that is 0), with the layout, contract and failure mode of
 *   sq_w8a8_linear's workspace: for shapes whose K is split over several
 *   workgroups (the decode and prefill cases of sq_w8a8_linear) it holds the
 *   ticket counters (first 1 KiB, zero when a call starts: the caller
 *   zero-fills once, every call leaves them at zero) and binary32 partial
 *   tiles; one call at a time per workspace. The partial tiles are added in
 *   a fixed order (deterministic results), each sum rounded to binary32.
 * sq_fp8_linear_dyn: sq_quant_act_fp8 then sq_fp8_linear on the same stream,
 *   with the codes, row scales and the GEMM's workspace in ws
 *   (sq_fp8_linear_dyn_workspace_size; no initialisation needed: the
 *   quantisation launch clears the split-K counters).
 */
sq_status sq_quant_act_fp8(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, uint8_t* xq,
                           float* x_scale, sq_stream_t stream);
size_t sq_quant_weights_fp8_workspace_size(int64_t k, int64_t n);
sq_status sq_quant_weights_fp8(const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw, uint8_t* wq,
                               float* w_scale, void* ws, size_t ws_bytes, sq_stream_t stream);
size_t sq_fp8_linear_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_fp8_linear(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                        int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes,
                        sq_stream_t stream);
size_t sq_fp8_linear_dyn_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_fp8_linear_dyn(const void* x, sq_dtype xt, int64_t ldx, const uint8_t* wq, const float* w_scale,
                            int64_t m, int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws,
                            size_t ws_bytes, sq_stream_t stream);

/*
 * GPTQ weight rounding, the weight half of the pages' compression pipeline,
 * run once at load time in place of round-to-nearest.
 * [W8A8] "How GPTQ improves on naive quantization" (quantise one weight,
 * measure its error, spread it over the weights not yet quantised as the
 * Hessian of the calibration activations directs); "How the smoothing
 * factor is computed" (it starts from the smoothed weights); the GPTQ paper
 * cited there (input order, damping by 1% of the mean diagonal).
 *
 * sq_gptq_hessian:   h[a][b] += sum_t xh_ta * xh_tb,  xh = fl32(x / s_j)
 *   (x itself when smooth == NULL), in binary64. Call it once per batch of
 *   calibration rows; the caller zero-fills h once before the first call.
 *   x: [T x ldx] SQ_F32, SQ_BF16 or SQ_F16, element-aligned. smooth: [K] or
 *   NULL. h: [K x K] binary64, row-major, 8-byte aligned, written whole and
 *   symmetric. K % 128 == 0 and K <= SQ_MAX_K_GPTQ (SQ_ERR_SHAPE /
 *   SQ_ERR_RANGE otherwise).
 *
 * sq_gptq_quantize: from h and the weights W [K x N] (row j = input j):
 *   W'_jn = fl32(s_j * W_jn) (W itself when smooth == NULL); inputs with
 *   h_jj == 0 are dead: W'_j = 0 and h_jj taken as 1;
 *   sw_n  = fl32(max_j |W'_jn| / 127), as sq_smooth_fold_weights;
 *   lambda = damp * mean_j h_jj, added to the diagonal;
 *   for j = 0 .. K-1, every n:  q_jn = clamp(round_half_even(z_jn / sw_n), -127, 127)
 *   where z_jn is W'_jn plus the errors of the earlier inputs of channel n
 *   passed on through the damped h (the GPTQ update), all in binary64.
 *   Only the lower triangle of h (row >= column) is read. The result is
 *   deterministic; it equals a sequential binary64 GPTQ except where a
 *   quotient lies within rounding of a half-integer.
 *   w: [K x ldw] SQ_F32, SQ_BF16 or SQ_F16, element-aligned. damp: in
 *   (0, 1] (SQ_ERR_RANGE otherwise; 0.01 is the usual value). wq: [N x K]
 *   int8 output (transposed, like sq_smooth_fold_weights), 16-byte aligned.
 *   w_scale: [N] binary32 output. ws: sq_gptq_quantize_workspace_size(k, n)
 *   bytes, 16-byte aligned, no initialisation needed (it holds the K x K
 *   factor, W' and the running corrections: 12 K N + 8 K^2 bytes and a
 *   little more). About 3 K/64 + 4 launches.
 */
sq_status sq_gptq_hessian(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, const float* smooth,
                          double* h, sq_stream_t stream);
size_t sq_gptq_quantize_workspace_size(int64_t k, int64_t n);
sq_status sq_gptq_quantize(const double* h, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                           const float* smooth, float damp, int8_t* wq, float* w_scale, void* ws, size_t ws_bytes,
                           sq_stream_t stream);

/*
 * LLM.int8() outlier detection over the feature columns of X.
 * [INT8] "The architecture: every piece explained", top row (a column is an
 * outlier when some |x| in it exceeds the threshold; 6.0 is the usual value).
 *
 *   mask[c] = (max_i |x[i][c]| > threshold) ? 1 : 0          (strictly greater)
 *   idx[0 .. count-1] = the outlier columns in ascending order; *count = their number
 *
 * x: [M x ldx] SQ_F16 or SQ_BF16 or SQ_F32. mask: [K] uint8 output. idx: [K]
 * int32 output (only the first *count entries are defined). count: one int32
 * in device memory. ws: sq_outlier_detect_workspace_size(k) bytes.
 */
size_t sq_outlier_detect_workspace_size(int64_t k);
sq_status sq_outlier_detect(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, float threshold,
                            uint8_t* mask, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                            sq_stream_t stream);

/*
 * LLM.int8() row-wise (vectorwise) int8 quantisation of the regular columns.
 * [INT8] "End-to-end flow" (each row's scale is its absolute maximum over the
 * regular features only).
 *
 *   d_i   = fl32(max_{c : mask[c]==0} |x_ic| / 127)
 *   xq_ic = mask[c] ? 0 : clamp(round_half_even(fl32(x_ic / d_i)), -127, 127); 0 when d_i == 0
 *
 * Setting the outlier columns of Xq to zero gives the same int8 product as
 * removing them from X and from W.
 */
sq_status sq_quant_act_rows_masked(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx,
                                   const uint8_t* mask, int8_t* xq, float* x_scale, sq_stream_t stream);

/*
 * LLM.int8() decomposed linear layer, fp16 in and out.
 * [INT8] "The architecture: every piece explained" and "End-to-end flow":
 * detection, column split, int8 path with row scales over the regular
 * columns and load-time column scales of W, fp16 path over the outlier slice,
 * element-wise sum of the two fp16 partial products.
 *
 *   y_int  = fp16( fl32( fl32(fl32(acc_in) * d_i) * w_scale_n ) )
 *   y_out  = fp16( sum over outlier columns c in ascending order of x_ic * w16[c][n] ),
 *            each product and each partial sum rounded to binary32
 *   y[i][n] = fp16( y_int + y_out )        (the exact sum of the two fp16 values, rounded once)
 *
 * x: [M x ldx] SQ_F16. wq: [N x K] int8 and w_scale: [N] from
 * sq_smooth_fold_weights(..., SQ_SMOOTH_NONE) on the same fp16 W. w16: [K x
 * ldw16] fp16 weights (only the outlier rows are read). y: [M x ldy] fp16.
 * n_outliers: one int32 in device memory, the number of outlier columns found.
 * ws: sq_int8_decomp_workspace_size(m, n, k) bytes.
 */
size_t sq_int8_decomp_workspace_size(int64_t m, int64_t n, int64_t k);
sq_status sq_int8_decomp_linear(const void* x, int64_t ldx, const int8_t* wq, const float* w_scale,
                                const void* w16, int64_t ldw16, int64_t m, int64_t n, int64_t k,
                                float threshold, void* y, int64_t ldy, int32_t* n_outliers,
                                void* ws, size_t ws_bytes, sq_stream_t stream);

/*
 * The second half of sq_int8_decomp_linear on its own, for callers that run
 * detection (sq_outlier_detect) and the masked quantisation
 * (sq_quant_act_rows_masked) themselves, e.g. to reuse one detection:
 * the int8 GEMM of the masked, row-quantised X with the fp16 outlier slice
 * added in the epilogue.
 * [INT8] "The architecture: every piece explained" (int8 path with the outer
 * product of row and column scales, fp16 path over the outlier slice, sum in
 * fp16); "End-to-end flow".
 *
 *   y[i][n] = fp16( y_int + y_out ) with y_int and y_out as defined for
 *   sq_int8_decomp_linear, the outlier columns being idx[0 .. *n_outliers-1]
 *
 * xq: [M x K] int8 with the outlier columns zero, x_scale: [M] (both from
 * sq_quant_act_rows_masked). x: [M x ldx] fp16 activations (only the outlier
 * columns are read). wq: [N x K] int8, w_scale: [N]. w16: [K x ldw16] fp16
 * (only the outlier rows are read). idx, n_outliers: from sq_outlier_detect
 * (device memory). y: [M x ldy] fp16 output. Pointers to fp16 data need
 * 2-byte alignment, xq and wq 16-byte alignment. Results equal those of
 * sq_int8_decomp_linear bit for bit.
 */
sq_status sq_int8_decomp_gemm(const int8_t* xq, const float* x_scale, const void* x, int64_t ldx, const int8_t* wq,
                              const float* w_scale, const void* w16, int64_t ldw16, const int32_t* idx,
                              const int32_t* n_outliers, int64_t m, int64_t n, int64_t k, void* y, int64_t ldy,
                              sq_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H_ */
