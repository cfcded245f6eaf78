// C ABI of the W8A8 library: argument validation and dispatch to the gfx950
// kernels. Every check runs before the first launch, so a call that returns
// an error has enqueued nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "sq.h"
#include "sq_launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

// A C caller may pass any int for an enum argument, but in C++ an enum object
// holds only values within its enumerators' bit range (loading another is
// undefined behaviour, which the host-sanitized build reports). Enum
// arguments are therefore read as plain ints (memcpy, not a load of the enum)
// and range-checked before any other use.
template <class E>
int enum_value(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "enum arguments are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}
bool dtype_in_range(const sq_dtype& t) {
  const int v = enum_value(t);
  return v >= (int)SQ_F32 && v <= (int)SQ_I8;
}

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(sq_dtype t) {
  switch (t) {
    case SQ_F32: case SQ_I32: return 4;
    case SQ_BF16: case SQ_F16: return 2;
    case SQ_I8: return 1;
  }
  return 0;
}

bool float_input(sq_dtype t) { return t == SQ_F32 || t == SQ_BF16 || t == SQ_F16; }

sq_status check_k(int64_t k) { return (k < 64 || k % 64 != 0) ? SQ_ERR_SHAPE : SQ_OK; }

// A float matrix [rows x ld] read with 16-byte vectors.
sq_status check_vec_matrix(const void* p, sq_dtype t, int64_t rows, int64_t cols, int64_t ld) {
  if (!float_input(t)) return SQ_ERR_DTYPE;
  if (rows < 0 || cols < 0) return SQ_ERR_SHAPE;
  if (ld < cols) return SQ_ERR_SHAPE;
  if (rows == 0 || cols == 0) return SQ_OK;
  if (!p) return SQ_ERR_NULL;
  if (!aligned16(p) || (ld * elem_bytes(t)) % 16 != 0) return SQ_ERR_ALIGN;
  return SQ_OK;
}

sq_status hip_status(hipError_t e) {
  if (e == hipSuccess) return SQ_OK;
  g_last_hip_error = (int)e;
  return SQ_ERR_HIP;
}

#define SQ_TRY(expr)              \
  do {                            \
    const sq_status st_ = (expr); \
    if (st_ != SQ_OK) return st_; \
  } while (0)

// Quantisation (by `quant`, which writes Xq and the row scales and clears the
// given counter words) followed by the GEMM, with Xq, the scales and the
// GEMM's workspace carved out of ws.
template <class Quant>
sq_status quant_then_gemm(Quant quant, const int8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k,
                          void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  int8_t* xq = reinterpret_cast<int8_t*>(ws);
  float* dx = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + round_up((size_t)m * (size_t)k));
  void* gws = reinterpret_cast<char*>(ws) + round_up((size_t)m * (size_t)k) + round_up((size_t)m * 4);
  if (sqh::gemm_decode_suits(m, n, k, false)) {
    // the quantisation launch also clears the GEMM's split-K counters
    uint32_t* counters;
    int64_t ncount;
    sqh::gemm_decode_counters(m, n, k, false, gws, &counters, &ncount);
    hipError_t e = quant(xq, dx, counters, ncount);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(sqh::gemm_i8_decode(xq, dx, wq, w_scale, m, n, k, y, yt, ldy, gws, s));
  }
  // prefill shapes split over K: the quantisation launch clears the tile counters
  uint32_t* counters;
  int64_t ncount;
  sqh::gemm_big_counters(m, n, k, false, gws, &counters, &ncount);
  hipError_t e = quant(xq, dx, counters, ncount);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(sqh::gemm_i8(xq, dx, wq, w_scale, m, n, k, y, yt, ldy, nullptr, gws, s));
}

}  // namespace

namespace sqh {
void set_last_hip_error(int e) { g_last_hip_error = e; }
}  // namespace sqh

extern "C" {

const char* sq_status_string(sq_status status) {
  switch (enum_value(status)) {
    case SQ_OK: return "ok";
    case SQ_ERR_NULL: return "a required pointer is NULL";
    case SQ_ERR_DTYPE: return "element type not supported by this call";
    case SQ_ERR_SHAPE: return "bad shape (negative size, K not a positive multiple of 64, or leading dimension too small)";
    case SQ_ERR_ALIGN: return "pointer or row not 16-byte aligned";
    case SQ_ERR_RANGE: return "value out of range (alpha, K beyond the int32 accumulator headroom, or flags)";
    case SQ_ERR_WORKSPACE: return "workspace missing or too small";
    case SQ_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int sq_last_hip_error(void) { return g_last_hip_error; }

int sq_version(void) { return 10000; }

sq_status sq_calibrate_absmax(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, float* absmax,
                              sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  SQ_TRY(check_vec_matrix(x, xt, t, k, ldx));
  if (!absmax) return SQ_ERR_NULL;
  if (t == 0) return SQ_OK;
  return hip_status(sqh::absmax_cols(x, xt, t, k, ldx, absmax, (hipStream_t)stream));
}

size_t sq_smooth_fold_workspace_size(int64_t k, int64_t n) {
  (void)k;
  return n > 0 ? round_up((size_t)n * 4) : 0;
}

sq_status sq_smooth_fold_weights(const float* absmax, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                                 double alpha, uint32_t flags, float* smooth, int8_t* wq, float* w_scale, void* ws,
                                 size_t ws_bytes, sq_stream_t stream) {
  if (!dtype_in_range(wt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  if (n < 0) return SQ_ERR_SHAPE;
  if (!float_input(wt)) return SQ_ERR_DTYPE;
  if (ldw < n) return SQ_ERR_SHAPE;
  if (n > 0 && !w) return SQ_ERR_NULL;
  // W may have any row pitch (element loads are used when rows are not 16-byte aligned)
  if (reinterpret_cast<uintptr_t>(w) % (uintptr_t)elem_bytes(wt) != 0) return SQ_ERR_ALIGN;
  if (flags != SQ_SMOOTH_COMPUTE && flags != SQ_SMOOTH_GIVEN && flags != SQ_SMOOTH_NONE) return SQ_ERR_RANGE;
  if (flags == SQ_SMOOTH_COMPUTE && !(alpha >= 0.0 && alpha <= 1.0)) return SQ_ERR_RANGE;
  if (flags == SQ_SMOOTH_COMPUTE && !absmax) return SQ_ERR_NULL;
  if (flags != SQ_SMOOTH_NONE && !smooth) return SQ_ERR_NULL;
  if (n == 0) {
    // No weights: every row maximum is 0, so a computed s is 1 (no smoothing).
    if (flags != SQ_SMOOTH_COMPUTE) return SQ_OK;
    return hip_status(sqh::fill_u32(smooth, 0x3F800000u, k, (hipStream_t)stream));
  }
  if (!wq || !w_scale) return SQ_ERR_NULL;
  if (!aligned16(wq)) return SQ_ERR_ALIGN;
  if (ws_bytes < sq_smooth_fold_workspace_size(k, n) || !ws) return SQ_ERR_WORKSPACE;
  return hip_status(sqh::fold_weights(absmax, w, wt, k, n, ldw, alpha, flags, smooth, wq, w_scale, (float*)ws,
                                      (hipStream_t)stream));
}

sq_status sq_quant_act_per_token(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* smooth,
                                 int8_t* xq, float* x_scale, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (m == 0) return SQ_OK;
  if (!xq || !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq) || (smooth && !aligned16(smooth))) return SQ_ERR_ALIGN;
  return hip_status(sqh::quant_rows(x, xt, m, k, ldx, smooth, nullptr, xq, x_scale, (hipStream_t)stream));
}

size_t sq_w8a8_linear_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0 || k % 64 != 0) return 0;
  if (sqh::gemm_decode_suits(m, n, k, false)) return sqh::gemm_decode_workspace(m, n, k, false);
  return sqh::gemm_big_workspace(m, n, k, false);
}

// Shapes, output type and the weight-side pointers of the GEMM.
static sq_status check_gemm_common(const int8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k,
                                   const void* y, sq_dtype yt, int64_t ldy) {
  SQ_TRY(check_k(k));
  if (k > SQ_MAX_K_INT32) return SQ_ERR_RANGE;
  if (m < 0 || n < 0) return SQ_ERR_SHAPE;
  if (yt != SQ_F32 && yt != SQ_BF16 && yt != SQ_F16 && yt != SQ_I32) return SQ_ERR_DTYPE;
  if (ldy < n) return SQ_ERR_SHAPE;
  if (m == 0 || n == 0) return SQ_OK;
  if (m > INT32_MAX || n > INT32_MAX) return SQ_ERR_SHAPE;
  if (!wq || !y) return SQ_ERR_NULL;
  if (yt != SQ_I32 && !w_scale) return SQ_ERR_NULL;
  if (!aligned16(wq)) return SQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(y) % (uintptr_t)elem_bytes(yt)) != 0) return SQ_ERR_ALIGN;
  return SQ_OK;
}

static sq_status check_linear(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale,
                              int64_t m, int64_t n, int64_t k, const void* y, sq_dtype yt, int64_t ldy) {
  SQ_TRY(check_gemm_common(wq, w_scale, m, n, k, y, yt, ldy));
  if (m == 0 || n == 0) return SQ_OK;
  if (!xq) return SQ_ERR_NULL;
  if (yt != SQ_I32 && !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_ALIGN;
  return SQ_OK;
}

sq_status sq_w8a8_linear(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                         int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes,
                         sq_stream_t stream) {
  if (!dtype_in_range(yt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_linear(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy));
  if (m == 0 || n == 0) return SQ_OK;
  const size_t need = sq_w8a8_linear_workspace_size(m, n, k);
  if (need > 0 && (!ws || ws_bytes < need)) return SQ_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return SQ_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  // decode shapes: the workspace's split-K counters are zero on entry (the
  // caller's contract) and restored to zero by the kernel
  if (sqh::gemm_decode_suits(m, n, k, false))
    return hip_status(sqh::gemm_i8_decode(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, ws, s));
  // prefill shapes split over K: the same contract for the tile counters
  return hip_status(sqh::gemm_i8(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, nullptr, ws, s));
}

size_t sq_w8a8_linear_dyn_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  return round_up((size_t)m * (size_t)k) + round_up((size_t)m * 4) + sq_w8a8_linear_workspace_size(m, n, k);
}

sq_status sq_w8a8_linear_dyn(const void* x, sq_dtype xt, int64_t ldx, const float* smooth, const int8_t* wq,
                             const float* w_scale, int64_t m, int64_t n, int64_t k, void* y, sq_dtype yt,
                             int64_t ldy, void* ws, size_t ws_bytes, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  if (!dtype_in_range(yt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (yt == SQ_I32) return SQ_ERR_DTYPE;
  if (smooth && !aligned16(smooth)) return SQ_ERR_ALIGN;
  SQ_TRY(check_gemm_common(wq, w_scale, m, n, k, y, yt, ldy));
  if (m == 0 || n == 0) return SQ_OK;
  if (!ws || ws_bytes < sq_w8a8_linear_dyn_workspace_size(m, n, k)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  // one token on the weight-streaming path: one launch (the quantisation
  // runs inside the GEMM; the workspace is not touched)
  if (sqh::decode1_suits(m, n, k, xt))
    return hip_status(sqh::decode1_linear(x, xt, smooth, wq, w_scale, n, k, y, yt, s));
  auto quant = [&](int8_t* xq, float* dx, uint32_t* zero, int64_t nzero) {
    return sqh::quant_rows(x, xt, m, k, ldx, smooth, nullptr, xq, dx, s, zero, nzero);
  };
  return quant_then_gemm(quant, wq, w_scale, m, n, k, y, yt, ldy, ws, s);
}

// ---------------------------------------------------------------- RMSNorm with the folded gain
static sq_status check_norm(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* gain,
                            float eps) {
  SQ_TRY(check_k(k));
  if (k > SQ_MAX_K_NORM) return SQ_ERR_RANGE;
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (!(eps >= 0.f && eps <= 3.4028234663852886e38f)) return SQ_ERR_RANGE;
  if (m == 0) return SQ_OK;
  if (!gain) return SQ_ERR_NULL;
  if (!aligned16(gain)) return SQ_ERR_ALIGN;
  return SQ_OK;
}

sq_status sq_fold_norm_gain(const void* gamma, sq_dtype gt, const float* smooth, int64_t k, float* gain,
                            sq_stream_t stream) {
  if (!dtype_in_range(gt)) return SQ_ERR_DTYPE;
  if (k < 0) return SQ_ERR_SHAPE;
  if (!float_input(gt)) return SQ_ERR_DTYPE;
  if (k == 0) return SQ_OK;
  if (!gamma || !gain) return SQ_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(gamma) % (uintptr_t)elem_bytes(gt) != 0) return SQ_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(gain) % 4 != 0 || reinterpret_cast<uintptr_t>(smooth) % 4 != 0)
    return SQ_ERR_ALIGN;
  return hip_status(sqh::fold_norm_gain(gamma, gt, smooth, k, gain, (hipStream_t)stream));
}

sq_status sq_rmsnorm_quant(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* gain,
                           float eps, int8_t* xq, float* x_scale, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_norm(x, xt, m, k, ldx, gain, eps));
  if (m == 0) return SQ_OK;
  if (!xq || !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_ALIGN;
  return hip_status(sqh::rmsnorm_quant(x, xt, m, k, ldx, gain, eps, xq, x_scale, (hipStream_t)stream));
}

size_t sq_rmsnorm_w8a8_linear_workspace_size(int64_t m, int64_t n, int64_t k) {
  return sq_w8a8_linear_dyn_workspace_size(m, n, k);
}

sq_status sq_rmsnorm_w8a8_linear(const void* x, sq_dtype xt, int64_t ldx, const float* gain, float eps,
                                 const int8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k, void* y,
                                 sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  if (!dtype_in_range(yt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_norm(x, xt, m, k, ldx, gain, eps));
  if (yt == SQ_I32) return SQ_ERR_DTYPE;
  SQ_TRY(check_gemm_common(wq, w_scale, m, n, k, y, yt, ldy));
  if (m == 0 || n == 0) return SQ_OK;
  if (!ws || ws_bytes < sq_rmsnorm_w8a8_linear_workspace_size(m, n, k)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  auto quant = [&](int8_t* xq, float* dx, uint32_t* zero, int64_t nzero) {
    return sqh::rmsnorm_quant(x, xt, m, k, ldx, gain, eps, xq, dx, s, zero, nzero);
  };
  return quant_then_gemm(quant, wq, w_scale, m, n, k, y, yt, ldy, ws, s);
}

// ---------------------------------------------------------------- gated activation -> down projection
static sq_status check_silu(const void* gate, const void* up, sq_dtype t, int64_t m, int64_t k, int64_t ldg,
                            int64_t ldu, const float* smooth) {
  SQ_TRY(check_k(k));
  if (k > SQ_MAX_K_SILU) return SQ_ERR_RANGE;
  if (t != SQ_BF16) return SQ_ERR_DTYPE;
  SQ_TRY(check_vec_matrix(gate, t, m, k, ldg));
  SQ_TRY(check_vec_matrix(up, t, m, k, ldu));
  if (smooth && !aligned16(smooth)) return SQ_ERR_ALIGN;
  return SQ_OK;
}

sq_status sq_silu_mul_quant(const void* gate, const void* up, sq_dtype t, int64_t m, int64_t k, int64_t ldg,
                            int64_t ldu, const float* smooth, int8_t* xq, float* x_scale, sq_stream_t stream) {
  if (!dtype_in_range(t)) return SQ_ERR_DTYPE;
  SQ_TRY(check_silu(gate, up, t, m, k, ldg, ldu, smooth));
  if (m == 0) return SQ_OK;
  if (!xq || !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_ALIGN;
  return hip_status(sqh::silu_quant(gate, up, m, k, ldg, ldu, smooth, xq, x_scale, (hipStream_t)stream));
}

size_t sq_silu_mul_w8a8_linear_workspace_size(int64_t m, int64_t n, int64_t k) {
  return sq_w8a8_linear_dyn_workspace_size(m, n, k);
}

sq_status sq_silu_mul_w8a8_linear(const void* gate, const void* up, sq_dtype t, int64_t ldg, int64_t ldu,
                                  const float* smooth, const int8_t* wq, const float* w_scale, int64_t m, int64_t n,
                                  int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes,
                                  sq_stream_t stream) {
  if (!dtype_in_range(t)) return SQ_ERR_DTYPE;
  if (!dtype_in_range(yt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_silu(gate, up, t, m, k, ldg, ldu, smooth));
  if (yt == SQ_I32) return SQ_ERR_DTYPE;
  SQ_TRY(check_gemm_common(wq, w_scale, m, n, k, y, yt, ldy));
  if (m == 0 || n == 0) return SQ_OK;
  if (!ws || ws_bytes < sq_silu_mul_w8a8_linear_workspace_size(m, n, k)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  auto quant = [&](int8_t* xq, float* dx, uint32_t* zero, int64_t nzero) {
    return sqh::silu_quant(gate, up, m, k, ldg, ldu, smooth, xq, dx, s, zero, nzero);
  };
  return quant_then_gemm(quant, wq, w_scale, m, n, k, y, yt, ldy, ws, s);
}

// ---------------------------------------------------------------- FP8 (E4M3) variant
sq_status sq_quant_act_fp8(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, uint8_t* xq,
                           float* x_scale, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  if (k > SQ_MAX_K_FP8) return SQ_ERR_RANGE;
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (m == 0) return SQ_OK;
  if (!xq || !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_ALIGN;
  return hip_status(sqh::quant_f8_rows(x, xt, m, k, ldx, xq, x_scale, (hipStream_t)stream));
}

size_t sq_quant_weights_fp8_workspace_size(int64_t k, int64_t n) {
  (void)k;
  return n > 0 ? round_up((size_t)n * 4) : 0;
}

sq_status sq_quant_weights_fp8(const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw, uint8_t* wq,
                               float* w_scale, void* ws, size_t ws_bytes, sq_stream_t stream) {
  if (!dtype_in_range(wt)) return SQ_ERR_DTYPE;
  if (k < 0) return SQ_ERR_SHAPE;
  // the column maxima read W with 16-byte vectors along N
  SQ_TRY(check_k(n));
  SQ_TRY(check_vec_matrix(w, wt, k, n, ldw));
  if (k == 0) return SQ_OK;
  if (!wq || !w_scale) return SQ_ERR_NULL;
  if (!ws || ws_bytes < sq_quant_weights_fp8_workspace_size(k, n)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  return hip_status(sqh::quant_f8_weights(w, wt, k, n, ldw, reinterpret_cast<float*>(ws), wq, w_scale,
                                          (hipStream_t)stream));
}

static sq_status check_fp8_gemm(const uint8_t* wq, const float* w_scale, int64_t m, int64_t n, int64_t k,
                                 const void* y, sq_dtype yt, int64_t ldy) {
  if (k < 128 || k % 128 != 0) return SQ_ERR_SHAPE;
  if (k > SQ_MAX_K_FP8) return SQ_ERR_RANGE;
  if (m < 0 || n < 0) return SQ_ERR_SHAPE;
  if (yt != SQ_F32 && yt != SQ_BF16 && yt != SQ_F16) return SQ_ERR_DTYPE;
  if (ldy < n) return SQ_ERR_SHAPE;
  if (m == 0 || n == 0) return SQ_OK;
  if (m > INT32_MAX || n > INT32_MAX) return SQ_ERR_SHAPE;
  if (!wq || !w_scale || !y) return SQ_ERR_NULL;
  if (!aligned16(wq)) return SQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(y) % (uintptr_t)elem_bytes(yt)) != 0) return SQ_ERR_ALIGN;
  return SQ_OK;
}

size_t sq_fp8_linear_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || n <= 0 || k <= 0) return 0;
  if (sqh::gemm_decode_suits(m, n, k, true)) return sqh::gemm_decode_workspace(m, n, k, true);
  return sqh::gemm_big_workspace(m, n, k, true);
}

sq_status sq_fp8_linear(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                        int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, size_t ws_bytes,
                        sq_stream_t stream) {
  if (!dtype_in_range(yt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_fp8_gemm(wq, w_scale, m, n, k, y, yt, ldy));
  if (m == 0 || n == 0) return SQ_OK;
  if (!xq || !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_ALIGN;
  const size_t need = sq_fp8_linear_workspace_size(m, n, k);
  if (need > 0 && (!ws || ws_bytes < need)) return SQ_ERR_WORKSPACE;
  if (need > 0 && !aligned16(ws)) return SQ_ERR_ALIGN;
  const hipStream_t s = (hipStream_t)stream;
  // decode shapes: the workspace's split-K counters are zero on entry (the
  // caller's contract) and restored to zero by the kernel
  if (sqh::gemm_decode_suits(m, n, k, true))
    return hip_status(sqh::gemm_f8_decode(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, ws, s));
  return hip_status(sqh::gemm_f8(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, ws, s));
}

size_t sq_fp8_linear_dyn_workspace_size(int64_t m, int64_t n, int64_t k) {
  if (m <= 0 || k <= 0) return 0;
  return round_up((size_t)m * (size_t)k) + round_up((size_t)m * 4) + sq_fp8_linear_workspace_size(m, n, k);
}

sq_status sq_fp8_linear_dyn(const void* x, sq_dtype xt, int64_t ldx, const uint8_t* wq, const float* w_scale,
                            int64_t m, int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws,
                            size_t ws_bytes, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  if (!dtype_in_range(yt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_fp8_gemm(wq, w_scale, m, n, k, y, yt, ldy));
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (m == 0 || n == 0) return SQ_OK;
  if (!ws || ws_bytes < sq_fp8_linear_dyn_workspace_size(m, n, k)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  uint8_t* xq = reinterpret_cast<uint8_t*>(ws);
  float* dx = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + round_up((size_t)m * (size_t)k));
  void* gws = reinterpret_cast<char*>(ws) + round_up((size_t)m * (size_t)k) + round_up((size_t)m * 4);
  const hipStream_t s = (hipStream_t)stream;
  if (sqh::gemm_decode_suits(m, n, k, true)) {
    // the quantisation launch also clears the GEMM's split-K counters
    uint32_t* counters;
    int64_t ncount;
    sqh::gemm_decode_counters(m, n, k, true, gws, &counters, &ncount);
    hipError_t e = sqh::quant_f8_rows(x, xt, m, k, ldx, xq, dx, s, counters, ncount);
    if (e != hipSuccess) return hip_status(e);
    return hip_status(sqh::gemm_f8_decode(xq, dx, wq, w_scale, m, n, k, y, yt, ldy, gws, s));
  }
  uint32_t* counters;
  int64_t ncount;
  sqh::gemm_big_counters(m, n, k, true, gws, &counters, &ncount);
  hipError_t e = sqh::quant_f8_rows(x, xt, m, k, ldx, xq, dx, s, counters, ncount);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(sqh::gemm_f8(xq, dx, wq, w_scale, m, n, k, y, yt, ldy, gws, s));
}

// ---------------------------------------------------------------- GPTQ
static sq_status check_gptq_k(int64_t k) {
  if (k < 128 || k % 128 != 0) return SQ_ERR_SHAPE;
  if (k > SQ_MAX_K_GPTQ) return SQ_ERR_RANGE;
  return SQ_OK;
}

static bool elem_aligned(const void* p, sq_dtype t) {
  return (reinterpret_cast<uintptr_t>(p) % (uintptr_t)elem_bytes(t)) == 0;
}

sq_status sq_gptq_hessian(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, const float* smooth,
                          double* h, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  if (!float_input(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_gptq_k(k));
  if (t < 0 || ldx < k) return SQ_ERR_SHAPE;
  if (t == 0) return SQ_OK;
  if (!x || !h) return SQ_ERR_NULL;
  if (!elem_aligned(x, xt) || (reinterpret_cast<uintptr_t>(h) & 7u) != 0 ||
      (reinterpret_cast<uintptr_t>(smooth) & 3u) != 0)
    return SQ_ERR_ALIGN;
  return hip_status(sqh::gptq_hessian(x, xt, t, k, ldx, smooth, h, (hipStream_t)stream));
}

size_t sq_gptq_quantize_workspace_size(int64_t k, int64_t n) { return sqh::gptq_workspace(k, n); }

sq_status sq_gptq_quantize(const double* h, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                           const float* smooth, float damp, int8_t* wq, float* w_scale, void* ws, size_t ws_bytes,
                           sq_stream_t stream) {
  if (!dtype_in_range(wt)) return SQ_ERR_DTYPE;
  if (!float_input(wt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_gptq_k(k));
  if (n < 0 || ldw < n) return SQ_ERR_SHAPE;
  if (!(damp > 0.f && damp <= 1.f)) return SQ_ERR_RANGE;
  if (n == 0) return SQ_OK;
  if (!h || !w || !wq || !w_scale) return SQ_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(h) & 7u) != 0 || !elem_aligned(w, wt) || !aligned16(wq) ||
      (reinterpret_cast<uintptr_t>(w_scale) & 3u) != 0 || (reinterpret_cast<uintptr_t>(smooth) & 3u) != 0)
    return SQ_ERR_ALIGN;
  if (!ws || ws_bytes < sq_gptq_quantize_workspace_size(k, n)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  return hip_status(sqh::gptq_quantize(h, w, wt, k, n, ldw, smooth, (double)damp, wq, w_scale, ws,
                                       (hipStream_t)stream));
}

size_t sq_outlier_detect_workspace_size(int64_t k) { return k > 0 ? round_up((size_t)k * 4) : 0; }

sq_status sq_outlier_detect(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, float threshold,
                            uint8_t* mask, int32_t* idx, int32_t* count, void* ws, size_t ws_bytes,
                            sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (std::isnan(threshold)) return SQ_ERR_RANGE;
  if (!mask || !idx || !count) return SQ_ERR_NULL;
  if (!ws || ws_bytes < sq_outlier_detect_workspace_size(k)) return SQ_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  float* colmax = (float*)ws;
  hipError_t e = sqh::fill_u32(colmax, 0u, k, s);
  if (e == hipSuccess) e = sqh::absmax_cols(x, xt, m, k, ldx, colmax, s);
  if (e == hipSuccess) e = sqh::outlier_select(colmax, k, threshold, mask, idx, count, s);
  return hip_status(e);
}

sq_status sq_quant_act_rows_masked(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx,
                                   const uint8_t* mask, int8_t* xq, float* x_scale, sq_stream_t stream) {
  if (!dtype_in_range(xt)) return SQ_ERR_DTYPE;
  SQ_TRY(check_k(k));
  SQ_TRY(check_vec_matrix(x, xt, m, k, ldx));
  if (!mask) return SQ_ERR_NULL;
  if (m == 0) return SQ_OK;
  if (!xq || !x_scale) return SQ_ERR_NULL;
  if (!aligned16(xq)) return SQ_ERR_ALIGN;
  return hip_status(sqh::quant_rows(x, xt, m, k, ldx, nullptr, mask, xq, x_scale, (hipStream_t)stream));
}

size_t sq_int8_decomp_workspace_size(int64_t m, int64_t n, int64_t k) {
  (void)n;
  if (k <= 0) return 0;
  const size_t mm = m > 0 ? (size_t)m : 0;
  return round_up((size_t)k * 4) + round_up((size_t)k) + round_up((size_t)k * 4) + round_up(mm * (size_t)k) +
         round_up(mm * 4);
}

sq_status sq_int8_decomp_linear(const void* x, int64_t ldx, const int8_t* wq, const float* w_scale, const void* w16,
                                int64_t ldw16, int64_t m, int64_t n, int64_t k, float threshold, void* y,
                                int64_t ldy, int32_t* n_outliers, void* ws, size_t ws_bytes, sq_stream_t stream) {
  SQ_TRY(check_k(k));
  SQ_TRY(check_vec_matrix(x, SQ_F16, m, k, ldx));
  if (k > SQ_MAX_K_INT32) return SQ_ERR_RANGE;
  if (n < 0) return SQ_ERR_SHAPE;
  if (ldw16 < n || ldy < n) return SQ_ERR_SHAPE;
  if (std::isnan(threshold)) return SQ_ERR_RANGE;
  if (!n_outliers) return SQ_ERR_NULL;
  if (m > INT32_MAX || n > INT32_MAX) return SQ_ERR_SHAPE;
  if (m > 0 && n > 0) {
    if (!w16 || !wq || !w_scale || !y) return SQ_ERR_NULL;
    if (!aligned16(wq)) return SQ_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(w16) & 1u) || (reinterpret_cast<uintptr_t>(y) & 1u)) return SQ_ERR_ALIGN;
  }
  if (!ws || ws_bytes < sq_int8_decomp_workspace_size(m, n, k)) return SQ_ERR_WORKSPACE;
  if (!aligned16(ws)) return SQ_ERR_ALIGN;
  char* p = reinterpret_cast<char*>(ws);
  float* colmax = reinterpret_cast<float*>(p);
  p += round_up((size_t)k * 4);
  uint8_t* mask = reinterpret_cast<uint8_t*>(p);
  p += round_up((size_t)k);
  int32_t* idx = reinterpret_cast<int32_t*>(p);
  p += round_up((size_t)k * 4);
  int8_t* xq = reinterpret_cast<int8_t*>(p);
  p += round_up((size_t)m * (size_t)k);
  float* dx = reinterpret_cast<float*>(p);
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = sqh::fill_u32(colmax, 0u, k, s);
  if (e == hipSuccess) e = sqh::absmax_cols(x, SQ_F16, m, k, ldx, colmax, s);
  if (e == hipSuccess) e = sqh::outlier_select(colmax, k, threshold, mask, idx, n_outliers, s);
  if (e == hipSuccess) e = sqh::quant_rows(x, SQ_F16, m, k, ldx, nullptr, mask, xq, dx, s);
  if (e != hipSuccess) return hip_status(e);
  if (m == 0 || n == 0) return SQ_OK;
  sqh::DecompArgs d{(const uint16_t*)x, ldx, (const uint16_t*)w16, ldw16, idx, n_outliers};
  return hip_status(sqh::gemm_i8(xq, dx, wq, w_scale, m, n, k, y, SQ_F16, ldy, &d, nullptr, s));
}

sq_status sq_int8_decomp_gemm(const int8_t* xq, const float* x_scale, const void* x, int64_t ldx, const int8_t* wq,
                              const float* w_scale, const void* w16, int64_t ldw16, const int32_t* idx,
                              const int32_t* n_outliers, int64_t m, int64_t n, int64_t k, void* y, int64_t ldy,
                              sq_stream_t stream) {
  SQ_TRY(check_k(k));
  if (k > SQ_MAX_K_INT32) return SQ_ERR_RANGE;
  if (m < 0 || n < 0) return SQ_ERR_SHAPE;
  if (ldx < k || ldw16 < n || ldy < n) return SQ_ERR_SHAPE;
  if (m > INT32_MAX || n > INT32_MAX) return SQ_ERR_SHAPE;
  if (m == 0 || n == 0) return SQ_OK;
  if (!xq || !x_scale || !x || !wq || !w_scale || !w16 || !idx || !n_outliers || !y) return SQ_ERR_NULL;
  if (!aligned16(xq) || !aligned16(wq)) return SQ_ERR_ALIGN;
  if ((reinterpret_cast<uintptr_t>(x) & 1u) || (reinterpret_cast<uintptr_t>(w16) & 1u) ||
      (reinterpret_cast<uintptr_t>(y) & 1u))
    return SQ_ERR_ALIGN;
  sqh::DecompArgs d{(const uint16_t*)x, ldx, (const uint16_t*)w16, ldw16, idx, n_outliers};
  return hip_status(sqh::gemm_i8(xq, x_scale, wq, w_scale, m, n, k, y, SQ_F16, ldy, &d, nullptr, (hipStream_t)stream));
}

}  // extern "C"
