// Host-side launchers of the gfx950 kernels (internal to the library).
// Each returns the HIP error of its launches; arguments are validated by the
// C-ABI layer before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_index.hpp"
#include "sq.h"

namespace sqh {

// Split-K workspaces: fixed counter region, then partial tiles (see
// gemm_index.hpp).
using sqi::kSplitCounterBytes;
using sqi::kSplitMaxCounters;

// Extra inputs of the LLM.int8() epilogue: the fp16 outlier slice.
struct DecompArgs {
  const uint16_t* x;    // [M x ldx] fp16 activations
  int64_t ldx;
  const uint16_t* w16;  // [K x ldw] fp16 weights
  int64_t ldw;
  const int32_t* idx;   // ascending outlier columns
  const int32_t* count; // number of outlier columns (device)
};

hipError_t fill_u32(void* p, uint32_t value, int64_t count, hipStream_t s);

// Records the HIP error behind an SQ_ERR_HIP (what sq_last_hip_error() returns
// on this thread).
void set_last_hip_error(int e);

hipError_t absmax_cols(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, float* absmax,
                       hipStream_t s);

hipError_t outlier_select(const float* colmax, int64_t k, float threshold, uint8_t* mask, int32_t* idx,
                          int32_t* count, hipStream_t s);

hipError_t fold_weights(const float* absmax, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                        double alpha, uint32_t flags, float* smooth, int8_t* wq, float* w_scale,
                        float* colmax_ws, hipStream_t s);

// zero / nzero: optional words the launch also clears (the split-K counters of
// a decode GEMM that follows on the same stream).
hipError_t quant_rows(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* smooth,
                      const uint8_t* mask, int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero = nullptr,
                      int64_t nzero = 0);

// RMSNorm with the folded gain, then per-token quantisation (zero / nzero as above).
hipError_t rmsnorm_quant(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* gain, float eps,
                         int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero = nullptr, int64_t nzero = 0);
hipError_t fold_norm_gain(const void* gamma, sq_dtype gt, const float* smooth, int64_t k, float* out,
                          hipStream_t s);

// SiLU(gate) * up (bf16), smoothing divide and per-token quantisation (zero / nzero as above).
hipError_t silu_quant(const void* gate, const void* up, int64_t m, int64_t k, int64_t ldg, int64_t ldu,
                      const float* smooth, int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero = nullptr,
                      int64_t nzero = 0);

// FP8 (E4M3) quantisers and GEMM.
// zero[0 .. nzero-1] are cleared on the way (the decode GEMM's split-K counters).
hipError_t quant_f8_rows(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, uint8_t* xq, float* x_scale,
                         hipStream_t s, uint32_t* zero = nullptr, int64_t nzero = 0);
hipError_t quant_f8_weights(const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw, float* colmax,
                            uint8_t* wq, float* w_scale, hipStream_t s);
hipError_t gemm_f8(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                   int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s);

// GPTQ (binary64): Hessian accumulation and the quantisation sweep.
hipError_t gptq_hessian(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, const float* smooth, double* h,
                        hipStream_t s);
size_t gptq_workspace(int64_t k, int64_t n);
hipError_t gptq_quantize(const double* h, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                         const float* smooth, double damp, int8_t* wq, float* w_scale, void* ws, hipStream_t s);

// ws: the prefill kernel's split-K workspace (gemm_big_workspace bytes; may
// be null when that is 0 or when dec is given).
hipError_t gemm_i8(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                   int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, const DecompArgs* dec, void* ws,
                   hipStream_t s);

// Large-tile prefill GEMM (256-row tiles); gemm_i8 routes to it when it suits.
// Whether the 256-row-tile prefill kernel takes this GEMM (split_ok: the
// call may split K, i.e. it is not the LLM.int8() epilogue).
bool gemm_big_suits(int64_t m, int64_t n, int64_t k, bool split_ok = true);
hipError_t gemm_i8_big(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, const DecompArgs* dec, void* ws,
                       hipStream_t s);
// Split-K workspace of the prefill kernel (0 when the shape is not split):
// ticket counters (zero at launch, restored by the kernel) and partial tiles.
size_t gemm_big_workspace(int64_t m, int64_t n, int64_t k, bool f8);
void gemm_big_counters(int64_t m, int64_t n, int64_t k, bool f8, void* ws, uint32_t** counters, int64_t* count);
// The same kernel on E4M3 operands (binary32 accumulators); gemm_f8 routes to it when it suits.
hipError_t gemm_f8_big(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s);

// One-token decode step (quantisation fused into the weight-streaming GEMM;
// no workspace): whether it takes this shape, and the call.
bool decode1_suits(int64_t m, int64_t n, int64_t k, sq_dtype xt);
hipError_t decode1_linear(const void* x, sq_dtype xt, const float* smooth, const int8_t* wq, const float* w_scale,
                          int64_t n, int64_t k, void* y, sq_dtype yt, hipStream_t s);

// Decode GEMM (up to 256 tokens; f8: E4M3 operands, else int8): split-K over
// workgroups, partial tiles and ticket counters in the workspace. The
// counters must be zero at launch.
bool gemm_decode_suits(int64_t m, int64_t n, int64_t k, bool f8);
size_t gemm_decode_workspace(int64_t m, int64_t n, int64_t k, bool f8);
void gemm_decode_counters(int64_t m, int64_t n, int64_t k, bool f8, void* ws, uint32_t** counters, int64_t* count);
hipError_t gemm_i8_decode(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                          int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s);
// The same decode GEMM on E4M3 operands (binary32 partial tiles in the same workspace layout).
hipError_t gemm_f8_decode(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                          int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s);

}  // namespace sqh
