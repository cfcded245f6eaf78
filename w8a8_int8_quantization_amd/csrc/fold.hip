// Load-time weight preparation: smoothing factor, fold into W, per-output-
// channel symmetric int8 quantisation with a transposed [N x K] store.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization":
//   * "How the smoothing factor is computed": s_j from the activation absmax
//     A_j, the largest weight magnitude W_j of row j and alpha; row j of W is
//     multiplied by s_j;
//   * "How the Model Was Compressed" / "Why Naive Weight Quantization Doesn't
//     Work": one scale per weight column, max|column| / 127, q = round(w/scale).
//
// Two passes over W [K x ldw]:
//   1. fold_rows: a workgroup takes kRows consecutive rows; it reduces each
//      row's |W| maximum, forms s_j in binary64 (rounded once to binary32),
//      then takes the maximum of |fl32(s_j * W_jn)| over its rows per column
//      and merges it into colmax[n] with an integer atomicMax.
//   2. fold_quant: 64 x 64 tiles; q = clamp(rint(fl32(W'_jn / sw_n)), +-127)
//      with sw_n = fl32(colmax_n / 127), transposed through LDS so that Wq
//      [N x K] is written with 16-byte row-contiguous stores.
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

constexpr int kFoldRows = 8;

// Elements [vi*V, vi*V + V) of a row, zero beyond column n. kAligned: the row
// is 16-byte aligned and one vector load serves; otherwise element loads.
template <class In, bool kAligned>
__device__ __forceinline__ void load_vec_masked(const uint8_t* row, int64_t vi, int64_t n, float* f) {
  constexpr int V = In::kVec;
  if (!kAligned) {
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = vi * V + e < n ? In::load1(row + (vi * V + e) * In::kBytes) : 0.f;
    return;
  }
  if (vi * V < n) {
    In::unpack(load16(row + vi * 16), f);
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (vi * V + e >= n) f[e] = 0.f;
  } else {
#pragma unroll
    for (int e = 0; e < V; ++e) f[e] = 0.f;
  }
}

template <class In, bool kAligned>
__global__ __launch_bounds__(256) void fold_rows_kernel(const uint8_t* __restrict__ w, int64_t k, int64_t n,
                                                        int64_t ldw_bytes, const float* __restrict__ absmax,
                                                        double alpha, uint32_t flags, float* __restrict__ smooth,
                                                        float* __restrict__ colmax) {
  constexpr int V = In::kVec;
  __shared__ float red[4];
  __shared__ float s_rows[kFoldRows];
  const int64_t j0 = (int64_t)blockIdx.x * kFoldRows;
  const int64_t nvec = (n + V - 1) / V;

  for (int r = 0; r < kFoldRows; ++r) {
    const int64_t j = j0 + r;
    if (j >= k) break;  // uniform across the workgroup
    float s = 1.f;
    if (flags == SQ_SMOOTH_GIVEN) {
      s = smooth[j];
    } else if (flags == SQ_SMOOTH_COMPUTE) {
      const uint8_t* row = w + j * ldw_bytes;
      float m = 0.f;
      for (int64_t vi = threadIdx.x; vi < nvec; vi += 256) {
        float f[V];
        load_vec_masked<In, kAligned>(row, vi, n, f);
#pragma unroll
        for (int e = 0; e < V; ++e) m = fmaxf(m, fabsf(f[e]));
      }
      m = block_max<256>(m, red);
      const float a = absmax[j];
      if (a > 0.f && m > 0.f) {
        const double num = pow((double)a, alpha);
        const double den = pow((double)m, 1.0 - alpha);
        s = (float)(num / den);
      }
      if (threadIdx.x == 0) smooth[j] = s;
    }
    if (threadIdx.x == 0) s_rows[r] = s;
  }
  __syncthreads();

  const int nr = (int)((k - j0) < kFoldRows ? (k - j0) : kFoldRows);
  for (int64_t vi = threadIdx.x; vi < nvec; vi += 256) {
    float cm[V];
#pragma unroll
    for (int e = 0; e < V; ++e) cm[e] = 0.f;
    for (int r = 0; r < nr; ++r) {
      float f[V];
      load_vec_masked<In, kAligned>(w + (j0 + r) * ldw_bytes, vi, n, f);
      const float s = s_rows[r];
#pragma unroll
      for (int e = 0; e < V; ++e) cm[e] = fmaxf(cm[e], fabsf(__fmul_rn(s, f[e])));
    }
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (vi * V + e < n && cm[e] > 0.f) atomic_max_nonneg(colmax + vi * V + e, cm[e]);
  }
}

// 64 x 64 tile of W (rows j, columns n) -> 64 rows of Wq (n) x 64 bytes (j).
template <class In, bool kAligned>
__global__ __launch_bounds__(256) void fold_quant_kernel(const uint8_t* __restrict__ w, int64_t k, int64_t n,
                                                         int64_t ldw_bytes, uint32_t flags,
                                                         const float* __restrict__ smooth,
                                                         const float* __restrict__ colmax, int8_t* __restrict__ wq,
                                                         float* __restrict__ w_scale) {
  constexpr int V = In::kVec;
  constexpr int kLd = 80;  // LDS row stride in bytes (16-byte aligned, staggers banks)
  __shared__ __attribute__((aligned(16))) int8_t tile[64 * kLd];
  const int64_t n0 = (int64_t)blockIdx.x * 64;
  const int64_t j0 = (int64_t)blockIdx.y * 64;
  const int tid = threadIdx.x;
  const int jj = tid >> 2;          // tile row (input channel)
  const int c0 = (tid & 3) * 16;    // first of this thread's 16 tile columns
  const int64_t j = j0 + jj;
  const float s = flags == SQ_SMOOTH_NONE ? 1.f : smooth[j];
  const uint8_t* row = w + j * ldw_bytes;
#pragma unroll
  for (int g = 0; g < 16 / V; ++g) {
    const int64_t col0 = n0 + c0 + g * V;
    float f[V];
    load_vec_masked<In, kAligned>(row, col0 / V, n, f);
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const int64_t col = col0 + e;
      int q = 0;
      if (col < n) {
        const float sw = colmax[col] / (float)kQMax;
        const float wf = __fmul_rn(s, f[e]);
        if (sw > 0.f) q = quant_rne_clamp(wf / sw);
      }
      tile[(c0 + g * V + e) * kLd + jj] = (int8_t)q;
    }
  }
  __syncthreads();
  // 64 output rows x 64 bytes: 4 threads per row, 16 bytes each
  const int orow = tid >> 2;
  const int oseg = (tid & 3) * 16;
  const int64_t nn = n0 + orow;
  if (nn < n) store16(wq + nn * k + j0 + oseg, load16(tile + orow * kLd + oseg));
  if (blockIdx.y == 0 && tid < 64 && n0 + tid < n) w_scale[n0 + tid] = colmax[n0 + tid] / (float)kQMax;
}

}  // namespace sqk

namespace sqh {

template <class In, bool kAligned>
static void launch_fold_a(const float* absmax, const void* w, int64_t k, int64_t n, int64_t ldw, double alpha,
                          uint32_t flags, float* smooth, int8_t* wq, float* w_scale, float* colmax, hipStream_t s) {
  const int64_t ldb = ldw * In::kBytes;
  hipLaunchKernelGGL((sqk::fold_rows_kernel<In, kAligned>),
                     dim3((unsigned)((k + sqk::kFoldRows - 1) / sqk::kFoldRows)), dim3(256), 0, s,
                     (const uint8_t*)w, k, n, ldb, absmax, alpha, flags, smooth, colmax);
  hipLaunchKernelGGL((sqk::fold_quant_kernel<In, kAligned>), dim3((unsigned)((n + 63) / 64), (unsigned)(k / 64)),
                     dim3(256), 0, s, (const uint8_t*)w, k, n, ldb, flags, (const float*)smooth,
                     (const float*)colmax, wq, w_scale);
}

template <class In>
static void launch_fold(const float* absmax, const void* w, int64_t k, int64_t n, int64_t ldw, double alpha,
                        uint32_t flags, float* smooth, int8_t* wq, float* w_scale, float* colmax, hipStream_t s) {
  const bool aligned = (reinterpret_cast<uintptr_t>(w) % 16 == 0) && ((ldw * In::kBytes) % 16 == 0);
  if (aligned)
    launch_fold_a<In, true>(absmax, w, k, n, ldw, alpha, flags, smooth, wq, w_scale, colmax, s);
  else
    launch_fold_a<In, false>(absmax, w, k, n, ldw, alpha, flags, smooth, wq, w_scale, colmax, s);
}

hipError_t fold_weights(const float* absmax, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                        double alpha, uint32_t flags, float* smooth, int8_t* wq, float* w_scale,
                        float* colmax_ws, hipStream_t s) {
  hipError_t e = fill_u32(colmax_ws, 0u, n, s);
  if (e != hipSuccess) return e;
  switch (wt) {
    case SQ_F32: launch_fold<sqk::F32In>(absmax, w, k, n, ldw, alpha, flags, smooth, wq, w_scale, colmax_ws, s); break;
    case SQ_BF16: launch_fold<sqk::BF16In>(absmax, w, k, n, ldw, alpha, flags, smooth, wq, w_scale, colmax_ws, s); break;
    default: launch_fold<sqk::F16In>(absmax, w, k, n, ldw, alpha, flags, smooth, wq, w_scale, colmax_ws, s); break;
  }
  return hipGetLastError();
}

}  // namespace sqh
