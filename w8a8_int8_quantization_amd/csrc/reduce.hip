// Column-wise absolute maxima (calibration statistics, LLM.int8() outlier
// detection) and the outlier-column selection.
//
// Calibration: "Half the Size, Better Performance, Same Accuracy:
// Understanding W8A8 INT8 LLM Quantization", section "How the smoothing
// factor is computed" -- A_j is the largest activation magnitude seen in
// input channel j over the calibration samples.
// Detection: the LLM.int8() page, section "The architecture: every piece
// explained" -- a feature column whose magnitude exceeds the threshold is an
// outlier column.
//
// Layout: X is row-major [T x ldx]. One thread owns one 16-byte column vector
// (4 fp32 or 8 bf16/fp16 columns) and walks a slab of rows, so every wave
// reads 1 KiB of contiguous row memory per step; partial maxima of a slab are
// merged with one integer atomicMax per column (non-negative binary32 values
// order like their bit patterns, so the result is exact and order free).
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

template <class In>
__global__ __launch_bounds__(256) void absmax_cols_kernel(const uint8_t* __restrict__ x, int64_t t, int64_t nvec,
                                                          int64_t ldx_bytes, int64_t rows_per_block,
                                                          float* __restrict__ absmax) {
  constexpr int V = In::kVec;
  const int64_t v = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (v >= nvec) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < t ? r0 + rows_per_block : t;
  float m[V];
#pragma unroll
  for (int e = 0; e < V; ++e) m[e] = 0.f;
  const uint8_t* p = x + r0 * ldx_bytes + v * 16;
  int64_t r = r0;
  for (; r + 4 <= r1; r += 4) {
    u32x4 q[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) q[u] = load16(p + u * ldx_bytes);
    p += 4 * ldx_bytes;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float f[V];
      In::unpack(q[u], f);
#pragma unroll
      for (int e = 0; e < V; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
    }
  }
  for (; r < r1; ++r) {
    float f[V];
    In::unpack(load16(p), f);
    p += ldx_bytes;
#pragma unroll
    for (int e = 0; e < V; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
  }
#pragma unroll
  for (int e = 0; e < V; ++e)
    if (m[e] > 0.f) atomic_max_nonneg(absmax + v * V + e, m[e]);
}

// One workgroup: mask, ascending index list and count of the columns whose
// maximum magnitude is strictly above the threshold.
__global__ __launch_bounds__(1024) void outlier_select_kernel(const float* __restrict__ colmax, int64_t k, float thr,
                                                              uint8_t* __restrict__ mask, int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ count) {
  __shared__ int sums[1024];
  const int tid = threadIdx.x;
  const int64_t seg = (k + 1023) / 1024;
  const int64_t b = tid * seg;
  const int64_t e = b + seg < k ? b + seg : k;
  int c = 0;
  for (int64_t j = b; j < e; ++j) c += colmax[j] > thr ? 1 : 0;
  sums[tid] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += add;
    __syncthreads();
  }
  int pos = sums[tid] - c;
  for (int64_t j = b; j < e; ++j) {
    const bool o = colmax[j] > thr;
    mask[j] = o ? 1 : 0;
    if (o) idx[pos++] = (int32_t)j;
  }
  if (tid == 1023) *count = sums[1023];
}

}  // namespace sqk

namespace sqh {

hipError_t fill_u32(void* p, uint32_t value, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  int64_t blocks = (count + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(sqk::fill_u32_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, value, count);
  return hipGetLastError();
}

hipError_t absmax_cols(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, float* absmax,
                       hipStream_t s) {
  if (t <= 0) return hipSuccess;
  const int bytes = xt == SQ_F32 ? 4 : 2;
  const int vec = 16 / bytes;
  const int64_t nvec = k / vec;
  const int64_t gx = (nvec + 255) / 256;
  // about 2048 workgroups, each over a slab of at least 8 rows
  int64_t rpb = (t * gx + 2047) / 2048;
  if (rpb < 8) rpb = 8;
  int64_t gy = (t + rpb - 1) / rpb;
  if (gy > 65535) {
    rpb = (t + 65534) / 65535;
    gy = (t + rpb - 1) / rpb;
  }
  const dim3 grid((unsigned)gx, (unsigned)gy);
  const int64_t ldb = ldx * bytes;
  switch (xt) {
    case SQ_F32:
      hipLaunchKernelGGL(sqk::absmax_cols_kernel<sqk::F32In>, grid, dim3(256), 0, s, (const uint8_t*)x, t, nvec, ldb,
                         rpb, absmax);
      break;
    case SQ_BF16:
      hipLaunchKernelGGL(sqk::absmax_cols_kernel<sqk::BF16In>, grid, dim3(256), 0, s, (const uint8_t*)x, t, nvec,
                         ldb, rpb, absmax);
      break;
    default:
      hipLaunchKernelGGL(sqk::absmax_cols_kernel<sqk::F16In>, grid, dim3(256), 0, s, (const uint8_t*)x, t, nvec, ldb,
                         rpb, absmax);
      break;
  }
  return hipGetLastError();
}

hipError_t outlier_select(const float* colmax, int64_t k, float threshold, uint8_t* mask, int32_t* idx,
                          int32_t* count, hipStream_t s) {
  hipLaunchKernelGGL(sqk::outlier_select_kernel, dim3(1), dim3(1024), 0, s, colmax, k, threshold, mask, idx, count);
  return hipGetLastError();
}

}  // namespace sqh
