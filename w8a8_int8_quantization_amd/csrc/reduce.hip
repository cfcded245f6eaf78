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
// Layout: X is row-major [T x ldx]. A lane owns one 16-byte column vector
// (4 fp32 or 8 bf16/fp16 columns) and walks rows of a slab, so every wave
// reads 1 KiB of contiguous row memory per step; the slab maxima are merged
// with one integer atomicMax per column and workgroup (non-negative binary32
// values order like their bit patterns, so the result is exact and order
// free).
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

__global__ __launch_bounds__(256) void fill_u32_kernel(uint32_t* __restrict__ p, uint32_t v, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) p[i] = v;
}

// A 256-thread workgroup covers 64 column vectors (1 KiB of a row) and a slab
// of rows: wave w reads rows w, w+4, ... of the slab, eight loads in flight
// per thread; the four waves' maxima meet in LDS and one atomicMax per column
// leaves the workgroup.
template <class In>
__global__ __launch_bounds__(256) void absmax_cols_kernel(const uint8_t* __restrict__ x, int64_t t, int64_t nvec,
                                                          int64_t ldx_bytes, int64_t rows_per_block,
                                                          float* __restrict__ absmax) {
  constexpr int V = In::kVec;
  constexpr int kU = 8;
  __shared__ float part[4][64][V + 1];
  const int lane = threadIdx.x & 63;
  const int wid = threadIdx.x >> 6;
  const int64_t v = (int64_t)blockIdx.x * 64 + lane;
  const bool active = v < nvec;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = r0 + rows_per_block < t ? r0 + rows_per_block : t;
  float m[V];
#pragma unroll
  for (int e = 0; e < V; ++e) m[e] = 0.f;
  if (active) {
    const uint8_t* p = x + v * 16;
    int64_t r = r0 + wid;
    for (; r + 4 * (kU - 1) < r1; r += 4 * kU) {
      u32x4 q[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) q[u] = load16(p + (r + 4 * u) * ldx_bytes);
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        float f[V];
        In::unpack(q[u], f);
#pragma unroll
        for (int e = 0; e < V; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
      }
    }
    for (; r < r1; r += 4) {
      float f[V];
      In::unpack(load16(p + r * ldx_bytes), f);
#pragma unroll
      for (int e = 0; e < V; ++e) m[e] = fmaxf(m[e], fabsf(f[e]));
    }
  }
#pragma unroll
  for (int e = 0; e < V; ++e) part[wid][lane][e] = m[e];
  __syncthreads();
  if (wid == 0 && active) {
#pragma unroll
    for (int e = 0; e < V; ++e) {
      const float mm = fmaxf(fmaxf(part[0][lane][e], part[1][lane][e]), fmaxf(part[2][lane][e], part[3][lane][e]));
      if (mm > 0.f) atomic_max_nonneg(absmax + v * V + e, mm);
    }
  }
}

// One workgroup: mask, ascending index list and count of the columns whose
// maximum magnitude is strictly above the threshold. Rounds of 1024 columns,
// one per thread in order: a wave's ballot gives each outlier lane its rank
// among the wave's outliers, the 16 wave counts in LDS give the wave offsets,
// and a running total carries across rounds, so the list comes out ascending.
__global__ __launch_bounds__(1024) void outlier_select_kernel(const float* __restrict__ colmax, int64_t k, float thr,
                                                              uint8_t* __restrict__ mask, int32_t* __restrict__ idx,
                                                              int32_t* __restrict__ count) {
  __shared__ int wcount[2][16];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  int base = 0;
  int parity = 0;
  for (int64_t j0 = 0; j0 < k; j0 += 1024) {
    const int64_t j = j0 + tid;
    const bool o = j < k && colmax[j] > thr;
    if (j < k) mask[j] = o ? 1 : 0;
    const uint64_t bal = __ballot(o);
    if (lane == 0) wcount[parity][wid] = __popcll(bal);
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 16; ++w) {
      const int c = wcount[parity][w];
      before += w < wid ? c : 0;
      total += c;
    }
    if (o) idx[base + before + __popcll(bal & ((1ull << lane) - 1ull))] = (int32_t)j;
    base += total;
    parity ^= 1;  // the next round writes the other buffer, so one barrier per round suffices
  }
  if (tid == 0) *count = base;
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
  const int64_t gx = (nvec + 63) / 64;
  // about 1024 workgroups (four per CU), each over a slab of at least 32 rows
  int64_t rpb = (t * gx + 1023) / 1024;
  if (rpb < 32) rpb = 32;
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
