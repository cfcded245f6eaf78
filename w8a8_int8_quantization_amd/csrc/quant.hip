// Run-time per-token dynamic int8 activation quantisation.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization":
//   * "How the Model Was Compressed": one scale per token over all channels,
//     found at run time;
//   * "Why Activation Quantization Is Hard": scale = max|x| / 127,
//     q = round(x / scale);
//   * "How the smoothing factor is computed": the activation is divided by s.
// The LLM.int8() page, "End-to-end flow": the row scale of the int8 path is
// taken over the regular (non-outlier) columns only; the outlier columns of
// Xq are zero.
//
// One 256-thread workgroup owns a row at a time (grid-stride over rows). Each
// thread loads kCh 16-byte vectors of the row (coalesced: consecutive threads
// read consecutive 16 bytes), keeps the smoothed values in registers, the
// workgroup reduces the row maximum through LDS, then each thread writes its
// int8 values with one 4- or 8-byte store per vector. X is read from HBM once
// and Xq written once. Rows longer than 8 vectors per thread use a two-pass
// variant that reads the row a second time.
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

template <class In, bool kSmooth, bool kMask>
__device__ __forceinline__ void load_smoothed(const uint8_t* __restrict__ xr, const float* __restrict__ smooth,
                                              const uint8_t* __restrict__ mask, int64_t vi, float* f) {
  constexpr int V = In::kVec;
  In::unpack(load16(xr + vi * 16), f);
  if (kSmooth) {
    const float* sp = smooth + vi * V;
#pragma unroll
    for (int e = 0; e < V; e += 4) {
      const u32x4 sv = load16(sp + e);
      f[e + 0] = f[e + 0] / __uint_as_float(sv.x);
      f[e + 1] = f[e + 1] / __uint_as_float(sv.y);
      f[e + 2] = f[e + 2] / __uint_as_float(sv.z);
      f[e + 3] = f[e + 3] / __uint_as_float(sv.w);
    }
  }
  if (kMask) {
    const uint8_t* mp = mask + vi * V;
#pragma unroll
    for (int e = 0; e < V; ++e)
      if (mp[e]) f[e] = 0.f;
  }
}

template <int V>
__device__ __forceinline__ void store_q(int8_t* __restrict__ dst, const float* f, float d) {
  uint32_t packed[V / 4];
#pragma unroll
  for (int w = 0; w < V / 4; ++w) {
    uint32_t p = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int q = d > 0.f ? quant_rne_clamp(f[4 * w + b] / d) : 0;
      p |= ((uint32_t)q & 0xFFu) << (8 * b);
    }
    packed[w] = p;
  }
  if constexpr (V == 8) {
    *reinterpret_cast<uint2*>(dst) = make_uint2(packed[0], packed[1]);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = packed[0];
  }
}

template <class In, int kCh, bool kSmooth, bool kMask>
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint8_t* __restrict__ x, int64_t m, int64_t nvec,
                                                         int64_t ldx_bytes, const float* __restrict__ smooth,
                                                         const uint8_t* __restrict__ mask, int8_t* __restrict__ xq,
                                                         float* __restrict__ x_scale) {
  constexpr int V = In::kVec;
  __shared__ float red[4];
  const int64_t k = nvec * V;
  for (int64_t row = blockIdx.x; row < m; row += gridDim.x) {
    const uint8_t* xr = x + row * ldx_bytes;
    float f[kCh][V];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int64_t vi = threadIdx.x + c * 256;
      if (vi < nvec) {
        load_smoothed<In, kSmooth, kMask>(xr, smooth, mask, vi, f[c]);
#pragma unroll
        for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(f[c][e]));
      }
    }
    amax = block_max<256>(amax, red);
    const float d = amax / (float)kQMax;
    if (threadIdx.x == 0) x_scale[row] = d;
    int8_t* qr = xq + row * k;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int64_t vi = threadIdx.x + c * 256;
      if (vi < nvec) store_q<V>(qr + vi * V, f[c], d);
    }
  }
}

// Rows of any length: pass 1 finds the maximum, pass 2 re-reads and quantises.
template <class In, bool kSmooth, bool kMask>
__global__ __launch_bounds__(256) void quant_rows_long_kernel(const uint8_t* __restrict__ x, int64_t m, int64_t nvec,
                                                              int64_t ldx_bytes, const float* __restrict__ smooth,
                                                              const uint8_t* __restrict__ mask,
                                                              int8_t* __restrict__ xq, float* __restrict__ x_scale) {
  constexpr int V = In::kVec;
  __shared__ float red[4];
  const int64_t k = nvec * V;
  for (int64_t row = blockIdx.x; row < m; row += gridDim.x) {
    const uint8_t* xr = x + row * ldx_bytes;
    float amax = 0.f;
    for (int64_t vi = threadIdx.x; vi < nvec; vi += 256) {
      float f[V];
      load_smoothed<In, kSmooth, kMask>(xr, smooth, mask, vi, f);
#pragma unroll
      for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(f[e]));
    }
    amax = block_max<256>(amax, red);
    const float d = amax / (float)kQMax;
    if (threadIdx.x == 0) x_scale[row] = d;
    int8_t* qr = xq + row * k;
    for (int64_t vi = threadIdx.x; vi < nvec; vi += 256) {
      float f[V];
      load_smoothed<In, kSmooth, kMask>(xr, smooth, mask, vi, f);
      store_q<V>(qr + vi * V, f, d);
    }
  }
}

}  // namespace sqk

namespace sqh {

template <class In, bool kSmooth, bool kMask>
static void launch_quant(const void* x, int64_t m, int64_t k, int64_t ldx, const float* smooth, const uint8_t* mask,
                         int8_t* xq, float* x_scale, hipStream_t s) {
  const int64_t nvec = k / In::kVec;
  const int64_t ldb = ldx * In::kBytes;
  const int64_t per_thread = (nvec + 255) / 256;
  unsigned grid = (unsigned)(m < 4096 ? m : 4096);
  const uint8_t* xb = (const uint8_t*)x;
  if (per_thread <= 1)
    hipLaunchKernelGGL((sqk::quant_rows_kernel<In, 1, kSmooth, kMask>), dim3(grid), dim3(256), 0, s, xb, m, nvec, ldb,
                       smooth, mask, xq, x_scale);
  else if (per_thread <= 2)
    hipLaunchKernelGGL((sqk::quant_rows_kernel<In, 2, kSmooth, kMask>), dim3(grid), dim3(256), 0, s, xb, m, nvec, ldb,
                       smooth, mask, xq, x_scale);
  else if (per_thread <= 4)
    hipLaunchKernelGGL((sqk::quant_rows_kernel<In, 4, kSmooth, kMask>), dim3(grid), dim3(256), 0, s, xb, m, nvec, ldb,
                       smooth, mask, xq, x_scale);
  else if (per_thread <= 8)
    hipLaunchKernelGGL((sqk::quant_rows_kernel<In, 8, kSmooth, kMask>), dim3(grid), dim3(256), 0, s, xb, m, nvec, ldb,
                       smooth, mask, xq, x_scale);
  else
    hipLaunchKernelGGL((sqk::quant_rows_long_kernel<In, kSmooth, kMask>), dim3(grid), dim3(256), 0, s, xb, m, nvec,
                       ldb, smooth, mask, xq, x_scale);
}

template <class In>
static void launch_quant_t(const void* x, int64_t m, int64_t k, int64_t ldx, const float* smooth, const uint8_t* mask,
                           int8_t* xq, float* x_scale, hipStream_t s) {
  if (mask)
    launch_quant<In, false, true>(x, m, k, ldx, nullptr, mask, xq, x_scale, s);
  else if (smooth)
    launch_quant<In, true, false>(x, m, k, ldx, smooth, nullptr, xq, x_scale, s);
  else
    launch_quant<In, false, false>(x, m, k, ldx, nullptr, nullptr, xq, x_scale, s);
}

hipError_t quant_rows(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* smooth,
                      const uint8_t* mask, int8_t* xq, float* x_scale, hipStream_t s) {
  if (m <= 0) return hipSuccess;
  switch (xt) {
    case SQ_F32: launch_quant_t<sqk::F32In>(x, m, k, ldx, smooth, mask, xq, x_scale, s); break;
    case SQ_BF16: launch_quant_t<sqk::BF16In>(x, m, k, ldx, smooth, mask, xq, x_scale, s); break;
    default: launch_quant_t<sqk::F16In>(x, m, k, ldx, smooth, mask, xq, x_scale, s); break;
  }
  return hipGetLastError();
}

}  // namespace sqh
