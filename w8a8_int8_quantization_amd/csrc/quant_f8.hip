// FP8 (E4M3) quantisers: per-token activations at run time, per-output-channel
// weights at load time.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization", section "Conclusion" (FP8 skips the calibration
// algorithms); the scales follow the int8 path's "How the Model Was
// Compressed" and "Why Activation Quantization Is Hard" with 448, the largest
// E4M3 magnitude, in place of 127:
//   d_i = fl32(max_j |x_ij| / 448),  q_ij = E4M3(fl32(x_ij / d_i))
//   sw_n = fl32(max_k |W_kn| / 448), Wq_nk = E4M3(fl32(W_kn / sw_n))
// E4M3 is the OCP encoding (bias 7, largest finite 448). gfx950's
// v_cvt_pk_fp8_f32 converts with round-to-nearest-even (checked on MI355X
// against a nearest-value search over all codes, midpoints included); every
// quotient here is at most 448 up to one rounding, below the conversion's
// overflow point (464).
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

constexpr float kE4M3Max = 448.0f;

// four binary32 values -> four E4M3 bytes (little-endian)
__device__ __forceinline__ uint32_t f8x4(float a, float b, float c, float d) {
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
  return (uint32_t)r;
}

// One workgroup per row (grid-stride); thread t owns the 16-byte vectors t,
// t + kT, ... of the row, kept in registers between the maximum and the codes.
template <class In, int kCh, int kT>
__global__ __launch_bounds__(kT) void quant_f8_rows_kernel(const uint8_t* __restrict__ x, int64_t m, int nvec,
                                                           int64_t ldx_bytes, uint8_t* __restrict__ xq,
                                                           float* __restrict__ x_scale, uint32_t* __restrict__ zero,
                                                           int nzero) {
  constexpr int V = In::kVec;
  constexpr int kW = kT / 64;
  __shared__ uint32_t red[kW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t k = (int64_t)nvec * V;
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += kT) zero[i] = 0u;
  for (int64_t row = blockIdx.x; row < m; row += gridDim.x) {
    const uint8_t* xr = x + row * ldx_bytes;
    float f[kCh][V];
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int vi = tid + kT * c;
      const u32x4 rv = vi < nvec ? load16(xr + (int64_t)vi * 16) : u32x4{0u, 0u, 0u, 0u};
      In::unpack(rv, f[c]);
#pragma unroll
      for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(f[c][e]));
    }
    uint32_t ab = wave_max_u32(__float_as_uint(amax));
    if (lane == 0) red[wid] = ab;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kW; ++w) ab = red[w] > ab ? red[w] : ab;
    amax = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)ab));
    const float d = amax / kE4M3Max;
    const float rd = d > 0.f ? rcp_scale(d) : 0.f;
    if (tid == 0) x_scale[row] = d;
    uint8_t* qr = xq + row * k;
    auto emit = [&](auto quot) {
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        const int vi = tid + kT * c;
        if (vi >= nvec) continue;
        if constexpr (V == 8) {
          *reinterpret_cast<uint2*>(qr + (int64_t)vi * V) =
              make_uint2(f8x4(quot(f[c][0]), quot(f[c][1]), quot(f[c][2]), quot(f[c][3])),
                         f8x4(quot(f[c][4]), quot(f[c][5]), quot(f[c][6]), quot(f[c][7])));
        } else {
          *reinterpret_cast<uint32_t*>(qr + (int64_t)vi * V) =
              f8x4(quot(f[c][0]), quot(f[c][1]), quot(f[c][2]), quot(f[c][3]));
        }
      }
    };
    // Markstein quotients inside the range where they equal IEEE division;
    // the correction step turns a zero quotient into +0, and the sign of
    // zero is part of an E4M3 code, so it is taken from the dividend
    if (d >= kFastDMin && amax <= kFastAMax)
      emit([&](float v) { return __builtin_copysignf(div_mk(v, d, rd), v); });
    else if (d > 0.f)
      emit([&](float v) { return v / d; });
    else
      emit([](float) { return 0.f; });
    lds_barrier();  // every wave has read red[] before the next row writes it
  }
}

// Weights W [K x N] (row pitch ldw elements) -> Wq [N x K] E4M3 codes, given the
// column maxima: 64 x 64 tiles transposed through LDS.
template <class In>
__global__ __launch_bounds__(256) void quant_f8_weights_kernel(const uint8_t* __restrict__ w, int64_t k, int64_t n,
                                                               int64_t ldw, const float* __restrict__ colmax,
                                                               uint8_t* __restrict__ wq, float* __restrict__ w_scale) {
  __shared__ uint8_t tile[64][65];
  const int64_t k0 = (int64_t)blockIdx.x * 64, n0 = (int64_t)blockIdx.y * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t nn = n0 + tx;
  const float sw = nn < n ? colmax[nn] / kE4M3Max : 0.f;
  if (blockIdx.x == 0 && ty == 0 && nn < n) w_scale[nn] = sw;
  for (int r = ty; r < 64; r += 4) {
    const int64_t kk = k0 + r;
    float v = 0.f;
    if (kk < k && nn < n && sw > 0.f) v = In::load1(w + (kk * ldw + nn) * In::kBytes) / sw;
    tile[tx][r] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xFF);
  }
  __syncthreads();
  for (int r = ty; r < 64; r += 4) {
    const int64_t on = n0 + r, ok = k0 + tx;
    if (on < n && ok < k) wq[on * k + ok] = tile[r][tx];
  }
}

}  // namespace sqk

namespace sqh {

template <class In, int kCh, int kT>
static void launch_f8_rows(const void* x, int64_t m, int64_t nvec, int64_t ldb, uint8_t* xq, float* x_scale,
                           hipStream_t s, uint32_t* zero, int nzero) {
  const int64_t grid = m < 1024 ? m : 1024;
  hipLaunchKernelGGL((sqk::quant_f8_rows_kernel<In, kCh, kT>), dim3((unsigned)grid), dim3(kT), 0, s,
                     (const uint8_t*)x, m, (int)nvec, ldb, xq, x_scale, zero, nzero);
}

template <class In>
static void quant_f8_t(const void* x, int64_t m, int64_t k, int64_t ldx, uint8_t* xq, float* x_scale, hipStream_t s,
                       uint32_t* zero, int nzero) {
  const int64_t nvec = k / In::kVec;
  const int64_t ldb = ldx * In::kBytes;
  const int64_t per_thread = (nvec + 255) / 256;
  if ((m < 1024 && nvec > 256) || per_thread > 4) {
    const int64_t pt = (nvec + 1023) / 1024;
    if (pt <= 1) launch_f8_rows<In, 1, 1024>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
    else if (pt <= 2) launch_f8_rows<In, 2, 1024>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
    else if (pt <= 4) launch_f8_rows<In, 4, 1024>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
    else launch_f8_rows<In, 8, 1024>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
    return;
  }
  if (per_thread <= 1) launch_f8_rows<In, 1, 256>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
  else if (per_thread <= 2) launch_f8_rows<In, 2, 256>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
  else launch_f8_rows<In, 4, 256>(x, m, nvec, ldb, xq, x_scale, s, zero, nzero);
}

hipError_t quant_f8_rows(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, uint8_t* xq, float* x_scale,
                         hipStream_t s, uint32_t* zero, int64_t nzero) {
  if (m <= 0) return hipSuccess;
  const int nz = (int)nzero;
  switch (xt) {
    case SQ_F32: quant_f8_t<sqk::F32In>(x, m, k, ldx, xq, x_scale, s, zero, nz); break;
    case SQ_BF16: quant_f8_t<sqk::BF16In>(x, m, k, ldx, xq, x_scale, s, zero, nz); break;
    default: quant_f8_t<sqk::F16In>(x, m, k, ldx, xq, x_scale, s, zero, nz); break;
  }
  return hipGetLastError();
}

hipError_t quant_f8_weights(const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw, float* colmax,
                            uint8_t* wq, float* w_scale, hipStream_t s) {
  if (k <= 0 || n <= 0) return hipSuccess;
  hipError_t e = fill_u32(colmax, 0u, n, s);
  if (e == hipSuccess) e = absmax_cols(w, wt, k, n, ldw, colmax, s);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((k + 63) / 64), (unsigned)((n + 63) / 64)), block(256);
  const uint8_t* wb = (const uint8_t*)w;
  switch (wt) {
    case SQ_F32:
      hipLaunchKernelGGL(sqk::quant_f8_weights_kernel<sqk::F32In>, grid, block, 0, s, wb, k, n, ldw, colmax, wq, w_scale);
      break;
    case SQ_BF16:
      hipLaunchKernelGGL(sqk::quant_f8_weights_kernel<sqk::BF16In>, grid, block, 0, s, wb, k, n, ldw, colmax, wq,
                         w_scale);
      break;
    default:
      hipLaunchKernelGGL(sqk::quant_f8_weights_kernel<sqk::F16In>, grid, block, 0, s, wb, k, n, ldw, colmax, wq,
                         w_scale);
      break;
  }
  return hipGetLastError();
}

}  // namespace sqh
