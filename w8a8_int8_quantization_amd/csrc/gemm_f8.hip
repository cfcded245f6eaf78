// FP8 (E4M3) W8A8 GEMM on the gfx950 matrix cores, with the per-token x
// per-channel dequantisation epilogue.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization", section "Conclusion": FP8 is the W8A8 alternative that
// skips calibration and needs newer hardware. The dequantisation is the int8
// path's (the LLM.int8() page, "The architecture: every piece explained":
// scale the accumulator by the product of its row and column scales).
//
//   acc_in = sum_k E4M3(xq_ik) * E4M3(wq_nk)        (matrix-core binary32 sums)
//   y_in   = out(fl32(fl32(acc_in * x_scale_i) * w_scale_n))
//
// The products of two E4M3 values are exact in binary32, but the matrix
// cores' FP8 dot products do not round their sums to nearest: measured on
// MI355X against the exact sums (E4M3 operands of every magnitude), both the
// 32x32x64 and 16x16x128 forms (and the older 32x32x16 one) deviate by up to
// ~2^-12 of the sum of |products| per instruction on random codes and ~2^-16
// on quantised Gaussian data. The results are deterministic, but only equal to
// the exact product within such a bound, which the parity tests state.
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a 128 x 128 tile,
// each wave 64 x 64 = 2 x 2 blocks of v_mfma_scale_f32_32x32x64_f8f6f4 (both
// operands E4M3, unit block scales). K advances 128 bytes per step through a
// double-buffered LDS (2 x 32 KiB) with 128-byte rows whose 16-byte chunks are
// XOR-swizzled with (row >> 1) & 7; the next step's global loads are issued
// before the MFMAs of the current one. Lane l supplies row l % 32 and the 32
// k-bytes 32 * (l / 32) .. +31 of a 64-k half-step (two 16-byte chunks).

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

typedef int v8i_t __attribute__((ext_vector_type(8)));
typedef float v16f_t __attribute__((ext_vector_type(16)));

constexpr int kF8BM = 128, kF8BN = 128, kF8BK = 128;

__device__ __forceinline__ int f8_off(int row, int chunk) { return row * kF8BK + ((chunk ^ ((row >> 1) & 7)) << 4); }

template <int kOut>  // 0 f32, 1 bf16, 2 f16
__global__ __launch_bounds__(256) void gemm_f8_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
                                                      int M, int N, int K, const float* __restrict__ x_scale,
                                                      const float* __restrict__ w_scale, void* __restrict__ Y,
                                                      int64_t ldy) {
  __shared__ __attribute__((aligned(16))) uint8_t sA[2][kF8BM * kF8BK];
  __shared__ __attribute__((aligned(16))) uint8_t sB[2][kF8BN * kF8BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = (N + kF8BN - 1) / kF8BN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kF8BM, n0 = tn * kF8BN;

  // global -> LDS: 1024 16-byte chunks per operand tile and step, 4 per thread;
  // 8 consecutive threads read one row's 128 bytes
  const uint8_t* pa[4];
  const uint8_t* pb[4];
  int soff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int g = tid + 256 * i;
    const int row = g >> 3, ch = g & 7;
    pa[i] = A + (int64_t)min(m0 + row, M - 1) * K + ch * 16;
    pb[i] = B + (int64_t)min(n0 + row, N - 1) * K + ch * 16;
    soff[i] = f8_off(row, ch);
  }

  v16f_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4 ga[4], gb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ga[i] = load16(pa[i]);
    gb[i] = load16(pb[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    store16(&sA[0][soff[i]], ga[i]);
    store16(&sB[0][soff[i]], gb[i]);
  }
  __syncthreads();

  const int nk = K / kF8BK;
  const int frow = lane & 31, fhalf = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ga[i] = load16(pa[i] + (int64_t)(kt + 1) * kF8BK);
        gb[i] = load16(pb[i] + (int64_t)(kt + 1) * kF8BK);
      }
    }
#pragma unroll
    for (int hs = 0; hs < 2; ++hs) {
      const int c0 = 4 * hs + 2 * fhalf;  // the lane's two chunks of this 64-byte half-step
      v8i_t af[2], bf[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const int row = wm * 64 + bi * 32 + frow;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&sA[cur][f8_off(row, c0)]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&sA[cur][f8_off(row, c0 + 1)]);
        af[bi] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int row = wn * 64 + bj * 32 + frow;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(&sB[cur][f8_off(row, c0)]);
        const u32x4 hi = *reinterpret_cast<const u32x4*>(&sB[cur][f8_off(row, c0 + 1)]);
        bf[bj] = v8i_t{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(af[bi], bf[bj], acc[bi][bj], 0, 0, 0, 127,
                                                                         0, 127);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        store16(&sA[cur ^ 1][soff[i]], ga[i]);
        store16(&sB[cur ^ 1][soff[i]], gb[i]);
      }
    }
    __syncthreads();
  }

  // Epilogue. 32x32 block output layout: lane l holds column l % 32 and rows
  // 8 (r / 4) + 4 (l / 32) + r % 4 for r = 0..15.
#pragma unroll
  for (int bj = 0; bj < 2; ++bj) {
    const int col = n0 + wn * 64 + bj * 32 + frow;
    if (col >= N) continue;
    const float sw = w_scale[col];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + bi * 32 + 8 * (r >> 2) + 4 * fhalf + (r & 3);
        if (row >= M) continue;
        const float y = __fmul_rn(__fmul_rn(acc[bi][bj][r], x_scale[row]), sw);
        const int64_t o = (int64_t)row * ldy + col;
        if (kOut == 0)
          reinterpret_cast<float*>(Y)[o] = y;
        else if (kOut == 1)
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(y);
        else
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_f16(y);
      }
    }
  }
}

}  // namespace sqk

namespace sqh {

hipError_t gemm_f8(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                   int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  if (gemm_big_suits(m, n, k))
    return gemm_f8_big(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, ws, s);
  const int64_t tiles = ((m + sqk::kF8BM - 1) / sqk::kF8BM) * ((n + sqk::kF8BN - 1) / sqk::kF8BN);
  const dim3 grid((unsigned)tiles), block(256);
  const int M = (int)m, N = (int)n, K = (int)k;
  switch (yt) {
    case SQ_F32:
      hipLaunchKernelGGL(sqk::gemm_f8_kernel<0>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y, ldy);
      break;
    case SQ_BF16:
      hipLaunchKernelGGL(sqk::gemm_f8_kernel<1>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y, ldy);
      break;
    default:
      hipLaunchKernelGGL(sqk::gemm_f8_kernel<2>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y, ldy);
      break;
  }
  return hipGetLastError();
}

}  // namespace sqh
