// int8 x int8 -> int32 GEMM on the gfx950 matrix cores with the fused
// dequantisation epilogue.
//
// The LLM.int8() page, "The architecture: every piece explained": int8
// operands, int32 accumulation, dequantisation by the product of the
// per-row (token) and per-column (output channel) scales; the fp16 outlier
// slice of the decomposition is added in the same epilogue. "Half the Size,
// Better Performance, Same Accuracy: Understanding W8A8 INT8 LLM
// Quantization", "Performance After Quantization" (Inter-Token Latency): the
// product is converted back to bf16.
//
// Operands: A = Xq [M x K] and B = Wq [N x K], both K-contiguous, so one
// 16-byte load brings 16 consecutive k of one row and the same k-to-slot
// assignment serves both operands of v_mfma_i32_32x32x32_i8 (lane l supplies
// row l%32 and k-slice l/32 of its 32x32 block).
//
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a 128 x 128 tile;
// each wave a 64 x 64 sub-tile with 2 x 2 MFMA blocks. K advances 64 bytes
// per step through double-buffered LDS (2 x 16 KiB); the next step's global
// loads are issued before the MFMAs of the current one. LDS rows are 64
// bytes and the four 16-byte chunks of a row are XOR-swizzled with bits 1..2
// of the row so that the 16-byte fragment reads of 8 consecutive rows hit
// distinct bank groups.
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutF16 = 2, kOutI32 = 3, kOutDecomp = 4 };

constexpr int kBM = 128, kBN = 128, kBK = 64;

__device__ __forceinline__ int swz(int row, int chunk) { return row * kBK + ((chunk ^ ((row >> 1) & 3)) << 4); }

template <int kOut>
__global__ __launch_bounds__(256) void gemm_i8_kernel(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                      int M, int N, int K, const float* __restrict__ x_scale,
                                                      const float* __restrict__ w_scale, void* __restrict__ Y,
                                                      int64_t ldy, sqh::DecompArgs dec) {
  __shared__ __attribute__((aligned(16))) int8_t sA[2][kBM * kBK];
  __shared__ __attribute__((aligned(16))) int8_t sB[2][kBN * kBK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;
  const int tiles_n = (N + kBN - 1) / kBN;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  // Global -> LDS assignment: 512 16-byte chunks per operand tile, 2 per thread.
  const int8_t* pa[2];
  const int8_t* pb[2];
  int soff[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int g = tid + 256 * i;
    const int row = g >> 2, ch = g & 3;
    const int ra = min(m0 + row, M - 1);
    const int rb = min(n0 + row, N - 1);
    pa[i] = A + (int64_t)ra * K + ch * 16;
    pb[i] = B + (int64_t)rb * K + ch * 16;
    soff[i] = swz(row, ch);
  }

  v16i acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

  u32x4 ga[2], gb[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    ga[i] = load16(pa[i]);
    gb[i] = load16(pb[i]);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    store16(&sA[0][soff[i]], ga[i]);
    store16(&sB[0][soff[i]], gb[i]);
  }
  __syncthreads();

  const int nk = K / kBK;
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ga[i] = load16(pa[i] + (int64_t)(kt + 1) * kBK);
        gb[i] = load16(pb[i] + (int64_t)(kt + 1) * kBK);
      }
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int ch = ks * 2 + (lane >> 5);
      v4i af[2], bf[2];
#pragma unroll
      for (int bi = 0; bi < 2; ++bi) {
        const int row = wm * 64 + bi * 32 + (lane & 31);
        af[bi] = *reinterpret_cast<const v4i*>(&sA[cur][swz(row, ch)]);
      }
#pragma unroll
      for (int bj = 0; bj < 2; ++bj) {
        const int row = wn * 64 + bj * 32 + (lane & 31);
        bf[bj] = *reinterpret_cast<const v4i*>(&sB[cur][swz(row, ch)]);
      }
#pragma unroll
      for (int bi = 0; bi < 2; ++bi)
#pragma unroll
        for (int bj = 0; bj < 2; ++bj)
          acc[bi][bj] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[bi], bf[bj], acc[bi][bj], 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        store16(&sA[cur ^ 1][soff[i]], ga[i]);
        store16(&sB[cur ^ 1][soff[i]], gb[i]);
      }
    }
    __syncthreads();
  }

  // Epilogue. 32x32 block output layout: lane l holds column l%32 and rows
  // 8*(r/4) + 4*(l/32) + r%4 for r = 0..15.
  int cnt = 0;
  if (kOut == kOutDecomp) cnt = *dec.count;
#pragma unroll
  for (int bj = 0; bj < 2; ++bj) {
    const int col = n0 + wn * 64 + bj * 32 + (lane & 31);
    if (col >= N) continue;
    const float sw = kOut == kOutI32 ? 0.f : w_scale[col];
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 64 + bi * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row >= M) continue;
        const int a = acc[bi][bj][r];
        const int64_t o = (int64_t)row * ldy + col;
        if (kOut == kOutI32) {
          reinterpret_cast<int32_t*>(Y)[o] = a;
          continue;
        }
        const float y = __fmul_rn(__fmul_rn((float)a, x_scale[row]), sw);
        if (kOut == kOutF32) {
          reinterpret_cast<float*>(Y)[o] = y;
        } else if (kOut == kOutBF16) {
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(y);
        } else if (kOut == kOutF16) {
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_f16(y);
        } else {
          const float yi = f16_to_f32(f32_to_f16(y));
          float yo = 0.f;
          for (int c = 0; c < cnt; ++c) {
            const int64_t jc = dec.idx[c];
            const float xv = f16_to_f32(dec.x[(int64_t)row * dec.ldx + jc]);
            const float wv = f16_to_f32(dec.w16[jc * dec.ldw + col]);
            yo = __fadd_rn(yo, __fmul_rn(xv, wv));
          }
          const float ys = __fadd_rn(yi, f16_to_f32(f32_to_f16(yo)));
          reinterpret_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_f16(ys);
        }
      }
    }
  }
}

}  // namespace sqk

namespace sqh {

hipError_t gemm_i8(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                   int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, const DecompArgs* dec, void* ws,
                   hipStream_t s) {
  if (m <= 0 || n <= 0) return hipSuccess;
  if (gemm_big_suits(m, n, k, dec == nullptr))
    return gemm_i8_big(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, dec, ws, s);
  const int64_t tiles = ((m + sqk::kBM - 1) / sqk::kBM) * ((n + sqk::kBN - 1) / sqk::kBN);
  const dim3 grid((unsigned)tiles), block(256);
  DecompArgs d{};
  if (dec) d = *dec;
  const int M = (int)m, N = (int)n, K = (int)k;
  if (dec) {
    hipLaunchKernelGGL(sqk::gemm_i8_kernel<sqk::kOutDecomp>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y,
                       ldy, d);
  } else {
    switch (yt) {
      case SQ_F32:
        hipLaunchKernelGGL(sqk::gemm_i8_kernel<sqk::kOutF32>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y,
                           ldy, d);
        break;
      case SQ_BF16:
        hipLaunchKernelGGL(sqk::gemm_i8_kernel<sqk::kOutBF16>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale,
                           y, ldy, d);
        break;
      case SQ_F16:
        hipLaunchKernelGGL(sqk::gemm_i8_kernel<sqk::kOutF16>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y,
                           ldy, d);
        break;
      default:
        hipLaunchKernelGGL(sqk::gemm_i8_kernel<sqk::kOutI32>, grid, block, 0, s, xq, wq, M, N, K, x_scale, w_scale, y,
                           ldy, d);
        break;
    }
  }
  return hipGetLastError();
}

}  // namespace sqh
