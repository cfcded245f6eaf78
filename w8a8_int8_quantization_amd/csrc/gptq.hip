// GPTQ weight rounding on gfx950, in binary64.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization":
//  * "How GPTQ improves on naive quantization": a Hessian from the
//    calibration activations; quantise one weight, measure its error, spread
//    the error over the weights not yet quantised as the Hessian directs,
//    repeat;
//  * "How the smoothing factor is computed": it runs on the smoothed weights;
//  * the reference it cites (Frantar et al., GPTQ): per input index in order,
//    with H damped by 1% of its mean diagonal.
//
// Formulation used here. Write H = V V^T with V upper triangular (the
// Cholesky factor of H taken from the last index backwards). The compensated
// weight that step j rounds is
//     z_j = w_j + sum_{i<j} (V_ij / V_jj) * delta_i,   delta_i = w_i - q_i * sw
// where w are the smoothed weights and q_i the codes already chosen. This is
// the same sequence of minimisers as the usual update with the upper factor U
// of H^-1: U = V^-1, so U^T e = delta for the scaled errors e, and
// z_j - q_j = U_jj e_j. No inverse is formed. Per output channel the sweep is
// sequential in j; across channels it is independent. So a block of 64
// inputs is rounded by one thread per channel, with the block's coefficients
// in LDS. A binary64 GEMM then passes the block's deltas on to every later
// input.
//
// Kernels, all on one stream:
//  1. gptq_hessian_kernel: H += Xh^T Xh, Xh = fl32(x / s), 128 x 128 lower
//     tiles mirrored, fp64 FMA with 8 x 8 outputs per thread;
//  2. gptq_weights_kernel: W' = fl32(s_j W_jn) as binary32 (0 on dead
//     inputs), with the column maxima;
//  3. gptq_damp_kernel, gptq_reverse_kernel: lambda = damp * mean(diag H)
//     (dead diagonal entries counted as 1), and A = P (H + dead + lambda I) P
//     with P the index reversal;
//  4. blocked lower Cholesky of A, 64 columns at a time: diagonal block in
//     LDS (one wave, left-looking), panel by forward substitution, trailing
//     update as an fp64 GEMM;
//  5. gptq_unit_kernel: C_ij = V_ij / V_jj into the upper triangle;
//  6. per block of 64 inputs: gptq_block_kernel (codes, deltas; one lane per
//     output channel), then gptq_trailing_kernel (Z += C^T D for the later
//     inputs).
#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

// v - sum_{p<c} x(p) * y(p) over four interleaved partial sums (four
// independent FMA chains instead of one), added in a fixed order
template <class X, class Y>
__device__ __forceinline__ double dot_sub(double v, int c, X x, Y y) {
  double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
  int p = 0;
  for (; p + 4 <= c; p += 4) {
    s0 = __builtin_fma(x(p), y(p), s0);
    s1 = __builtin_fma(x(p + 1), y(p + 1), s1);
    s2 = __builtin_fma(x(p + 2), y(p + 2), s2);
    s3 = __builtin_fma(x(p + 3), y(p + 3), s3);
  }
  for (; p < c; ++p) s0 = __builtin_fma(x(p), y(p), s0);
  return v - ((s0 + s1) + (s2 + s3));
}

constexpr int kGB = 64;   // Cholesky panel width and sweep block
constexpr int kGT = 128;  // GEMM output tile
constexpr int kGP = 16;   // GEMM k-chunk staged in LDS

// One 128 x 128 tile of acc += sum_p a[p][r] * b[p][c] from k-chunks staged
// p-major in LDS; thread (ty, tx) of 16 x 16 owns rows 8 ty .. and columns
// 8 tx ...
__device__ __forceinline__ void tile_fma(const double (*sa)[kGT], const double (*sb)[kGT], int ty, int tx,
                                         double (*acc)[8]) {
#pragma unroll 4
  for (int p = 0; p < kGP; ++p) {
    double a[8], b[8];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      const double2 va = *reinterpret_cast<const double2*>(&sa[p][8 * ty + i]);
      const double2 vb = *reinterpret_cast<const double2*>(&sb[p][8 * tx + i]);
      a[i] = va.x; a[i + 1] = va.y;
      b[i] = vb.x; b[i + 1] = vb.y;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fma(a[i], b[j], acc[i][j]);
  }
}

// ---- 1. Hessian over 128 x 128 tiles (ti >= tj); x rows t, t < T
template <class In, bool kSmooth>
__global__ __launch_bounds__(256) void gptq_hessian_kernel(const uint8_t* __restrict__ x, int64_t t_rows,
                                                           int64_t ldx_bytes, const float* __restrict__ smooth,
                                                           double* __restrict__ h, int64_t k) {
  const int nt = (int)(k / kGT);
  const int ti = blockIdx.x / nt, tj = blockIdx.x % nt;
  if (tj > ti) return;
  __shared__ __attribute__((aligned(16))) double sa[kGP][kGT];
  __shared__ __attribute__((aligned(16))) double sb[kGP][kGT];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t a0 = (int64_t)ti * kGT, b0 = (int64_t)tj * kGT;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  // loader: 16 rows x 128 columns per operand, 8 elements per thread; the
  // 128 threads of a row half read consecutive columns
  const int lc = tid & 127, lr = tid >> 7;
  const float sa_s = kSmooth ? smooth[a0 + lc] : 1.f;
  const float sb_s = kSmooth ? smooth[b0 + lc] : 1.f;
  // the next chunk's raw values are loaded into registers while the current
  // one is multiplied out of LDS
  float ra[kGP / 2], rb[kGP / 2];
  // loads from a clamped (valid) row, then a select: unconditional loads are
  // issued together instead of one branch and one wait each
  auto fetch = [&](int64_t t0) {
#pragma unroll
    for (int i = 0; i < kGP / 2; ++i) {
      const int64_t t = t0 + lr + 2 * i;
      const uint8_t* row = x + (t < t_rows ? t : t_rows - 1) * ldx_bytes;
      const float va = In::load1(row + (a0 + lc) * In::kBytes);
      const float vb = In::load1(row + (b0 + lc) * In::kBytes);
      ra[i] = t < t_rows ? va : 0.f;
      rb[i] = t < t_rows ? vb : 0.f;
    }
  };
  fetch(0);
  for (int64_t t0 = 0; t0 < t_rows; t0 += kGP) {
#pragma unroll
    for (int i = 0; i < kGP / 2; ++i) {
      const int p = lr + 2 * i;
      sa[p][lc] = (double)(kSmooth ? ra[i] / sa_s : ra[i]);
      sb[p][lc] = (double)(kSmooth ? rb[i] / sb_s : rb[i]);
    }
    __syncthreads();
    if (t0 + kGP < t_rows) fetch(t0 + kGP);
    tile_fma(sa, sb, ty, tx, acc);
    __syncthreads();
  }
  // read-modify-write a row of 8 at a time: the 8 (16) loads go out together
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t a = a0 + 8 * ty + i;
    double o1[8], o2[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t b = b0 + 8 * tx + j;
      o1[j] = h[a * k + b];
      o2[j] = h[b * k + a];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t b = b0 + 8 * tx + j;
      h[a * k + b] = o1[j] + acc[i][j];
      if (ti != tj) h[b * k + a] = o2[j] + acc[i][j];
    }
  }
}

// ---- 2. smoothed weights (binary32) and their column maxima
template <class In, bool kSmooth>
__global__ __launch_bounds__(256) void gptq_weights_kernel(const uint8_t* __restrict__ w, int64_t ldw, int64_t k,
                                                           int64_t n, const float* __restrict__ smooth,
                                                           const double* __restrict__ h, float* __restrict__ wp,
                                                           uint32_t* __restrict__ colmax) {
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col >= n) return;
  const int64_t j0 = (int64_t)blockIdx.y * kGB;
  float m = 0.f;
  for (int64_t j = j0; j < j0 + kGB; ++j) {
    float v = In::load1(w + (j * ldw + col) * In::kBytes);
    if (kSmooth) v = __fmul_rn(smooth[j], v);
    if (h[j * k + j] == 0.0) v = 0.f;  // dead input
    wp[j * n + col] = v;
    m = fmaxf(m, fabsf(v));
  }
  atomicMax(colmax + col, __float_as_uint(m));
}

// ---- 3. damping and the reversed, damped copy (lower triangle)
__global__ __launch_bounds__(256) void gptq_damp_kernel(const double* __restrict__ h, int64_t k, double damp,
                                                        double* __restrict__ lam) {
  __shared__ double part[256];
  const int tid = threadIdx.x;
  double s = 0.0;
  for (int64_t j = tid; j < k; j += 256) {
    const double d = h[j * k + j];
    s += d == 0.0 ? 1.0 : d;
  }
  part[tid] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (tid < w) part[tid] += part[tid + w];
    __syncthreads();
  }
  if (tid == 0) lam[0] = damp * (part[0] / (double)k);
}

// A[a][b] = H[K-1-b][K-1-a] for a >= b (reads the lower triangle of H), the
// diagonal with dead entries set to 1 and lambda added
__global__ __launch_bounds__(256) void gptq_reverse_kernel(const double* __restrict__ h, int64_t k,
                                                           const double* __restrict__ lam, double* __restrict__ a) {
  const int64_t row = (int64_t)blockIdx.y;
  const int64_t col = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (col > row) return;
  double v = h[(k - 1 - col) * k + (k - 1 - row)];
  if (col == row) v = (v == 0.0 ? 1.0 : v) + lam[0];
  a[row * k + col] = v;
}

// ---- 4. blocked Cholesky (lower) of A, panel kb
// Diagonal block, left-looking, one wave: lane r owns row r;
// column c: v_r = A_rc - sum_{p<c} L_rp L_cp, L_cc = sqrt(v_c), L_rc = v_r / L_cc.
__global__ __launch_bounds__(64) void chol_diag_kernel(double* __restrict__ a, int64_t k, int64_t o) {
  __shared__ double l[kGB][kGB + 1];
  const int r = threadIdx.x;
  // unconditional loads (every address is inside the block), then a select
#pragma unroll 16
  for (int i = 0; i < kGB; ++i) {
    const double v = a[(o + i) * k + (o + r)];
    l[i][r] = r <= i ? v : 0.0;
  }
  __syncthreads();
  for (int c = 0; c < kGB; ++c) {
    double v = 0.0;
    if (r >= c) v = dot_sub(l[r][c], c, [&](int p) { return l[r][p]; }, [&](int p) { return l[c][p]; });
    if (r == c) l[c][c] = sqrt(v);
    __syncthreads();
    if (r > c) l[r][c] = v / l[c][c];
    __syncthreads();
  }
#pragma unroll 16
  for (int i = 0; i < kGB; ++i)
    if (r <= i) a[(o + i) * k + (o + r)] = l[i][r];
}

// rows i0 .. i0+63 below the diagonal block: L21 = A21 L11^-T, one thread per row
__global__ __launch_bounds__(64) void chol_panel_kernel(double* __restrict__ a, int64_t k, int64_t o) {
  __shared__ double l11[kGB][kGB + 1];
  __shared__ double p[kGB][kGB + 1];  // p[c][r]: column c of row r
  const int r = threadIdx.x;
  const int64_t i0 = o + kGB + (int64_t)blockIdx.x * kGB;
  // row by row, the 64 lanes reading one row's 64 consecutive columns
#pragma unroll 16
  for (int i = 0; i < kGB; ++i) {
    const double v = a[(o + i) * k + (o + r)];
    l11[i][r] = r <= i ? v : 0.0;
    p[r][i] = a[(i0 + i) * k + (o + r)];
  }
  __syncthreads();
  for (int c = 0; c < kGB; ++c) {
    const double v = dot_sub(p[c][r], c, [&](int q) { return p[q][r]; }, [&](int q) { return l11[c][q]; });
    p[c][r] = v / l11[c][c];
  }
  __syncthreads();
#pragma unroll 16
  for (int i = 0; i < kGB; ++i) a[(i0 + i) * k + (o + r)] = p[r][i];
}

// trailing update of rows/columns [s, K), s = o + 64: A[r][c] -= sum_p L[r][o+p] L[c][o+p], lower tiles
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ a, int64_t k, int64_t o) {
  const int64_t s = o + kGB;
  const int nt = (int)((k - s + kGT - 1) / kGT);
  const int ti = blockIdx.x / nt, tj = blockIdx.x % nt;
  if (tj > ti) return;
  __shared__ __attribute__((aligned(16))) double sa[kGP][kGT];
  __shared__ __attribute__((aligned(16))) double sb[kGP][kGT];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t r0 = s + (int64_t)ti * kGT, c0 = s + (int64_t)tj * kGT;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  // loader: element (row q of the tile, column p of the panel); 16 consecutive
  // threads read one row's 16 panel columns (128 bytes)
  const int lp = tid & 15, lq = tid >> 4;
  double va[kGT / 16], vb[kGT / 16];
  auto fetch = [&](int p0) {
#pragma unroll
    for (int i = 0; i < kGT / 16; ++i) {
      const int64_t ra = r0 + lq + 16 * i, rb = c0 + lq + 16 * i;
      const double x0 = a[(ra < k ? ra : k - 1) * k + o + p0 + lp];
      const double x1 = a[(rb < k ? rb : k - 1) * k + o + p0 + lp];
      va[i] = ra < k ? x0 : 0.0;
      vb[i] = rb < k ? x1 : 0.0;
    }
  };
  fetch(0);
  for (int p0 = 0; p0 < kGB; p0 += kGP) {
#pragma unroll
    for (int i = 0; i < kGT / 16; ++i) {
      sa[lp][lq + 16 * i] = va[i];
      sb[lp][lq + 16 * i] = vb[i];
    }
    __syncthreads();
    if (p0 + kGP < kGB) fetch(p0 + kGP);
    tile_fma(sa, sb, ty, tx, acc);
    __syncthreads();
  }
  // A -= acc on and below the diagonal. With an even K and a 16-byte aligned
  // A the thread's 8 columns go as four 16-byte accesses (c is even, so
  // c < k implies c + 1 < k); a pair that straddles the diagonal stores its
  // first element only.
  if ((k & 1) == 0 && (reinterpret_cast<uintptr_t>(a) & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + 8 * ty + i;
      const int64_t rr = r < k ? r : k - 1;
      double2 old[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + 8 * tx + 2 * j;
        old[j] = *reinterpret_cast<const double2*>(&a[rr * k + (c < k ? c : k - 2)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + 8 * tx + 2 * j;
        if (r < k && c + 1 <= r)
          *reinterpret_cast<double2*>(&a[r * k + c]) =
              double2{old[j].x - acc[i][2 * j], old[j].y - acc[i][2 * j + 1]};
        else if (r < k && c == r)
          a[r * k + c] = old[j].x - acc[i][2 * j];
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + 8 * ty + i;
    const int64_t rr = r < k ? r : k - 1;
    double old[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + 8 * tx + j;
      old[j] = a[rr * k + (c < k ? c : k - 1)];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + 8 * tx + j;
      if (r < k && c <= r) a[r * k + c] = old[j] - acc[i][j];
    }
  }
}

// ---- 5. C[i][j] = V_ij / V_jj for i < j, with V_ij = L[K-1-i][K-1-j], into the upper triangle
__global__ __launch_bounds__(256) void gptq_unit_kernel(double* __restrict__ a, int64_t k) {
  const int64_t i = (int64_t)blockIdx.y;
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j <= i || j >= k) return;
  const int64_t ri = k - 1 - i, rj = k - 1 - j;
  a[i * k + j] = a[ri * k + rj] / a[rj * k + rj];
}

// ---- 6a. one block of 64 inputs, one lane per output channel (one wave per
// workgroup): z_q = w_q + Z_q + sum_{p<q} C[j0+p][j0+q] delta_p, left-looking,
// with the block's coefficients, this lane's deltas and codes in LDS
__global__ __launch_bounds__(64) void gptq_block_kernel(const float* __restrict__ wp, const double* __restrict__ z,
                                                        const double* __restrict__ a,
                                                        const uint32_t* __restrict__ colmax, int64_t k, int64_t n,
                                                        int64_t j0, double* __restrict__ dblk,
                                                        int8_t* __restrict__ wq, float* __restrict__ w_scale) {
  __shared__ double cb[kGB][kGB];  // cb[p][q] = C[j0+p][j0+q], p < q
  __shared__ double ds[kGB][64];   // ds[q][lane]: z_q's running correction, then delta_q
  __shared__ float wsh[kGB][64];   // this lane's smoothed weights of the block
  __shared__ uint32_t cs[kGB][64];  // codes, one per word
  const int lane = threadIdx.x;
  for (int e = lane; e < kGB * kGB; e += 64) {
    const int p = e / kGB, q = e % kGB;
    cb[p][q] = p < q ? a[(j0 + p) * k + (j0 + q)] : 0.0;
  }
  __syncthreads();
  const int64_t col = (int64_t)blockIdx.x * 64 + lane;
  if (col >= n) return;  // no barrier below
  const float sw = __uint_as_float(colmax[col]) / 127.f;
  if (j0 == 0) w_scale[col] = sw;
  const double sw64 = (double)sw;
  // the block's corrections and weights of this channel, every load in flight at once
#pragma unroll 16
  for (int q = 0; q < kGB; ++q) {
    ds[q][lane] = z[(j0 + q) * n + col];
    wsh[q][lane] = wp[(j0 + q) * n + col];
  }
  for (int q = 0; q < kGB; ++q) {
    const double acc = -dot_sub(-ds[q][lane], q, [&](int p) { return cb[p][q]; }, [&](int p) { return ds[p][lane]; });
    const double w = (double)wsh[q][lane];
    const double zq = w + acc;
    double code = 0.0;
    if (sw > 0.f) code = fmin(fmax(rint(zq / sw64), -127.0), 127.0);
    const double delta = w - code * sw64;
    ds[q][lane] = delta;
    dblk[(int64_t)q * n + col] = delta;
    cs[q][lane] = (uint32_t)(int32_t)code & 0xFFu;
  }
  uint4* dst = reinterpret_cast<uint4*>(wq + col * k + j0);
#pragma unroll
  for (int v = 0; v < kGB / 16; ++v) {
    uint32_t wv[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = 16 * v + 4 * u;
      wv[u] = cs[q][lane] | (cs[q + 1][lane] << 8) | (cs[q + 2][lane] << 16) | (cs[q + 3][lane] << 24);
    }
    dst[v] = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// ---- 6b. Z[j][n] += sum_p C[j0+p][j] * D[p][n] for j >= j0 + 64
__global__ __launch_bounds__(256) void gptq_trailing_kernel(const double* __restrict__ a,
                                                            const double* __restrict__ dblk, double* __restrict__ z,
                                                            int64_t k, int64_t n, int64_t j0) {
  const int64_t s = j0 + kGB;
  const int ntn = (int)((n + kGT - 1) / kGT);
  const int ti = blockIdx.x / ntn, tj = blockIdx.x % ntn;
  __shared__ __attribute__((aligned(16))) double sa[kGP][kGT];
  __shared__ __attribute__((aligned(16))) double sb[kGP][kGT];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int64_t r0 = s + (int64_t)ti * kGT, c0 = (int64_t)tj * kGT;
  double acc[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.0;
  const int lc = tid & 127, lr = tid >> 7;
  double va[kGP / 2], vb[kGP / 2];
  auto fetch = [&](int p0) {
    const int64_t r = r0 + lc, c = c0 + lc;
    const int64_t rr = r < k ? r : k - 1, cc = c < n ? c : n - 1;
#pragma unroll
    for (int i = 0; i < kGP / 2; ++i) {
      const int p = lr + 2 * i;
      const double x0 = a[(j0 + p0 + p) * k + rr];
      const double x1 = dblk[(int64_t)(p0 + p) * n + cc];
      va[i] = r < k ? x0 : 0.0;
      vb[i] = c < n ? x1 : 0.0;
    }
  };
  fetch(0);
  for (int p0 = 0; p0 < kGB; p0 += kGP) {
#pragma unroll
    for (int i = 0; i < kGP / 2; ++i) {
      sa[lr + 2 * i][lc] = va[i];
      sb[lr + 2 * i][lc] = vb[i];
    }
    __syncthreads();
    if (p0 + kGP < kGB) fetch(p0 + kGP);
    tile_fma(sa, sb, ty, tx, acc);
    __syncthreads();
  }
  // Z += acc. With an even row length and a 16-byte aligned Z the thread's 8
  // columns go as four 16-byte accesses (column pairs never straddle the end:
  // c is even, so c < n implies c + 1 < n); otherwise one element at a time.
  if ((n & 1) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int64_t r = r0 + 8 * ty + i;
      const int64_t rr = r < k ? r : k - 1;
      double2 old[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + 8 * tx + 2 * j;
        old[j] = *reinterpret_cast<const double2*>(&z[rr * n + (c < n ? c : n - 2)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t c = c0 + 8 * tx + 2 * j;
        if (r < k && c < n)
          *reinterpret_cast<double2*>(&z[r * n + c]) =
              double2{old[j].x + acc[i][2 * j], old[j].y + acc[i][2 * j + 1]};
      }
    }
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int64_t r = r0 + 8 * ty + i;
    const int64_t rr = r < k ? r : k - 1;
    double old[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + 8 * tx + j;
      old[j] = z[rr * n + (c < n ? c : n - 1)];
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int64_t c = c0 + 8 * tx + j;
      if (r < k && c < n) z[r * n + c] = old[j] + acc[i][j];
    }
  }
}

}  // namespace sqk

namespace sqh {

namespace {

template <class In>
hipError_t hessian_t(const void* x, int64_t t, int64_t k, int64_t ldx, const float* smooth, double* h,
                     hipStream_t s) {
  const int64_t nt = k / sqk::kGT;
  const dim3 grid((unsigned)(nt * nt)), block(256);
  const uint8_t* xb = (const uint8_t*)x;
  const int64_t ldb = ldx * In::kBytes;
  if (smooth)
    hipLaunchKernelGGL((sqk::gptq_hessian_kernel<In, true>), grid, block, 0, s, xb, t, ldb, smooth, h, k);
  else
    hipLaunchKernelGGL((sqk::gptq_hessian_kernel<In, false>), grid, block, 0, s, xb, t, ldb, smooth, h, k);
  return hipGetLastError();
}

template <class In>
void weights_t(const void* w, int64_t ldw, int64_t k, int64_t n, const float* smooth, const double* h, float* wp,
               uint32_t* colmax, hipStream_t s) {
  const dim3 grid((unsigned)((n + 255) / 256), (unsigned)(k / sqk::kGB)), block(256);
  if (smooth)
    hipLaunchKernelGGL((sqk::gptq_weights_kernel<In, true>), grid, block, 0, s, (const uint8_t*)w, ldw, k, n, smooth,
                       h, wp, colmax);
  else
    hipLaunchKernelGGL((sqk::gptq_weights_kernel<In, false>), grid, block, 0, s, (const uint8_t*)w, ldw, k, n,
                       smooth, h, wp, colmax);
}

size_t align256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

hipError_t gptq_hessian(const void* x, sq_dtype xt, int64_t t, int64_t k, int64_t ldx, const float* smooth, double* h,
                        hipStream_t s) {
  if (t <= 0 || k <= 0) return hipSuccess;
  switch (xt) {
    case SQ_F32: return hessian_t<sqk::F32In>(x, t, k, ldx, smooth, h, s);
    case SQ_BF16: return hessian_t<sqk::BF16In>(x, t, k, ldx, smooth, h, s);
    default: return hessian_t<sqk::F16In>(x, t, k, ldx, smooth, h, s);
  }
}

size_t gptq_workspace(int64_t k, int64_t n) {
  if (k <= 0 || n <= 0) return 0;
  return 256 + align256((size_t)n * 4) + align256((size_t)k * k * 8) + align256((size_t)k * n * 4) +
         align256((size_t)k * n * 8) + align256((size_t)sqk::kGB * n * 8);
}

hipError_t gptq_quantize(const double* h, const void* w, sq_dtype wt, int64_t k, int64_t n, int64_t ldw,
                         const float* smooth, double damp, int8_t* wq, float* w_scale, void* ws, hipStream_t s) {
  if (k <= 0 || n <= 0) return hipSuccess;
  char* p = reinterpret_cast<char*>(ws);
  double* lam = reinterpret_cast<double*>(p);
  p += 256;
  uint32_t* colmax = reinterpret_cast<uint32_t*>(p);
  p += align256((size_t)n * 4);
  double* a = reinterpret_cast<double*>(p);
  p += align256((size_t)k * k * 8);
  float* wp = reinterpret_cast<float*>(p);
  p += align256((size_t)k * n * 4);
  double* z = reinterpret_cast<double*>(p);
  p += align256((size_t)k * n * 8);
  double* dblk = reinterpret_cast<double*>(p);

  hipError_t e = fill_u32(colmax, 0u, n, s);
  if (e == hipSuccess) e = fill_u32(z, 0u, 2 * k * n, s);
  if (e != hipSuccess) return e;
  switch (wt) {
    case SQ_F32: weights_t<sqk::F32In>(w, ldw, k, n, smooth, h, wp, colmax, s); break;
    case SQ_BF16: weights_t<sqk::BF16In>(w, ldw, k, n, smooth, h, wp, colmax, s); break;
    default: weights_t<sqk::F16In>(w, ldw, k, n, smooth, h, wp, colmax, s); break;
  }
  hipLaunchKernelGGL(sqk::gptq_damp_kernel, dim3(1), dim3(256), 0, s, h, k, damp, lam);
  hipLaunchKernelGGL(sqk::gptq_reverse_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, h, k,
                     lam, a);
  const int64_t nb = k / sqk::kGB;
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t o = b * sqk::kGB;
    hipLaunchKernelGGL(sqk::chol_diag_kernel, dim3(1), dim3(64), 0, s, a, k, o);
    if (b + 1 < nb) {
      hipLaunchKernelGGL(sqk::chol_panel_kernel, dim3((unsigned)(nb - 1 - b)), dim3(64), 0, s, a, k, o);
      const int64_t nt = (k - o - sqk::kGB + sqk::kGT - 1) / sqk::kGT;
      hipLaunchKernelGGL(sqk::chol_update_kernel, dim3((unsigned)(nt * nt)), dim3(256), 0, s, a, k, o);
    }
  }
  hipLaunchKernelGGL(sqk::gptq_unit_kernel, dim3((unsigned)((k + 255) / 256), (unsigned)k), dim3(256), 0, s, a, k);
  const unsigned ncol = (unsigned)((n + 63) / 64);
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t j0 = b * sqk::kGB;
    hipLaunchKernelGGL(sqk::gptq_block_kernel, dim3(ncol), dim3(64), 0, s, wp, z, a, colmax, k, n, j0, dblk, wq,
                       w_scale);
    if (b + 1 < nb) {
      const int64_t ntr = (k - j0 - sqk::kGB + sqk::kGT - 1) / sqk::kGT;
      const int64_t ntn = (n + sqk::kGT - 1) / sqk::kGT;
      hipLaunchKernelGGL(sqk::gptq_trailing_kernel, dim3((unsigned)(ntr * ntn)), dim3(256), 0, s, a, dblk, z, k, n,
                         j0);
    }
  }
  return hipGetLastError();
}

}  // namespace sqh
