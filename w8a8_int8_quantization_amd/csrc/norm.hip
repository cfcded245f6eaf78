// RMSNorm whose gain carries the smoothing factor, fused with per-token int8
// quantisation.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization":
//   * "Where the outlier actually comes from": RMSNorm divides a token's
//     vector by its root-mean-square, then scales channel j by a gain gamma_j;
//   * "How the smoothing factor is computed": SmoothQuant divides gamma by s
//     (the matching weight rows are multiplied by s), so the norm's output is
//     already the smoothed activation and the quantiser needs no division by s;
//   * "How the Model Was Compressed" / "Why Activation Quantization Is Hard":
//     one scale per token, d = max|a| / 127, q = round(a / d).
//
// What one row computes (x: M x K of bf16, fp16 or binary32; g = gamma / s):
//   S     = sum_j x_j^2, exact, rounded once to binary64
//   v     = RN64(RN64(S / K) + eps);  inv = RN32(RN64(1 / RN64(sqrt(v))))
//   a_j   = RN32(RN32(x_j * inv) * g_j)
//   d     = RN32(max_j |a_j| / 127);  q_j = clamp(round_half_even(RN32(a_j / d)))
// A row with v == 0, or whose inv overflows binary32, normalises to zero.
//
// Exact sum of squares. A value is m * 2^(e - off) with an integer
// significand m (hidden bit included) and the exponent field e (1 for
// subnormals), so its square is m^2 * 2^(2e - 2 off) with m^2 < 2^48. With emax
// the row's largest exponent field, d = 2 (emax - e) is the square's distance
// below the largest square in binades. Chunk c holds the squares with
// d in [64c, 64c + 64) as the 128-bit integer sum of m^2 << (64(c+1) - d),
// in units of 2^(2 emax - 2 off - 64(c+1)): every such term is exact
// (m^2 << 64 < 2^112) and K <= 32768 terms cannot overflow 128 bits. Integer
// sums do not depend on order, so the wave and workgroup reductions give the
// same bits however the row is split. Chunk 0 covers every square within 2^-64
// of the largest one, which is all of them in practice; when a row has smaller
// nonzero squares the workgroup forms the further chunks one reduction at a
// time. The chunks then form one wide integer (Horner: W = W * 2^64 + B_c),
// and its round-to-nearest-even binary64 value, scaled by the unit, is S.
// fp16 squares span 2^58 at most, so fp16 rows never need a second chunk.
//
// Layout: a kT-thread workgroup walks a grid-stride list of rows; thread t
// owns the 16-byte vectors t, t + kT, ... of every row, keeps them in
// registers through the three row reductions (largest exponent, sum of
// squares, largest |a|), and loads the next row's vectors while it works on
// the current one. The gains of its columns stay in registers for every row.
#include <math.h>

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

// Integer significand and exponent field of the element formats.
template <class In>
struct NormBits;
template <>
struct NormBits<BF16In> {
  static constexpr int kManBits = 7, kOff = 134, kMaxChunks = 8;
  static constexpr uint32_t kMagMask = 0x7FFFu;
};
template <>
struct NormBits<F16In> {
  static constexpr int kManBits = 10, kOff = 25, kMaxChunks = 1;
  static constexpr uint32_t kMagMask = 0x7FFFu;
};
template <>
struct NormBits<F32In> {
  static constexpr int kManBits = 23, kOff = 150, kMaxChunks = 8;
  static constexpr uint32_t kMagMask = 0x7FFFFFFFu;
};

// Element e of a 16-byte vector as raw magnitude bits (sign dropped).
template <class In>
__device__ __forceinline__ uint32_t mag_bits(const u32x4& v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (In::kVec == 8)
    return ((e & 1) ? (w[e >> 1] >> 16) : w[e >> 1]) & NormBits<In>::kMagMask;
  else
    return w[e] & NormBits<In>::kMagMask;
}

struct U128 {
  uint64_t lo, hi;
};

__device__ __forceinline__ void add128(U128& a, uint64_t lo, uint64_t hi) {
  const uint64_t s = a.lo + lo;
  a.hi += hi + (s < lo ? 1u : 0u);
  a.lo = s;
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int off) {
  const uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
  const uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
  return ((uint64_t)hi << 32) | lo;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = __shfl_xor(v, off, 64);
    v = o > v ? o : v;
  }
  return v;
}

__device__ __forceinline__ U128 wave_sum128(U128 a) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) add128(a, shfl_xor_u64(a.lo, off), shfl_xor_u64(a.hi, off));
  return a;
}

// Round-to-nearest-even binary64 of the integer W[0] + W[1] 2^64 + ... times 2^unit.
template <int kW>
__device__ __forceinline__ double wide_to_f64(const uint64_t (&w)[kW], int unit) {
  uint64_t top = 0, nxt = 0;
  bool found = false, have_nxt = false, sticky = false;
  int t = 0;
#pragma unroll
  for (int j = kW - 1; j >= 0; --j) {
    if (found) {
      if (have_nxt) sticky |= w[j] != 0;
      else nxt = w[j];
      have_nxt = true;
    } else if (w[j] != 0) {
      found = true;
      top = w[j];
      t = j;
    }
  }
  if (!found) return 0.0;
  const int lz = __builtin_clzll(top);
  const uint64_t mant = lz ? (top << lz) | (nxt >> (64 - lz)) : top;  // most significant bit at bit 63
  sticky |= (lz ? (nxt << lz) : nxt) != 0;
  uint64_t keep = mant >> 11;
  const uint64_t rest = mant & 0x7FFu;
  const bool up = (rest > 0x400u) || (rest == 0x400u && (sticky || (keep & 1u)));
  keep += up ? 1u : 0u;  // may reach 2^53, still exact as a double
  const int msb = 64 * t + 63 - lz;
  return ldexp((double)keep, msb - 52 + unit);
}

template <class In, int kCh, int kT>
__global__ __launch_bounds__(kT) void rmsnorm_quant_kernel(const uint8_t* __restrict__ x, int64_t m, int nvec,
                                                            int64_t ldx_bytes, const float* __restrict__ gain,
                                                            float eps, int8_t* __restrict__ xq,
                                                            float* __restrict__ x_scale, uint32_t* __restrict__ zero,
                                                            int nzero) {
  using NB = NormBits<In>;
  constexpr int V = In::kVec;
  constexpr int kW = kT / 64;
  __shared__ uint32_t red_e[kW];
  __shared__ uint64_t red_s[kW][2];
  __shared__ uint32_t red_more[kW];
  __shared__ float red_a[kW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t k = (int64_t)nvec * V;

  auto load_row = [&](int64_t row, u32x4* dst) {
    const uint8_t* xr = x + row * ldx_bytes;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int vi = tid + kT * c;
      dst[c] = vi < nvec ? load16(xr + (int64_t)vi * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 nxt[kCh];
  int64_t row = blockIdx.x;
  if (row < m) load_row(row, nxt);
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += kT) zero[i] = 0u;

  float g[kCh][V];
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    const int vi = tid + kT * c;
#pragma unroll
    for (int e = 0; e < V; e += 4) {
      const u32x4 gv = vi < nvec ? load16(gain + (int64_t)vi * V + e) : u32x4{0u, 0u, 0u, 0u};
      g[c][e] = __uint_as_float(gv.x); g[c][e + 1] = __uint_as_float(gv.y);
      g[c][e + 2] = __uint_as_float(gv.z); g[c][e + 3] = __uint_as_float(gv.w);
    }
  }
  const double kd = (double)k;
  const double epsd = (double)eps;

  for (; row < m; row += gridDim.x) {
    u32x4 raw[kCh];
#pragma unroll
    for (int c = 0; c < kCh; ++c) raw[c] = nxt[c];
    if (row + gridDim.x < m) load_row(row + gridDim.x, nxt);

    // 1. largest magnitude (bit patterns of non-negative values order like the values)
    uint32_t mx = 0;
#pragma unroll
    for (int c = 0; c < kCh; ++c)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint32_t b = mag_bits<In>(raw[c], e);
        mx = b > mx ? b : mx;
      }
    mx = wave_max_u32(mx);
    if (lane == 0) red_e[wid] = mx;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kW; ++w) mx = red_e[w] > mx ? red_e[w] : mx;
    const int emax_f = (int)(mx >> NB::kManBits);
    const int emax = emax_f > 1 ? emax_f : 1;

    // 2. exact sum of squares: chunk 0 from the registers; the rare further
    //    chunks re-read the row (uniform across the workgroup)
    auto term = [&](uint32_t b, int c0, U128& acc, bool& mr) {
      const uint32_t ef = b >> NB::kManBits;
      const uint32_t mn = b & ((1u << NB::kManBits) - 1u);
      const uint64_t mant = ef ? (mn | (1u << NB::kManBits)) : mn;
      const int ex = ef ? (int)ef : 1;
      const uint64_t m2 = mant * mant;
      const int d = 2 * (emax - ex) - 64 * c0;  // negative: an earlier chunk's term
      const bool in = d >= 0 && d < 64;
      mr |= d >= 64 && m2 != 0;
      const int dd = in ? d : 0;
      const uint64_t hi = in ? (m2 >> dd) : 0u;
      const uint64_t lo = (in && dd > 0) ? (m2 << (64 - dd)) : 0u;
      add128(acc, lo, hi);
    };
    auto block_sum = [&](U128 acc, bool mr, bool& more) {
      acc = wave_sum128(acc);
      const uint32_t wmore = __any(mr) ? 1u : 0u;
      if (lane == 0) {
        red_s[wid][0] = acc.lo;
        red_s[wid][1] = acc.hi;
        red_more[wid] = wmore;
      }
      lds_barrier();
      U128 tot = {0u, 0u};
      uint32_t anym = 0;
#pragma unroll
      for (int w = 0; w < kW; ++w) {
        add128(tot, red_s[w][0], red_s[w][1]);
        anym |= red_more[w];
      }
      more = anym != 0;
      return tot;
    };
    bool more = false;
    U128 b0;
    {
      U128 acc = {0u, 0u};
      bool mr = false;
#pragma unroll
      for (int c = 0; c < kCh; ++c)
#pragma unroll
        for (int e = 0; e < V; ++e) term(mag_bits<In>(raw[c], e), 0, acc, mr);
      b0 = block_sum(acc, mr, more);
    }
    double ss;
    if (NB::kMaxChunks == 1 || !more) {
      const uint64_t w2[2] = {b0.lo, b0.hi};
      ss = wide_to_f64<2>(w2, 2 * (emax - NB::kOff) - 64);
    } else {
      // squares below 2^-64 of the largest: Horner over the chunks, W = W * 2^64 + B_c
      uint64_t wide[NB::kMaxChunks + 1];
#pragma unroll
      for (int j = 0; j <= NB::kMaxChunks; ++j) wide[j] = 0u;
      wide[0] = b0.lo;
      wide[1] = b0.hi;
      int nchunks = 1;
      const uint8_t* xr = x + row * ldx_bytes;
#pragma unroll 1
      for (int c = 1; c < NB::kMaxChunks && more; ++c) {
        lds_barrier();  // the previous chunk's LDS reads are done before lane 0 writes again
        U128 acc = {0u, 0u};
        bool mr = false;
#pragma unroll 1
        for (int vi = tid; vi < nvec; vi += kT) {
          const u32x4 rv = load16(xr + (int64_t)vi * 16);
#pragma unroll
          for (int e = 0; e < V; ++e) term(mag_bits<In>(rv, e), c, acc, mr);
        }
        const U128 bc = block_sum(acc, mr, more);
#pragma unroll
        for (int j = NB::kMaxChunks; j > 0; --j) wide[j] = wide[j - 1];
        wide[0] = bc.lo;
        uint64_t carry = bc.hi;
#pragma unroll
        for (int j = 1; j <= NB::kMaxChunks; ++j) {
          const uint64_t t = wide[j] + carry;
          carry = t < carry ? 1u : 0u;
          wide[j] = t;
        }
        ++nchunks;
      }
      ss = wide_to_f64<NB::kMaxChunks + 1>(wide, 2 * (emax - NB::kOff) - 64 * nchunks);
    }

    // 3. 1/rms, binary64 chain, one IEEE operation at a time
    float inv = 0.f;
    const double v = ss / kd + epsd;
    if (v > 0.0) {
      const double r = sqrt(v);
      const float i32 = (float)(1.0 / r);
      inv = i32 <= 3.4028234663852886e38f ? i32 : 0.f;
    }

    // 4. a = (x * inv) * g and the row maximum of |a| (a is formed again for the codes)
    auto act = [&](int c, float* a) {
      In::unpack(raw[c], a);
#pragma unroll
      for (int e = 0; e < V; ++e) a[e] = (a[e] * inv) * g[c][e];
    };
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      float a[V];
      act(c, a);
#pragma unroll
      for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(a[e]));
    }
    amax = wave_max(amax);
    if (lane == 0) red_a[wid] = amax;
    lds_barrier();
#pragma unroll
    for (int w = 0; w < kW; ++w) amax = fmaxf(amax, red_a[w]);

    // 5. per-token scale and int8 codes (Markstein quotients inside the checked range)
    const float dsc = amax / (float)kQMax;
    const bool fast = dsc >= kFastDMin && amax <= kFastAMax;
    const float rd = dsc > 0.f ? 1.0f / dsc : 0.f;
    if (tid == 0) x_scale[row] = dsc;
    int8_t* qr = xq + row * k;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int vi = tid + kT * c;
      if (vi >= nvec) continue;
      float a[V];
      act(c, a);
      uint32_t code[V];
#pragma unroll
      for (int e = 0; e < V; ++e) {
        float qv = 0.f;
        if (dsc > 0.f) qv = fast ? div_mk(a[e], dsc, rd) : a[e] / dsc;
        code[e] = q_code(qv);
      }
      if constexpr (V == 8) {
        *reinterpret_cast<uint2*>(qr + (int64_t)vi * V) =
            make_uint2(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]));
      } else {
        *reinterpret_cast<uint32_t*>(qr + (int64_t)vi * V) = pack4(code[0], code[1], code[2], code[3]);
      }
    }
  }
}

// g_j = RN32(gamma_j / s_j), IEEE division (gamma_j itself without s).
template <class In>
__global__ __launch_bounds__(256) void fold_gain_kernel(const uint8_t* __restrict__ gamma,
                                                        const float* __restrict__ smooth, int64_t k,
                                                        float* __restrict__ out) {
  for (int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x; j < k; j += (int64_t)gridDim.x * 256) {
    const float gv = In::load1(gamma + j * In::kBytes);
    out[j] = smooth ? gv / smooth[j] : gv;
  }
}

}  // namespace sqk

namespace sqh {

template <class In, int kCh, int kT>
static void launch_norm(const uint8_t* xb, int64_t m, int64_t nvec, int64_t ldb, const float* gain, float eps,
                        int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero, int nzero) {
  int64_t grid = m;
  if (m >= 1024) {
    const int64_t cap = (kT == 256 && kCh <= 4) ? 1024 : 512;
    grid = m < cap ? m : cap;
  }
  hipLaunchKernelGGL((sqk::rmsnorm_quant_kernel<In, kCh, kT>), dim3((unsigned)grid), dim3(kT), 0, s, xb, m,
                     (int)nvec, ldb, gain, eps, xq, x_scale, zero, nzero);
}

template <class In>
static void launch_norm_t(const void* x, int64_t m, int64_t k, int64_t ldx, const float* gain, float eps, int8_t* xq,
                          float* x_scale, hipStream_t s, uint32_t* zero, int nzero) {
  const int64_t nvec = k / In::kVec;
  const int64_t ldb = ldx * In::kBytes;
  const uint8_t* xb = (const uint8_t*)x;
  // decode-sized inputs: 1024 threads, so that one row's work spreads over a whole CU
  if ((m < 1024 && nvec > 256) || nvec > 2048) {
    if (nvec <= 1024)
      launch_norm<In, 1, 1024>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
    else if (nvec <= 2048)
      launch_norm<In, 2, 1024>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
    else if (nvec <= 4096)
      launch_norm<In, 4, 1024>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
    else
      launch_norm<In, 8, 1024>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
    return;
  }
  const int64_t per_thread = (nvec + 255) / 256;
  if (per_thread <= 1)
    launch_norm<In, 1, 256>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
  else if (per_thread <= 2)
    launch_norm<In, 2, 256>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
  else if (per_thread <= 4)
    launch_norm<In, 4, 256>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
  else
    launch_norm<In, 8, 256>(xb, m, nvec, ldb, gain, eps, xq, x_scale, s, zero, nzero);
}

hipError_t rmsnorm_quant(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* gain, float eps,
                         int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero, int64_t nzero) {
  if (m <= 0) return nzero > 0 ? fill_u32(zero, 0u, nzero, s) : hipSuccess;
  if (!zero) nzero = 0;
  switch (xt) {
    case SQ_F32: launch_norm_t<sqk::F32In>(x, m, k, ldx, gain, eps, xq, x_scale, s, zero, (int)nzero); break;
    case SQ_BF16: launch_norm_t<sqk::BF16In>(x, m, k, ldx, gain, eps, xq, x_scale, s, zero, (int)nzero); break;
    default: launch_norm_t<sqk::F16In>(x, m, k, ldx, gain, eps, xq, x_scale, s, zero, (int)nzero); break;
  }
  return hipGetLastError();
}

hipError_t fold_norm_gain(const void* gamma, sq_dtype gt, const float* smooth, int64_t k, float* out,
                          hipStream_t s) {
  if (k <= 0) return hipSuccess;
  const int64_t blocks = (k + 255) / 256;
  const unsigned grid = (unsigned)(blocks < 1024 ? blocks : 1024);
  const uint8_t* gb = (const uint8_t*)gamma;
  switch (gt) {
    case SQ_F32: hipLaunchKernelGGL(sqk::fold_gain_kernel<sqk::F32In>, dim3(grid), dim3(256), 0, s, gb, smooth, k, out); break;
    case SQ_BF16: hipLaunchKernelGGL(sqk::fold_gain_kernel<sqk::BF16In>, dim3(grid), dim3(256), 0, s, gb, smooth, k, out); break;
    default: hipLaunchKernelGGL(sqk::fold_gain_kernel<sqk::F16In>, dim3(grid), dim3(256), 0, s, gb, smooth, k, out); break;
  }
  return hipGetLastError();
}

}  // namespace sqh
