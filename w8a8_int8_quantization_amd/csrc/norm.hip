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
// Fast path (bf16 and fp16). With kDh = 53 - log2(max m^2) - log2(values per
// thread), rounded down to even, every square within 2^-kDh of the row's
// largest is a multiple of 2^(2 emax - 2 off - kDh) and below
// 2^(2 emax - 2 off + log2(max m^2)), so one thread's binary64 FMA sum of such
// squares is exact whatever its order. A thread converts that exact sum to
// chunk 0's 128-bit integer once per row; only squares further down (a wave
// whose smallest non-zero magnitude is below the window: rare) take the
// integer path one by one. binary32 rows have 48-bit square significands and
// always take the integer path.
//
// Layout: a kT-thread workgroup walks a grid-stride list of rows; thread t
// owns the 16-byte vectors t, t + kT, ... of every row, keeps them in
// registers through the three row reductions (largest exponent, sum of
// squares, largest |a|), and loads the next row's vectors while it works on
// the current one. The gains of its columns stay in registers for every row.
// Wave reductions use DPP row shifts and broadcasts (no LDS traffic), the
// workgroup step one LDS word per wave and one barrier.
#include <math.h>

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

// Integer significand and exponent field of the element formats. kSqBits
// bounds the significand of a square (m^2 < 2^kSqBits); kBias is the
// format's exponent bias.
template <class In>
struct NormBits;
template <>
struct NormBits<BF16In> {
  static constexpr int kManBits = 7, kOff = 134, kMaxChunks = 8, kSqBits = 16, kBias = 127;
  static constexpr uint32_t kMagMask = 0x7FFFu;
};
template <>
struct NormBits<F16In> {
  static constexpr int kManBits = 10, kOff = 25, kMaxChunks = 1, kSqBits = 22, kBias = 15;
  static constexpr uint32_t kMagMask = 0x7FFFu;
};
template <>
struct NormBits<F32In> {
  static constexpr int kManBits = 23, kOff = 150, kMaxChunks = 8, kSqBits = 48, kBias = 127;
  static constexpr uint32_t kMagMask = 0x7FFFFFFFu;
};

constexpr int ceil_log2(int v) { return v <= 1 ? 0 : 1 + ceil_log2((v + 1) / 2); }

// Element e of a 16-byte vector as raw magnitude bits (sign dropped).
template <class In>
__device__ __forceinline__ uint32_t mag_bits(const u32x4& v, int e) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (In::kVec == 8)
    return ((e & 1) ? (w[e >> 1] >> 16) : w[e >> 1]) & NormBits<In>::kMagMask;
  else
    return w[e] & NormBits<In>::kMagMask;
}

typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

struct U128 {
  uint64_t lo, hi;
};

__device__ __forceinline__ void add128(U128& a, uint64_t lo, uint64_t hi) {
  const uint64_t s = a.lo + lo;
  a.hi += hi + (s < lo ? 1u : 0u);
  a.lo = s;
}

template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ void add128_dpp(U128& a) {
  const uint32_t w0 = dpp0<kCtrl, kRowMask>((uint32_t)a.lo), w1 = dpp0<kCtrl, kRowMask>((uint32_t)(a.lo >> 32));
  const uint32_t w2 = dpp0<kCtrl, kRowMask>((uint32_t)a.hi), w3 = dpp0<kCtrl, kRowMask>((uint32_t)(a.hi >> 32));
  add128(a, ((uint64_t)w1 << 32) | w0, ((uint64_t)w3 << 32) | w2);
}

__device__ __forceinline__ U128 wave_sum128(U128 a) {
  add128_dpp<0x111>(a);
  add128_dpp<0x112>(a);
  add128_dpp<0x114>(a);
  add128_dpp<0x118>(a);
  add128_dpp<0x142, 0xA>(a);
  add128_dpp<0x143, 0xC>(a);
  const uint32_t w0 = __builtin_amdgcn_readlane((int)(uint32_t)a.lo, 63);
  const uint32_t w1 = __builtin_amdgcn_readlane((int)(uint32_t)(a.lo >> 32), 63);
  const uint32_t w2 = __builtin_amdgcn_readlane((int)(uint32_t)a.hi, 63);
  const uint32_t w3 = __builtin_amdgcn_readlane((int)(uint32_t)(a.hi >> 32), 63);
  return U128{((uint64_t)w1 << 32) | w0, ((uint64_t)w3 << 32) | w2};
}

// Maximum of the kW per-wave values in LDS (and v): unrolled for a few waves,
// one value per lane and a wave reduction for many.
template <int kW>
__device__ __forceinline__ uint32_t block_max_lds(const uint32_t* red, int lane, uint32_t v) {
  if constexpr (kW <= 4) {
#pragma unroll
    for (int w = 0; w < kW; ++w) v = red[w] > v ? red[w] : v;
    return v;
  } else {
    const uint32_t r = lane < kW ? red[lane] : 0u;
    return wave_max_u32(r > v ? r : v);
  }
}

// A non-negative binary64 that is an integer multiple of 2^unit and below
// 2^(unit + 84), as the 128-bit integer acc / 2^unit (exact).
__device__ __forceinline__ U128 f64_to_fixed(double acc, int unit) {
  if (!(acc > 0.0)) return U128{0u, 0u};
  const uint64_t bits = (uint64_t)__double_as_longlong(acc);
  const int ex = (int)((bits >> 52) & 0x7FF);
  const uint64_t mant = (bits & 0xFFFFFFFFFFFFFull) | (1ull << 52);
  const int sh = ex - 1075 - unit;  // acc = mant * 2^(sh + unit); sh in [-52, 32)
  if (sh >= 0) return U128{mant << sh, sh > 0 ? mant >> (64 - sh) : 0u};
  return U128{mant >> (-sh), 0u};
}

// Round to nearest even: the integer whose most significant non-zero 64-bit
// word is `top` (word index t), followed by the word `nxt`, with `sticky` set
// when any lower word is non-zero; the value is scaled by 2^unit.
__device__ __forceinline__ double round_top(uint64_t top, uint64_t nxt, bool sticky, int t, int unit) {
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

// Round-to-nearest-even binary64 of the integer w[0] + w[1] 2^64 + ... +
// w[n-1] 2^(64(n-1)) times 2^unit.
__device__ __forceinline__ double wide_to_f64_lds(const uint64_t* w, int n, int unit) {
  int t = n - 1;
#pragma unroll 1
  while (t >= 0 && w[t] == 0) --t;
  if (t < 0) return 0.0;
  const uint64_t top = w[t];
  const uint64_t nxt = t > 0 ? w[t - 1] : 0u;
  bool sticky = false;
#pragma unroll 1
  for (int j = t - 2; j >= 0; --j) sticky |= w[j] != 0;
  return round_top(top, nxt, sticky, t, unit);
}

// The same for two words held in registers.
__device__ __forceinline__ double u128_to_f64(U128 v, int unit) {
  if (v.hi != 0) return round_top(v.hi, v.lo, false, 1, unit);
  if (v.lo != 0) return round_top(v.lo, 0u, false, 0, unit);
  return 0.0;
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
  // Fast window of the sum of squares (bf16 and fp16): the squares within 2^-kDh
  // of the largest one, summed per thread in binary64. Every such square is a
  // multiple of 2^(2 emax - 2 off - kDh) below 2^(2 emax - 2 off + kSqBits), so
  // a thread's kCh * V of them sum exactly when kDh + kSqBits + log2(kCh V) <= 53.
  constexpr bool kF64Win = NB::kSqBits <= 22;
  constexpr int kDh = kF64Win ? ((53 - NB::kSqBits - ceil_log2(kCh * V)) & ~1) : 0;
  static_assert(!kF64Win || (kDh >= 8 && kDh <= 64), "fast window");
  __shared__ uint32_t red_e[kW];
  __shared__ uint64_t red_s[kW][2];
  __shared__ uint32_t red_more[kW];
  __shared__ uint32_t red_a[kW];
  __shared__ uint64_t wide_s[NB::kMaxChunks + 1];
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

    // 1. largest magnitude (bit patterns of non-negative values order like the
    //    values) and, for the 16-bit formats, the smallest non-zero one; two
    //    elements per packed 16-bit operation
    uint32_t mx = 0, mnz = 0xFFFFFFFFu;
    if constexpr (In::kVec == 8) {
      u16x2 pmax = {0, 0}, pmin = {0xFFFF, 0xFFFF};
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        const uint32_t w[4] = {raw[c].x, raw[c].y, raw[c].z, raw[c].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const u16x2 b = __builtin_bit_cast(u16x2, w[i] & 0x7FFF7FFFu);
          pmax = __builtin_elementwise_max(pmax, b);
          pmin = __builtin_elementwise_min(pmin, b - u16x2{1, 1});  // zero wraps to 0xFFFF
        }
      }
      mx = pmax.x > pmax.y ? pmax.x : pmax.y;
      mnz = (uint32_t)(pmin.x < pmin.y ? pmin.x : pmin.y) + 1u;  // 0x10000: no non-zero element
    } else {
#pragma unroll
      for (int c = 0; c < kCh; ++c)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          const uint32_t b = mag_bits<In>(raw[c], e);
          mx = b > mx ? b : mx;
        }
    }
    mx = wave_max_u32(mx);
    if (lane == 0) red_e[wid] = mx;
    lds_barrier();
    mx = block_max_lds<kW>(red_e, lane, mx);
    const int emax_f = (int)(mx >> NB::kManBits);
    const int emax = emax_f > 1 ? emax_f : 1;
    const int unit0 = 2 * (emax - NB::kOff) - 64;  // chunk 0's unit, 2^unit0

    // 2. exact sum of squares. Chunk 0 (squares within 2^-64 of the largest)
    //    from the registers; the rare further chunks re-read the row.
    // Integer term of chunk c0 (zero outside it); mr: the square lies below chunk c0.
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
      if constexpr (kW <= 4) {
#pragma unroll
        for (int w = 0; w < kW; ++w) {
          add128(tot, red_s[w][0], red_s[w][1]);
          anym |= red_more[w];
        }
      } else {
        // one wave's partial per lane, then the wave reduction again
        if (lane < kW) {
          tot = U128{red_s[lane][0], red_s[lane][1]};
          anym = red_more[lane];
        }
        tot = wave_sum128(tot);
        anym = wave_max_u32(anym);
      }
      more = anym != 0;
      return tot;
    };
    bool more = false;
    U128 b0;
    float fv[kCh][V];  // the row as binary32, later the activations a
#pragma unroll
    for (int c = 0; c < kCh; ++c) In::unpack(raw[c], fv[c]);
    {
      U128 acc = {0u, 0u};
      bool mr = false;
      if constexpr (kF64Win) {
        // exponent fields >= t_hi lie in the binary64 window (d < kDh)
        const int t_hi = emax - kDh / 2 + 1;
        const uint32_t thr_b = t_hi <= 1 ? 0u : (uint32_t)t_hi << NB::kManBits;
        if (!__any(mnz < thr_b)) {
          // every square of the wave is in the window: no selection needed;
          // four independent FMA chains (the sums are exact, so their
          // grouping cannot change the result)
          double s4[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
          for (int c = 0; c < kCh; ++c)
#pragma unroll
            for (int e = 0; e < V; ++e) {
              const double fd = (double)fv[c][e];
              s4[e & 3] = __builtin_fma(fd, fd, s4[e & 3]);
            }
          acc = f64_to_fixed((s4[0] + s4[1]) + (s4[2] + s4[3]), unit0);
        } else {
          // rare: squares in [2^-64, 2^-kDh) of the largest go to integer
          // terms; the row is read again (L2) rather than kept in registers
          const uint8_t* xr = x + row * ldx_bytes;
          double s64 = 0.0;
#pragma unroll
          for (int c = 0; c < kCh; ++c) {
            const int vi = tid + kT * c;
            const u32x4 rv = vi < nvec ? load16(xr + (int64_t)vi * 16) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int e = 0; e < V; ++e) {
              const uint32_t b = mag_bits<In>(rv, e);
              const bool in = b >= thr_b;
              const double fd = (double)(in ? fv[c][e] : 0.f);
              s64 = __builtin_fma(fd, fd, s64);
              if (!in) term(b, 0, acc, mr);
            }
          }
          const U128 hi = f64_to_fixed(s64, unit0);
          add128(acc, hi.lo, hi.hi);
        }
      } else {
#pragma unroll
        for (int c = 0; c < kCh; ++c)
#pragma unroll
          for (int e = 0; e < V; ++e) term(mag_bits<In>(raw[c], e), 0, acc, mr);
      }
      b0 = block_sum(acc, mr, more);
    }
    double ss;
    if (NB::kMaxChunks == 1 || !more) {
      ss = u128_to_f64(b0, unit0);
    } else {
      // squares below 2^-64 of the largest (rare): Horner over the chunks,
      // W = W * 2^64 + B_c, kept by thread 0 in LDS
      if (tid == 0) {
        wide_s[0] = b0.lo;
        wide_s[1] = b0.hi;
        for (int j = 2; j <= NB::kMaxChunks; ++j) wide_s[j] = 0u;
      }
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
        if (tid == 0) {
#pragma unroll 1
          for (int j = NB::kMaxChunks; j > 0; --j) wide_s[j] = wide_s[j - 1];
          wide_s[0] = bc.lo;
          uint64_t carry = bc.hi;
#pragma unroll 1
          for (int j = 1; j <= NB::kMaxChunks; ++j) {
            const uint64_t t = wide_s[j] + carry;
            carry = t < carry ? 1u : 0u;
            wide_s[j] = t;
          }
        }
        ++nchunks;
      }
      lds_barrier();
      ss = wide_to_f64_lds(wide_s, NB::kMaxChunks + 1, 2 * (emax - NB::kOff) - 64 * nchunks);
    }

    // 3. 1/rms, binary64 chain, one IEEE operation at a time
    float inv = 0.f;
    const double v = ss / kd + epsd;
    if (v > 0.0) {
      const double r = sqrt(v);
      const float i32 = (float)(1.0 / r);
      inv = i32 <= 3.4028234663852886e38f ? i32 : 0.f;
    }

    // 4. a = (x * inv) * g and the row maximum of |a|
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c)
#pragma unroll
      for (int e = 0; e < V; ++e) {
        fv[c][e] = (fv[c][e] * inv) * g[c][e];
        amax = fmaxf(amax, fabsf(fv[c][e]));
      }
    uint32_t abits = wave_max_u32(__float_as_uint(amax));
    if (lane == 0) red_a[wid] = abits;
    lds_barrier();
    abits = block_max_lds<kW>(red_a, lane, abits);
    amax = __uint_as_float(abits);

    // 5. per-token scale and int8 codes (Markstein quotients inside the
    //    checked range). The row maximum is uniform; one branch per row
    //    picks the quotient, not one per element.
    amax = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(amax)));
    const float dsc = amax / (float)kQMax;
    const float rd = dsc > 0.f ? rcp_scale(dsc) : 0.f;
    if (tid == 0) x_scale[row] = dsc;
    int8_t* qr = xq + row * k;
    auto emit = [&](auto quot) {
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        const int vi = tid + kT * c;
        if (vi >= nvec) continue;
        uint32_t code[V];
#pragma unroll
        for (int e = 0; e < V; ++e) code[e] = q_code(quot(fv[c][e]));
        if constexpr (V == 8) {
          *reinterpret_cast<uint2*>(qr + (int64_t)vi * V) =
              make_uint2(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]));
        } else {
          *reinterpret_cast<uint32_t*>(qr + (int64_t)vi * V) = pack4(code[0], code[1], code[2], code[3]);
        }
      }
    };
    if (dsc >= kFastDMin && amax <= kFastAMax)
      emit([&](float v) { return div_mk(v, dsc, rd); });
    else if (dsc > 0.f)
      emit([&](float v) { return v / dsc; });
    else
      emit([](float) { return 0.f; });
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
