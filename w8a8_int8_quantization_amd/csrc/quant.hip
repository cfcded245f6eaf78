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
// Two kernels. quant_rows_kernel (the fast one, below) keeps up to eight
// 16-byte vectors of a row per thread in registers: one 256-thread workgroup
// owns a row at a time (grid-stride over rows), loads it coalesced, reduces
// the row maximum through LDS and writes its int8 values with one 4- or
// 8-byte store per vector. Longer rows use quant_rows_long_kernel, which
// reads the row a second time instead of keeping it.
// Either kernel can also clear a few words of device memory in its first
// workgroup (the split-K ticket counters of a decode GEMM launched next on
// the same stream), which saves that GEMM a launch.
#include <type_traits>

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

// Rows of any length: pass 1 finds the maximum, pass 2 re-reads and quantises.
template <class In, bool kSmooth, bool kMask>
__global__ __launch_bounds__(256) void quant_rows_long_kernel(const uint8_t* __restrict__ x, int64_t m, int64_t nvec,
                                                              int64_t ldx_bytes, const float* __restrict__ smooth,
                                                              const uint8_t* __restrict__ mask,
                                                              int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                              uint32_t* __restrict__ zero, int nzero) {
  constexpr int V = In::kVec;
  __shared__ float red[4];
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0u;
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


// ---------------------------------------------------------------------------
// Fast row kernel. Correctly rounded binary32 division costs about eleven VALU
// instructions on gfx950 (v_div_scale / v_rcp / FMA refinement / v_div_fmas /
// v_div_fixup), which made a straightforward kernel ALU-bound at ~20% of HBM
// bandwidth. Every quotient here uses Markstein's FMA correction instead:
// with r = RN(1/b),
//     q0 = a*r,  e = fma(-q0, b, a) (exact),  q = fma(e, r, q0),
// gives q = RN(a/b) whenever no step leaves the normal range. The divisors are
// the s_j and the row scale d. Each thread forms r_j = RN(1/s_j) for its own
// columns once and keeps s_j and r_j in registers for every row it visits:
// r_j is v_rcp_f32(s_j) refined by one FMA Newton step, e = fma(-s, y, 1),
// r = fma(e, y, y), which equals the IEEE reciprocal for every s_j in
// [2^-20, 2^21) (checked exhaustively on MI355X: all 2^23 significands of each
// of the 41 binades, zero mismatches). RN(1/d) is one IEEE division per row.
// Range argument for the fast path of a whole row: all s_j in [2^-20, 2^20],
// d >= 2^-30 and max|x/s| <= 2^50. Then any |x| < 2^-60 (where the remainder
// could underflow) gives |x/s| < 2^-40 and a quantised value of 0 under either
// division; every other operand stays well inside the normal range. A row
// outside these bounds is redone with IEEE division, and a launch whose s_j
// leave the bounds uses IEEE division throughout.
// Layout: a kT-thread workgroup walks a grid-stride list of rows; thread t
// owns the 16-byte vectors t, t+kT, ... of every row (coalesced loads,
// 8- or 4-byte coalesced stores), prefetches its vectors of the next row
// while working on the current one (short rows), and the row maximum is a
// wave reduction plus one barrier on double-buffered LDS partials. Prefill
// shapes use 256 threads and many rows per CU; decode shapes (one row per
// workgroup, the row's VALU work on a single CU) use 1024 threads for long
// rows so that four waves per SIMD overlap their dependent chains.
template <class In, int kCh, int kR, bool kSmooth, bool kMask, bool kMk, int kT>
__global__ __launch_bounds__(kT) void quant_rows_kernel(const uint8_t* __restrict__ x, int64_t m, int nvec,
                                                         int64_t ldx_bytes, const float* __restrict__ smooth,
                                                         const uint8_t* __restrict__ mask, int8_t* __restrict__ xq,
                                                         float* __restrict__ x_scale, uint32_t* __restrict__ zero,
                                                         int nzero) {
  constexpr int V = In::kVec;
  constexpr bool kSmall = kCh * kR <= 8 && kCh <= 4;  // keep x/s between passes and prefetch the next rows
  constexpr int kW = kT / 64;                          // waves per workgroup
  __shared__ float red[2][kR][kW];
  __shared__ int any_bad[kW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t k = (int64_t)nvec * V;
  const int64_t ngroups = (m + kR - 1) / kR;

  auto load_rows = [&](int64_t g, u32x4 (*raw)[kCh]) {
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int64_t row = g * kR + j;
      if (row >= m) continue;
      const uint8_t* xr = x + row * ldx_bytes;
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        const int vi = tid + kT * c;
        if (vi < nvec) raw[j][c] = load16(xr + (int64_t)vi * 16);
      }
    }
  };
  // the first rows' loads go out before the reciprocals are formed
  u32x4 raw[kR][kCh];
  u32x4 nxt[kSmall ? kR : 1][kCh];
  int64_t g = blockIdx.x;
  if (kSmall && g < ngroups) load_rows(g, nxt);
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += kT) zero[i] = 0u;

  float sreg[kSmooth ? kCh : 1][V];
  float rreg[(kSmooth && kMk) ? kCh : 1][V];
  uint32_t mreg[kMask ? kCh : 1][2];
  int bad = 0;
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    const int vi = tid + kT * c;
    if (vi >= nvec) continue;
    if (kSmooth) {
#pragma unroll
      for (int e = 0; e < V; e += 4) {
        const u32x4 sv = load16(smooth + (int64_t)vi * V + e);
        sreg[c][e] = __uint_as_float(sv.x); sreg[c][e + 1] = __uint_as_float(sv.y);
        sreg[c][e + 2] = __uint_as_float(sv.z); sreg[c][e + 3] = __uint_as_float(sv.w);
      }
      if (kMk) {
#pragma unroll
        for (int e = 0; e < V; ++e) {
          rreg[c][e] = rcp_rn(sreg[c][e]);  // used only when every s_j is in the fast range
          bad |= !(sreg[c][e] >= kFastSMin && sreg[c][e] <= kFastSMax);
        }
      }
    }
    if (kMask) {
      const uint8_t* mp = mask + (int64_t)vi * V;
      uint32_t w0 = 0, w1 = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) w0 |= (uint32_t)(mp[e] != 0) << (8 * e);
#pragma unroll
      for (int e = 4; e < V; ++e) w1 |= (uint32_t)(mp[e] != 0) << (8 * (e - 4));
      mreg[c][0] = w0; mreg[c][1] = w1;
    }
  }
  bool s_ok = kMk;
  if (kMk && kSmooth) {
    // workgroup-wide "some s_j outside the fast range", without draining the prefetch
    const int wbad = __any(bad);
    if (lane == 0) any_bad[wid] = wbad;
    lds_barrier();
    int anyb = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) anyb |= any_bad[w];
    s_ok = !anyb;
  }

  auto smoothed = [&](const u32x4& rv, int c, float* f, bool fast) {
    In::unpack(rv, f);
    if (kSmooth) {
      if (kMk && fast) {
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = div_mk(f[e], sreg[c][e], rreg[kMk ? c : 0][e]);
      } else {
#pragma unroll
        for (int e = 0; e < V; ++e) f[e] = f[e] / sreg[c][e];
      }
    }
    if (kMask) {
#pragma unroll
      for (int e = 0; e < V; ++e)
        if ((mreg[c][e >> 2] >> (8 * (e & 3))) & 0xFFu) f[e] = 0.f;
    }
  };
  int parity = 0;
  // maximum over the workgroup of each of the kR per-row values
  auto block_amax = [&](float* v) {
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      v[j] = wave_max(v[j]);
      if (lane == 0) red[parity][j][wid] = v[j];
    }
    lds_barrier();  // keeps the next rows' prefetched loads in flight
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      float r = red[parity][j][0];
#pragma unroll
      for (int w = 1; w < kW; ++w) r = fmaxf(r, red[parity][j][w]);
      v[j] = r;
    }
    parity ^= 1;
  };
  auto pass1 = [&](float* amax, float (*keep)[kCh][V], bool fast) {
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      amax[j] = 0.f;
#pragma unroll
      for (int c = 0; c < kCh; ++c) {
        if (tid + kT * c < nvec) {
          float f[V];
          smoothed(raw[j][c], c, f, fast);
#pragma unroll
          for (int e = 0; e < V; ++e) {
            amax[j] = fmaxf(amax[j], fabsf(f[e]));
            if (kSmall) keep[kSmall ? j : 0][c][e] = f[e];
          }
        }
      }
    }
    block_amax(amax);
  };

  for (; g < ngroups; g += gridDim.x) {
    if (kSmall) {
#pragma unroll
      for (int j = 0; j < kR; ++j)
#pragma unroll
        for (int c = 0; c < kCh; ++c) raw[j][c] = nxt[kSmall ? j : 0][c];
      if (g + gridDim.x < ngroups) load_rows(g + gridDim.x, nxt);
    } else {
      load_rows(g, raw);
    }
    float keep[kSmall ? kR : 1][kCh][V];
    float amax[kR];
    if (s_ok)
      pass1(amax, keep, true);
    else
      pass1(amax, keep, false);
    float d[kR];
    bool all_fast = s_ok;
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      d[j] = amax[j] / (float)kQMax;
      all_fast = all_fast && d[j] >= kFastDMin && amax[j] <= kFastAMax;
    }
    // a row outside the fast bounds (g*kR+j >= m rows are zero, also "slow"
    // only through d == 0, which needs no quotient) sends the group to IEEE division
    bool fast = all_fast;
    if (s_ok && !all_fast) {
      fast = true;
#pragma unroll
      for (int j = 0; j < kR; ++j)
        if (g * kR + j < m && !(d[j] >= kFastDMin && amax[j] <= kFastAMax)) fast = false;
      if (!fast && kSmooth) {
        pass1(amax, keep, false);
#pragma unroll
        for (int j = 0; j < kR; ++j) d[j] = amax[j] / (float)kQMax;
      }
    }
    // The row scale and the fast flag are uniform: one branch per row picks
    // the quotient, instead of one per element.
    const bool fast_u = __builtin_amdgcn_readfirstlane((int)fast) != 0;
#pragma unroll
    for (int j = 0; j < kR; ++j) {
      const int64_t row = g * kR + j;
      if (row >= m) continue;
      const float dj = __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(d[j])));
      if (tid == 0) x_scale[row] = dj;
      const float rd = (kMk && dj > 0.f) ? rcp_scale(dj) : 0.f;
      int8_t* qr = xq + row * k;
      auto emit = [&](auto fast_c, auto quot) {
        constexpr bool kF = decltype(fast_c)::value;
#pragma unroll
        for (int c = 0; c < kCh; ++c) {
          const int vi = tid + kT * c;
          if (vi >= nvec) continue;
          float f[V];
          if (kSmall) {
#pragma unroll
            for (int e = 0; e < V; ++e) f[e] = keep[kSmall ? j : 0][c][e];
          } else {
            smoothed(raw[j][c], c, f, kF);
          }
          uint32_t code[V];
#pragma unroll
          for (int e = 0; e < V; ++e) code[e] = q_code(quot(f[e]));
          if constexpr (V == 8) {
            *reinterpret_cast<uint2*>(qr + (int64_t)vi * V) =
                make_uint2(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]));
          } else {
            *reinterpret_cast<uint32_t*>(qr + (int64_t)vi * V) = pack4(code[0], code[1], code[2], code[3]);
          }
        }
      };
      if (kMk && fast_u && dj > 0.f)
        emit(std::true_type{}, [&](float v) { return div_mk(v, dj, rd); });
      else if (dj > 0.f)
        emit(std::false_type{}, [&](float v) { return v / dj; });
      else
        emit(std::false_type{}, [](float) { return 0.f; });
    }
  }
}

// ---------------------------------------------------------------------------
// Rows that fill the workgroup exactly (kCh 16-byte vectors per thread, no
// outlier mask): the prefill shapes' rows. The same arithmetic as
// quant_rows_kernel, in fewer instructions per element:
//  * the row loop is unrolled twice, so the current row and the prefetched
//    next one live in fixed registers (no copies between rows);
//  * every load is unconditional (the last row of a workgroup prefetches
//    itself again), so the compiler's wait counts are exact;
//  * the row scale d = RN(amax / 127) is Markstein's quotient with the
//    constant RN(1/127) (exact in the checked range, like every other
//    quotient here) instead of an IEEE division.
// Rows outside the fast range take the IEEE path of quant_rows_kernel.
constexpr float kRcp127 = 0x1.020408p-7f;  // RN(1/127)

template <class In, int kCh, int kT, bool kSmooth>
__global__ __launch_bounds__(kT) void quant_rows_full_kernel(const uint8_t* __restrict__ x, int64_t m,
                                                              int64_t ldx_bytes, const float* __restrict__ smooth,
                                                              int8_t* __restrict__ xq, float* __restrict__ x_scale,
                                                              uint32_t* __restrict__ zero, int nzero) {
  constexpr int kW = kT / 64;
  constexpr int V = In::kVec;
  constexpr int64_t k = (int64_t)kCh * kT * V;
  __shared__ float red[2][kW];
  __shared__ int any_bad[kW];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t grid = gridDim.x;

  auto load_row = [&](int64_t r, u32x4* raw) {
    const uint8_t* xr = x + r * ldx_bytes;
#pragma unroll
    for (int c = 0; c < kCh; ++c) raw[c] = load16(xr + (int64_t)(tid + kT * c) * 16);
  };
  u32x4 buf_a[kCh], buf_b[kCh];
  load_row(blockIdx.x, buf_a);  // grid <= m
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += kT) zero[i] = 0u;

  float sreg[kSmooth ? kCh : 1][V];
  float rreg[kSmooth ? kCh : 1][V];
  bool s_ok = true;
  if constexpr (kSmooth) {
    int bad = 0;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
#pragma unroll
      for (int e = 0; e < V; e += 4) {
        const u32x4 sv = load16(smooth + (int64_t)(tid + kT * c) * V + e);
        sreg[c][e] = __uint_as_float(sv.x); sreg[c][e + 1] = __uint_as_float(sv.y);
        sreg[c][e + 2] = __uint_as_float(sv.z); sreg[c][e + 3] = __uint_as_float(sv.w);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        rreg[c][e] = rcp_rn(sreg[c][e]);  // used only when every s_j is in the fast range
        bad |= !(sreg[c][e] >= kFastSMin && sreg[c][e] <= kFastSMax);
      }
    }
    const int wbad = __any(bad);
    if (lane == 0) any_bad[wid] = wbad;
    lds_barrier();
    int anyb = 0;
#pragma unroll
    for (int w = 0; w < kW; ++w) anyb |= any_bad[w];
    s_ok = !anyb;
  }
  const bool s_ok_u = __builtin_amdgcn_readfirstlane((int)s_ok) != 0;

  int parity = 0;
  auto block_amax = [&](float v) {
    v = wave_max(v);
    if (lane == 0) red[parity][wid] = v;
    lds_barrier();
    float r = red[parity][0];
#pragma unroll
    for (int w = 1; w < kW; ++w) r = fmaxf(r, red[parity][w]);
    parity ^= 1;
    return r;
  };
  // x / s of the row held in raw: Markstein quotients (fast) or IEEE division
  auto smooth_row = [&](const u32x4* raw, float (*f)[V], bool fast) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      In::unpack(raw[c], f[c]);
      if constexpr (kSmooth) {
        if (fast) {
#pragma unroll
          for (int e = 0; e < V; ++e) f[c][e] = div_mk(f[c][e], sreg[c][e], rreg[c][e]);
        } else {
#pragma unroll
          for (int e = 0; e < V; ++e) f[c][e] = f[c][e] / sreg[c][e];
        }
      }
#pragma unroll
      for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(f[c][e]));
    }
    return amax;
  };
  auto emit = [&](int8_t* qr, const float (*f)[V], auto quot) {
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      uint32_t code[V];
#pragma unroll
      for (int e = 0; e < V; ++e) code[e] = q_code(quot(f[c][e]));
      int8_t* dst = qr + (int64_t)(tid + kT * c) * V;
      if constexpr (V == 8)
        *reinterpret_cast<uint2*>(dst) =
            make_uint2(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]));
      else
        *reinterpret_cast<uint32_t*>(dst) = pack4(code[0], code[1], code[2], code[3]);
    }
  };
  auto body = [&](const u32x4* cur, u32x4* nxt, int64_t row) {
    load_row(row + grid < m ? row + grid : row, nxt);
    float f[kCh][V];
    float amax = block_amax(smooth_row(cur, f, s_ok_u));
    float d = div_mk(amax, (float)kQMax, kRcp127);
    const bool fast = s_ok_u && d >= kFastDMin && amax <= kFastAMax;
    int8_t* qr = xq + row * k;
    if (fast) {
      const float rd = rcp_scale(d);
      emit(qr, f, [&](float v) { return div_mk(v, d, rd); });
    } else {
      // the whole row again with IEEE quotients (the Markstein ones may be
      // inexact outside the checked range)
      if (s_ok_u && kSmooth) amax = block_amax(smooth_row(cur, f, false));
      d = amax / (float)kQMax;
      if (d > 0.f)
        emit(qr, f, [&](float v) { return v / d; });
      else
        emit(qr, f, [](float) { return 0.f; });
    }
    if (tid == 0) x_scale[row] = d;
  };
  for (int64_t row = blockIdx.x;;) {
    body(buf_a, buf_b, row);
    row += grid;
    if (row >= m) break;
    body(buf_b, buf_a, row);
    row += grid;
    if (row >= m) break;
  }
}

}  // namespace sqk

namespace sqh {

template <class In, int kCh, int kT, bool kSmooth, bool kMask>
static void launch_rows(const uint8_t* xb, int64_t m, int64_t nvec, int64_t ldb, const float* smooth,
                        const uint8_t* mask, int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero, int nzero) {
  // Measured on MI355X: one row per iteration with ~4 resident workgroups per
  // CU beats fewer workgroups with more rows each (the per-row work is about
  // one wave per SIMD, so latency hiding wins); below 1024 rows every row gets
  // its own workgroup.
  int64_t grid = m;
  if (m >= 1024) {
    const int64_t cap = (kT == 256 && kCh <= 4) ? 1024 : 512;
    grid = m < cap ? m : cap;
  }
  hipLaunchKernelGGL((sqk::quant_rows_kernel<In, kCh, 1, kSmooth, kMask, true, kT>), dim3((unsigned)grid), dim3(kT),
                     0, s, xb, m, (int)nvec, ldb, smooth, mask, xq, x_scale, zero, nzero);
}

template <class In, bool kSmooth, bool kMask>
static void launch_quant(const void* x, int64_t m, int64_t k, int64_t ldx, const float* smooth, const uint8_t* mask,
                         int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero, int nzero) {
  const int64_t nvec = k / In::kVec;
  const int64_t ldb = ldx * In::kBytes;
  const uint8_t* xb = (const uint8_t*)x;
  // Prefill rows of 1792 vectors (14336 bf16 or fp16 values): 448 threads of
  // 4 vectors, full rows (8192 x 14336 bf16: 74.7 us back to back, against
  // 84.3 us for 1024 threads of 2 vectors with an eighth of them idle)
  if (!kMask && m >= 1024 && nvec == 1792) {
    const int64_t grid = m < 512 ? m : 512;
    hipLaunchKernelGGL((sqk::quant_rows_full_kernel<In, 4, 448, kSmooth>), dim3((unsigned)grid), dim3(448), 0, s, xb,
                       m, ldb, smooth, xq, x_scale, zero, nzero);
    return;
  }
  // 1024 threads per row: decode-sized inputs (the row's work lands on one
  // CU), and rows too long to keep in registers at 256 threads
  if (nvec <= 2048 && ((m < 1024 && nvec > 256) || nvec > 1024)) {
    if (nvec <= 1024)
      launch_rows<In, 1, 1024, kSmooth, kMask>(xb, m, nvec, ldb, smooth, mask, xq, x_scale, s, zero, nzero);
    else
      launch_rows<In, 2, 1024, kSmooth, kMask>(xb, m, nvec, ldb, smooth, mask, xq, x_scale, s, zero, nzero);
    return;
  }
  const int64_t per_thread = (nvec + 255) / 256;
  // Rows of exactly 1, 2 or 4 vectors per thread: the full-row kernel. Grids
  // measured back to back (bf16, smoothing): 2048 x 4096 6.79 us at 1024
  // workgroups, 6.27 at 768; 8192 x 4096 18.5 / 18.4 us.
  if (!kMask && nvec == per_thread * 256 && (per_thread == 1 || per_thread == 2 || per_thread == 4)) {
    const int64_t cap = per_thread == 2 ? 768 : 1024;
    const int64_t grid = m < cap ? m : cap;
    if (per_thread == 1)
      hipLaunchKernelGGL((sqk::quant_rows_full_kernel<In, 1, 256, kSmooth>), dim3((unsigned)grid), dim3(256), 0, s, xb, m,
                         ldb, smooth, xq, x_scale, zero, nzero);
    else if (per_thread == 2)
      hipLaunchKernelGGL((sqk::quant_rows_full_kernel<In, 2, 256, kSmooth>), dim3((unsigned)grid), dim3(256), 0, s, xb, m,
                         ldb, smooth, xq, x_scale, zero, nzero);
    else
      hipLaunchKernelGGL((sqk::quant_rows_full_kernel<In, 4, 256, kSmooth>), dim3((unsigned)grid), dim3(256), 0, s, xb, m,
                         ldb, smooth, xq, x_scale, zero, nzero);
    return;
  }
  if (per_thread <= 1)
    launch_rows<In, 1, 256, kSmooth, kMask>(xb, m, nvec, ldb, smooth, mask, xq, x_scale, s, zero, nzero);
  else if (per_thread <= 2)
    launch_rows<In, 2, 256, kSmooth, kMask>(xb, m, nvec, ldb, smooth, mask, xq, x_scale, s, zero, nzero);
  else if (per_thread <= 4)
    launch_rows<In, 4, 256, kSmooth, kMask>(xb, m, nvec, ldb, smooth, mask, xq, x_scale, s, zero, nzero);
  else if (per_thread <= 8)
    launch_rows<In, 8, 256, kSmooth, kMask>(xb, m, nvec, ldb, smooth, mask, xq, x_scale, s, zero, nzero);
  else
    hipLaunchKernelGGL((sqk::quant_rows_long_kernel<In, kSmooth, kMask>), dim3((unsigned)(m < 4096 ? m : 4096)),
                       dim3(256), 0, s, xb, m, nvec, ldb, smooth, mask, xq, x_scale, zero, nzero);
}

template <class In>
static void launch_quant_t(const void* x, int64_t m, int64_t k, int64_t ldx, const float* smooth, const uint8_t* mask,
                           int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero, int nzero) {
  if (mask)
    launch_quant<In, false, true>(x, m, k, ldx, nullptr, mask, xq, x_scale, s, zero, nzero);
  else if (smooth)
    launch_quant<In, true, false>(x, m, k, ldx, smooth, nullptr, xq, x_scale, s, zero, nzero);
  else
    launch_quant<In, false, false>(x, m, k, ldx, nullptr, nullptr, xq, x_scale, s, zero, nzero);
}

hipError_t quant_rows(const void* x, sq_dtype xt, int64_t m, int64_t k, int64_t ldx, const float* smooth,
                      const uint8_t* mask, int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero,
                      int64_t nzero) {
  if (m <= 0) return nzero > 0 ? fill_u32(zero, 0u, nzero, s) : hipSuccess;
  if (!zero) nzero = 0;
  switch (xt) {
    case SQ_F32: launch_quant_t<sqk::F32In>(x, m, k, ldx, smooth, mask, xq, x_scale, s, zero, (int)nzero); break;
    case SQ_BF16: launch_quant_t<sqk::BF16In>(x, m, k, ldx, smooth, mask, xq, x_scale, s, zero, (int)nzero); break;
    default: launch_quant_t<sqk::F16In>(x, m, k, ldx, smooth, mask, xq, x_scale, s, zero, (int)nzero); break;
  }
  return hipGetLastError();
}

}  // namespace sqh
