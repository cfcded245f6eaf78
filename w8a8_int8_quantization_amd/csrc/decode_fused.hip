// One-launch decode step for a single token: per-token quantisation fused
// into the weight-streaming int8 GEMM.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization": "How the Model Was Compressed" and "Why Activation
// Quantization Is Hard" (one scale per token, max|x/s| / 127, round to
// nearest); "Performance After Quantization", Inter-Token Latency (per decoded
// token the weights are read once and the quantisation is per-token overhead:
// here it costs no launch of its own). The LLM.int8() page, "The
// architecture: every piece explained" (int32 accumulation, dequantisation by
// the row scale times the column scale).
//
// Layout on gfx950: a 256-thread workgroup owns 64 rows of Wq (output
// columns) and the whole of K; its 4 waves take the 128-byte k-steps round-
// robin (wave w: steps w, w+4, ...), with up to kDepth steps of loads in
// flight (straight into registers in the v_mfma_i32_16x16x64_i8 A layout, as
// in the decode GEMM). Before its first MFMA every workgroup reads the token's
// row of X and the smoothing factors (L2-resident after the first workgroup),
// forms the row scale exactly as the quantisation kernel does (the same
// Markstein quotients, fast-range rule and IEEE fallback), and writes the
// row's int8 codes to LDS; the MFMA B operand then comes from LDS, the token's
// codes in lanes 0-15 of column 0 and zeros elsewhere. The x and s loads go
// out before the Wq loads, so waiting for them never waits for weights. The
// 4 waves' int32 tiles are summed through LDS. There is no split over K, so
// no workspace and no counters: the results are those of the two-launch path
// bit for bit. Without a split the grid has one workgroup per 64 output
// columns, so the path is taken for layers at least 192 x 64 wide (the
// up-projection shape, 224 workgroups); narrower layers keep the split-K
// decode GEMM after the quantisation launch, which measured faster there
// (14336 -> 4096 at one token: 19.0 us in two launches, 20.2 us fused with
// 16-column workgroups over all of K).
#include <type_traits>

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

struct Decode1Args {
  const uint8_t* x;     // the token's row (K values of the input type)
  const float* smooth;  // [K] or null
  const int8_t* wq;     // [N][K]
  const float* w_scale; // [N]
  void* y;              // [N] outputs of type out
  int N, K;
  int out;              // 0 f32, 1 bf16, 2 f16
};

constexpr int kD1MaxC = 8;  // 16-byte input vectors per thread: K <= 2048 x (values per vector)

template <class In, int kC, bool kSmooth>
__global__ __launch_bounds__(256, 1) void gemm_decode1_kernel(Decode1Args a) {
  constexpr int V = In::kVec;
  constexpr int kG = 4;                        // 16-row groups of Wq
  constexpr int kRowsT = 16 * kG;              // Wq rows (outputs) of the workgroup
  // steps of Wq loads in flight per wave: as many as the registers hold next
  // to the row's values (K up to 4096 bf16: all 8 steps of a wave)
  constexpr int kDepth = kC <= 2 ? 8 : 4;
  constexpr int kMaxK = 256 * kC * V;
  __shared__ __attribute__((aligned(16))) int8_t codes[kMaxK + 64];
  __shared__ int32_t red[4][kRowsT];
  __shared__ float red_f[4];
  __shared__ int red_i[4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n0 = (int)blockIdx.x * kRowsT;
  const int K = a.K;
  const int nvec = K / V;
  const int nsteps = K / 128;

  // ---- the token's row and the smoothing factors (issued first)
  u32x4 xr[kC];
  float sv[kSmooth ? kC : 1][V];
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int vi = tid + 256 * c;
    if (vi < nvec) {
      xr[c] = load16(a.x + (int64_t)vi * 16);
      if (kSmooth) {
#pragma unroll
        for (int e = 0; e < V; e += 4) {
          const u32x4 s4 = load16(a.smooth + (int64_t)vi * V + e);
          sv[c][e] = __uint_as_float(s4.x); sv[c][e + 1] = __uint_as_float(s4.y);
          sv[c][e + 2] = __uint_as_float(s4.z); sv[c][e + 3] = __uint_as_float(s4.w);
        }
      }
    }
  }

  // ---- Wq: the first kDepth steps of this wave
  const int kb = 16 * (lane >> 4);
  const int8_t* wp[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) wp[g] = a.wq + (int64_t)min(n0 + 16 * g + (lane & 15), a.N - 1) * K + kb;
  u32x4 wb[kDepth][kG][2];
  auto load = [&](int i, int slot) {
    const int64_t off = (int64_t)min(wid + 4 * i, nsteps - 1) * 128;
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      wb[slot][g][0] = load16(wp[g] + off);
      wb[slot][g][1] = load16(wp[g] + off + 64);
    }
  };
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load(i, i);

  // ---- row scale: d = fl32(max_j |fl32(x_j / s_j)| / 127), the quantiser's arithmetic
  float xh[kC][V];
  int bad = 0;
  if (kSmooth) {
#pragma unroll
    for (int c = 0; c < kC; ++c)
#pragma unroll
      for (int e = 0; e < V; ++e) bad |= !(sv[c][e] >= kFastSMin && sv[c][e] <= kFastSMax);
  }
  const int wbad = __any(bad);
  if (lane == 0) red_i[wid] = wbad;
  auto smooth_pass = [&](bool fast) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if (tid + 256 * c >= nvec) continue;
      In::unpack(xr[c], xh[c]);
      if (kSmooth) {
#pragma unroll
        for (int e = 0; e < V; ++e)
          xh[c][e] = fast ? div_mk(xh[c][e], sv[c][e], rcp_rn(sv[c][e])) : xh[c][e] / sv[c][e];
      }
#pragma unroll
      for (int e = 0; e < V; ++e) amax = fmaxf(amax, fabsf(xh[c][e]));
    }
    return amax;
  };
  lds_barrier();
  const bool s_ok = !(red_i[0] | red_i[1] | red_i[2] | red_i[3]);
  auto block_max = [&](float v) {
    v = wave_max(v);
    lds_barrier();  // the previous readers of red_f are done
    if (lane == 0) red_f[wid] = v;
    lds_barrier();
    return fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
  };
  float amax = block_max(s_ok ? smooth_pass(true) : smooth_pass(false));
  float d = amax / (float)kQMax;
  const bool fast = s_ok && d >= kFastDMin && amax <= kFastAMax;
  if (kSmooth && s_ok && !fast && d > 0.f) {
    amax = block_max(smooth_pass(false));
    d = amax / (float)kQMax;
  }

  // ---- the row's codes into LDS (then 64 zero bytes: the other 15 token columns)
  const float rd = (fast && d > 0.f) ? rcp_scale(d) : 0.f;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int vi = tid + 256 * c;
    if (vi >= nvec) continue;
    uint32_t code[V];
#pragma unroll
    for (int e = 0; e < V; ++e)
      code[e] = d > 0.f ? q_code(fast ? div_mk(xh[c][e], d, rd) : xh[c][e] / d) : 0u;
    if constexpr (V == 8) {
      *reinterpret_cast<uint2*>(&codes[vi * 8]) =
          make_uint2(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]));
    } else {
      *reinterpret_cast<uint32_t*>(&codes[vi * 4]) = pack4(code[0], code[1], code[2], code[3]);
    }
  }
  if (tid < 4) *reinterpret_cast<u32x4*>(&codes[K + 16 * tid]) = u32x4{0u, 0u, 0u, 0u};
  lds_barrier();

  // ---- the GEMM: step i of this wave is k-step wid + 4 i; the B fragment of
  // lane l is the token's 16 codes at the lane's k bytes when l % 16 == 0,
  // zeros otherwise
  const int bsel = (lane & 15) == 0 ? kb : K;  // zero bytes for the empty token columns
  v4i acc[kG];
#pragma unroll
  for (int g = 0; g < kG; ++g) acc[g] = v4i{0, 0, 0, 0};
  const int ns = (nsteps - wid + 3) / 4;  // steps of this wave
  for (int i0 = 0; i0 < ns; i0 += kDepth) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int i = i0 + u;
      u32x4 w[kG][2];
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        w[g][0] = wb[u][g][0];
        w[g][1] = wb[u][g][1];
      }
      if (i + kDepth < ns) load(i + kDepth, u);
      const int koff = (bsel == K) ? K : (wid + 4 * i) * 128 + bsel;
      const v4i x0 = *reinterpret_cast<const v4i*>(&codes[min(koff, K)]);
      const v4i x1 = *reinterpret_cast<const v4i*>(&codes[bsel == K ? K : min(koff + 64, K)]);
      const bool valid = i < ns;
#pragma unroll
      for (int g = 0; g < kG; ++g) {
        acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, w[g][0]), valid ? x0 : v4i{0, 0, 0, 0},
                                                       acc[g], 0, 0, 0);
        acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, w[g][1]), valid ? x1 : v4i{0, 0, 0, 0},
                                                       acc[g], 0, 0, 0);
      }
    }
  }

  // 16x16 result layout: lane l holds token l % 16 and rows 16 g + 4 (l / 16)
  // + r, r = 0..3; the token is column 0, lanes 0, 16, 32 and 48
  if ((lane & 15) == 0) {
#pragma unroll
    for (int g = 0; g < kG; ++g)
      *reinterpret_cast<v4i*>(&red[wid][16 * g + 4 * (lane >> 4)]) = acc[g];
  }
  __syncthreads();
  if (tid < kRowsT / 4) {
    const int nl = 4 * tid;
    const int n = n0 + nl;
    if (n < a.N) {
      int32_t s4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) s4[e] = red[0][nl + e] + red[1][nl + e] + red[2][nl + e] + red[3][nl + e];
      const int nv = min(4, a.N - n);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = e < nv ? __fmul_rn(__fmul_rn((float)s4[e], d), a.w_scale[n + e]) : 0.f;
      if (a.out == 0) {
        float* p = reinterpret_cast<float*>(a.y) + n;
        for (int e = 0; e < nv; ++e) p[e] = v[e];
      } else if (a.out == 1) {
        uint16_t* p = reinterpret_cast<uint16_t*>(a.y) + n;
        for (int e = 0; e < nv; ++e) p[e] = (uint16_t)f32_to_bf16(v[e]);
      } else {
        uint16_t* p = reinterpret_cast<uint16_t*>(a.y) + n;
        for (int e = 0; e < nv; ++e) p[e] = (uint16_t)f32_to_f16(v[e]);
      }
    }
  }
}

}  // namespace sqk

namespace sqh {

namespace {

template <class In, bool kSmooth>
void launch_d1(const sqk::Decode1Args& a, int c, hipStream_t s) {
  const dim3 grid((unsigned)((a.N + 63) / 64));
  switch (c) {
    case 1: hipLaunchKernelGGL((sqk::gemm_decode1_kernel<In, 1, kSmooth>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((sqk::gemm_decode1_kernel<In, 2, kSmooth>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((sqk::gemm_decode1_kernel<In, 4, kSmooth>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((sqk::gemm_decode1_kernel<In, 8, kSmooth>), grid, dim3(256), 0, s, a); break;
  }
}

template <class In>
hipError_t decode1(const sqk::Decode1Args& a, bool smooth, hipStream_t s) {
  const int nvec = a.K / In::kVec;
  const int per = (nvec + 255) / 256;
  const int c = per <= 1 ? 1 : per <= 2 ? 2 : per <= 4 ? 4 : 8;
  if (smooth)
    launch_d1<In, true>(a, c, s);
  else
    launch_d1<In, false>(a, c, s);
  return hipGetLastError();
}

}  // namespace

bool decode1_suits(int64_t m, int64_t n, int64_t k, sq_dtype xt) {
  if (m != 1 || n > INT32_MAX || (n + 63) / 64 < 192 || k % 128 != 0) return false;
  const int64_t per_vec = xt == SQ_F32 ? 4 : 8;
  return k <= 256 * sqk::kD1MaxC * per_vec;
}

hipError_t decode1_linear(const void* x, sq_dtype xt, const float* smooth, const int8_t* wq, const float* w_scale,
                          int64_t n, int64_t k, void* y, sq_dtype yt, hipStream_t s) {
  sqk::Decode1Args a{};
  a.x = reinterpret_cast<const uint8_t*>(x);
  a.smooth = smooth;
  a.wq = wq;
  a.w_scale = w_scale;
  a.y = y;
  a.N = (int)n;
  a.K = (int)k;
  a.out = yt == SQ_F32 ? 0 : yt == SQ_BF16 ? 1 : 2;
  switch (xt) {
    case SQ_F32: return decode1<sqk::F32In>(a, smooth != nullptr, s);
    case SQ_BF16: return decode1<sqk::BF16In>(a, smooth != nullptr, s);
    default: return decode1<sqk::F16In>(a, smooth != nullptr, s);
  }
}

}  // namespace sqh
