// The gated-MLP activation feeding the down projection, h = SiLU(gate) * up,
// fused with the smoothing divide and the per-token int8 quantisation of h.
//
// "Half the Size, Better Performance, Same Accuracy: Understanding W8A8 INT8
// LLM Quantization": every linear layer's input is quantised per token at
// run time ("How the Model Was Compressed", "Why Activation Quantization Is
// Hard"), divided by the smoothing factor first ("How the smoothing factor is
// computed"), and these memory-bound steps are what costs inter-token latency
// ("Performance After Quantization", Inter-Token Latency). Here the down
// projection's input never goes to memory in floating point: the kernel reads
// the gate/up projection's bf16 outputs and writes Xq and the row scales.
//
// Per element (every step one IEEE binary32 operation, no fused multiply-add):
//   e   = exp(-g) by a fixed algorithm: k = rint(t * RN32(1/ln2)) clamped to
//         [-256, 256], r = (t - k L1) - k L2 (ln2 = L1 + L2, L1 with 16
//         significant bits), p = degree-7 Taylor polynomial of e^r in Horner
//         form with coefficients RN32(1/n!), e = ldexp(p, k); t > 100 gives
//         +inf and t < -110 gives 0
//   sig = 1 / (1 + e);  h = bf16(RN32(RN32(g * sig) * u))
//   xh  = RN32(h / s_j);  d = RN32(max |xh| / 127);  q = clamp(rne(RN32(xh / d)))
// sigma(g) = 1 / (1 + e) of every bf16 g comes from a per-workgroup LDS table
// built with exactly these steps (IEEE division), or from its exact value
// where the steps give 0.5, 0 or 1 (see sigma_of): one LDS read per element
// instead of ~30 instructions.
//
// Layout as the other row kernels: a kT-thread workgroup per row (grid-
// stride), thread t owns the 16-byte vectors t, t + kT, ... of the row in both
// inputs and keeps its columns' s_j and RN(1/s_j) in registers for every row.
#include <math.h>

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

constexpr float kLn2Hi = 0.693145751953125f;       // 16 significant bits
constexpr float kLn2Lo = 1.428606765330187e-06f;  // ln2 - kLn2Hi
constexpr float kInvLn2 = 1.4426950408889634f;

// e^t by the fixed algorithm above (exactly the oracle's steps).
__device__ __forceinline__ float exp_fixed(float t) {
  float k = __builtin_rintf(t * kInvLn2);
  k = __builtin_amdgcn_fmed3f(k, -256.0f, 256.0f);
  const float r = (t - k * kLn2Hi) - k * kLn2Lo;
  float p = (float)(1.0 / 5040.0);
  p = p * r + (float)(1.0 / 720.0);
  p = p * r + (float)(1.0 / 120.0);
  p = p * r + (float)(1.0 / 24.0);
  p = p * r + (float)(1.0 / 6.0);
  p = p * r + 0.5f;
  p = p * r + 1.0f;
  p = p * r + 1.0f;
  float e = __builtin_ldexpf(p, (int)k);
  e = t > 100.0f ? __builtin_huge_valf() : e;
  e = t < -110.0f ? 0.0f : e;
  return e;
}

// sigma(g) = 1 / (1 + e^-g) over the bf16 inputs, tabulated. A bf16 g with
// exponent field below 102 (|g| < 2^-25) has e^-g == 1 exactly in the fixed
// algorithm (k = 0, and the polynomial rounds to 1), so sigma == 0.5; with
// exponent field 134 or more (|g| >= 128), e^-g is 0 (g > 0: t < -110) or
// +inf (g < 0: t > 100), so sigma is 1 or 0. The 2 x 32 x 128 = 8192 bf16
// values in between are tabulated per workgroup in LDS (32 KiB), each entry
// computed by the same steps as the direct evaluation.
constexpr int kSigLo = 102, kSigHi = 134;  // tabulated exponent fields [kSigLo, kSigHi)
constexpr int kSigHalf = (kSigHi - kSigLo) * 128;
constexpr int kSigEntries = 2 * kSigHalf;

__device__ __forceinline__ float sigma_direct(float g) { return 1.0f / (1.0f + exp_fixed(-g)); }

template <int kCh, int kT>
__global__ __launch_bounds__(kT) void silu_quant_kernel(const uint8_t* __restrict__ gate,
                                                        const uint8_t* __restrict__ up, int64_t m, int nvec,
                                                        int64_t ldg_bytes, int64_t ldu_bytes,
                                                        const float* __restrict__ smooth, int8_t* __restrict__ xq,
                                                        float* __restrict__ x_scale, uint32_t* __restrict__ zero,
                                                        int nzero) {
  constexpr int V = 8;  // bf16 values per 16-byte vector
  constexpr int kW = kT / 64;
  __shared__ uint32_t red_a[kW];
  __shared__ int any_bad[kW];
  __shared__ float sig_tab[kSigEntries];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int64_t k = (int64_t)nvec * V;

  // sigma of a bf16 bit pattern: the table, or its exact value outside it
  auto sigma_of = [&](uint32_t b) {
    const uint32_t mag = b & 0x7FFFu;
    const uint32_t off = mag - (uint32_t)(kSigLo << 7);  // wraps for small magnitudes
    const bool neg = (b & 0x8000u) != 0;
    const bool in = off < (uint32_t)kSigHalf;
    // always an in-range read (no per-element branch); the value is used only when in
    const float tv = sig_tab[(in ? off : 0u) + (neg ? (uint32_t)kSigHalf : 0u)];
    return in ? tv : (mag < (uint32_t)(kSigLo << 7) ? 0.5f : (neg ? 0.0f : 1.0f));
  };

  auto load_row = [&](int64_t row, u32x4* dg, u32x4* du) {
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const int vi = tid + kT * c;
      const bool ok = vi < nvec;
      dg[c] = ok ? load16(gate + row * ldg_bytes + (int64_t)vi * 16) : u32x4{0u, 0u, 0u, 0u};
      du[c] = ok ? load16(up + row * ldu_bytes + (int64_t)vi * 16) : u32x4{0u, 0u, 0u, 0u};
    }
  };
  u32x4 ng[kCh], nu[kCh];
  int64_t row = blockIdx.x;
  if (row < m) load_row(row, ng, nu);
  if (blockIdx.x == 0)
    for (int i = tid; i < nzero; i += kT) zero[i] = 0u;
  // the sigma table, built while the first row's loads are in flight
  for (int i = tid; i < kSigEntries; i += kT) {
    const uint32_t mag = (uint32_t)(kSigLo << 7) + (uint32_t)(i % kSigHalf);
    const uint32_t b = mag | (i >= kSigHalf ? 0x8000u : 0u);
    sig_tab[i] = sigma_direct(__uint_as_float(b << 16));
  }

  // the thread's smoothing factors and their reciprocals (1 without smoothing)
  float sreg[kCh][V], rreg[kCh][V];
  int bad = 0;
#pragma unroll
  for (int c = 0; c < kCh; ++c) {
    const int vi = tid + kT * c;
#pragma unroll
    for (int e = 0; e < V; e += 4) {
      u32x4 sv = {0x3F800000u, 0x3F800000u, 0x3F800000u, 0x3F800000u};
      if (smooth && vi < nvec) sv = load16(smooth + (int64_t)vi * V + e);
      sreg[c][e] = __uint_as_float(sv.x); sreg[c][e + 1] = __uint_as_float(sv.y);
      sreg[c][e + 2] = __uint_as_float(sv.z); sreg[c][e + 3] = __uint_as_float(sv.w);
    }
#pragma unroll
    for (int e = 0; e < V; ++e) {
      rreg[c][e] = rcp_rn(sreg[c][e]);
      bad |= !(sreg[c][e] >= kFastSMin && sreg[c][e] <= kFastSMax);
    }
  }
  {
    const int wbad = __any(bad);
    if (lane == 0) any_bad[wid] = wbad;
    lds_barrier();
  }
  int anyb = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) anyb |= any_bad[w];
  const bool s_fast = __builtin_amdgcn_readfirstlane(anyb) == 0;

  for (; row < m; row += gridDim.x) {
    u32x4 rg[kCh], ru[kCh];
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      rg[c] = ng[c];
      ru[c] = nu[c];
    }
    if (row + gridDim.x < m) load_row(row + gridDim.x, ng, nu);

    // h = bf16(SiLU(g) * u), as binary32; sigma(g) from the table
    float h[kCh][V];
#pragma unroll
    for (int c = 0; c < kCh; ++c) {
      const uint32_t w[4] = {rg[c].x, rg[c].y, rg[c].z, rg[c].w};
      float u[V];
      BF16In::unpack(ru[c], u);
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const uint32_t b = (e & 1) ? (w[e >> 1] >> 16) : (w[e >> 1] & 0xFFFFu);
        h[c][e] = __uint_as_float(f32_to_bf16((__uint_as_float(b << 16) * sigma_of(b)) * u[e]) << 16);
      }
    }

    // xh = h / s and the row maximum; IEEE division when the row leaves the fast range
    auto smooth_pass = [&](bool fast, float (*xh)[V]) {
      float amax = 0.f;
#pragma unroll
      for (int c = 0; c < kCh; ++c)
#pragma unroll
        for (int e = 0; e < V; ++e) {
          xh[c][e] = fast ? div_mk(h[c][e], sreg[c][e], rreg[c][e]) : h[c][e] / sreg[c][e];
          amax = fmaxf(amax, fabsf(xh[c][e]));
        }
      uint32_t ab = wave_max_u32(__float_as_uint(amax));
      if (lane == 0) red_a[wid] = ab;
      lds_barrier();
#pragma unroll
      for (int w = 0; w < kW; ++w) ab = red_a[w] > ab ? red_a[w] : ab;
      return __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)ab));
    };
    float xh[kCh][V];
    float amax;
    if (s_fast) {
      amax = smooth_pass(true, xh);
      const float d0 = amax / (float)kQMax;
      if (!(d0 >= kFastDMin && amax <= kFastAMax) && d0 > 0.f) {
        lds_barrier();  // every wave has read red_a before it is written again
        amax = smooth_pass(false, xh);
      }
    } else {
      amax = smooth_pass(false, xh);
    }
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
        for (int e = 0; e < V; ++e) code[e] = q_code(quot(xh[c][e]));
        *reinterpret_cast<uint2*>(qr + (int64_t)vi * V) =
            make_uint2(pack4(code[0], code[1], code[2], code[3]), pack4(code[4], code[5], code[6], code[7]));
      }
    };
    if (s_fast && dsc >= kFastDMin && amax <= kFastAMax)
      emit([&](float v) { return div_mk(v, dsc, rd); });
    else if (dsc > 0.f)
      emit([&](float v) { return v / dsc; });
    else
      emit([](float) { return 0.f; });
    lds_barrier();  // red_a is read by every wave before the next row writes it
  }
}

}  // namespace sqk

namespace sqh {

template <int kCh, int kT>
static void launch_silu(const uint8_t* g, const uint8_t* u, int64_t m, int64_t nvec, int64_t ldg, int64_t ldu,
                        const float* smooth, int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero, int nzero) {
  int64_t grid = m;
  if (m >= 1024) {
    const int64_t cap = (kT == 256 && kCh <= 4) ? 1024 : 512;
    grid = m < cap ? m : cap;
  }
  hipLaunchKernelGGL((sqk::silu_quant_kernel<kCh, kT>), dim3((unsigned)grid), dim3(kT), 0, s, g, u, m, (int)nvec, ldg,
                     ldu, smooth, xq, x_scale, zero, nzero);
}

hipError_t silu_quant(const void* gate, const void* up, int64_t m, int64_t k, int64_t ldg, int64_t ldu,
                      const float* smooth, int8_t* xq, float* x_scale, hipStream_t s, uint32_t* zero,
                      int64_t nzero) {
  if (m <= 0) return nzero > 0 ? fill_u32(zero, 0u, nzero, s) : hipSuccess;
  if (!zero) nzero = 0;
  const int64_t nvec = k / 8;
  const uint8_t* g = (const uint8_t*)gate;
  const uint8_t* u = (const uint8_t*)up;
  const int64_t lg = ldg * 2, lu = ldu * 2;
  const int nz = (int)nzero;
  if ((m < 1024 && nvec > 256) || nvec > 1024) {
    if (nvec <= 1024)
      launch_silu<1, 1024>(g, u, m, nvec, lg, lu, smooth, xq, x_scale, s, zero, nz);
    else if (nvec <= 2048)
      launch_silu<2, 1024>(g, u, m, nvec, lg, lu, smooth, xq, x_scale, s, zero, nz);
    else
      launch_silu<4, 1024>(g, u, m, nvec, lg, lu, smooth, xq, x_scale, s, zero, nz);
  } else {
    const int64_t per_thread = (nvec + 255) / 256;
    if (per_thread <= 1)
      launch_silu<1, 256>(g, u, m, nvec, lg, lu, smooth, xq, x_scale, s, zero, nz);
    else if (per_thread <= 2)
      launch_silu<2, 256>(g, u, m, nvec, lg, lu, smooth, xq, x_scale, s, zero, nz);
    else
      launch_silu<4, 256>(g, u, m, nvec, lg, lu, smooth, xq, x_scale, s, zero, nz);
  }
  return hipGetLastError();
}

}  // namespace sqh
