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
// Layout on gfx950: one token makes the product a matrix-vector product, so
// the matrix cores would idle on 15 of their 16 token columns; the dot
// products run on the vector ALUs instead (v_dot4_i32_i8: four int8 products
// summed into an int32 per instruction), and the weight stream is laid out
// for full cache lines. A workgroup of kW waves owns 8 or 16 rows of Wq
// (output columns); within a wave, lanes 8r .. 8r + 7 read the 16-byte pieces
// of one 128-byte line of row r, so each load instruction covers 8 whole
// lines (the matrix-core layout reads half lines, 16 rows x 64 bytes, and
// needs two requests per line). The waves take the 128-byte k-steps round-
// robin (wave w: steps w, w + kW, ...), up to eight steps per wave with every
// load of the wave in flight before the first product; kW grows with K (4
// waves for K up to 4096, 8 up to 8192, 16 up to 16384) so that the row's
// quantisation below is spread over enough threads.
//
// Before its first product every workgroup reads the token's row of X and the
// smoothing factors (L2-resident after the first workgroup), forms the row
// scale exactly as the quantisation kernel does (the same Markstein quotients,
// fast-range rule and IEEE fallback), and writes the row's int8 codes to LDS,
// from where every lane reads the 16 codes of its k-piece. The x and s loads
// go out before the Wq loads, so waiting for them never waits for weights.
// Each lane's int32 sums are added over the 8 lanes of its row (lane
// shuffles) and over the waves (LDS). There is no split over K, so no
// workspace and no counters: the results are those of the two-launch path bit
// for bit (int32 sums are exact in any order).
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

// kW waves of kNS 128-byte k-steps each (all loads of a tile in flight; K <=
// 128 kW kNS) over kG 8-row groups of Wq per tile, kR tiles one after the
// other (the row is quantised once per workgroup; the next tile's loads go
// out before the current tile's products); each thread keeps kC 16-byte
// vectors of the row (16 / bytes per value, so K <= 64 kW x 16 values).
// kXFirst: the x and s loads complete before the first weight load goes out
// (with 1024-thread workgroups the weight requests of every CU otherwise
// queue in front of them, and the quantisation, which needs them, waits).
template <class In, bool kSmooth, int kW, int kG, int kNS, int kR, bool kXFirst>
__global__ __launch_bounds__(64 * kW, 1) void gemv_decode1_kernel(Decode1Args a) {
  constexpr int kT = 64 * kW;
  constexpr int V = In::kVec;
  constexpr int kC = 16 / V;
  constexpr int kD1Rows = 8 * kG;  // Wq rows (outputs) of a tile
  constexpr int kD1Steps = kNS;
  constexpr int kMaxK = kT * kC * V;
  __shared__ __attribute__((aligned(16))) int8_t codes[kMaxK];
  __shared__ int32_t red[2][kW][kD1Rows];
  __shared__ float red_f[kW];
  __shared__ int red_i[kW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int nfirst = (int)blockIdx.x * kD1Rows * kR;
  const int K = a.K;
  const int nvec = K / V;
  const int nsteps = K / 128;

  // ---- the token's row and the smoothing factors (issued first)
  u32x4 xr[kC];
  float sv[kSmooth ? kC : 1][V];
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int vi = tid + kT * c;
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

  if constexpr (kXFirst) __builtin_amdgcn_s_waitcnt(0);

  // ---- Wq: all kD1Steps steps of this wave for the row groups of tile r
  // (into register buffer buf); steps past the end reload the last step, and
  // rows past N the last row (valid memory; their products are not stored)
  const int piece = 16 * (lane & 7);
  u32x4 wb[kR > 1 ? 2 : 1][kD1Steps][kG];
  auto wload = [&](int r, int buf) {
    const int n0 = nfirst + r * kD1Rows;
    const int8_t* wp[kG];
#pragma unroll
    for (int g = 0; g < kG; ++g) wp[g] = a.wq + (int64_t)min(n0 + 8 * g + (lane >> 3), a.N - 1) * K + piece;
#pragma unroll
    for (int i = 0; i < kD1Steps; ++i) {
      const int64_t off = (int64_t)min(wid + kW * i, nsteps - 1) * 128;
#pragma unroll
      for (int g = 0; g < kG; ++g) wb[buf][i][g] = load16(wp[g] + off);
    }
  };
  wload(0, 0);
  // keep the scheduler from moving the weight loads behind the quantisation
  __builtin_amdgcn_sched_barrier(0);

  // ---- row scale: d = fl32(max_j |fl32(x_j / s_j)| / 127), the quantiser's arithmetic
  float xh[kC][V];
  int bad = 0;
  if (kSmooth) {
#pragma unroll
    for (int c = 0; c < kC; ++c)
      if (tid + kT * c < nvec)
#pragma unroll
        for (int e = 0; e < V; ++e) bad |= !(sv[c][e] >= kFastSMin && sv[c][e] <= kFastSMax);
  }
  const int wbad = __any(bad);
  if (lane == 0) red_i[wid] = wbad;
  auto smooth_pass = [&](bool fast) {
    float amax = 0.f;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if (tid + kT * c >= nvec) continue;
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
  int anyb = 0;
#pragma unroll
  for (int w = 0; w < kW; ++w) anyb |= red_i[w];
  const bool s_ok = !anyb;
  auto block_max = [&](float v) {
    v = wave_max(v);
    lds_barrier();  // the previous readers of red_f are done
    if (lane == 0) red_f[wid] = v;
    lds_barrier();
    float r = red_f[0];
#pragma unroll
    for (int w = 1; w < kW; ++w) r = fmaxf(r, red_f[w]);
    return r;
  };
  float amax = block_max(s_ok ? smooth_pass(true) : smooth_pass(false));
  float d = amax / (float)kQMax;
  const bool fast = s_ok && d >= kFastDMin && amax <= kFastAMax;
  if (kSmooth && s_ok && !fast && d > 0.f) {
    amax = block_max(smooth_pass(false));
    d = amax / (float)kQMax;
  }

  // ---- the row's codes into LDS
  const float rd = (fast && d > 0.f) ? rcp_scale(d) : 0.f;
#pragma unroll
  for (int c = 0; c < kC; ++c) {
    const int vi = tid + kT * c;
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
  lds_barrier();

  // ---- dot products (step i of this wave is k-step wid + kW i), the 8
  // lanes of a row, then the waves through LDS; with several tiles the next
  // tile's loads go out first and the LDS partials are double-buffered (one
  // barrier per tile, none of which waits for the loads in flight). The
  // single-tile form is kept separate: folded into the loop, the 16-wave
  // instance spilled a weight register and waited for every load first.
  auto dots = [&](int buf, int* acc) {
#pragma unroll
    for (int g = 0; g < kG; ++g) acc[g] = 0;
#pragma unroll
    for (int i = 0; i < kD1Steps; ++i) {
      const int st = wid + kW * i;
      if (st < nsteps) {
        const u32x4 xv = *reinterpret_cast<const u32x4*>(&codes[st * 128 + piece]);
#pragma unroll
        for (int g = 0; g < kG; ++g) {
          acc[g] = __builtin_amdgcn_sdot4((int)wb[buf][i][g].x, (int)xv.x, acc[g], false);
          acc[g] = __builtin_amdgcn_sdot4((int)wb[buf][i][g].y, (int)xv.y, acc[g], false);
          acc[g] = __builtin_amdgcn_sdot4((int)wb[buf][i][g].z, (int)xv.z, acc[g], false);
          acc[g] = __builtin_amdgcn_sdot4((int)wb[buf][i][g].w, (int)xv.w, acc[g], false);
        }
      }
    }
#pragma unroll
    for (int g = 0; g < kG; ++g) {
      acc[g] += __shfl_xor(acc[g], 1);
      acc[g] += __shfl_xor(acc[g], 2);
      acc[g] += __shfl_xor(acc[g], 4);
    }
  };
  auto store = [&](int n, int32_t sum, float ws) {
    const float v = __fmul_rn(__fmul_rn((float)sum, d), ws);
    if (a.out == 0)
      reinterpret_cast<float*>(a.y)[n] = v;
    else if (a.out == 1)
      reinterpret_cast<uint16_t*>(a.y)[n] = (uint16_t)f32_to_bf16(v);
    else
      reinterpret_cast<uint16_t*>(a.y)[n] = (uint16_t)f32_to_f16(v);
  };
  if constexpr (kR == 1) {
    int acc[kG];
    dots(0, acc);
#pragma unroll
    for (int g = 0; g < kG; ++g)
      if ((lane & 7) == 0) red[0][wid][8 * g + (lane >> 3)] = acc[g];
    __syncthreads();
    if (tid < kD1Rows) {
      const int n = nfirst + tid;
      if (n < a.N) {
        int32_t sum = red[0][0][tid];
#pragma unroll
        for (int w = 1; w < kW; ++w) sum += red[0][w][tid];
        store(n, sum, a.w_scale[n]);
      }
    }
  } else {
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int buf = r & 1;
      // the tile's channel scale first: a load issued after the next tile's
      // weight loads would make the epilogue wait for all of them
      const int ns = min(nfirst + r * kD1Rows + (tid < kD1Rows ? tid : 0), a.N - 1);
      const float wsc = a.w_scale[ns];
      if (r + 1 < kR) wload(r + 1, buf ^ 1);
      int acc[kG];
      dots(buf, acc);
#pragma unroll
      for (int g = 0; g < kG; ++g)
        if ((lane & 7) == 0) red[buf][wid][8 * g + (lane >> 3)] = acc[g];
      lds_barrier();
      if (tid < kD1Rows) {
        const int n = nfirst + r * kD1Rows + tid;
        if (n < a.N) {
          int32_t sum = red[buf][0][tid];
#pragma unroll
          for (int w = 1; w < kW; ++w) sum += red[buf][w][tid];
          store(n, sum, wsc);
        }
      }
    }
  }
}

}  // namespace sqk

namespace sqh {

namespace {

// 4 waves of 8 steps and 8-row tiles up to K = 4096, 8 waves of 8 steps up
// to 8192, 16 waves of 8 steps and 16-row tiles up to 16384. Measured on
// MI355X, us per launch back to back over rotating weight copies, one tile
// per workgroup, 4096 -> 14336 layer (waves / rows per workgroup / steps per
// wave): 4/8/8 13.5, 8/8/4 14.2, 8/16/4 13.8, 16/16/2 14.8, 16/32/2 14.2,
// 16/8/2 18.5; 14336 -> 4096 layer: 16/16/8 15.2, 16/8/8 17.5 (two rounds of
// workgroups, each quantising the row), 16/24/8 23.7 and 16/32/8 32.8
// (registers spilled). Without the quantisation the product alone takes
// 10.7-11.0 / 11.4 with 8 rows, and a plain stream of the same bytes
// 10.1-10.4: the row's quantisation in every workgroup costs the rest.
// Publishing the codes from one workgroup to the others through the
// workspace measured slower (15.6 / 16.1: the publication adds two dependent
// memory round trips to every other workgroup's path).
//
// Several tiles per workgroup (the row quantised once, the next tile's loads
// in flight during the current tile's products), up to K = 8192: kR tiles
// per workgroup with the grid nearest 448 workgroups measured fastest or
// within noise of it (us, one tile -> kR): 4096 -> 14336 14.2 -> 12.4 (kR
// 4; kR 2, 3, 5, 6, 8: 13.5, 14.1, 13.6, 15.0, 14.3), 4096 -> 6144 8.1 ->
// 7.5 (kR 2), 4096 -> 28672 22.8 -> 22.6 (kR 8), 8192 -> 14336 25.8 ->
// 23.0 (kR 4), 8192 -> 28672 45.4 -> 41.0 (kR 8). The 16-wave form (one
// workgroup per CU) takes as many 8-row tiles per workgroup as keep the grid
// within 256, and waits for x and s before its weight loads: 14336 -> 4096
// with 16-row tiles 15.0, two 8-row tiles 13.9, and with the x-first wait
// 13.6 (the wait made no difference at 4096 -> 14336: 12.65 / 12.59).
inline int d1_tiles_per_wg(int64_t n, int rows) {
  const int64_t tiles = (n + rows - 1) / rows;
  int best = 1;
  int64_t err = tiles > 448 ? tiles - 448 : 448 - tiles;
  for (int r = 2; r <= 8; r *= 2) {
    const int64_t wgs = (tiles + r - 1) / r;
    const int64_t e = wgs > 448 ? wgs - 448 : 448 - wgs;
    if (e < err) {
      best = r;
      err = e;
    }
  }
  return best;
}

// The 16-wave form (K above 8192) holds a whole CU: up to 256 workgroups,
// as few tiles each as that allows.
inline int d1_tiles_per_wg16(int64_t n) {
  const int64_t tiles = (n + 7) / 8;
  int r = 1;
  while (r < 8 && (tiles + r - 1) / r > 256) r *= 2;
  return r;
}

template <class In, bool kSmooth, int kW>
void launch_d1_r(const sqk::Decode1Args& a, hipStream_t s) {
  const int r = kW == 16 ? d1_tiles_per_wg16(a.N) : d1_tiles_per_wg(a.N, 8);
  const unsigned grid = (unsigned)((a.N + 8 * r - 1) / (8 * r));
  switch (r) {
    case 1: hipLaunchKernelGGL((sqk::gemv_decode1_kernel<In, kSmooth, kW, 1, 8, 1, kW == 16>), dim3(grid), dim3(64 * kW), 0, s, a); break;
    case 2: hipLaunchKernelGGL((sqk::gemv_decode1_kernel<In, kSmooth, kW, 1, 8, 2, kW == 16>), dim3(grid), dim3(64 * kW), 0, s, a); break;
    case 4: hipLaunchKernelGGL((sqk::gemv_decode1_kernel<In, kSmooth, kW, 1, 8, 4, kW == 16>), dim3(grid), dim3(64 * kW), 0, s, a); break;
    default: hipLaunchKernelGGL((sqk::gemv_decode1_kernel<In, kSmooth, kW, 1, 8, 8, kW == 16>), dim3(grid), dim3(64 * kW), 0, s, a); break;
  }
}

template <class In, bool kSmooth>
void launch_d1(const sqk::Decode1Args& a, hipStream_t s) {
  if (a.K <= 4096)
    launch_d1_r<In, kSmooth, 4>(a, s);
  else if (a.K <= 8192)
    launch_d1_r<In, kSmooth, 8>(a, s);
  else if constexpr (In::kVec == 8)  // binary32 rows stop at 8192 (decode1_suits)
    launch_d1_r<In, kSmooth, 16>(a, s);
}

template <class In>
hipError_t decode1(const sqk::Decode1Args& a, bool smooth, hipStream_t s) {
  if (smooth)
    launch_d1<In, true>(a, s);
  else
    launch_d1<In, false>(a, s);
  return hipGetLastError();
}

}  // namespace

// One token, K a multiple of 128 up to 16384 values (16 waves x 64 lanes x
// 16 values; the eight k-steps per wave then cover K), and layers at least
// 2048 wide (128 workgroups or more).
bool decode1_suits(int64_t m, int64_t n, int64_t k, sq_dtype xt) {
  // binary32 rows up to 8192 (beyond, the 16-wave form would need more
  // registers than it has)
  return m == 1 && n >= 2048 && n <= INT32_MAX && k % 128 == 0 && k <= (xt == SQ_F32 ? 8192 : 16384);
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
