// Decode-shaped int8 GEMM (M <= 64 tokens, and up to 256 where the tiled
// kernels would cover few CUs): Y = dequant(Xq . Wq^T), where the cost is
// streaming the weight matrix Wq [N x K] from HBM.
//
// The LLM.int8() page, "The architecture: every piece explained" (int8
// operands, int32 accumulation, dequantisation by the outer product of the row
// and column scales); "Half the Size, Better Performance, Same Accuracy:
// Understanding W8A8 INT8 LLM Quantization", "Performance After Quantization"
// (per decoded token the weights are read once; the layer is memory-bound).
//
// Layout of the work on gfx950:
//  * A 256-thread workgroup owns 64 rows of Wq (output columns n) and one
//    slice of K. The grid is (ceil(N/64), S): S slices of K, chosen so that a
//    few hundred workgroups keep every CU streaming.
//  * Inside the workgroup the 4 waves split the slice's 128-byte k-steps
//    round-robin (wave w takes steps w, w+4, ...), so the 4 waves read
//    adjacent 128-byte pieces of the same rows, and every wave covers all 64
//    rows: one Xq fragment feeds 4 row groups, so Xq (L2-resident) costs no
//    more load bandwidth than Wq.
//  * Operands go straight from global memory into registers in the
//    v_mfma_i32_16x16x64_i8 layout: A = Wq (lane l: row l%16, 16 bytes at
//    k-offset 16*(l/16) of each 64-byte half step), B = Xq (token l%16, same
//    k bytes). The step count per wave is a template constant, so the whole
//    pipeline is unrolled: kDepth steps of loads stay in flight ahead of the
//    MFMAs. Rows of Wq beyond N and tokens beyond M read a clamped (valid)
//    row whose results are never stored.
//  * The 4 waves' int32 tiles are summed through LDS; one thread then owns 4
//    consecutive outputs of one token (16 threads = 64 contiguous outputs).
//  * With S > 1 each workgroup writes its int32 partial tile to a workspace,
//    then takes a ticket from the tile's counter; the workgroup drawing the
//    last ticket sums the S partials in slice order and runs the epilogue.
//    All partial sums are int32 additions, so the result equals the unsplit
//    product bit for bit. The counters must be zero at launch; the last
//    workgroup of a tile sets its counter back to zero, so a zeroed workspace
//    stays zeroed from call to call.
//  * The same kernel takes E4M3 operands (kF8): one
//    v_mfma_scale_f32_16x16x128_f8f6f4 per 128-byte step (lane l: row l%16,
//    the 32 bytes at k-offset 32*(l/16)), binary32 accumulators and partial
//    tiles. The waves' tiles and the slices' partials are added in a fixed
//    order (wave 0..3, slice 0..S-1), so results are deterministic; they
//    differ from an unsplit product by binary32 roundings of those sums.
#include <type_traits>

#include "sq_common.hpp"
#include "sq_launch.hpp"

#include <stdlib.h>

namespace sqk {

constexpr int kDecRows = 64;    // Wq rows per workgroup
constexpr int kDecStep = 128;   // k bytes per pipeline step
constexpr int kDecWaves = 4;
constexpr int kDecMaxNS = 8;    // most steps per wave (template range)
// Buffer descriptor word 3 of a raw byte buffer on gfx9 (32-bit data format),
// and the cache-policy operand of device-coherent (sc1) buffer accesses.
constexpr int kBufDword3 = 0x00020000;
constexpr int kCoherent = 16;

struct DecodeArgs {
  const int8_t* xq;
  const int8_t* wq;
  const float* x_scale;
  const float* w_scale;
  void* y;
  int64_t ldy;
  int32_t* partial;    // [S][M][N] int32 (S > 1)
  uint32_t* counter;   // [ceil(N/64)], zero at launch and at exit (S > 1)
  int M, N, K;
  int S;               // number of K slices
  int slice_steps;     // 128-byte steps per slice
  int out;             // 0 f32, 1 bf16, 2 f16, 3 i32
};

typedef int v8i_d __attribute__((ext_vector_type(8)));
typedef float v4f_d __attribute__((ext_vector_type(4)));

// acc: int32 sums, or (kF8) the bits of binary32 sums
template <bool kF8>
__device__ __forceinline__ void dec_epilogue(const DecodeArgs& a, int m, int n, const int32_t* acc) {
  if (m >= a.M || n >= a.N) return;
  const int nv = min(4, a.N - n);
  const int64_t off = (int64_t)m * a.ldy + n;
  if (a.out == 3) {
    int32_t* p = reinterpret_cast<int32_t*>(a.y) + off;
    if (nv == 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      *reinterpret_cast<int4*>(p) = make_int4(acc[0], acc[1], acc[2], acc[3]);
    } else {
      for (int e = 0; e < nv; ++e) p[e] = acc[e];
    }
    return;
  }
  const float xs = a.x_scale[m];
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float av = kF8 ? __int_as_float(acc[e]) : (float)acc[e];
    v[e] = e < nv ? __fmul_rn(__fmul_rn(av, xs), a.w_scale[n + e]) : 0.f;
  }
  if (a.out == 0) {
    float* p = reinterpret_cast<float*>(a.y) + off;
    if (nv == 4 && (reinterpret_cast<uintptr_t>(p) & 15) == 0) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int e = 0; e < nv; ++e) p[e] = v[e];
    }
    return;
  }
  uint16_t h[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) h[e] = a.out == 1 ? f32_to_bf16(v[e]) : f32_to_f16(v[e]);
  uint16_t* p = reinterpret_cast<uint16_t*>(a.y) + off;
  if (nv == 4 && (reinterpret_cast<uintptr_t>(p) & 7) == 0) {
    *reinterpret_cast<uint2*>(p) = make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                              (uint32_t)h[2] | ((uint32_t)h[3] << 16));
  } else {
    for (int e = 0; e < nv; ++e) p[e] = h[e];
  }
}

template <int kMB, int kNS, bool kF8>
__global__ __launch_bounds__(256, 1) void gemm_decode_kernel(DecodeArgs a) {
  using AccT = typename std::conditional<kF8, v4f_d, v4i>::type;
  constexpr int kTok = 16 * kMB;
  // steps of loads in flight: all of them when the registers allow (the
  // workgroup's whole share of Wq is requested at once). The caps keep the
  // compiler from spilling: measured on MI355X, the int8 form at 64 tokens
  // with depth 6 spilled 12 registers and ran its 64 x 4096 x 14336 GEMM in
  // 26.4 us, with depth 4 in 23.5 us; at 16 tokens depth 8 spilled (14336 x
  // 4096 down projection, M 1: 17.5 -> 16.5 us with depth 5). The E4M3 form
  // (one MFMA per step) fits depth 6 / 8 without spilling.
  constexpr int kMaxDepth = kF8 ? (kMB == 4 ? 6 : 8) : (kMB == 4 ? 4 : (kMB == 1 ? 5 : 8));
  constexpr int kDepth = kNS < kMaxDepth ? kNS : kMaxDepth;
  __shared__ int32_t red[kDecWaves][kTok][kDecRows];
  __shared__ uint32_t last_ticket;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int tile = blockIdx.x;
  const int slice = blockIdx.y;
  const int n0 = tile * kDecRows;
  // tokens m0 .. m0 + 63 (blockIdx.z: one grid layer per 64 tokens; every
  // layer streams the same Wq, whose re-reads hit the last-level cache)
  const int m0 = (int)blockIdx.z * 64;
  const int ctr = (int)blockIdx.z * (int)gridDim.x + tile;
  const int step0 = slice * a.slice_steps;
  const int nsl = min(a.slice_steps, a.K / kDecStep - step0);  // >= 1 by construction of S

  // the lane's k bytes of a step: int8, [kb, kb+16) and [64+kb, 64+kb+16);
  // E4M3, [kb, kb+32)
  const int kb = (kF8 ? 32 : 16) * (lane >> 4);
  constexpr int kHalf = kF8 ? 16 : 64;
  const int8_t* wp[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) wp[g] = a.wq + (int64_t)min(n0 + 16 * g + (lane & 15), a.N - 1) * a.K + kb;
  const int8_t* xp[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) xp[mb] = a.xq + (int64_t)min(m0 + 16 * mb + (lane & 15), a.M - 1) * a.K + kb;

  AccT acc[4][kMB];
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) acc[g][mb] = AccT{0, 0, 0, 0};

  u32x4 wb[kDepth][4][2];
  u32x4 xb[kDepth][kMB][2];
  // step i of this wave is slice step wid + 4 i; past the slice end it reloads
  // the last step (valid memory) and its product is skipped
  auto load = [&](int i, int slot) {
    const int64_t off = (int64_t)(step0 + min(wid + kDecWaves * i, nsl - 1)) * kDecStep;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      wb[slot][g][0] = load16(wp[g] + off);
      wb[slot][g][1] = load16(wp[g] + off + kHalf);
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      xb[slot][mb][0] = load16(xp[mb] + off);
      xb[slot][mb][1] = load16(xp[mb] + off + kHalf);
    }
  };
#pragma unroll
  for (int i = 0; i < kDepth; ++i) load(i, i);
  // keep the scheduler from trading the loads in flight for registers
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < kNS; ++i) {
    const int slot = i % kDepth;
    u32x4 w[4][2], x[kMB][2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      w[g][0] = wb[slot][g][0];
      w[g][1] = wb[slot][g][1];
    }
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      x[mb][0] = xb[slot][mb][0];
      x[mb][1] = xb[slot][mb][1];
    }
    if (i + kDepth < kNS) load(i + kDepth, slot);
    // a step past the slice end contributes zero (a select, not a branch, so
    // that the compiler keeps every load at its place in the pipeline)
    const bool valid = wid + kDecWaves * i < nsl;
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      x[mb][0] = valid ? x[mb][0] : u32x4{0u, 0u, 0u, 0u};
      x[mb][1] = valid ? x[mb][1] : u32x4{0u, 0u, 0u, 0u};
    }
    if constexpr (kF8) {
      auto cat = [](const u32x4& lo, const u32x4& hi) {
        return v8i_d{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      };
#pragma unroll
      for (int g = 0; g < 4; ++g)
#pragma unroll
        for (int mb = 0; mb < kMB; ++mb)
          acc[g][mb] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cat(w[g][0], w[g][1]), cat(x[mb][0], x[mb][1]),
                                                                        acc[g][mb], 0, 0, 0, 127, 0, 127);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int mb = 0; mb < kMB; ++mb)
            acc[g][mb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(v4i, w[g][h]),
                                                               __builtin_bit_cast(v4i, x[mb][h]), acc[g][mb], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // 16x16 result layout: lane l holds token 16 mb + l%16 and rows
  // 16 g + 4 (l/16) + r, r = 0..3. Quads of rows are XOR-swizzled by the
  // token so that both this store and the row-wise reads below are free of
  // bank conflicts.
#pragma unroll
  for (int g = 0; g < 4; ++g)
#pragma unroll
    for (int mb = 0; mb < kMB; ++mb) {
      const int tok = 16 * mb + (lane & 15);
      const int quad = (4 * g + (lane >> 4)) ^ (tok & 15);
      *reinterpret_cast<v4i*>(&red[wid][tok][4 * quad]) = __builtin_bit_cast(v4i, acc[g][mb]);
    }
  __syncthreads();

  const int q = tid & 15;
  int32_t sum[kMB][4];
#pragma unroll
  for (int j = 0; j < kMB; ++j) {
    const int tok = (tid >> 4) + 16 * j;
    const int sq = q ^ (tok & 15);
    AccT s = __builtin_bit_cast(AccT, *reinterpret_cast<const v4i*>(&red[0][tok][4 * sq]));
#pragma unroll
    for (int w = 1; w < kDecWaves; ++w) s += __builtin_bit_cast(AccT, *reinterpret_cast<const v4i*>(&red[w][tok][4 * sq]));
    const v4i sb = __builtin_bit_cast(v4i, s);
    sum[j][0] = sb[0]; sum[j][1] = sb[1]; sum[j][2] = sb[2]; sum[j][3] = sb[3];
  }
  const int n = n0 + 4 * q;
  if (a.S == 1) {
#pragma unroll
    for (int j = 0; j < kMB; ++j) dec_epilogue<kF8>(a, m0 + (tid >> 4) + 16 * j, n, sum[j]);
    return;
  }

  // Split K: publish this slice's tile; the last workgroup of the tile
  // reduces. The partial tiles cross XCDs, whose L2 caches are not coherent
  // with each other, so they are written and read with device-coherent (sc1)
  // buffer accesses; a device-scope fence would instead write back and
  // invalidate the whole L2 of the XCD in every workgroup. Order: coherent
  // stores, wait until every store of the workgroup has completed, then the
  // ticket (an agent-scope atomic); the holder of the last ticket then reads
  // the partials coherently.
  const uint32_t pbytes = (uint32_t)((size_t)a.S * a.M * a.N * 4);
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(a.partial, (short)0, pbytes, kBufDword3);
  const bool vec = (a.N & 3) == 0;
#pragma unroll
  for (int j = 0; j < kMB; ++j) {
    const int m = m0 + (tid >> 4) + 16 * j;
    if (m < a.M && n < a.N) {
      const uint32_t off = (uint32_t)((((size_t)slice * a.M + m) * a.N + n) * 4);
      if (vec) {
        const v4i v = {sum[j][0], sum[j][1], sum[j][2], sum[j][3]};
        __builtin_amdgcn_raw_buffer_store_b128(v, pr, off, 0, kCoherent);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) __builtin_amdgcn_raw_buffer_store_b32(sum[j][e], pr, off + 4 * e, 0, kCoherent);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0)
    last_ticket = __hip_atomic_fetch_add(a.counter + ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (last_ticket != (uint32_t)(a.S - 1)) return;
#pragma unroll
  for (int j = 0; j < kMB; ++j) {
    const int m = m0 + (tid >> 4) + 16 * j;
    if (m >= a.M || n >= a.N) continue;
    AccT t = {0, 0, 0, 0};
    const uint32_t off0 = (uint32_t)(((size_t)m * a.N + n) * 4);
    const uint32_t sstride = (uint32_t)((size_t)a.M * a.N * 4);
    if (vec) {
      // eight slices per round trip; slices past S read beyond the buffer's
      // range, which a raw buffer load returns as zero
      for (int s = 0; s < a.S; s += 8) {
        v4i part[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          part[u] = __builtin_amdgcn_raw_buffer_load_b128(pr, off0 + (uint32_t)(s + u) * sstride, 0, kCoherent);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (!kF8 || s + u < a.S) t += __builtin_bit_cast(AccT, part[u]);
      }
    } else {
      for (int s = 0; s < a.S; ++s)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (n + e < a.N) {
            const int32_t pv = __builtin_amdgcn_raw_buffer_load_b32(pr, off0 + s * sstride + 4 * e, 0, kCoherent);
            if constexpr (kF8)
              t[e] += __int_as_float(pv);
            else
              t[e] += pv;
          }
    }
    const v4i tb = __builtin_bit_cast(v4i, t);
    const int32_t tt[4] = {tb[0], tb[1], tb[2], tb[3]};
    dec_epilogue<kF8>(a, m, n, tt);
  }
  // every ticket of this tile has been drawn: restore the counter for the next call
  if (tid == 0) __hip_atomic_store(a.counter + ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace sqk

namespace sqh {

namespace {

struct DecodePlan {
  int S = 1;
  int slice_steps = 0;
  int ns = 0;      // steps per wave
  int tiles = 0;
  int tb = 1;      // 64-token blocks (grid z)
};

DecodePlan decode_plan(int64_t m, int64_t n, int64_t k) {
  DecodePlan p;
  const int steps = (int)(k / sqk::kDecStep);
  p.tiles = (int)((n + sqk::kDecRows - 1) / sqk::kDecRows);
  p.tb = (int)((m + 63) / 64);
  // at least one workgroup per CU (256 CUs), with at most kDecMaxNS steps
  // per wave; measured on MI355X, more slices than that only add partial-tile
  // traffic and reduction latency. Where the unsplit grid already has 192
  // workgroups, three in four of the CUs streaming unsplit K are faster than a
  // second round of workgroups (4096 -> 14336, 224 column tiles, GEMM us
  // unsplit / 2 slices: M 1 13.8 / 15.0, M 8 13.9 / 16.0, M 32 16.4 / 18.4,
  // M 64 20.6 / 27.0).
  const int wgs = p.tiles * p.tb;
  int want = (256 + wgs - 1) / wgs;
  if (wgs >= 192) want = 1;
#ifdef SQ_TUNE
  if (const char* e = getenv("SQ_DECODE_SPLIT")) want = atoi(e);
#endif
  if (want < 1) want = 1;
  if (want > steps) want = steps;
  int per = (steps + want - 1) / want;
  const int cap = sqk::kDecWaves * sqk::kDecMaxNS;
  if (per > cap) per = cap;
  p.slice_steps = per;
  p.S = (steps + per - 1) / per;
  p.ns = (per + sqk::kDecWaves - 1) / sqk::kDecWaves;
  return p;
}

size_t counter_bytes(int tiles) { return ((size_t)tiles * 4 + 255) / 256 * 256; }

template <int kMB, bool kF8>
hipError_t launch_decode(const sqk::DecodeArgs& a, int ns, dim3 grid, hipStream_t s) {
  switch (ns) {
    case 1: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 1, kF8>), grid, dim3(256), 0, s, a); break;
    case 2: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 2, kF8>), grid, dim3(256), 0, s, a); break;
    case 3: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 3, kF8>), grid, dim3(256), 0, s, a); break;
    case 4: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 4, kF8>), grid, dim3(256), 0, s, a); break;
    case 5: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 5, kF8>), grid, dim3(256), 0, s, a); break;
    case 6: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 6, kF8>), grid, dim3(256), 0, s, a); break;
    case 7: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 7, kF8>), grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL((sqk::gemm_decode_kernel<kMB, 8, kF8>), grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

template <bool kF8>
hipError_t decode_gemm(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  const DecodePlan p = decode_plan(m, n, k);
  sqk::DecodeArgs a{};
  a.xq = xq; a.wq = wq; a.x_scale = x_scale; a.w_scale = w_scale; a.y = y; a.ldy = ldy;
  a.M = (int)m; a.N = (int)n; a.K = (int)k;
  a.S = p.S;
  a.slice_steps = p.slice_steps;
  a.out = yt == SQ_F32 ? 0 : yt == SQ_BF16 ? 1 : yt == SQ_F16 ? 2 : 3;
  if (p.S > 1) {
    a.counter = reinterpret_cast<uint32_t*>(ws);
    a.partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + counter_bytes(p.tiles * p.tb));
  }
  const dim3 grid((unsigned)p.tiles, (unsigned)p.S, (unsigned)p.tb);
  bool mb1 = m <= 16;
#ifdef SQ_TUNE
  if (getenv("SQ_DECODE_MB2")) mb1 = false;
#endif
  if (mb1) return launch_decode<1, kF8>(a, p.ns, grid, s);
  if (m <= 32) return launch_decode<2, kF8>(a, p.ns, grid, s);
  return launch_decode<4, kF8>(a, p.ns, grid, s);
}

}  // namespace

// Up to 256 tokens the decode kernel runs one grid layer per 64 tokens.
constexpr int64_t kDecodeMaxM = 256;

// Whether 65..256 tokens go to the decode kernel rather than the tiled
// kernels. The decode kernel streams Wq once per 64-token layer (time grows
// about linearly with the layers); the tiled kernels are slow when their
// output tiles cover few CUs. Counted in 128 x 128 tile units (a 256 x 192
// prefill tile is 3), decode wins when the tiled kernel has at most 128 units:
// measured on MI355X (GEMM us, tiled -> decode), 4096 -> 14336 columns:
// M 96 42.4 -> 36.0, M 128 43.5 -> 39.8 (decode), M 192 43.3 vs 57.5, M 256
// 43.9 vs 75.0 (tiled); 14336 -> 4096: M 96 113.8 -> 42.7, M 128 125.2 ->
// 47.6, M 192 111.8 -> 68.3 (decode). Where the 256-row prefill kernel
// applies (gemm_big_suits), it splits K over enough workgroups to cover the
// CUs and beats the decode kernel: 14336 -> 4096 at 256 tokens 60.4 us
// against 89.6, at 192 tokens 57.1 against 69.2.
static bool decode_beats_prefill(int64_t m, int64_t n, int64_t k) {
  if (gemm_big_suits(m, n, k)) return false;
  const int64_t units = ((m + 127) / 128) * ((n + 127) / 128);
  return units <= 128;
}

bool gemm_decode_suits(int64_t m, int64_t n, int64_t k) {
  if (!(m >= 1 && m <= kDecodeMaxM && n >= 1 && n <= INT32_MAX && k % sqk::kDecStep == 0)) return false;
  if (m <= 64) return true;
  // beyond one 64-token block only where the prefill kernels get few tiles
  // (see the dispatch notes); the partial tiles must fit 32-bit offsets
  const DecodePlan p = decode_plan(m, n, k);
  if ((size_t)p.S * (size_t)m * (size_t)n * 4 >= ((size_t)1 << 31)) return false;
  return decode_beats_prefill(m, n, k);
}

size_t gemm_decode_workspace(int64_t m, int64_t n, int64_t k) {
  if (!gemm_decode_suits(m, n, k)) return 0;
  const DecodePlan p = decode_plan(m, n, k);
  if (p.S == 1) return 0;
  return counter_bytes(p.tiles * p.tb) + (size_t)p.S * (size_t)m * (size_t)n * 4;
}

void gemm_decode_counters(int64_t m, int64_t n, int64_t k, void* ws, uint32_t** counters, int64_t* count) {
  *counters = nullptr;
  *count = 0;
  if (!gemm_decode_suits(m, n, k)) return;
  const DecodePlan p = decode_plan(m, n, k);
  if (p.S == 1) return;
  *counters = reinterpret_cast<uint32_t*>(ws);
  *count = (int64_t)p.tiles * p.tb;
}

hipError_t gemm_i8_decode(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                          int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  return decode_gemm<false>(xq, x_scale, wq, w_scale, m, n, k, y, yt, ldy, ws, s);
}

hipError_t gemm_f8_decode(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                          int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  return decode_gemm<true>(reinterpret_cast<const int8_t*>(xq), x_scale, reinterpret_cast<const int8_t*>(wq), w_scale,
                           m, n, k, y, yt, ldy, ws, s);
}

}  // namespace sqh
