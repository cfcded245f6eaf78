// Decode-shaped int8 GEMM (M <= 64 tokens, and up to 256 where the tiled
// kernels would cover few CUs): Y = dequant(Xq . Wq^T), where the cost is
// streaming the weight matrix Wq [N x K] from HBM. Two forms: the unrolled
// register-pipeline kernel below (up to 16 tokens), and the LDS-ring kernel
// further down (17 tokens and more); both take int8 and E4M3 operands.
//
// The LLM.int8() page, "The architecture: every piece explained" (int8
// operands, int32 accumulation, dequantisation by the product of the row
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


namespace sqk {

using sqi::kDecMaxNS;
using sqi::kDecRows;
using sqi::kDecStep;
using sqi::kDecWaves;
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
  const sqi::DecSlice sl = sqi::dec_slice(slice, a.slice_steps, a.K);
  const int step0 = sl.step0;
  const int nsl = sl.nsl;  // >= 1 by construction of S

  // the lane's k bytes of a step: int8, [kb, kb+16) and [64+kb, 64+kb+16);
  // E4M3, [kb, kb+32)
  const int kb = sqi::dec_kb(kF8, lane);
  constexpr int kHalf = sqi::dec_khalf(kF8);
  const int8_t* wp[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) wp[g] = a.wq + (int64_t)sqi::dec_w_row(n0, g, lane, a.N) * a.K + kb;
  const int8_t* xp[kMB];
#pragma unroll
  for (int mb = 0; mb < kMB; ++mb) xp[mb] = a.xq + (int64_t)sqi::dec_x_row(m0, mb, lane, a.M) * a.K + kb;

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
    const int64_t off = (int64_t)(step0 + sqi::dec_step(wid, i, nsl)) * kDecStep;
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
    const bool valid = sqi::dec_step_valid(wid, i, nsl);
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
      const int quad = sqi::dec_red_quad(g, lane, tok);
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
      const uint32_t off = sqi::dec_partial_off(slice, a.M, a.N, m, n);
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
    const uint32_t off0 = sqi::dec_partial_off(0, a.M, a.N, m, n);
    const uint32_t sstride = sqi::dec_partial_off(1, a.M, a.N, 0, 0);
    if (vec) {
      // eight slices per round trip; slices past S read beyond the buffer's
      // range (a raw buffer load returns zero there) and are not added
      for (int s = 0; s < a.S; s += 8) {
        v4i part[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          part[u] = __builtin_amdgcn_raw_buffer_load_b128(pr, off0 + (uint32_t)(s + u) * sstride, 0, kCoherent);
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (s + u < a.S) t += __builtin_bit_cast(AccT, part[u]);
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

// ---- LDS-ring form (17 tokens and more; index maps: sqi::RingCfg)
//
// With 32 or 64 tokens the register form spends its load bandwidth on
// 64-byte pieces (its operand layout gives each row 4 lanes of 16 bytes per
// instruction) and re-reads the whole token tile per wave. Here every
// 128-byte k-step of the 64 Wq rows and the kTok Xq rows is one stage,
// brought into LDS by direct-to-LDS transfers over whole 128-byte lines;
// kRing - 1 stages are in flight while the four waves multiply the current
// one, each wave its own 32-byte quarter of the step. Per stage and wave:
// one vmcnt wait for the wave's own transfers of the stage, one barrier (all
// waves' transfers landed; the slot of the stage before is free), the next
// transfers into that slot, then the fragment reads and MFMAs.
//
// The kernel keeps a single LDS array (the ticket word at its end): with a
// second LDS variable the accesses carry alias scopes, and the compiler then
// waits for every transfer in flight before each fragment read.
template <int kN>
__device__ __forceinline__ void ring_wait_vm() {
  __builtin_amdgcn_s_waitcnt((kN & 0xF) | ((kN >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
// wait until at most `after` stages of kDma transfers are in flight (after
// is wave-uniform, in [0, kMax])
template <int kDma, int kMax, int kI = 0>
__device__ __forceinline__ void ring_wait_stages(int after) {
  if constexpr (kI >= kMax) {
    ring_wait_vm<kMax * kDma>();
  } else {
    if (after == kI) {
      ring_wait_vm<kI * kDma>();
      return;
    }
    ring_wait_stages<kDma, kMax, kI + 1>(after);
  }
}

typedef __attribute__((address_space(3))) void lds_void_d;
typedef float v16f_d __attribute__((ext_vector_type(16)));

// kF8: E4M3 operands; each wave takes one 64-byte k-half of every stage for
// one Wq block (sqi::ring_f8_*), binary32 accumulators. The two k-halves of
// an output are added in a fixed order (wave 2 bn, then 2 bn + 1), and the
// S slices' partial tiles in slice order, so results are deterministic.
template <int kTok, bool kF8>
__global__ __launch_bounds__(256, 1) void gemm_decode_ring_kernel(DecodeArgs a) {
  using C = sqi::RingCfg<kTok>;
  constexpr int kR = C::kRing;
  static_assert((kR - 2) * C::kDma <= 63, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) int8_t smem[C::kLds + 16];
  uint32_t& last_ticket = *reinterpret_cast<uint32_t*>(smem + C::kLds);
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int tile = blockIdx.x, slice = blockIdx.y;
  const int n0 = tile * C::kRows;
  const int m0 = (int)blockIdx.z * 64;
  const int ctr = (int)blockIdx.z * (int)gridDim.x + tile;
  const sqi::DecSlice sl = sqi::dec_slice(slice, a.slice_steps, a.K);
  const int nk = sl.nsl;

  const int8_t* src[C::kDma];
  int dst[C::kDma];
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) {
    const sqi::RingDma d = sqi::ring_dma<kTok>(i, wid, lane);
    src[i] = d.w ? a.wq + sqi::big_dma_src(n0, d.row, a.N, a.K, sl.step0, d.chunk)
                 : a.xq + sqi::big_dma_src(m0, d.row, a.M, a.K, sl.step0, d.chunk);
    dst[i] = d.dst;
  }
  // stage s of the slice into ring slot b
  auto issue = [&](int s, int b) {
    int8_t* st = smem + b * C::kStage;
    const int64_t koff = (int64_t)s * kDecStep;
#pragma unroll
    for (int i = 0; i < C::kDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + koff), (lds_void_d*)(st + dst[i]), 16, 0, 0);
  };

  constexpr int kNBW = kF8 ? 1 : C::kNB;  // Wq blocks per wave
  int offw[kNBW][kF8 ? 2 : 1], offx[C::kMB][kF8 ? 2 : 1];
#pragma unroll
  for (int h = 0; h < (kF8 ? 2 : 1); ++h) {
#pragma unroll
    for (int bn = 0; bn < kNBW; ++bn)
      offw[bn][h] = kF8 ? sqi::ring_f8_frag_w<kTok>(wid, lane, h) : sqi::ring_frag_w<kTok>(bn, wid, lane);
#pragma unroll
    for (int bm = 0; bm < C::kMB; ++bm)
      offx[bm][h] = kF8 ? sqi::ring_f8_frag_x<kTok>(bm, wid, lane, h) : sqi::ring_frag_x<kTok>(bm, wid, lane);
  }

  using AccT = typename std::conditional<kF8, v16f_d, v16i>::type;
  AccT acc[kNBW][C::kMB];
#pragma unroll
  for (int bn = 0; bn < kNBW; ++bn)
#pragma unroll
    for (int bm = 0; bm < C::kMB; ++bm)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[bn][bm][r] = 0;

  int ib = 0;  // slot of the next transfer
  for (int s = 0; s < kR - 1 && s < nk; ++s) {
    issue(s, ib);
    ib = ib + 1 == kR ? 0 : ib + 1;
  }
  int rb = 0;  // slot of stage s
  for (int s = 0; s < nk; ++s) {
    // stages s+1 .. min(s + kR - 2, nk - 1) may stay in flight
    ring_wait_stages<C::kDma, kR - 2>(sqi::imin(kR - 2, nk - 1 - s));
    lds_barrier();
    if (s + kR - 1 < nk) {
      issue(s + kR - 1, ib);
      ib = ib + 1 == kR ? 0 : ib + 1;
    }
    const int8_t* st = smem + rb * C::kStage;
    if constexpr (kF8) {
      auto frag = [&](const int* off) {
        const v4i lo = *reinterpret_cast<const v4i*>(st + off[0]);
        const v4i hi = *reinterpret_cast<const v4i*>(st + off[1]);
        return v8i_d{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      };
      const v8i_d fw = frag(offw[0]);
      v8i_d fx[C::kMB];
#pragma unroll
      for (int bm = 0; bm < C::kMB; ++bm) fx[bm] = frag(offx[bm]);
#pragma unroll
      for (int bm = 0; bm < C::kMB; ++bm)
        acc[0][bm] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw, fx[bm], acc[0][bm], 0, 0, 0, 127, 0, 127);
    } else {
      v4i fw[C::kNB], fx[C::kMB];
#pragma unroll
      for (int bn = 0; bn < C::kNB; ++bn) fw[bn] = *reinterpret_cast<const v4i*>(st + offw[bn][0]);
#pragma unroll
      for (int bm = 0; bm < C::kMB; ++bm) fx[bm] = *reinterpret_cast<const v4i*>(st + offx[bm][0]);
#pragma unroll
      for (int bn = 0; bn < C::kNB; ++bn)
#pragma unroll
        for (int bm = 0; bm < C::kMB; ++bm)
          acc[bn][bm] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[bn], fx[bm], acc[bn][bm], 0, 0, 0);
    }
    rb = rb + 1 == kR ? 0 : rb + 1;
  }

  // the waves' k-parts, added through LDS (the ring is free once every
  // transfer has landed and every wave is past its last reads): int8, the
  // four k-quarters of each output; E4M3, its two k-halves in wave order
  __syncthreads();
  int32_t* red = reinterpret_cast<int32_t*>(smem);
  constexpr int kSlots = kF8 ? C::kSlotsF8 : C::kSlots;
#pragma unroll
  for (int bn = 0; bn < kNBW; ++bn)
#pragma unroll
    for (int bm = 0; bm < C::kMB; ++bm) {
      const v16i bits = __builtin_bit_cast(v16i, acc[bn][bm]);
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const v4i v = {bits[4 * rg], bits[4 * rg + 1], bits[4 * rg + 2], bits[4 * rg + 3]};
        const int slot = kF8 ? sqi::ring_f8_slot<kTok>(bm, rg, lane) : sqi::ring_slot<kTok>(bn, bm, rg, lane);
        *reinterpret_cast<v4i*>(red + 4 * (wid * kSlots + slot)) = v;
      }
    }
  __syncthreads();
  const int ml = sqi::ring_tok<kTok>(tid);
  v4i sum[C::kNG];  // int32 sums, or the bits of binary32 sums
#pragma unroll
  for (int g = 0; g < C::kNG; ++g) {
    const int nl = sqi::ring_col<kTok>(tid, g);
    if constexpr (kF8) {
      const int slot = sqi::ring_f8_read_slot<kTok>(ml, nl);
      const int w0 = 2 * (nl >> 5);
      v4f_d t = __builtin_bit_cast(v4f_d, *reinterpret_cast<const v4i*>(red + 4 * (w0 * kSlots + slot)));
      t += __builtin_bit_cast(v4f_d, *reinterpret_cast<const v4i*>(red + 4 * ((w0 + 1) * kSlots + slot)));
      sum[g] = __builtin_bit_cast(v4i, t);
    } else {
      const int slot = sqi::ring_read_slot<kTok>(ml, nl);
      v4i t = *reinterpret_cast<const v4i*>(red + 4 * slot);
#pragma unroll
      for (int w = 1; w < kDecWaves; ++w) t += *reinterpret_cast<const v4i*>(red + 4 * (w * kSlots + slot));
      sum[g] = t;
    }
  }

  if (a.S > 1) {
    // Split K: publish this slice's tile, take a ticket; the last workgroup
    // of the tile adds the slices (device-coherent accesses, as in the
    // unrolled kernel; int32 sums are exact in any order, so the own slice
    // stays in registers; E4M3 partials are added in slice order)
    const int nctr = (int)(gridDim.x * gridDim.z);
    const uint32_t pbytes = (uint32_t)a.S * (uint32_t)nctr * C::kTileBytes;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(a.partial, (short)0, pbytes, kBufDword3);
#pragma unroll
    for (int g = 0; g < C::kNG; ++g)
      __builtin_amdgcn_raw_buffer_store_b128(
          sum[g], pr, sqi::ring_partial_off(slice, nctr, ctr, g, tid, C::kTileBytes), 0, kCoherent);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last_ticket = __hip_atomic_fetch_add(a.counter + ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (last_ticket != (uint32_t)(a.S - 1)) return;
    if constexpr (kF8) {
      // all S partial tiles in slice order (this slice's from registers)
      v4f_d tot[C::kNG];
#pragma unroll
      for (int g = 0; g < C::kNG; ++g) tot[g] = v4f_d{0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < a.S; ++s) {
        v4i part[C::kNG];
#pragma unroll
        for (int g = 0; g < C::kNG; ++g)
          part[g] = s == slice ? sum[g]
                               : __builtin_amdgcn_raw_buffer_load_b128(
                                     pr, sqi::ring_partial_off(s, nctr, ctr, g, tid, C::kTileBytes), 0, kCoherent);
#pragma unroll
        for (int g = 0; g < C::kNG; ++g) tot[g] += __builtin_bit_cast(v4f_d, part[g]);
      }
#pragma unroll
      for (int g = 0; g < C::kNG; ++g) sum[g] = __builtin_bit_cast(v4i, tot[g]);
    } else {
      for (int s = 0; s < a.S; ++s) {
        if (s == slice) continue;
        v4i part[C::kNG];
#pragma unroll
        for (int g = 0; g < C::kNG; ++g)
          part[g] = __builtin_amdgcn_raw_buffer_load_b128(
              pr, sqi::ring_partial_off(s, nctr, ctr, g, tid, C::kTileBytes), 0, kCoherent);
#pragma unroll
        for (int g = 0; g < C::kNG; ++g) sum[g] += part[g];
      }
    }
    // every ticket of this tile has been drawn: restore the counter
    if (tid == 0) __hip_atomic_store(a.counter + ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int g = 0; g < C::kNG; ++g) {
    const int32_t t[4] = {sum[g][0], sum[g][1], sum[g][2], sum[g][3]};
    dec_epilogue<kF8>(a, m0 + ml, n0 + sqi::ring_col<kTok>(tid, g), t);
  }
}

}  // namespace sqk

namespace sqh {

namespace {

using sqi::decode_plan;
using sqi::DecodePlan;

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
    a.partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + kSplitCounterBytes);
  }
  const dim3 grid((unsigned)p.tiles, (unsigned)p.S, (unsigned)p.tb);
  if (sqi::dec_ring(m, kF8)) {
    if (sqi::dec_ring_tok(m) == 32)
      hipLaunchKernelGGL((sqk::gemm_decode_ring_kernel<32, kF8>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((sqk::gemm_decode_ring_kernel<64, kF8>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
  }
  if (m <= 16) return launch_decode<1, kF8>(a, p.ns, grid, s);
  return hipErrorInvalidValue;  // beyond 16 tokens the ring form always runs
}

}  // namespace

bool gemm_decode_suits(int64_t m, int64_t n, int64_t k, bool f8) { return sqi::decode_suits(m, n, k, f8); }

size_t gemm_decode_workspace(int64_t m, int64_t n, int64_t k, bool f8) {
  if (!gemm_decode_suits(m, n, k, f8)) return 0;
  return sqi::dec_workspace_bytes(decode_plan(m, n, k), m, n, sqi::dec_ring(m, f8));
}

void gemm_decode_counters(int64_t m, int64_t n, int64_t k, bool f8, void* ws, uint32_t** counters, int64_t* count) {
  *counters = nullptr;
  *count = 0;
  if (!gemm_decode_suits(m, n, k, f8)) return;
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
