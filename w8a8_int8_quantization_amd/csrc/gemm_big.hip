// Large-tile int8 MFMA GEMM for prefill-sized problems, with the fused
// dequantisation epilogue (and the LLM.int8() fp16 outlier slice).
//
// The LLM.int8() page, "The architecture: every piece explained": int8 x int8
// products accumulated in int32, scaled by the product of the row
// (token) and column (output channel) scales; the fp16 outlier slice is added
// to the dequantised product. "Half the Size, Better Performance, Same
// Accuracy: Understanding W8A8 INT8 LLM Quantization", "Performance After
// Quantization" (Inter-Token Latency): the result goes back to bf16.
//
// Design for gfx950 (256 CUs, 160 KiB LDS per CU, 64-wide waves):
//  * one 512-thread workgroup per CU computes a 256 x BN output tile
//    (BN = 256, or 192 when that fills the 256 CUs better); 8 waves, two per
//    SIMD, in a 4 x 2 grid, each owning 64 x BN/2 outputs = 2 x BN/64 blocks
//    of v_mfma_i32_32x32x32_i8 with int32 accumulators in AGPRs.
//  * K advances 128 bytes per stage through a double-buffered LDS (2 x 64
//    KiB) filled by gfx950's direct global-to-LDS transfers (global_load_lds,
//    16 bytes per lane): no registers stage the tiles, every tile row is one
//    full 128-byte line per stage (full-line requests: the L1 sustains only
//    a bounded number of requests in flight, so 64-byte requests halve the
//    bandwidth), and each stage's transfers start a full stage before it is
//    consumed. Completion is tracked with explicit vmcnt waits and one
//    barrier per stage.
//  * LDS rows are 128 bytes; the eight 16-byte chunks of row r are XOR-
//    swizzled with (r >> 1) & 7, and each transfer lane fetches the chunk
//    that belongs at its fixed LDS slot. ds_read_b128 is served 16 lanes at a
//    time: the 16 rows of such a group then hit 16 distinct bank groups.
//  * The MFMA A operand is the Wq fragment and B the Xq fragment, so a lane's
//    four consecutive accumulator registers are four consecutive output
//    columns of one token; the epilogue assembles whole output rows in LDS.
//  * Workgroups are dispatched round-robin over the 8 XCDs; the tile order
//    gives each XCD a contiguous range of tiles, grouped 4 tile-rows at a time,
//    so that tiles sharing Xq and Wq panels run under the same L2.
#include <type_traits>

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

using sqi::BigCfg;
using sqi::kBigBK;
using sqi::kBigBM;
using sqi::kBigMaxSplit;
using sqi::kBigStages;
constexpr int kSliceCols = 16;  // outlier columns staged in LDS by the LLM.int8() epilogue

enum BigOut { kBigF32 = 0, kBigBF16 = 1, kBigF16 = 2, kBigI32 = 3, kBigDecomp = 4 };

// LDS layout of a stage: 128-byte rows, 16-byte chunks XOR-swizzled by
// (row >> 1) & 7 (sqi::big_lds_off). kW waves in a (kW/2) x 2 grid over the
// 256 x BN tile (sqi::BigCfg). Eight waves (two per SIMD, 64 x BN/2 each):
// while one wave of a SIMD waits on its fragment reads or the stage barrier,
// the other keeps the matrix core busy. Four waves (one per SIMD, 128 x BN/2
// each): every fragment read feeds twice the MFMAs, so the LDS carries less
// per MFMA, and the schedule alone has to hide waits.

struct BigEpi {
  const float* x_scale;
  const float* w_scale;
  void* y;
  int64_t ldy;
  sqh::DecompArgs dec;
  bool rows16;  // y and every output row start 16-byte aligned: staged full-row stores
  // split K (kSplit kernels): S slices of slice_stages stages each; partial
  // tiles [S][tiles][256 x BN] (int32, or binary32 bits, in accumulator
  // order) and one ticket counter per tile, zero at launch and restored to
  // zero by the tile's last workgroup
  int32_t* partial;
  uint32_t* counter;
  int S;
  int slice_stages;
};

// Buffer descriptor word 3 of a raw byte buffer on gfx9, and the cache-policy
// operand of device-coherent (sc1) buffer accesses: partial tiles cross XCDs,
// whose L2 caches are not coherent with each other.
constexpr int kBigBufDword3 = 0x00020000;
constexpr int kBigCoherent = 16;

// s_waitcnt vmcnt(n) with the lgkm and exp counters left alone (gfx9 encoding).
template <int kN>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((kN & 0xF) | ((kN >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

template <int kOut>
__device__ __forceinline__ void store4(void* y, int64_t off, const float* v, const int* a, bool vec, int nvalid) {
  if (kOut == kBigI32) {
    int32_t* p = reinterpret_cast<int32_t*>(y) + off;
    if (vec) {
      *reinterpret_cast<int4*>(p) = make_int4(a[0], a[1], a[2], a[3]);
    } else {
      for (int e = 0; e < nvalid; ++e) p[e] = a[e];
    }
  } else if (kOut == kBigF32) {
    float* p = reinterpret_cast<float*>(y) + off;
    if (vec) {
      *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
      for (int e = 0; e < nvalid; ++e) p[e] = v[e];
    }
  } else {
    uint32_t h[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = kOut == kBigBF16 ? f32_to_bf16(v[e]) : f32_to_f16(v[e]);
    uint16_t* p = reinterpret_cast<uint16_t*>(y) + off;
    if (vec) {
      *reinterpret_cast<uint2*>(p) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
    } else {
      for (int e = 0; e < nvalid; ++e) p[e] = (uint16_t)h[e];
    }
  }
}

typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from a buffer resource into LDS at M0 + 16 lane (the
// builtin exists only in the device compilation).
__device__ __forceinline__ void buffer_load_lds16(__amdgpu_buffer_rsrc_t r, lds_void* dst, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// kF8: E4M3 operands (one code per byte) on v_mfma_scale_f32_32x32x64_f8f6f4
// with binary32 accumulators, two 64-k substeps per stage instead of four
// 32-k ones; everything else is shared with the int8 kernel.
// kSplit: the K range is split over blockIdx.y (see BigEpi); the tile's last
// workgroup adds the S partial tiles in slice order, then runs the epilogue.
template <int BN, int kW, int kOut, bool kVec, bool kF8 = false, bool kSplit = false>
__global__ __launch_bounds__(64 * kW, 1) void gemm_big_kernel(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                              int M, int N, int K, BigEpi ep) {
  using C = BigCfg<BN, kW>;
  using AccT = typename std::conditional<kF8, v16f, v16i>::type;
  using FragT = typename std::conditional<kF8, v8i, v4i>::type;
  constexpr int kSub = kF8 ? 2 : 4;  // MFMA k-substeps per 128-byte stage
  // Two stage buffers; stage kt lives in buffer kt % 2. The epilogue stages
  // its output bands in them as well.
  __shared__ __attribute__((aligned(1024))) int8_t smem[kBigStages * C::kStage];
  // LLM.int8(): the tile's fp16 outlier slices of X and W, gathered once
  __shared__ uint16_t slice_x[kOut == kBigDecomp ? kBigBM * kSliceCols : 1];
  __shared__ __attribute__((aligned(16))) uint16_t slice_w[kOut == kBigDecomp ? kSliceCols * BN : 1];
  // the tile's output-channel scales, read by the epilogue
  __shared__ __attribute__((aligned(16))) float scale_w[kOut == kBigI32 ? 4 : BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- tile schedule: contiguous tile ranges per XCD, grouped along M
  const int nbm = (M + kBigBM - 1) / kBigBM;
  const int nbn = (N + BN - 1) / BN;
  const int total = nbm * nbn;
  const sqi::BigTile tile = sqi::big_tile((int)blockIdx.x, nbm, nbn);
  const int tm = tile.tm, tn = tile.tn;
  const int m0 = tm * kBigBM, n0 = tn * BN;
  // this workgroup's stages: kt0 .. kt0 + nk - 1
  const sqi::BigSlice slice = sqi::big_slice(kSplit, (int)blockIdx.y, ep.slice_stages, K / kBigBK);
  const int kt0 = slice.kt0;
  const int nk = slice.nk;

  // ---- direct-to-LDS transfers: lane L of a 1 KiB transfer fills LDS bytes
  // [16L, 16L+16) of an 8-row block (sqi::big_dma), read through buffer
  // resources over the tile's rows of Xq and Wq: the lane's offset is fixed,
  // the stage is a scalar offset and the LDS destination a scalar (M0), so a
  // transfer costs no vector instructions (with per-lane 64-bit addresses
  // and a readfirstlane for M0 each one held up its wave's matrix-core issue)
  const int uwid = __builtin_amdgcn_readfirstlane(wid);
  const int rows_a = sqi::big_tile_rows(m0, M, kBigBM), rows_b = sqi::big_tile_rows(n0, N, BN);
  const __amdgpu_buffer_rsrc_t ra =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + (int64_t)m0 * K), (short)0, rows_a * K, kBigBufDword3);
  const __amdgpu_buffer_rsrc_t rb =
      __builtin_amdgcn_make_buffer_rsrc((void*)(B + (int64_t)n0 * K), (short)0, rows_b * K, kBigBufDword3);
  int voff[C::kDma];
  int dst[C::kDma];
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) {
    const sqi::BigDma d = sqi::big_dma<BN, kW>(i, uwid, lane);
    voff[i] = sqi::big_dma_voff(d.row, d.a ? rows_a : rows_b, K, d.chunk);
    dst[i] = d.dst;
  }
  auto stage_ptr = [&](int kt) { return smem + (kt & 1) * C::kStage; };
  auto dma_one = [&](int kt, int i) {
    buffer_load_lds16(i < C::kDmaA ? ra : rb, (lds_void*)(stage_ptr(kt) + dst[i]), voff[i],
                      sqi::big_dma_soff(kt0 + kt));
  };
  auto issue = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::kDma; ++i) dma_one(kt, i);
  };

  AccT acc[C::kFN][C::kFM];
#pragma unroll
  for (int j = 0; j < C::kFN; ++j)
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

  // The epilogue's scales are fetched before the first transfers, so that
  // their latency hides behind the main loop: the lane's token scales in
  // registers, the tile's channel scales in LDS.
  const int frow = lane & 31;
  float xs[C::kFM];
#pragma unroll
  for (int i = 0; i < C::kFM; ++i) {
    const int m = m0 + sqi::big_frag_row<BN, kW>(wm, i, frow);
    xs[i] = (kOut != kBigI32 && m < M) ? ep.x_scale[m] : 0.f;
  }
  float4 w4 = make_float4(0.f, 0.f, 0.f, 0.f);
  if (kOut != kBigI32 && tid < BN / 4) {
    const int n = n0 + 4 * tid;
    if (kVec && n + 4 <= N) {
      w4 = *reinterpret_cast<const float4*>(ep.w_scale + n);
    } else {
      if (n < N) w4.x = ep.w_scale[n];
      if (n + 1 < N) w4.y = ep.w_scale[n + 1];
      if (n + 2 < N) w4.z = ep.w_scale[n + 2];
      if (n + 3 < N) w4.w = ep.w_scale[n + 3];
    }
  }

  issue(0);
  if (nk > 1) issue(1);

  const int fhalf = lane >> 5;
  // Fragment of tile row r for substep ks: int8, 16 bytes (chunk 2 ks + half);
  // E4M3, 32 bytes (chunks 4 ks + 2 half and the next one).
  auto frag = [&](const int8_t* base, int r, int ks) -> FragT {
    if constexpr (kF8) {
      const int c = 4 * ks + 2 * fhalf;
      const v4i lo = *reinterpret_cast<const v4i*>(base + sqi::big_lds_off(r, c));
      const v4i hi = *reinterpret_cast<const v4i*>(base + sqi::big_lds_off(r, c + 1));
      return FragT{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    } else {
      return *reinterpret_cast<const v4i*>(base + sqi::big_lds_off(r, 2 * ks + fhalf));
    }
  };
  // Fragments of one substep: Xq blocks for this wave's tokens and Wq blocks
  // for its BN/2 output channels.
  auto read_frags = [&](const int8_t* stage, int ks, FragT* xf, FragT* wf) {
#pragma unroll
    for (int i = 0; i < C::kFM; ++i) xf[i] = frag(stage, sqi::big_frag_row<BN, kW>(wm, i, frow), ks);
#pragma unroll
    for (int j = 0; j < C::kFN; ++j) wf[j] = frag(stage + C::kStageA, sqi::big_wfrag_row<BN, kW>(wn, j, frow), ks);
  };

  // Software pipeline over the 4 substeps of a stage: the fragments of the
  // next substep are read from LDS while the MFMAs of the current one run,
  // one read after each of the first MFMAs (so they have landed well before
  // the substep ends). The stage hand-over sits in front of
  // the last substep: wait for the next stage's transfers, retire this wave's
  // LDS reads, barrier (now no wave reads the current buffer any more); the
  // transfers of the stage after next into that buffer are then issued one
  // per MFMA, by half of the waves in the last substep and by the other half
  // in the next stage's first, so the address unit works while the matrix
  // cores do (issued in one burst they stall the wave for hundreds of cycles).
  constexpr int kQ = C::kFN * C::kFM > C::kDma ? C::kFN * C::kFM : C::kDma;
  auto frag_one = [&](const int8_t* stage, int ks, int q, FragT* xf, FragT* wf) {
    if (q < C::kFM)
      xf[q] = frag(stage, sqi::big_frag_row<BN, kW>(wm, q, frow), ks);
    else
      wf[q - C::kFM] = frag(stage + C::kStageA, sqi::big_wfrag_row<BN, kW>(wn, q - C::kFM, frow), ks);
  };
  FragT fx[2][C::kFM], fw[2][C::kFN];
  if (nk > 1)
    wait_vmcnt<C::kDma>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  read_frags(stage_ptr(0), 0, fx[0], fw[0]);
  wait_lgkmcnt0();
  // The stage hand-over (transfer wait, barrier) runs in front of the last
  // substep of every stage but the last; the stage after next is transferred
  // during that substep when it exists.
  for (int kt = 0; kt < nk; ++kt) {
    const int8_t* cur = stage_ptr(kt);
#pragma unroll
    for (int ks = 0; ks < kSub; ++ks) {
      const int p = ks & 1;
      const bool trans = ks == kSub - 1 && kt + 1 < nk;
      const bool more_dma = trans && kt + 2 < nk;
      if (trans) {
        wait_vmcnt<0>();
        lds_barrier();
      }
      const int8_t* nstage = ks < kSub - 1 ? cur : stage_ptr(kt + 1);
      const int nks = ks < kSub - 1 ? ks + 1 : 0;
      const bool do_frag = ks < kSub - 1 || trans;
#pragma unroll
      for (int q = 0; q < kQ; ++q) {
        if (q < C::kFN * C::kFM) {
          const int j = q / C::kFM, i = q % C::kFM;
          if constexpr (kF8)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fw[p][j], fx[p][i], acc[j][i], 0, 0, 0, 127, 0,
                                                                       127);
          else
            acc[j][i] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fw[p][j], fx[p][i], acc[j][i], 0, 0, 0);
        }
        if (do_frag && q < C::kFM + C::kFN) frag_one(nstage, nks, q, fx[p ^ 1], fw[p ^ 1]);
        // Waves 0 .. kW/2-1 issue their transfers of stage kt + 2 in the last
        // substep of stage kt, the others in the first substep of stage
        // kt + 1 (the buffer is free from the barrier before the last
        // substep of kt; either way the transfers land before the hand-over
        // of kt + 1 waits for them): the two waves of a SIMD never issue
        // transfers at the same time, so one of them keeps the matrix core busy.
        // With two substeps per stage (E4M3) the late half would issue its
        // transfers only one substep before the hand-over waits for them
        // (QKV 58 -> 69 us): there every wave issues in the last substep.
        const bool early = kSub < 4 || uwid < kW / 2;
        if (early && more_dma && q < C::kDma) dma_one(kt + 2, q);
        if (!early && ks == 0 && kt >= 1 && kt + 1 < nk && q < C::kDma) dma_one(kt + 1, q);
        __builtin_amdgcn_sched_barrier(0);
      }
      // retire the fragment reads (issued during the MFMAs above) before
      // the next substep uses them
      wait_lgkmcnt0();
    }
  }

  if constexpr (kSplit) {
    // ---- split K: publish this slice's tile (coherent buffer stores), take
    // a ticket; the last workgroup of the tile adds all S slices in order.
    // Partial tiles are kept in accumulator order, not as rows of the
    // output: slice s, tile t, wave w, block (j, i), register group rg, lane
    // l at 16 bytes each, so every store and load instruction of a wave
    // covers 1 KiB of consecutive bytes, and ragged tiles need no bounds
    // (their padding is never stored to y).
    __shared__ uint32_t last_ticket;
    const uint32_t pbytes = (uint32_t)ep.S * (uint32_t)total * C::kTileBytes;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(ep.partial, (short)0, pbytes, kBigBufDword3);
    const int tile_id = tm * nbn + tn;
    {
      const int sl = (int)blockIdx.y;
#pragma unroll
      for (int j = 0; j < C::kFN; ++j)
#pragma unroll
        for (int i = 0; i < C::kFM; ++i) {
          // bit_cast the whole accumulator, then pick elements: a bit_cast of
          // one vector element reads element 0 of the vector in this compiler
          const v16i bits = __builtin_bit_cast(v16i, acc[j][i]);
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const v4i v = {bits[4 * rg], bits[4 * rg + 1], bits[4 * rg + 2], bits[4 * rg + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(
                v, pr, sqi::big_partial_off<BN, kW>(sl, total, tile_id, wid, lane, j * C::kFM + i, rg), 0,
                kBigCoherent);
          }
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0)
      last_ticket = __hip_atomic_fetch_add(ep.counter + tile_id, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (last_ticket != (uint32_t)(ep.S - 1)) return;
    // slice by slice, a whole slice's loads in flight together. E4M3: all S
    // partials in slice order (binary32 sums in a fixed order: deterministic
    // results); int8: the own slice stays in registers (int32 sums are exact
    // in any order)
    if constexpr (kF8) {
#pragma unroll
      for (int j = 0; j < C::kFN; ++j)
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;
    }
    for (int sl = 0; sl < ep.S; ++sl) {
      if (!kF8 && sl == (int)blockIdx.y) continue;
#pragma unroll
      for (int j = 0; j < C::kFN; ++j)
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const v4i t = __builtin_amdgcn_raw_buffer_load_b128(
                pr, sqi::big_partial_off<BN, kW>(sl, total, tile_id, wid, lane, j * C::kFM + i, rg), 0,
                kBigCoherent);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if constexpr (kF8)
                acc[j][i][4 * rg + e] += __int_as_float(t[e]);
              else
                acc[j][i][4 * rg + e] += t[e];
            }
          }
    }
    // every ticket of this tile has been drawn: restore the counter
    if (tid == 0) __hip_atomic_store(ep.counter + tile_id, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- epilogue: lane holds D[n][m] with m = l%32 and n = 8*(r/4) + 4*(l/32) + r%4 of each 32x32 block
  int mrow[C::kFM];
#pragma unroll
  for (int i = 0; i < C::kFM; ++i) mrow[i] = m0 + sqi::big_frag_row<BN, kW>(wm, i, frow);
  if (kOut != kBigI32) {
    if (tid < BN / 4) *reinterpret_cast<float4*>(&scale_w[4 * tid]) = w4;
    __syncthreads();
  }
  const int cnt = kOut == kBigDecomp ? *ep.dec.count : 0;
  // Up to kSliceCols outlier columns: gather X[tile rows][idx] and
  // W16[idx][tile columns] into LDS once (the direct version below gathers
  // them from global memory for every 32-column block of every wave).
  const bool staged = kOut == kBigDecomp && cnt <= kSliceCols;
  if (kOut == kBigDecomp && staged && cnt > 0) {
    if (tid < kBigBM) {
      const int row = tid;  // one thread per tile row
      const int64_t m = (int64_t)m0 + row;
      for (int c = 0; c < cnt; ++c)
        slice_x[row * kSliceCols + c] = m < M ? ep.dec.x[m * ep.dec.ldx + ep.dec.idx[c]] : (uint16_t)0;
    }
    for (int e = tid; e < cnt * BN; e += C::kThreads) {
      const int c = e / BN, nl = e - c * BN;
      const int64_t n = (int64_t)n0 + nl;
      slice_w[c * BN + nl] = n < N ? ep.dec.w16[(int64_t)ep.dec.idx[c] * ep.dec.ldw + n] : (uint16_t)0;
    }
    __syncthreads();
  }
  // fp16 outlier-slice products of fragments i in [i0, i1) for column block j
  auto outlier_slice = [&](int j, int i0, int i1, float (*yo)[16]) {
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) yo[i][r] = 0.f;
    if (staged) {
      for (int c = 0; c < cnt; ++c) {
        float xv[C::kFM];
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
          xv[i] = (i >= i0 && i < i1) ? f16_to_f32(slice_x[sqi::big_frag_row<BN, kW>(wm, i, frow) * kSliceCols + c]) : 0.f;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int nl = sqi::big_frag_col<BN, kW>(wn, j, rg, fhalf);
          const uint2 wp = *reinterpret_cast<const uint2*>(&slice_w[c * BN + nl]);
          const float wv[4] = {f16_to_f32((uint16_t)(wp.x & 0xFFFFu)), f16_to_f32((uint16_t)(wp.x >> 16)),
                               f16_to_f32((uint16_t)(wp.y & 0xFFFFu)), f16_to_f32((uint16_t)(wp.y >> 16))};
          // fp16 x fp16 is exact in binary32 (22 significant bits), so one
          // fused multiply-add rounds exactly like product-then-sum
#pragma unroll
          for (int i = 0; i < C::kFM; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) yo[i][4 * rg + e] = __builtin_fmaf(xv[i], wv[e], yo[i][4 * rg + e]);
        }
      }
      return;
    }
    for (int c = 0; c < cnt; ++c) {
      const int64_t jc = ep.dec.idx[c];
      float xv[C::kFM];
#pragma unroll
      for (int i = 0; i < C::kFM; ++i)
        xv[i] = (i >= i0 && i < i1 && mrow[i] < M) ? f16_to_f32(ep.dec.x[(int64_t)mrow[i] * ep.dec.ldx + jc]) : 0.f;
      const uint16_t* wrow = ep.dec.w16 + jc * ep.dec.ldw;
#pragma unroll
      for (int rg = 0; rg < 4; ++rg) {
        const int n = n0 + sqi::big_frag_col<BN, kW>(wn, j, rg, fhalf);
        float wv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) wv[e] = n + e < N ? f16_to_f32(wrow[n + e]) : 0.f;
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
          for (int e = 0; e < 4; ++e) yo[i][4 * rg + e] = __fadd_rn(yo[i][4 * rg + e], __fmul_rn(xv[i], wv[e]));
      }
    }
  };
  // column scales of the 4 outputs a lane holds in row group rg of block j
  // (zero past N), from the LDS copy
  auto col_scales = [&](int n, int nvalid, float* ws) {
    if (kOut == kBigI32) {
      ws[0] = ws[1] = ws[2] = ws[3] = 0.f;
      return;
    }
    (void)nvalid;
    const float4 c4 = *reinterpret_cast<const float4*>(&scale_w[n - n0]);
    ws[0] = c4.x; ws[1] = c4.y; ws[2] = c4.z; ws[3] = c4.w;
  };
  // output values of fragment (j, i), row group rg: dequantised, plus the
  // outlier slice for LLM.int8()
  auto out_values = [&](int j, int i, int rg, const float* ws, const float (*yo)[16], float* v, int* a) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float av;
      if constexpr (kF8) {
        a[e] = 0;
        av = acc[j][i][4 * rg + e];
      } else {
        a[e] = acc[j][i][4 * rg + e];
        av = (float)a[e];
      }
      v[e] = __fmul_rn(__fmul_rn(av, xs[i]), ws[e]);
      if (kOut == kBigDecomp) {
        const float yi = f16_to_f32(f32_to_f16(v[e]));
        v[e] = __fadd_rn(yi, f16_to_f32(f32_to_f16(yo[i][4 * rg + e])));
      }
    }
  };

  if (ep.rows16) {
    // Staged through LDS, one band at a time: the lanes' 4-column pieces are
    // assembled into whole rows, which then leave as 16-byte chunks,
    // consecutive threads writing consecutive chunks of a row (whole 128-byte
    // lines; written straight from the fragments, 32 rows x 16 bytes per
    // instruction, the partial lines cost about three times the output size
    // in HBM writes). Band (i, h) holds fragment row block i of every wave
    // row (kW/2 x 32 tile rows) and, for 4-byte outputs, column half h (all
    // BN columns for 2-byte outputs). Bands alternate between the two stage
    // buffers, so one barrier per band separates its writes from its
    // copy-out: the copy-out of band b and the writes of band b + 1 use
    // different buffers. Chunk c of staged row r sits at chunk (c + r) mod
    // kCh, which spreads the 32 rows of a fragment write over the banks.
    constexpr int kEl = (kOut == kBigF32 || kOut == kBigI32) ? 4 : 2;
    using Band = sqi::BigBand<BN, kW, kEl>;
    constexpr int kRows = Band::kRows;    // rows per band
    constexpr int kParts = Band::kParts;  // column parts per band row block
    constexpr int kColsB = Band::kColsB;  // columns per band
    constexpr int kRowB = Band::kRowB;    // staged row bytes
    constexpr int kCh = Band::kCh;        // 16-byte chunks per staged row
    constexpr int kPer = Band::kPer;      // outputs per chunk
    __syncthreads();  // every wave is done with the stage buffers
#pragma unroll
    for (int b = 0; b < C::kFM * kParts; ++b) {
      const int i = b / kParts, h = b % kParts;
      int8_t* const buf = smem + (b & 1) * C::kStage;
      if (kParts == 1 || wn == h) {
        const int lr = wm * 32 + frow;  // row within the band
#pragma unroll
        for (int j = 0; j < C::kFN; ++j) {
          float yo[kOut == kBigDecomp ? C::kFM : 1][16];
          if (kOut == kBigDecomp) outlier_slice(j, i, i + 1, yo);
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const int nl = sqi::big_frag_col<BN, kW>(wn, j, rg, fhalf);
            float ws[4];
            col_scales(n0 + nl, 4, ws);
            int a[4];
            float v[4];
            out_values(j, i, rg, ws, yo, v, a);
            const int cb = (nl - h * kColsB) * kEl;  // byte offset within the staged row
            const int pc = sqi::band_chunk(cb >> 4, lr, kCh);
            int8_t* dst = buf + lr * kRowB + pc * 16 + (cb & 15);
            if (kOut == kBigI32) {
              *reinterpret_cast<int4*>(dst) = make_int4(a[0], a[1], a[2], a[3]);
            } else if (kOut == kBigF32) {
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else if (kOut == kBigBF16) {
              *reinterpret_cast<uint2*>(dst) = make_uint2(bf16x2_rn(v[0], v[1]), bf16x2_rn(v[2], v[3]));
            } else {
              uint32_t hb[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) hb[e] = f32_to_f16(v[e]);
              *reinterpret_cast<uint2*>(dst) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
            }
          }
        }
      }
      __syncthreads();
      for (int c = tid; c < kRows * kCh; c += C::kThreads) {
        const int lr = c / kCh, ch = c - lr * kCh;
        const int m = m0 + sqi::band_tile_row<BN, kW>(lr, i);
        const int n = n0 + h * kColsB + ch * kPer;
        if (m >= M || n >= N) continue;
        const int8_t* srcp = buf + lr * kRowB + sqi::band_chunk(ch, lr, kCh) * 16;
        int8_t* dst = reinterpret_cast<int8_t*>(ep.y) + ((int64_t)m * ep.ldy + n) * kEl;
        if (n + kPer <= N) {
          *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(srcp);
        } else {
          for (int e = 0; e < (N - n) * kEl; ++e) dst[e] = srcp[e];
        }
      }
    }
    return;
  }

  // Direct stores (output rows not 16-byte aligned): 4 outputs per lane.
#pragma unroll
  for (int j = 0; j < C::kFN; ++j) {
    float yo[kOut == kBigDecomp ? C::kFM : 1][16];
    if (kOut == kBigDecomp) outlier_slice(j, 0, C::kFM, yo);
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int n = n0 + sqi::big_frag_col<BN, kW>(wn, j, rg, fhalf);
      if (n >= N) continue;
      const int nvalid = min(4, N - n);
      float ws[4];
      col_scales(n, nvalid, ws);
#pragma unroll
      for (int i = 0; i < C::kFM; ++i) {
        const int m = mrow[i];
        if (m >= M) continue;
        int a[4];
        float v[4];
        out_values(j, i, rg, ws, yo, v, a);
        const int64_t off = (int64_t)m * ep.ldy + n;
        store4<kOut == kBigDecomp ? kBigF16 : kOut>(ep.y, off, v, a, kVec && nvalid == 4, nvalid);
      }
    }
  }
}

template <int BN, int kW, int kOut, bool kVec, bool kF8 = false>
static void launch_big(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, hipStream_t s) {
  const int tiles = ((M + kBigBM - 1) / kBigBM) * ((N + BN - 1) / BN);
  if (ep.S > 1 && kOut != kBigDecomp)
    hipLaunchKernelGGL((gemm_big_kernel<BN, kW, kOut, kVec, kF8, kOut != kBigDecomp>), dim3(tiles, ep.S),
                       dim3(64 * kW), 0, s, xq, wq, M, N, K, ep);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BN, kW, kOut, kVec, kF8, false>), dim3(tiles), dim3(64 * kW), 0, s, xq,
                       wq, M, N, K, ep);
}

template <int BN, int kW, int kOut, bool kF8 = false>
static void launch_big_v(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, bool vec,
                         hipStream_t s) {
  if (vec)
    launch_big<BN, kW, kOut, true, kF8>(xq, wq, M, N, K, ep, s);
  else
    launch_big<BN, kW, kOut, false, kF8>(xq, wq, M, N, K, ep, s);
}

template <int BN, int kW = 8>
static void launch_big_o(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, int out, bool vec,
                         hipStream_t s) {
  switch (out) {
    case kBigF32: launch_big_v<BN, kW, kBigF32>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigBF16: launch_big_v<BN, kW, kBigBF16>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigF16: launch_big_v<BN, kW, kBigF16>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigI32: launch_big_v<BN, kW, kBigI32>(xq, wq, M, N, K, ep, vec, s); break;
    default: launch_big_v<BN, kW, kBigDecomp>(xq, wq, M, N, K, ep, vec, s); break;
  }
}

// E4M3 operands, 256-column tiles on four waves (one per SIMD, 128 x 128
// outputs each: the accumulators and two fragment sets need more registers
// than a lane has at two waves per SIMD), K not split.
template <int kOut>
static void launch_big_f8_w4(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, bool vec,
                             hipStream_t s) {
  const int tiles = ((M + kBigBM - 1) / kBigBM) * ((N + 255) / 256);
  if (vec)
    hipLaunchKernelGGL((gemm_big_kernel<256, 4, kOut, true, true, false>), dim3(tiles), dim3(256), 0, s, xq, wq, M, N,
                       K, ep);
  else
    hipLaunchKernelGGL((gemm_big_kernel<256, 4, kOut, false, true, false>), dim3(tiles), dim3(256), 0, s, xq, wq, M,
                       N, K, ep);
}

// E4M3 operands: floating-point outputs only
template <int BN, int kW = 8>
static void launch_big_f8(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, int out,
                          bool vec, hipStream_t s) {
  switch (out) {
    case kBigF32: launch_big_v<BN, kW, kBigF32, true>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigBF16: launch_big_v<BN, kW, kBigBF16, true>(xq, wq, M, N, K, ep, vec, s); break;
    default: launch_big_v<BN, kW, kBigF16, true>(xq, wq, M, N, K, ep, vec, s); break;
  }
}

}  // namespace sqk

// The host code below is compiled twice (build.py): the int8 entry points,
// and, with SQ_BIG_E4M3 defined, the E4M3 one. The E4M3 object is built
// without LLVM's machine-code sinking: with it, the E4M3 main loop's matrix
// instructions sink past the conditional stage transfers of the hand-over
// substep, so a stage's twelve MFMAs issue back to back after all of its
// fragment reads instead of one between each pair (QKV prefill E4M3 GEMM
// 59.2 -> 48.4 us without the pass); the int8 instances keep the default
// pipeline.
namespace sqh {

#ifndef SQ_BIG_E4M3
bool gemm_big_suits(int64_t m, int64_t n, int64_t k, bool split_ok) { return sqi::big_suits(m, n, k, split_ok); }

namespace {
using sqi::BigSplit;
BigSplit big_split(int64_t m, int64_t n, int64_t k, bool f8, bool split_ok = true) {
  return sqi::big_split(m, n, k, f8, split_ok);
}
}  // namespace

size_t gemm_big_workspace(int64_t m, int64_t n, int64_t k, bool f8) {
  if (!gemm_big_suits(m, n, k)) return 0;
  return sqi::big_workspace_bytes(big_split(m, n, k, f8));
}

void gemm_big_counters(int64_t m, int64_t n, int64_t k, bool f8, void* ws, uint32_t** counters, int64_t* count) {
  *counters = nullptr;
  *count = 0;
  if (!gemm_big_suits(m, n, k)) return;
  const BigSplit p = big_split(m, n, k, f8);
  if (p.S == 1) return;
  *counters = reinterpret_cast<uint32_t*>(ws);
  *count = p.tiles;
}

hipError_t gemm_i8_big(const int8_t* xq, const float* x_scale, const int8_t* wq, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, const DecompArgs* dec, void* ws,
                       hipStream_t s) {
  sqk::BigEpi ep{x_scale, w_scale, y, ldy, dec ? *dec : DecompArgs{}, false, nullptr, nullptr, 1, 0};
  const BigSplit sp = big_split(m, n, k, false, dec == nullptr);
  if (sp.S > 1) {
    ep.S = sp.S;
    ep.slice_stages = sp.slice_stages;
    ep.counter = reinterpret_cast<uint32_t*>(ws);
    ep.partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + kSplitCounterBytes);
  }
  int out;
  int eb;
  if (dec) {
    out = sqk::kBigDecomp; eb = 2;
  } else {
    switch (yt) {
      case SQ_F32: out = sqk::kBigF32; eb = 4; break;
      case SQ_BF16: out = sqk::kBigBF16; eb = 2; break;
      case SQ_F16: out = sqk::kBigF16; eb = 2; break;
      default: out = sqk::kBigI32; eb = 4; break;
    }
  }
  const bool vec = (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % (uintptr_t)(4 * eb) == 0) &&
                   (out == sqk::kBigI32 || reinterpret_cast<uintptr_t>(w_scale) % 16 == 0);
  ep.rows16 = (ldy * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
  const int M = (int)m, N = (int)n, K = (int)k;
  if (sp.bn == 128)
    sqk::launch_big_o<128>(xq, wq, M, N, K, ep, out, vec, s);
  else if (sp.bn == 192)
    sqk::launch_big_o<192>(xq, wq, M, N, K, ep, out, vec, s);
  else
    sqk::launch_big_o<256>(xq, wq, M, N, K, ep, out, vec, s);
  return hipGetLastError();
}

#else  // SQ_BIG_E4M3

hipError_t gemm_f8_big(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  sqk::BigEpi ep{x_scale, w_scale, y, ldy, DecompArgs{}, false, nullptr, nullptr, 1, 0};
  const sqi::BigSplit sp = sqi::big_split(m, n, k, true, true);
  if (sp.S > 1) {
    ep.S = sp.S;
    ep.slice_stages = sp.slice_stages;
    ep.counter = reinterpret_cast<uint32_t*>(ws);
    ep.partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + kSplitCounterBytes);
  }
  const int out = yt == SQ_F32 ? sqk::kBigF32 : (yt == SQ_BF16 ? sqk::kBigBF16 : sqk::kBigF16);
  const int eb = yt == SQ_F32 ? 4 : 2;
  const bool vec = (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % (uintptr_t)(4 * eb) == 0) &&
                   reinterpret_cast<uintptr_t>(w_scale) % 16 == 0;
  ep.rows16 = (ldy * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
  const int M = (int)m, N = (int)n, K = (int)k;
  // 192- or 128-column tiles on eight waves: the E4M3 fragments are twice
  // the int8 ones, and with 256 columns the accumulators and two fragment
  // sets exceed the 256 registers a lane has at two waves per SIMD. Where
  // 256-column tiles fill the CUs at least once and K is not split, four
  // waves of 128 x 128 outputs take them instead (one wave per SIMD, 512
  // registers a lane): 8192 x 4096 -> 28672 903.5 -> 839.1 us, 8192 x 14336
  // -> 4096 447.0 -> 370.3 us (the same accumulation order per output, so
  // the same bits); QKV at 2048 tokens (192 such tiles) stays on 192 columns.
  const int64_t tiles256 = ((m + sqi::kBigBM - 1) / sqi::kBigBM) * ((n + 255) / 256);
  if (sp.S == 1 && tiles256 >= 256) {
    const int8_t* a8 = reinterpret_cast<const int8_t*>(xq);
    const int8_t* b8 = reinterpret_cast<const int8_t*>(wq);
    if (out == sqk::kBigF32)
      sqk::launch_big_f8_w4<sqk::kBigF32>(a8, b8, M, N, K, ep, vec, s);
    else if (out == sqk::kBigBF16)
      sqk::launch_big_f8_w4<sqk::kBigBF16>(a8, b8, M, N, K, ep, vec, s);
    else
      sqk::launch_big_f8_w4<sqk::kBigF16>(a8, b8, M, N, K, ep, vec, s);
  } else if (sp.bn == 128)
    sqk::launch_big_f8<128>(reinterpret_cast<const int8_t*>(xq), reinterpret_cast<const int8_t*>(wq), M, N, K, ep,
                            out, vec, s);
  else
    sqk::launch_big_f8<192>(reinterpret_cast<const int8_t*>(xq), reinterpret_cast<const int8_t*>(wq), M, N, K, ep,
                            out, vec, s);
  return hipGetLastError();
}

#endif  // SQ_BIG_E4M3

}  // namespace sqh
