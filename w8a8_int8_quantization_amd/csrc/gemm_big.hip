// Large-tile int8 MFMA GEMM for prefill-sized problems, with the fused
// dequantisation epilogue (and the LLM.int8() fp16 outlier slice).
//
// The LLM.int8() page, "The architecture: every piece explained": int8 x int8
// products accumulated in int32, scaled by the outer product of the row
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
#include <cstdlib>
#include <type_traits>

#include "sq_common.hpp"
#include "sq_launch.hpp"

namespace sqk {

constexpr int kBigBM = 256;
// Eight waves, two per SIMD, in a 4 x 2 grid over the tile: while one wave of
// a SIMD waits on its fragment reads or the stage barrier, the other keeps the
// matrix core busy (measured on MI355X against four waves of twice the
// sub-tile: QKV 62 -> 55 us, gate/up 1010 -> 942 us, down 425 -> 406 us), at
// the price of ~40% more LDS fragment reads, which the LDS has room for.
constexpr int kBigWaves = 8;
constexpr int kBigThreads = 64 * kBigWaves;
constexpr int kBigBK = 128;    // k bytes per pipeline stage: one 128-byte line per tile row
constexpr int kBigStages = 2;  // LDS double buffer
constexpr int kGroupM = 4;
constexpr int kSliceCols = 16;  // outlier columns staged in LDS by the LLM.int8() epilogue

enum BigOut { kBigF32 = 0, kBigBF16 = 1, kBigF16 = 2, kBigI32 = 3, kBigDecomp = 4 };

// Byte offset of 16-byte chunk c (0..7) of tile row r in a stage (128-byte
// rows). The chunk index is XOR-ed with (r >> 1) & 7: a 128-byte row covers
// half of the 64 banks, so rows r and r+1 fall in different halves, and the
// eight even (odd) rows of a 16-lane group get eight distinct chunks. Without
// it every lane of a half-wave would hit the same bank group; with r & 7,
// rows r and r + 8 collided (measured: 3.96M bank-conflict cycles per QKV
// dispatch, 0.29M with this one).
__device__ __forceinline__ int big_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int big_lds_off(int r, int c) { return r * kBigBK + ((c ^ big_swz(r)) << 4); }

template <int BN>
struct BigCfg {
  static constexpr int kWN = BN / 2;                  // output columns per wave
  static constexpr int kFN = kWN / 32;
  static constexpr int kWM = kBigBM / (kBigWaves / 2);  // tokens per wave
  static constexpr int kFM = kWM / 32;
  static constexpr int kStageA = kBigBM * kBigBK;
  static constexpr int kStage = (kBigBM + BN) * kBigBK;
  // 1 KiB direct-to-LDS transfers (8 rows each) per wave and stage
  static constexpr int kDmaA = kBigBM / 8 / kBigWaves;
  static constexpr int kDmaB = BN / 8 / kBigWaves;
  static constexpr int kDma = kDmaA + kDmaB;
};

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
// at most this many K slices per output tile
constexpr int kBigMaxSplit = 8;
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

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

// kF8: E4M3 operands (one code per byte) on v_mfma_scale_f32_32x32x64_f8f6f4
// with binary32 accumulators, two 64-k substeps per stage instead of four
// 32-k ones; everything else is shared with the int8 kernel.
// kSplit: the K range is split over blockIdx.y (see BigEpi); the tile's last
// workgroup adds the S partial tiles in slice order, then runs the epilogue.
template <int BN, int kOut, bool kVec, bool kF8 = false, bool kSplit = false>
__global__ __launch_bounds__(kBigThreads, 1) void gemm_big_kernel(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                          int M, int N, int K, BigEpi ep) {
  using C = BigCfg<BN>;
  using AccT = typename std::conditional<kF8, v16f, v16i>::type;
  using FragT = typename std::conditional<kF8, v8i, v4i>::type;
  constexpr int kSub = kF8 ? 2 : 4;  // MFMA k-substeps per 128-byte stage
  __shared__ __attribute__((aligned(1024))) int8_t smem[kBigStages * C::kStage];
  // LLM.int8(): the tile's fp16 outlier slices of X and W, gathered once
  __shared__ uint16_t slice_x[kOut == kBigDecomp ? kBigBM * kSliceCols : 1];
  __shared__ __attribute__((aligned(16))) uint16_t slice_w[kOut == kBigDecomp ? kSliceCols * BN : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  // ---- tile schedule: contiguous tile ranges per XCD, grouped along M
  const int nbm = (M + kBigBM - 1) / kBigBM;
  const int nbn = (N + BN - 1) / BN;
  const int total = nbm * nbn;
  int t = blockIdx.x;
  const int full = total & ~7;
  if (t < full) t = (t & 7) * (full >> 3) + (t >> 3);
  const int in_group = kGroupM * nbn;
  const int first_m = (t / in_group) * kGroupM;
  const int gm = min(nbm - first_m, kGroupM);
  const int tm = first_m + (t % in_group) % gm;
  const int tn = (t % in_group) / gm;
  const int m0 = tm * kBigBM, n0 = tn * BN;
  // this workgroup's stages: kt0 .. kt0 + nk - 1
  const int kt0 = kSplit ? (int)blockIdx.y * ep.slice_stages : 0;
  const int nk = kSplit ? min(ep.slice_stages, K / kBigBK - kt0) : K / kBigBK;

  // ---- direct-to-LDS transfers: lane L of a 1 KiB transfer fills LDS bytes
  // [16L, 16L+16) of an 8-row block, i.e. row L/8, physical chunk L%8, so it
  // fetches the logical chunk (L%8) ^ swizzle(row) of that row from HBM; the
  // 8 lanes of a row read one whole 128-byte line.
  const int8_t* src[C::kDma];
  int dst[C::kDma];
#pragma unroll
  for (int i = 0; i < C::kDma; ++i) {
    const bool is_a = i < C::kDmaA;
    const int blk = (is_a ? i : i - C::kDmaA) * kBigWaves + wid;  // 8-row block within the operand tile
    const int r = blk * 8 + (lane >> 3);
    const int c = (lane & 7) ^ big_swz(r);
    if (is_a) {
      src[i] = A + (int64_t)min(m0 + r, M - 1) * K + (int64_t)kt0 * kBigBK + c * 16;
      dst[i] = blk * 1024;
    } else {
      src[i] = B + (int64_t)min(n0 + r, N - 1) * K + (int64_t)kt0 * kBigBK + c * 16;
      dst[i] = C::kStageA + blk * 1024;
    }
  }
  auto issue = [&](int kt) {
    int8_t* stage = smem + (kt % kBigStages) * C::kStage;
    const int64_t koff = (int64_t)kt * kBigBK;
#pragma unroll
    for (int i = 0; i < C::kDma; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(src[i] + koff), (lds_void*)(stage + dst[i]), 16, 0, 0);
  };

  AccT acc[C::kFN][C::kFM];
#pragma unroll
  for (int j = 0; j < C::kFN; ++j)
#pragma unroll
    for (int i = 0; i < C::kFM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

  issue(0);
  if (nk > 1) issue(1);

  const int frow = lane & 31;
  const int fhalf = lane >> 5;
  // Fragment of tile row r for substep ks: int8, 16 bytes (chunk 2 ks + half);
  // E4M3, 32 bytes (chunks 4 ks + 2 half and the next one).
  auto frag = [&](const int8_t* base, int r, int ks) -> FragT {
    if constexpr (kF8) {
      const int c = 4 * ks + 2 * fhalf;
      const v4i lo = *reinterpret_cast<const v4i*>(base + big_lds_off(r, c));
      const v4i hi = *reinterpret_cast<const v4i*>(base + big_lds_off(r, c + 1));
      return FragT{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    } else {
      return *reinterpret_cast<const v4i*>(base + big_lds_off(r, 2 * ks + fhalf));
    }
  };
  // Fragments of one substep: Xq blocks for this wave's tokens and Wq blocks
  // for its BN/2 output channels.
  auto read_frags = [&](const int8_t* stage, int ks, FragT* xf, FragT* wf) {
#pragma unroll
    for (int i = 0; i < C::kFM; ++i) xf[i] = frag(stage, wm * C::kWM + 32 * i + frow, ks);
#pragma unroll
    for (int j = 0; j < C::kFN; ++j) wf[j] = frag(stage + C::kStageA, wn * C::kWN + 32 * j + frow, ks);
  };
  auto stage_ptr = [&](int kt) { return smem + (kt & 1) * C::kStage; };

  // Software pipeline over the 4 substeps of a stage: the fragments of the
  // next substep are read from LDS while the MFMAs of the current one run,
  // one read after each of the first MFMAs (so they have landed well before
  // the substep ends). The stage hand-over sits in front of
  // the last substep: wait for the next stage's transfers, retire this wave's
  // LDS reads, barrier (now no wave reads the current buffer any more); the
  // transfers of the stage after next into that buffer are then issued one
  // per MFMA of the last substep, so the address unit works while the matrix
  // cores do (issued in one burst they stall the wave for hundreds of cycles).
  constexpr int kQ = C::kFN * C::kFM > C::kDma ? C::kFN * C::kFM : C::kDma;
  auto dma_one = [&](int kt, int i) {
    int8_t* stage = smem + (kt & 1) * C::kStage;
    __builtin_amdgcn_global_load_lds((const void*)(src[i] + (int64_t)kt * kBigBK), (lds_void*)(stage + dst[i]), 16, 0,
                                     0);
  };
  auto frag_one = [&](const int8_t* stage, int ks, int q, FragT* xf, FragT* wf) {
    if (q < C::kFM)
      xf[q] = frag(stage, wm * C::kWM + 32 * q + frow, ks);
    else
      wf[q - C::kFM] = frag(stage + C::kStageA, wn * C::kWN + 32 * (q - C::kFM) + frow, ks);
  };
  FragT fx[2][C::kFM], fw[2][C::kFN];
  if (nk > 1)
    wait_vmcnt<C::kDma>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  read_frags(stage_ptr(0), 0, fx[0], fw[0]);
  wait_lgkmcnt0();
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
        if (more_dma && q < C::kDma) dma_one(kt + 2, q);
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
    constexpr uint32_t kTileBytes = kBigBM * BN * 4;
    constexpr uint32_t kWaveBytes = kTileBytes / kBigWaves;
    const uint32_t pbytes = (uint32_t)ep.S * (uint32_t)total * kTileBytes;
    const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(ep.partial, (short)0, pbytes, kBigBufDword3);
    const int tile_id = tm * nbn + tn;
    const uint32_t lane_off = (uint32_t)wid * kWaveBytes + (uint32_t)lane * 16;
    auto slice_base = [&](int sl) { return ((uint32_t)sl * (uint32_t)total + (uint32_t)tile_id) * kTileBytes + lane_off; };
    {
      const uint32_t base = slice_base((int)blockIdx.y);
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
            __builtin_amdgcn_raw_buffer_store_b128(v, pr, base + (uint32_t)((j * C::kFM + i) * 4 + rg) * 1024, 0,
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
      const uint32_t base = slice_base(sl);
#pragma unroll
      for (int j = 0; j < C::kFN; ++j)
#pragma unroll
        for (int i = 0; i < C::kFM; ++i)
#pragma unroll
          for (int rg = 0; rg < 4; ++rg) {
            const v4i t = __builtin_amdgcn_raw_buffer_load_b128(
                pr, base + (uint32_t)((j * C::kFM + i) * 4 + rg) * 1024, 0, kBigCoherent);
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
  const int mw = m0 + wm * C::kWM;
  const int nw = n0 + wn * C::kWN;
  int mrow[C::kFM];
  float xs[C::kFM];
#pragma unroll
  for (int i = 0; i < C::kFM; ++i) {
    mrow[i] = mw + 32 * i + frow;
    xs[i] = (kOut != kBigI32 && mrow[i] < M) ? ep.x_scale[mrow[i]] : 0.f;
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
    for (int e = tid; e < cnt * BN; e += kBigThreads) {
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
          xv[i] = (i >= i0 && i < i1) ? f16_to_f32(slice_x[(wm * C::kWM + 32 * i + frow) * kSliceCols + c]) : 0.f;
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int nl = wn * C::kWN + 32 * j + 8 * rg + 4 * fhalf;
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
        const int n = nw + 32 * j + 8 * rg + 4 * fhalf;
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
  auto col_scales = [&](int n, int nvalid, float* ws) {
    ws[0] = ws[1] = ws[2] = ws[3] = 0.f;
    if (kOut == kBigI32 || n >= N) return;
    if (kVec && nvalid == 4) {
      const float4 w4 = *reinterpret_cast<const float4*>(ep.w_scale + n);
      ws[0] = w4.x; ws[1] = w4.y; ws[2] = w4.z; ws[3] = w4.w;
    } else {
      for (int e = 0; e < nvalid; ++e) ws[e] = ep.w_scale[n + e];
    }
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
    // Staged through LDS, one band of tile rows at a time: the lanes' 4-column
    // pieces are assembled into whole tile rows, which then leave as 16-byte
    // chunks, consecutive threads writing consecutive chunks of a row (whole
    // 128-byte lines; written straight from the fragments, 32 rows x 16 bytes
    // per instruction, the partial lines cost about three times the output
    // size in HBM writes).
    constexpr int kEl = (kOut == kBigF32 || kOut == kBigI32) ? 4 : 2;
    constexpr int kRowB = BN * kEl + 16;  // staged row pitch; the pad spreads the row-strided writes over the banks
    constexpr int kBand = 128 * kRowB <= kBigStages * C::kStage ? 128 : 64;
    constexpr int kChunks = BN * kEl / 16;
    constexpr int kPer = 16 / kEl;  // outputs per chunk
#pragma unroll 1
    for (int band = 0; band < kBigBM / kBand; ++band) {
      __syncthreads();  // every wave is done with the LDS contents
#pragma unroll
      for (int j = 0; j < C::kFN; ++j) {
        // fragments of this wave inside the band (the test is uniform per wave)
        const int i0 = (band * kBand - wm * C::kWM) / 32;
        const int lo = i0 < 0 ? 0 : i0, hi = min(C::kFM, i0 + kBand / 32);
        if (lo >= hi) continue;
        float yo[kOut == kBigDecomp ? C::kFM : 1][16];
        if (kOut == kBigDecomp) outlier_slice(j, lo, hi, yo);
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int nl = wn * C::kWN + 32 * j + 8 * rg + 4 * fhalf;
          const int n = n0 + nl;
          float ws[4];
          col_scales(n, min(4, N - n), ws);
#pragma unroll
          for (int i = 0; i < C::kFM; ++i) {
            if (i < lo || i >= hi) continue;
            int a[4];
            float v[4];
            out_values(j, i, rg, ws, yo, v, a);
            int8_t* dst = smem + (wm * C::kWM + 32 * i + frow - band * kBand) * kRowB + nl * kEl;
            if (kOut == kBigI32) {
              *reinterpret_cast<int4*>(dst) = make_int4(a[0], a[1], a[2], a[3]);
            } else if (kOut == kBigF32) {
              *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
              uint32_t h[4];
#pragma unroll
              for (int e = 0; e < 4; ++e)
                h[e] = (kOut == kBigBF16) ? f32_to_bf16(v[e]) : f32_to_f16(v[e]);
              *reinterpret_cast<uint2*>(dst) = make_uint2(h[0] | (h[1] << 16), h[2] | (h[3] << 16));
            }
          }
        }
      }
      __syncthreads();
      for (int c = tid; c < kBand * kChunks; c += kBigThreads) {
        const int r = c / kChunks, ch = c - r * kChunks;
        const int m = m0 + band * kBand + r;
        const int n = n0 + ch * kPer;
        if (m >= M || n >= N) continue;
        const int8_t* srcp = smem + r * kRowB + ch * 16;
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
      const int n = nw + 32 * j + 8 * rg + 4 * fhalf;
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

template <int BN, int kOut, bool kVec, bool kF8 = false>
static void launch_big(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, hipStream_t s) {
  const int tiles = ((M + kBigBM - 1) / kBigBM) * ((N + BN - 1) / BN);
  if (ep.S > 1 && kOut != kBigDecomp)
    hipLaunchKernelGGL((gemm_big_kernel<BN, kOut, kVec, kF8, kOut != kBigDecomp>), dim3(tiles, ep.S),
                       dim3(kBigThreads), 0, s, xq, wq, M, N, K, ep);
  else
    hipLaunchKernelGGL((gemm_big_kernel<BN, kOut, kVec, kF8>), dim3(tiles), dim3(kBigThreads), 0, s, xq, wq, M, N,
                       K, ep);
}

template <int BN, int kOut, bool kF8 = false>
static void launch_big_v(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, bool vec,
                         hipStream_t s) {
  if (vec)
    launch_big<BN, kOut, true, kF8>(xq, wq, M, N, K, ep, s);
  else
    launch_big<BN, kOut, false, kF8>(xq, wq, M, N, K, ep, s);
}

template <int BN>
static void launch_big_o(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, int out, bool vec,
                         hipStream_t s) {
  switch (out) {
    case kBigF32: launch_big_v<BN, kBigF32>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigBF16: launch_big_v<BN, kBigBF16>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigF16: launch_big_v<BN, kBigF16>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigI32: launch_big_v<BN, kBigI32>(xq, wq, M, N, K, ep, vec, s); break;
    default: launch_big_v<BN, kBigDecomp>(xq, wq, M, N, K, ep, vec, s); break;
  }
}

// E4M3 operands: floating-point outputs only
template <int BN>
static void launch_big_f8(const int8_t* xq, const int8_t* wq, int M, int N, int K, const BigEpi& ep, int out,
                          bool vec, hipStream_t s) {
  switch (out) {
    case kBigF32: launch_big_v<BN, kBigF32, true>(xq, wq, M, N, K, ep, vec, s); break;
    case kBigBF16: launch_big_v<BN, kBigBF16, true>(xq, wq, M, N, K, ep, vec, s); break;
    default: launch_big_v<BN, kBigF16, true>(xq, wq, M, N, K, ep, vec, s); break;
  }
}

}  // namespace sqk

namespace sqh {

bool gemm_big_suits(int64_t m, int64_t n, int64_t k, bool split_ok) {
  if (n < 192 || k % sqk::kBigBK != 0) return false;
  if (m >= 256 && m * n >= ((int64_t)1 << 20)) return true;
  // 129..255 tokens over wide layers: one 256-row tile per column block with
  // K split over the CUs beats the decode and 128 x 128 kernels (GEMM us at
  // 136 / 192 tokens, decode / 128 x 128 / this: 14336 -> 4096 60.8 / 136.3 /
  // 49.9 and 69.2 / 138.0 / 57.1; 4096 -> 14336 48.9 / 48.6 / 38.0 and 55.4 /
  // 49.8 / 39.1; 4096 -> 28672 91.8 / 60.4 / 47.8 and 110.2 / 61.9 / 53.6),
  // except that the decode kernel streams weights under 32 MiB fast enough to
  // stay ahead up to about 176 tokens (4096 -> 6144: 24.0 / 38.6 / 30.9 at
  // 136 tokens, 36.6 / 39.3 / 31.3 at 192)
  if (!split_ok || n < 4096 || k / sqk::kBigBK < 20) return false;
  return m >= 176 || (m >= 129 && n * k >= ((int64_t)1 << 25));
}

namespace {

using sqk::kBigMaxSplit;

struct BigSplit {
  int bn = 256;
  int S = 1;
  int slice_stages = 0;
  int64_t tiles = 0;
};

// K slices for `tiles` output tiles: split when the tiles cover fewer than
// half of the 256 CUs, into at most as many slices as keep all workgroups in
// one wave with a CU to spare (a full 256 measured slower: 4096 -> 6144 at 512
// tokens, 64 tiles in 3 / 4 slices 34.8 / 37.1 us). Each slice costs its reducer one more partial tile to read and
// shortens every slice's main loop: with about 1.3 us per 128-deep stage and
// 3 us per slice (fitted on 14336 -> 4096 at 192 tokens: 4 / 8 / 10 slices
// 56.6 / 49.9 / 52.1 us), S = sqrt(0.45 x stages) balances the two (7 for
// K = 14336, 4 for K = 4096; 4096 -> 6144 at 256 tokens: 3 / 4 / 6 slices
// 32.1 / 31.9 / 34.8 us). Slices keep at least 8 stages. A second wave of
// workgroups costs more than the split saves (14336 -> 4096 at 1024 tokens
// in 3 slices: 112 us against 89 in 2), and so does splitting 128 tiles in
// two (4096 -> 6144 at 1024 tokens: 43.2 -> 46.5 us).
int split_for(int64_t tiles, int stages, int bn) {
  int want = tiles < 128 ? (int)(255 / tiles) : 1;
  int best = (int)(sqrtf(0.45f * (float)stages) + 0.5f);
#ifdef SQ_TUNE
  if (const char* e = getenv("SQ_BIG_SPLIT")) want = best = atoi(e);
#endif
  if (want > best) want = best;
  if (want > kBigMaxSplit) want = kBigMaxSplit;
  if (want > stages / 8) want = stages / 8;
  if (want < 2) return 1;
  const int per = (stages + want - 1) / want;
  const int S = (stages + per - 1) / per;
  if ((size_t)S * (size_t)tiles * (size_t)(sqk::kBigBM * bn * 4) >= ((size_t)1 << 31)) return 1;
  return S;
}

// Tile width (256, 192 or 128 columns) and K split, chosen together: the
// score is the fraction of the scheduled waves' workgroup slots doing useful
// work, useful outputs x S over (waves of tiles x S) x 256 x 256 x BN, times
// a measured efficiency: 0.8 for 128-column tiles (less operand reuse per
// fragment read), 0.8 for a split (0.7 with 256-column tiles). GEMM alone,
// us, tile width 192 / 256 / 128 (S: split into S slices): 4096 -> 6144 at
// 1024 tokens 44.2 / 59.4 (S2) / 36.9; 4096 -> 14336 at 512 tokens 47.8 /
// 63.4 (S2) / 41.6; 14336 -> 4096 at 2048 tokens 134.8 / 146.9 / 126.3, at
// 1024 tokens 97.5 (S2) / 105.9 (S3) / 118.4, at 3072 tokens 269.3 / 167.3 /
// 223.7; 4096 -> 6144 at 1536 tokens 46.2 / 52.9 / 71.0. The 128-column
// tile is taken only unsplit (the combination measured).
BigSplit big_split(int64_t m, int64_t n, int64_t k, bool f8, bool split_ok = true) {
  const int stages = (int)(k / sqk::kBigBK);
  const int cands[3] = {256, 192, 128};
  BigSplit best;
  double best_score = -1.0;
  for (int bn : cands) {
    if (f8 && bn == 256) continue;  // E4M3 tiles: 192 or 128 columns
#ifdef SQ_TUNE
    if (const char* e = getenv("SQ_BIG_BN"))
      if (atoi(e) != bn) continue;
#endif
    BigSplit p;
    p.bn = bn;
    p.tiles = ((m + sqk::kBigBM - 1) / sqk::kBigBM) * ((n + bn - 1) / bn);
    p.S = split_ok ? split_for(p.tiles, stages, bn) : 1;
    if (bn == 128 && p.S > 1) continue;
    p.slice_stages = (stages + p.S - 1) / p.S;
    const int64_t waves = (p.tiles * p.S + 255) / 256;
    double score = (double)m * (double)n * p.S / ((double)waves * 256.0 * sqk::kBigBM * bn);
    if (bn == 128) score *= 0.8;
    if (p.S > 1) score *= bn == 256 ? 0.7 : 0.8;
    if (score > best_score + 1e-9) {
      best = p;
      best_score = score;
    }
  }
  return best;
}

size_t big_counter_bytes(int64_t tiles) { return ((size_t)tiles * 4 + 255) / 256 * 256; }

}  // namespace

size_t gemm_big_workspace(int64_t m, int64_t n, int64_t k, bool f8) {
  if (!gemm_big_suits(m, n, k)) return 0;
  const BigSplit p = big_split(m, n, k, f8);
  if (p.S == 1) return 0;
  return big_counter_bytes(p.tiles) + (size_t)p.S * (size_t)p.tiles * (size_t)(sqk::kBigBM * p.bn * 4);
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
    ep.partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + big_counter_bytes(sp.tiles));
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

hipError_t gemm_f8_big(const uint8_t* xq, const float* x_scale, const uint8_t* wq, const float* w_scale, int64_t m,
                       int64_t n, int64_t k, void* y, sq_dtype yt, int64_t ldy, void* ws, hipStream_t s) {
  sqk::BigEpi ep{x_scale, w_scale, y, ldy, DecompArgs{}, false, nullptr, nullptr, 1, 0};
  const BigSplit sp = big_split(m, n, k, true);
  if (sp.S > 1) {
    ep.S = sp.S;
    ep.slice_stages = sp.slice_stages;
    ep.counter = reinterpret_cast<uint32_t*>(ws);
    ep.partial = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + big_counter_bytes(sp.tiles));
  }
  const int out = yt == SQ_F32 ? sqk::kBigF32 : (yt == SQ_BF16 ? sqk::kBigBF16 : sqk::kBigF16);
  const int eb = yt == SQ_F32 ? 4 : 2;
  const bool vec = (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % (uintptr_t)(4 * eb) == 0) &&
                   reinterpret_cast<uintptr_t>(w_scale) % 16 == 0;
  ep.rows16 = (ldy * eb) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
  const int M = (int)m, N = (int)n, K = (int)k;
  // 192- or 128-column tiles: the E4M3 fragments are twice the int8 ones,
  // and with 256 columns the accumulators and two fragment sets exceed the
  // 256 registers a lane has at two waves per SIMD
  if (sp.bn == 128)
    sqk::launch_big_f8<128>(reinterpret_cast<const int8_t*>(xq), reinterpret_cast<const int8_t*>(wq), M, N, K, ep,
                            out, vec, s);
  else
    sqk::launch_big_f8<192>(reinterpret_cast<const int8_t*>(xq), reinterpret_cast<const int8_t*>(wq), M, N, K, ep,
                            out, vec, s);
  return hipGetLastError();
}

}  // namespace sqh
