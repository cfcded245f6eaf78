// Measurement probes of the gfx950 ceilings that bound the int8 path: the
// matrix-core rate and shader clock with constant or changing operands, a
// plain streaming read/write kernel, the LDS fragment-read rate beside the
// MFMA rate, the LDS read throughput by instruction width, the MFMA rate of
// the prefill GEMM's main loop taken apart (fragment reads, barriers, stage
// transfers), and the summation error of the FP8 (E4M3) matrix instructions.
//
// None of this is part of the linear layer: the benchmark loads this library
// (libsq_probes.so) only in its probe modes. Every entry point launches on
// the caller's stream, takes device pointers sized by the caller and returns
// the HIP error of its launch (0 on success).
//
// Clock readings: lane 0 of wave 0 of every workgroup records s_memtime (the
// shader clock counter) and s_memrealtime (a constant 100 MHz counter) at its
// start and end; their ratio over the same interval gives the shader clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t mix(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

__device__ __forceinline__ void clock_mark(int64_t* clocks, int slot) {
  if (threadIdx.x == 0) {
    const uint64_t t = __builtin_amdgcn_s_memtime();
    const uint64_t r = __builtin_amdgcn_s_memrealtime();
    clocks[(int64_t)blockIdx.x * 4 + 2 * slot] = (int64_t)t;
    clocks[(int64_t)blockIdx.x * 4 + 2 * slot + 1] = (int64_t)r;
  }
}

// ---- matrix-core rate: one wave per SIMD, 8 independent 32x32x32 int8
// accumulators, 16 MFMAs per iteration. `random`: the operands of every MFMA
// differ (16 A and 16 B fragments of hashed bytes, combined in a rotating
// order); otherwise all operands are the same constant.
constexpr int kPool = 16;

__global__ __launch_bounds__(256, 1) void mfma_rate_kernel(int64_t* clocks, int32_t* sink, int iters, int random) {
  const int lane = threadIdx.x & 63;
  v4i a[kPool], b[kPool];
#pragma unroll
  for (int p = 0; p < kPool; ++p) {
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u + (uint32_t)p;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[p][e] = random ? (int)mix(seed * 8u + e) : 0x01010101;
      b[p][e] = random ? (int)mix(seed * 8u + 4 + e + 0x9e3779b9u) : 0x01010101;
    }
  }
  v16i acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0;
  __syncthreads();
  clock_mark(clocks, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      acc[q & 7] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[q], b[(q * 5 + 3) & (kPool - 1)], acc[q & 7], 0, 0, 0);
  }
  __syncthreads();
  clock_mark(clocks, 1);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= acc[j][r];
  sink[blockIdx.x * 256 + threadIdx.x] = s + lane;
}

// The same for the E4M3 matrix instruction (v_mfma_scale_f32_32x32x64_f8f6f4,
// unit scales): 8 operand pairs of 32 bytes per lane (constant 1.0 codes, or
// hashed bytes with the exponent's low bit cleared, so every code is finite).
constexpr int kPoolF8 = 8;
__global__ __launch_bounds__(256, 1) void mfma_rate_f8_kernel(int64_t* clocks, int32_t* sink, int iters, int random) {
  const int lane = threadIdx.x & 63;
  v8i a[kPoolF8], b[kPoolF8];
#pragma unroll
  for (int p = 0; p < kPoolF8; ++p) {
    const uint32_t seed = (blockIdx.x * 256u + threadIdx.x) * 64u + (uint32_t)p;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[p][e] = random ? (int)(mix(seed * 16u + e) & 0xF7F7F7F7u) : 0x38383838;
      b[p][e] = random ? (int)(mix(seed * 16u + 8 + e + 0x9e3779b9u) & 0xF7F7F7F7u) : 0x38383838;
    }
  }
  v16f acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  __syncthreads();
  clock_mark(clocks, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int q = 0; q < 16; ++q)
      acc[q & 7] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[q & 7], b[(q * 5 + 3) & 7], acc[q & 7], 0, 0, 0,
                                                                  127, 0, 127);
  }
  __syncthreads();
  clock_mark(clocks, 1);
  int32_t s = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= __float_as_int(acc[j][r]);
  sink[blockIdx.x * 256 + threadIdx.x] = s + lane;
}

// ---- streaming: each workgroup walks chunks of 256 x kD 16-byte vectors
// (grid-stride over chunks); thread t loads vectors t, t + 256, ... of a
// chunk, all kD in flight before their first use, folds them into one word
// and writes a pattern over the same vectors of `dst`.
template <int kD>
__global__ __launch_bounds__(256) void stream_kernel(const u32x4* __restrict__ src, int64_t nread,
                                                     u32x4* __restrict__ dst, int64_t nwrite,
                                                     uint32_t* __restrict__ sink) {
  constexpr int64_t kChunk = 256 * kD;
  const int t = threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t base = (int64_t)blockIdx.x * kChunk; base < nread; base += (int64_t)gridDim.x * kChunk) {
    if (base + kChunk <= nread) {
      u32x4 v[kD];
#pragma unroll
      for (int j = 0; j < kD; ++j) v[j] = src[base + t + 256 * j];
#pragma unroll
      for (int j = 0; j < kD; ++j) acc ^= v[j];
    } else {
      for (int64_t i = base + t; i < nread; i += 256) acc ^= src[i];
    }
  }
  const u32x4 pat = {(uint32_t)t, 1u, 2u, 3u};
  for (int64_t base = (int64_t)blockIdx.x * kChunk; base < nwrite; base += (int64_t)gridDim.x * kChunk) {
    if (base + kChunk <= nwrite) {
#pragma unroll
      for (int j = 0; j < kD; ++j) dst[base + t + 256 * j] = pat;
    } else {
      for (int64_t i = base + t; i < nwrite; i += 256) dst[i] = pat;
    }
  }
  const uint32_t s = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (s == 0x9e3779b9u) sink[(int64_t)blockIdx.x * 256 + t] = s;  // practically never: keeps the loads
}

// ---- LDS rate: 8 waves (two per SIMD) over 64 KiB of LDS, the prefill
// GEMM's fragment-read pattern (16-byte reads, 128-byte rows, chunks XOR-
// swizzled by (row >> 1) & 7). mode 0: 5 fragment reads per iteration;
// mode 1: 6 MFMAs (32x32x32 int8, constant operands) per iteration; mode 2:
// both, as the GEMM's substeps run them: the reads of one iteration fill the
// fragments the next iteration's MFMAs use (double-buffered registers);
// mode 3: mode 0 with linear addresses (lane l reads bytes [16 l, 16 l + 16)
// of a 1 KiB block), the instruction's rate without the row pattern.
__global__ __launch_bounds__(512, 1) void lds_rate_kernel(int64_t* clocks, int32_t* sink, int iters, int mode) {
  __shared__ __attribute__((aligned(16))) int8_t lds[65536];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < 65536 / 16; i += 512)
    *reinterpret_cast<u32x4*>(lds + 16 * i) = u32x4{(uint32_t)i, 0x01010101u, 0x01010101u, 0x01010101u};
  __syncthreads();
  v4i f[5];
#pragma unroll
  for (int q = 0; q < 5; ++q) f[q] = v4i{0x01010101, 0x01010101, 0x01010101, 0x01010101};
  v16i acc[6];
#pragma unroll
  for (int j = 0; j < 6; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0;
  clock_mark(clocks, 0);
  const int frow = lane & 31, fhalf = lane >> 5;
  for (int it = 0; it < iters; ++it) {
    const int ks = it & 3;
    v4i g[5];
#pragma unroll
    for (int q = 0; q < 6; ++q) {
      if (mode == 1 || mode == 2)
        acc[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[q % 5], f[(q + 2) % 5], acc[q], 0, 0, 0);
      if (mode != 1 && q < 5) {
        const int r = (wid * 5 + q) * 32 % 512 + frow;
        const int c = 2 * ks + fhalf;
        const int off = mode == 3 ? ((wid * 5 + q + 8 * ks) & 63) * 1024 + 16 * lane
                                  : r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
        g[q] = *reinterpret_cast<const v4i*>(lds + off);
      }
    }
    if (mode != 1) {
#pragma unroll
      for (int q = 0; q < 5; ++q) f[q] = mode == 2 ? g[q] : (f[q] ^ g[q]);
    }
  }
  __syncthreads();
  clock_mark(clocks, 1);
  int32_t s = 0;
#pragma unroll
  for (int q = 0; q < 5; ++q) s ^= f[q][0] ^ f[q][1] ^ f[q][2] ^ f[q][3];
#pragma unroll
  for (int j = 0; j < 6; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= acc[j][r];
  sink[blockIdx.x * 512 + tid] = s;
}

// ---- FP8 summation: one E4M3 MFMA per tile with zero accumulators and unit
// scales. Form 0: v_mfma_scale_f32_32x32x64_f8f6f4, tiles of A [32 x 64] and
// B [32 x 64] codes, D [32 x 32] with D[n][m] = sum_k A[n][k] B[m][k]. Form 1:
// v_mfma_scale_f32_16x16x128_f8f6f4, A [16 x 128], B [16 x 128], D [16 x 16].
// One wave per tile.
__global__ __launch_bounds__(64) void fp8_mfma_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                      float* __restrict__ d, int form) {
  const int lane = threadIdx.x;
  const int64_t t = blockIdx.x;
  if (form == 0) {
    const uint8_t* ap = a + t * 32 * 64 + (lane & 31) * 64 + 32 * (lane >> 5);
    const uint8_t* bp = b + t * 32 * 64 + (lane & 31) * 64 + 32 * (lane >> 5);
    const v8i av = *reinterpret_cast<const v8i*>(ap);
    const v8i bv = *reinterpret_cast<const v8i*>(bp);
    v16f acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int n = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3), m = lane & 31;
      d[t * 1024 + n * 32 + m] = acc[r];
    }
  } else {
    const uint8_t* ap = a + t * 16 * 128 + (lane & 15) * 128 + 32 * (lane >> 4);
    const uint8_t* bp = b + t * 16 * 128 + (lane & 15) * 128 + 32 * (lane >> 4);
    const v8i av = *reinterpret_cast<const v8i*>(ap);
    const v8i bv = *reinterpret_cast<const v8i*>(bp);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, acc, 0, 0, 0, 127, 0, 127);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int n = 4 * (lane >> 4) + r, m = lane & 15;
      d[t * 256 + n * 16 + m] = acc[r];
    }
  }
}

// ---- LDS read throughput: every lane reads kB bytes per instruction, kR
// independent reads per wave in flight, one wait per round; pattern 0: lanes
// consecutive in a 1 KiB block, 1: the prefill GEMM's fragment reads (32 rows
// of 128 bytes, chunk XOR (row >> 1) & 7, the lane halves in adjacent chunks).
// cycles: 16 x blocks (s_memtime per wave), sink: blockDim x blocks.
template <int kB, int kR>
__global__ __launch_bounds__(1024) void lds_bw_kernel(int64_t* cycles, int32_t* sink, int iters, int pattern) {
  __shared__ __attribute__((aligned(16))) int8_t lds[65536];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < 65536 / 4; i += blockDim.x) reinterpret_cast<uint32_t*>(lds)[i] = mix((uint32_t)i);
  __syncthreads();
  int off[kR];
#pragma unroll
  for (int r = 0; r < kR; ++r) {
    const int blk = (wid * kR + r) & 63;
    int o;
    if (pattern == 0) {
      o = blk * 1024 + lane * kB;
    } else {
      const int row = lane & 31, c = (2 * (r & 3) + (lane >> 5)) ^ ((row >> 1) & 7);
      o = (blk & 15) * 4096 + row * 128 + c * 16;
    }
    off[r] = o & 65535;
  }
  int acc = 0;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int it = 0; it < iters; ++it) {
    const int shift = (it & 7) * 64;
#pragma unroll
    for (int r = 0; r < kR; ++r) {
      const int o = (off[r] + shift) & (65535 & ~(kB - 1));
      if constexpr (kB == 16) {
        const v4i v = *reinterpret_cast<const v4i*>(lds + o);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
      } else if constexpr (kB == 8) {
        const int2 v = *reinterpret_cast<const int2*>(lds + o);
        acc ^= v.x ^ v.y;
      } else {
        acc ^= *reinterpret_cast<const int*>(lds + o);
      }
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  if (lane == 0) cycles[blockIdx.x * 16 + wid] = (int64_t)(t1 - t0);
  sink[blockIdx.x * blockDim.x + tid] = acc;
}

// ---- The prefill GEMM's main loop taken apart: 8 waves (two per SIMD), per
// 128-byte stage four substeps of 6 v_mfma_i32_32x32x32_i8 per wave on 6
// accumulators (the 256 x 192 tile's 64 x 96 wave tiles), with
//   mode 0: MFMAs only;
//   mode 1: + 5 fragment reads per substep from LDS in the GEMM's swizzled
//           pattern, each substep's reads feeding the next one;
//   mode 2: mode 1 + one workgroup barrier per stage;
//   mode 3: mode 2 + the stage's 56 KiB of direct-to-LDS transfers (7 per
//           wave, global_load_lds with per-lane 64-bit addresses) in the last
//           substep, waited for before the barrier of the next stage;
//   mode 4: mode 3 with the transfers through a buffer resource (fixed lane
//           offset, scalar stage offset, scalar LDS base);
//   mode 5: mode 4 with every stage of every workgroup reading a different
//           56 KiB (no L2 reuse).
// Sources: 8 x 16 stages x 56 KiB (modes 3, 4; each XCD's workgroups share
// theirs, L2-resident) or blocks x 16 x 56 KiB (mode 5).
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ void probe_buffer_load_lds16(__amdgpu_buffer_rsrc_t r, lds_void* dst, int voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
#endif
}
constexpr int kPartsStage = 57344;  // 448 rows x 128 bytes
template <int kMode>
__global__ __launch_bounds__(512) void gemm_parts_kernel(int64_t* cycles, int32_t* sink, int stages,
                                                         const int8_t* src, int64_t src_bytes) {
  __shared__ __attribute__((aligned(1024))) int8_t lds[65536 + kPartsStage];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  for (int i = tid; i < 65536 / 16; i += 512)
    *reinterpret_cast<v4i*>(lds + 16 * i) = v4i{(int)mix(i), i ^ 0x55aa55aa, i * 131, 3 * i};
  __syncthreads();
  const int frow = lane & 31, fhalf = lane >> 5;
  int off[4][5];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int q = 0; q < 5; ++q) {
      const int r = (wid * 5 + q) * 32 % 448 + frow;
      const int c = 2 * ks + fhalf;
      off[ks][q] = r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
    }
  v4i f[2][5];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 5; ++q) f[p][q] = *reinterpret_cast<const v4i*>(lds + off[p][q]);
  const int uwid = __builtin_amdgcn_readfirstlane(wid);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)src_bytes, 0x00020000);
  const int8_t* dsrc[7];
#pragma unroll
  for (int i = 0; i < 7; ++i) dsrc[i] = src + ((blockIdx.x & 7) * 56 + i * 8 + wid) * 1024 + lane * 16;
  v16i acc[6];
#pragma unroll
  for (int j = 0; j < 6; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0;
  __syncthreads();
  const uint64_t t0 = __builtin_amdgcn_s_memtime();
  for (int st = 0; st < stages; ++st) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int cs = ks & 1, ns = cs ^ 1;
      if (kMode >= 3 && ks == 3) {
        __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): the previous stage's transfers
      }
      if (kMode >= 2 && ks == 3) __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        acc[q] = __builtin_amdgcn_mfma_i32_32x32x32_i8(f[cs][q & 1], f[cs][2 + (q >> 1)], acc[q], 0, 0, 0);
        if (kMode >= 1 && q < 5) f[ns][q] = *reinterpret_cast<const v4i*>(lds + off[(ks + 1) & 3][q]);
        if (kMode >= 3 && ks == 3 && q < 7) {
          const int blk = q * 8 + uwid;
          if (kMode == 3) {
            __builtin_amdgcn_global_load_lds((const void*)(dsrc[q] + (int64_t)(st & 15) * 8 * kPartsStage),
                                             (lds_void*)(lds + 65536 + blk * 1024), 16, 0, 0);
          } else {
            const int soff = kMode == 4 ? (st & 15) * 8 * kPartsStage + (blockIdx.x & 7) * kPartsStage
                                        : ((int)blockIdx.x * 16 + (st & 15)) * kPartsStage;
            probe_buffer_load_lds16(rs, (lds_void*)(lds + 65536 + blk * 1024), blk * 1024 + lane * 16, soff);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kMode >= 3 && ks == 3 && 6 < 7) {  // the seventh transfer after the substep's MFMAs
        const int blk = 6 * 8 + uwid;
        if (kMode == 3) {
          __builtin_amdgcn_global_load_lds((const void*)(dsrc[6] + (int64_t)(st & 15) * 8 * kPartsStage),
                                           (lds_void*)(lds + 65536 + blk * 1024), 16, 0, 0);
        } else {
          const int soff = kMode == 4 ? (st & 15) * 8 * kPartsStage + (blockIdx.x & 7) * kPartsStage
                                      : ((int)blockIdx.x * 16 + (st & 15)) * kPartsStage;
          probe_buffer_load_lds16(rs, (lds_void*)(lds + 65536 + blk * 1024), blk * 1024 + lane * 16, soff);
        }
      }
      if (kMode >= 1) __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }
  }
  const uint64_t t1 = __builtin_amdgcn_s_memtime();
  __builtin_amdgcn_s_waitcnt(0x0070);
  int s = 0;
#pragma unroll
  for (int j = 0; j < 6; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s ^= acc[j][r];
#pragma unroll
  for (int p = 0; p < 2; ++p)
#pragma unroll
    for (int q = 0; q < 5; ++q) s ^= f[p][q].x;
  sink[blockIdx.x * 512 + tid] = s;
  if (lane == 0) cycles[blockIdx.x * 8 + wid] = (int64_t)(t1 - t0);
}

}  // namespace

extern "C" {

// clocks: 4 x blocks int64 (start memtime, start realtime, end memtime, end
// realtime per workgroup); sink: 256 x blocks int32. One 256-thread
// workgroup (4 waves) per CU for blocks = 256.
// random: 0 / 1 int8 with constant / changing operands, 2 / 3 the same for E4M3.
int sqp_mfma_rate(int64_t* clocks, int32_t* sink, int blocks, int iters, int random, hipStream_t s) {
  if (blocks <= 0 || iters <= 0 || random < 0 || random > 3) return (int)hipErrorInvalidValue;
  if (random >= 2)
    hipLaunchKernelGGL(mfma_rate_f8_kernel, dim3(blocks), dim3(256), 0, s, clocks, sink, iters, random - 2);
  else
    hipLaunchKernelGGL(mfma_rate_kernel, dim3(blocks), dim3(256), 0, s, clocks, sink, iters, random);
  return (int)hipGetLastError();
}

// src: read_bytes (a multiple of 16) of readable memory; dst: write_bytes (a
// multiple of 16); sink: 256 x blocks words; depth: 4, 8 or 16 loads in
// flight per thread.
int sqp_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes, uint32_t* sink, int blocks,
               int depth, hipStream_t s) {
  if (blocks <= 0 || read_bytes < 0 || write_bytes < 0 || read_bytes % 16 || write_bytes % 16)
    return (int)hipErrorInvalidValue;
  const u32x4* in = reinterpret_cast<const u32x4*>(src);
  u32x4* out = reinterpret_cast<u32x4*>(dst);
  switch (depth) {
    case 4: hipLaunchKernelGGL(stream_kernel<4>, dim3(blocks), dim3(256), 0, s, in, read_bytes / 16, out, write_bytes / 16, sink); break;
    case 8: hipLaunchKernelGGL(stream_kernel<8>, dim3(blocks), dim3(256), 0, s, in, read_bytes / 16, out, write_bytes / 16, sink); break;
    case 16: hipLaunchKernelGGL(stream_kernel<16>, dim3(blocks), dim3(256), 0, s, in, read_bytes / 16, out, write_bytes / 16, sink); break;
    default: return (int)hipErrorInvalidValue;
  }
  return (int)hipGetLastError();
}

// clocks: 4 x blocks int64; sink: 512 x blocks int32; mode 0 .. 3 as above.
int sqp_lds_rate(int64_t* clocks, int32_t* sink, int blocks, int iters, int mode, hipStream_t s) {
  if (blocks <= 0 || iters <= 0 || mode < 0 || mode > 3) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(lds_rate_kernel, dim3(blocks), dim3(512), 0, s, clocks, sink, iters, mode);
  return (int)hipGetLastError();
}

// cycles: 16 x blocks int64 (per wave); sink: threads x blocks int32;
// bytes: 16, 8 or 4 per lane per read; reads: 4, 8 or 16 in flight per wave;
// threads: 256, 512 or 1024; pattern 0 (linear) or 1 (GEMM fragments).
int sqp_lds_bw(int64_t* cycles, int32_t* sink, int blocks, int threads, int iters, int bytes, int reads, int pattern,
               hipStream_t s) {
  if (blocks <= 0 || iters <= 0 || (threads != 256 && threads != 512 && threads != 1024) || pattern < 0 ||
      pattern > 1)
    return (int)hipErrorInvalidValue;
#define SQP_LDS_BW(B, R)                                                                                         \
  if (bytes == B && reads == R) {                                                                              \
    hipLaunchKernelGGL((lds_bw_kernel<B, R>), dim3(blocks), dim3(threads), 0, s, cycles, sink, iters, pattern); \
    return (int)hipGetLastError();                                                                             \
  }
  SQP_LDS_BW(16, 4) SQP_LDS_BW(16, 8) SQP_LDS_BW(8, 8) SQP_LDS_BW(8, 16) SQP_LDS_BW(4, 16)
#undef SQP_LDS_BW
  return (int)hipErrorInvalidValue;
}

// cycles: 8 x blocks int64 (per wave); sink: 512 x blocks int32; src: at least
// 8 x 16 x 57344 bytes (modes 3, 4) or blocks x 16 x 57344 bytes (mode 5), and
// src_bytes < 2^31.
int sqp_gemm_parts(int64_t* cycles, int32_t* sink, int blocks, int stages, int mode, const int8_t* src,
                   int64_t src_bytes, hipStream_t s) {
  if (blocks <= 0 || stages <= 0 || mode < 0 || mode > 5 || src_bytes >= ((int64_t)1 << 31)) return (int)hipErrorInvalidValue;
  const int64_t need = mode == 5 ? (int64_t)blocks * 16 * kPartsStage : (mode >= 3 ? (int64_t)8 * 16 * kPartsStage : 0);
  if (src_bytes < need || (need > 0 && !src)) return (int)hipErrorInvalidValue;
  switch (mode) {
    case 0: hipLaunchKernelGGL(gemm_parts_kernel<0>, dim3(blocks), dim3(512), 0, s, cycles, sink, stages, src, src_bytes); break;
    case 1: hipLaunchKernelGGL(gemm_parts_kernel<1>, dim3(blocks), dim3(512), 0, s, cycles, sink, stages, src, src_bytes); break;
    case 2: hipLaunchKernelGGL(gemm_parts_kernel<2>, dim3(blocks), dim3(512), 0, s, cycles, sink, stages, src, src_bytes); break;
    case 3: hipLaunchKernelGGL(gemm_parts_kernel<3>, dim3(blocks), dim3(512), 0, s, cycles, sink, stages, src, src_bytes); break;
    case 4: hipLaunchKernelGGL(gemm_parts_kernel<4>, dim3(blocks), dim3(512), 0, s, cycles, sink, stages, src, src_bytes); break;
    default: hipLaunchKernelGGL(gemm_parts_kernel<5>, dim3(blocks), dim3(512), 0, s, cycles, sink, stages, src, src_bytes); break;
  }
  return (int)hipGetLastError();
}

// a, b: tiles x 2048 E4M3 codes each; d: tiles x 1024 (form 0) or 256 (form 1) floats.
int sqp_fp8_mfma(const uint8_t* a, const uint8_t* b, float* d, int tiles, int form, hipStream_t s) {
  if (tiles <= 0 || (form != 0 && form != 1)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(fp8_mfma_kernel, dim3(tiles), dim3(64), 0, s, a, b, d, form);
  return (int)hipGetLastError();
}

}  // extern "C"
