// Device-side helpers shared by the gfx950 kernels of the W8A8 library.
//
// Storage formats: bf16 and fp16 values travel as uint16_t bit patterns;
// 16-byte vectors carry 8 of them, or 4 binary32 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sq.h"

namespace sqk {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kQMax = 127;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// binary32 -> bf16, round to nearest, ties to even (NaN is outside the contract).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two binary32 values -> two bf16 (low half = a), round to nearest even, with
// gfx950's packed conversion (v_cvt_pk_bf16_f32): the same results as
// f32_to_bf16 on every finite value, in one instruction per pair.
__device__ __forceinline__ uint32_t bf16x2_rn(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  const f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// binary32 -> binary16 with the hardware conversion (round to nearest even).
// The empty asm pins f as a rounded binary32 value: without it the compiler
// folds "multiply, then convert to half" into one v_fma_mix instruction that
// rounds the exact product straight to binary16, which differs from rounding
// to binary32 first whenever the binary32 product sits on a binary16 tie.
__device__ __forceinline__ uint32_t f32_to_f16(float f) {
  asm volatile("" : "+v"(f));
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Element types of the activation / weight inputs.
struct F32In {
  static constexpr int kVec = 4;  // elements per 16-byte vector
  static constexpr int kBytes = 4;
  __device__ __forceinline__ static float load1(const uint8_t* p) { return *reinterpret_cast<const float*>(p); }
  __device__ __forceinline__ static void unpack(const u32x4& v, float* o) {
    o[0] = __uint_as_float(v.x); o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z); o[3] = __uint_as_float(v.w);
  }
};
struct BF16In {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load1(const uint8_t* p) {
    return bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  }
  __device__ __forceinline__ static void unpack(const u32x4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
struct F16In {
  static constexpr int kVec = 8;
  static constexpr int kBytes = 2;
  __device__ __forceinline__ static float load1(const uint8_t* p) {
    return f16_to_f32(*reinterpret_cast<const uint16_t*>(p));
  }
  __device__ __forceinline__ static void unpack(const u32x4& v, float* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = f16_to_f32(w[i] & 0xFFFFu);
      o[2 * i + 1] = f16_to_f32(w[i] >> 16);
    }
  }
};

// ---------------------------------------------------------------- loads
__device__ __forceinline__ u32x4 load16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void store16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

// ---------------------------------------------------------------- reductions
// ---------------------------------------------------------------- wave reductions over DPP
// Inclusive scan within each 16-lane row (row_shr 1, 2, 4, 8), then row_bcast
// 15 / 31 carry the row totals upwards; lane 63 ends with the wave's total,
// which readlane makes uniform. Lanes whose DPP source does not exist read 0,
// the identity of every reduction here (sums, and maxima of non-negative values).
template <int kCtrl, int kRowMask = 0xF>
__device__ __forceinline__ uint32_t dpp0(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, kCtrl, kRowMask, 0xF, false);
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp0<0x111>(v));
  v = op(v, dpp0<0x112>(v));
  v = op(v, dpp0<0x114>(v));
  v = op(v, dpp0<0x118>(v));
  v = op(v, dpp0<0x142, 0xA>(v));
  v = op(v, dpp0<0x143, 0xC>(v));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  return wave_reduce_u32(v, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

// Maximum over the 64 lanes of a wavefront of non-negative values (their bit
// patterns order like the values); every lane receives it.
__device__ __forceinline__ float wave_max(float v) { return __uint_as_float(wave_max_u32(__float_as_uint(v))); }

// Maximum over a workgroup of kThreads threads; `red` holds kThreads/64 floats of LDS.
template <int kThreads>
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wid = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wid] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// s_waitcnt lgkmcnt(0) (LDS and scalar loads) with vmcnt and expcnt left alone (gfx9 encoding).
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4)); }

// Workgroup barrier for LDS traffic only. __syncthreads() also waits for every
// outstanding global load (vmcnt(0)), which would drain prefetches issued
// before the barrier; here only this wave's LDS accesses are retired first.
// The empty asm statements stop the compiler from moving memory accesses
// across the barrier.
__device__ __forceinline__ void lds_barrier() {
  wait_lgkmcnt0();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Running maximum of non-negative binary32 values: their bit patterns order like the values.
__device__ __forceinline__ void atomic_max_nonneg(float* addr, float v) {
  atomicMax(reinterpret_cast<unsigned int*>(addr), __float_as_uint(v));
}

// ---------------------------------------------------------------- rounding
// round-half-to-even to an integer, then clamp to the symmetric int8 range.
__device__ __forceinline__ int quant_rne_clamp(float q) {
  float r = __builtin_rintf(q);
  r = fminf(fmaxf(r, -(float)kQMax), (float)kQMax);
  return (int)r;
}

// ---------------------------------------------------------------- quotients and int8 codes
// Markstein's FMA-corrected quotient: with r = RN(1/b), q0 = a*r,
// e = fma(-q0, b, a) (exact), q = fma(e, r, q0) gives q = RN(a/b) whenever no
// step leaves the normal range; the quantisation kernels check that range per
// row (below) and fall back to IEEE division outside it.
constexpr float kFastSMin = 0x1p-20f, kFastSMax = 0x1p20f;
constexpr float kFastDMin = 0x1p-30f, kFastAMax = 0x1p50f;

// RN(1/s) for s in [2^-20, 2^21): hardware reciprocal plus one Newton step.
__device__ __forceinline__ float rcp_rn(float s) {
  const float y = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, y, 1.0f);
  return __builtin_fmaf(e, y, y);
}

// RN(1/d) for a positive row scale: the refined hardware reciprocal inside the
// range where it equals the IEEE one, IEEE division outside it.
__device__ __forceinline__ float rcp_scale(float d) {
  return (d >= 0x1p-20f && d < 0x1p21f) ? rcp_rn(d) : 1.0f / d;
}

__device__ __forceinline__ float div_mk(float a, float b, float rb) {
  const float q0 = a * rb;
  const float e = __builtin_fmaf(-q0, b, a);
  return __builtin_fmaf(e, rb, q0);
}

// int8 code of one quotient v = fl32(a / d) with d = fl32(amax / 127) and
// |a| <= amax (a row's own values): |a / d| <= amax / d <= 127 (1 + 2^-23),
// so |v| < 127.0001 and round-half-even(v) already lies in [-127, 127]; the
// clamp of the definition never acts and is not applied. Adding 1.5 * 2^23
// rounds to the nearest integer with ties to even (the sum lies in
// [2^23, 2^24), where the binary32 spacing is 1) and leaves the two's-
// complement code in the low byte of the sum's bit pattern.
__device__ __forceinline__ uint32_t q_code(float v) { return __float_as_uint(v + 12582912.0f); }

// Low bytes of four codes -> one little-endian word (v_perm_b32 picks bytes).
__device__ __forceinline__ uint32_t pack4(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3) {
  const uint32_t lo = __builtin_amdgcn_perm(c1, c0, 0x0C0C0400u);  // c0.b0, c1.b0
  const uint32_t hi = __builtin_amdgcn_perm(c3, c2, 0x0C0C0400u);  // c2.b0, c3.b0
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

}  // namespace sqk
