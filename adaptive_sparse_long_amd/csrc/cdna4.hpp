// cdna4.hpp -- small device helpers for gfx950 (CDNA4) kernels: MFMA operand
// types and wrappers, wavefront reductions through DPP and the gfx950 permlane
// swaps, bfloat16 packing.
//
// MFMA register layouts used throughout (64-lane wavefront, lane l):
//   v_mfma_f32_32x32x16_bf16  A: row l%32, k = 8*(l/32) .. +7   (8 bf16)
//                             B: col l%32, k = 8*(l/32) .. +7   (8 bf16)
//                             D: col l%32, row 8*(r/4) + 4*(l/32) + r%4, r < 16
//   v_mfma_f32_16x16x32_bf16  A: row l%16, k = 8*(l/16) .. +7
//                             B: col l%16, k = 8*(l/16) .. +7
//                             D: col l%16, row 4*(l/16) + r, r < 4
//   v_mfma_f32_32x32x2_f32    A: row l%32, k = l/32;  B: col l%32, k = l/32
//                             D: as for 32x32x16
// A and B pair their k elements the same way, so any consistent relabelling of
// k on both operands gives the same product.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dash {

typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef uint32_t u32x4 __attribute__((__vector_size__(4 * sizeof(uint32_t))));
typedef uint32_t u32x2 __attribute__((__vector_size__(2 * sizeof(uint32_t))));

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1.0e30f;  // finite "minus infinity" for running maxima

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// v_exp_f32 / v_log_f32 (base 2) without the denormal range fix-ups of exp2f /
// log2f: results below 2^-126 flush to zero, which is harmless for attention
// weights and priors.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32x32x2f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// --- bfloat16 <-> float -----------------------------------------------------
__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Round two floats to bfloat16 (nearest even) and pack (a in the low half).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float round_bf16(float a) {
  return __uint_as_float(((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a)) << 16);
}

// --- fp16 <-> float (partial results) ----------------------------------------
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (_Float16)a);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (_Float16)b);
  return lo | (hi << 16);
}
__device__ __forceinline__ float f16lo(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u & 0xffffu)); }
__device__ __forceinline__ float f16hi(uint32_t u) { return (float)__builtin_bit_cast(_Float16, (uint16_t)(u >> 16)); }

// --- cross-lane moves -------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
// DPP controls: quad_perm [1,0,3,2] and [2,3,0,1], row_half_mirror, row_mirror.
constexpr int kDppXor1 = 0xB1;
constexpr int kDppXor2 = 0x4E;
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Sum over each group of 8 lanes; every lane of the group gets the result.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x;
}
// Pair reduction of lane l with lane l ^ 8 (row_ror:8 within each row of 16).
constexpr int kDppRor8 = 0x128;
__device__ __forceinline__ float sum_xor8(float x) { return x + dpp_f<kDppRor8>(x); }
__device__ __forceinline__ float max_xor8(float x) { return fmaxf(x, dpp_f<kDppRor8>(x)); }

// Sum / max over each row of 16 lanes; every lane of the row gets the result.
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  x += dpp_f<kDppMirror>(x);
  return x;
}
__device__ __forceinline__ float max16(float x) {
  x = fmaxf(x, dpp_f<kDppXor1>(x));
  x = fmaxf(x, dpp_f<kDppXor2>(x));
  x = fmaxf(x, dpp_f<kDppHalfMirror>(x));
  x = fmaxf(x, dpp_f<kDppMirror>(x));
  return x;
}

// v_permlane32_swap with both operands x: the two results hold x of lane l and
// x of lane l ^ 32 (in some order), so their sum / max is the pair reduction.
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Same for lane l ^ 16 (rows of 16 lanes swapped pairwise).
__device__ __forceinline__ float sum_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_sum(float x) { return sum_xor32(sum_xor16(sum16(x))); }
__device__ __forceinline__ float wave_max(float x) { return max_xor32(max_xor16(max16(x))); }

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Wave-uniform "any lane" / "all lanes".
__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }
__device__ __forceinline__ bool wave_all(bool p) { return __ballot(!p) == 0ull; }

// Orders this wave's own LDS writes before its later LDS reads (no block barrier).
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Exclusive prefix sum of v over a workgroup of NWAVES wavefronts; returns the
// total. Every thread of the workgroup calls it; s_tmp holds NWAVES ints and
// may be reused once it returns.
template <int NWAVES>
__device__ __forceinline__ int block_excl_scan(int v, int* s_tmp, int& excl) {
  const int lane = __lane_id();
  const int w = threadIdx.x / kWave;
  int x = v;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(x, off);
    x += lane >= off ? y : 0;
  }
  if (lane == kWave - 1) s_tmp[w] = x;
  __syncthreads();
  int wpre = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NWAVES; ++k) {
    const int t = s_tmp[k];
    wpre += k < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  excl = wpre + x - v;
  return tot;
}

// Number of workgroups the blockIdx -> XCD round robin spreads over.
constexpr int kNumXcd = 8;

}  // namespace dash
