// Shared device helpers for the gfx950 kernels of libdbsp.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbsp {

constexpr int kBlock = 128;  // tokens per block

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Round-to-nearest-even float -> bf16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Order-preserving map float32 -> uint32 (larger float, larger key). -0.0 is folded onto +0.0
// first so that the two zeros tie. Finite values and infinities map to keys >= 1.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0) u = 0;  // -0.0 -> +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Number of set bits of `mask` in lanes below the calling lane.
__device__ __forceinline__ int mbcnt64(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot64(bool p) { return __ballot(p); }

// Cross-lane steps through DPP (no LDS round trip). dpp<CTRL, ROW_MASK>(v) returns v moved as
// CTRL says, and 0 in lanes with no source or in rows outside ROW_MASK.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xf, false);
}
constexpr int kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114, kRowShr8 = 0x118;
constexpr int kRowBcast15 = 0x142, kRowBcast31 = 0x143;

// Inclusive prefix sum over the 64 lanes (lane i gets the sum of lanes 0..i).
__device__ __forceinline__ uint32_t wave_prefix_sum_u32(uint32_t v) {
  v += dpp_u32<kRowShr1>(v);
  v += dpp_u32<kRowShr2>(v);
  v += dpp_u32<kRowShr4>(v);
  v += dpp_u32<kRowShr8>(v);
  v += dpp_u32<kRowBcast15, 0xa>(v);
  v += dpp_u32<kRowBcast31, 0xc>(v);
  return v;
}

__device__ __forceinline__ uint64_t wave_prefix_sum_u64(uint64_t v) {
#define DBSP_ADD64(CTRL, MASK)                                                               \
  v += ((uint64_t)dpp_u32<CTRL, MASK>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL, MASK>((uint32_t)v);
  DBSP_ADD64(kRowShr1, 0xf)
  DBSP_ADD64(kRowShr2, 0xf)
  DBSP_ADD64(kRowShr4, 0xf)
  DBSP_ADD64(kRowShr8, 0xf)
  DBSP_ADD64(kRowBcast15, 0xa)
  DBSP_ADD64(kRowBcast31, 0xc)
#undef DBSP_ADD64
  return v;
}

__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int lane) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}

// Wave-wide reductions through the prefix scan; the result is wave-uniform.
__device__ __forceinline__ uint64_t wave_total_u64(uint64_t v) {
  v = wave_prefix_sum_u64(v);
  return ((uint64_t)lane_u32((uint32_t)(v >> 32), 63) << 32) | lane_u32((uint32_t)v, 63);
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f32(float v, float fill) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, fill),
                                                               __builtin_bit_cast(int, v), CTRL,
                                                               ROW_MASK, 0xf, false));
}
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ uint32_t dpp_fill_u32(uint32_t v, uint32_t fill) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)v, CTRL, ROW_MASK, 0xf, false);
}

// Wave-wide max / sum / min through the same scan pattern; the results are wave-uniform.
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = fmaxf(v, dpp_f32<kRowShr1>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowShr2>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowShr4>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowShr8>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowBcast15, 0xa>(v, -INFINITY));
  v = fmaxf(v, dpp_f32<kRowBcast31, 0xc>(v, -INFINITY));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_total_f32(float v) {
  v += dpp_f32<kRowShr1>(v, 0.f);
  v += dpp_f32<kRowShr2>(v, 0.f);
  v += dpp_f32<kRowShr4>(v, 0.f);
  v += dpp_f32<kRowShr8>(v, 0.f);
  v += dpp_f32<kRowBcast15, 0xa>(v, 0.f);
  v += dpp_f32<kRowBcast31, 0xc>(v, 0.f);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t v) {
  v = min(v, dpp_fill_u32<kRowShr1>(v, 0xffffffffu));
  v = min(v, dpp_fill_u32<kRowShr2>(v, 0xffffffffu));
  v = min(v, dpp_fill_u32<kRowShr4>(v, 0xffffffffu));
  v = min(v, dpp_fill_u32<kRowShr8>(v, 0xffffffffu));
  v = min(v, dpp_fill_u32<kRowBcast15, 0xa>(v, 0xffffffffu));
  v = min(v, dpp_fill_u32<kRowBcast31, 0xc>(v, 0xffffffffu));
  return lane_u32(v, 63);
}
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
  v = max(v, dpp_fill_u32<kRowShr1>(v, 0u));
  v = max(v, dpp_fill_u32<kRowShr2>(v, 0u));
  v = max(v, dpp_fill_u32<kRowShr4>(v, 0u));
  v = max(v, dpp_fill_u32<kRowShr8>(v, 0u));
  v = max(v, dpp_fill_u32<kRowBcast15, 0xa>(v, 0u));
  v = max(v, dpp_fill_u32<kRowBcast31, 0xc>(v, 0u));
  return lane_u32(v, 63);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t lo = __shfl_xor((uint32_t)v, off, 64);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), off, 64);
    v += ((uint64_t)hi << 32) | lo;
  }
  return v;
}

__device__ __forceinline__ u32x4 load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

}  // namespace dbsp
