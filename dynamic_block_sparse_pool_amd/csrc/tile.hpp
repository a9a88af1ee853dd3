// 128 x 128 bf16 tiles in LDS for the MFMA kernels: swizzles, global-to-LDS DMA of a tile, and
// the raw barrier / wait helpers that keep the DMA in flight across workgroup barriers.
#pragma once

#include "common.hpp"

namespace dbsp {

// LDS tiles hold one key block of K or V (128 rows x 256 bytes) unpadded. Global-to-LDS DMA
// writes 1 KiB per wave instruction contiguously, so bank conflicts are avoided by an XOR
// swizzle of the 16-byte chunk index within each row instead of padding:
//   K: physical chunk = c ^ (row & 15)      (16 consecutive rows read at one logical chunk)
//   V: physical chunk = c ^ (4 * (row & 3))  (transpose reads: 4 rows x 4 chunks per half wave)
__device__ __forceinline__ int k_swz(int row, int chunk) { return chunk ^ (row & 15); }
__device__ __forceinline__ int v_swz(int row, int chunk) { return chunk ^ ((row & 3) << 2); }

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(0xF | (0x3 << 14) | (0x7 << 4));
}
// Workgroup barrier without the implicit drain of outstanding vector-memory operations that a
// fenced barrier would add (the K/V prefetch must stay in flight across it). The empty asm
// statements keep the compiler from moving memory accesses across the barrier; the waits the
// algorithm needs are issued explicitly next to each barrier.
__device__ __forceinline__ void wg_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __attribute__((address_space(3))) void lds_void;

// Per-lane byte offsets (inside a 4-row slab) of the global source of a tile DMA, for K rows
// rbk bytes apart and V rows rbv bytes apart (256 for contiguous bf16 x 128 tensors). For slab i
// (rows 4 i .. 4 i + 3 of the wave's 32) the swizzle depends on the row only modulo 16 (K) or
// 4 (V), so K needs four offsets (i mod 4) and V one.
struct DmaOffsets {
  uint32_t k[4];
  uint32_t v;
};

__device__ __forceinline__ DmaOffsets dma_offsets(int lane, int rbk, int rbv) {
  DmaOffsets d;
  const int r = lane >> 4, pc = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) d.k[i] = (uint32_t)(r * rbk + k_swz(4 * i + r, pc) * 16);
  d.v = (uint32_t)(r * rbv + v_swz(r, pc) * 16);
  return d;
}

// Raw buffer resource over `bytes` bytes at `base` (gfx9 descriptor: 32-bit data format, no
// stride, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// Issue the DMA of one 128 x 128 bf16 tile (128 rows `rb` bytes apart, starting at byte
// `tile_off` of the head's K or V, wave-uniform) into LDS: wave w copies rows 32 w .. 32 w + 31,
// one 4-row slab (1 KiB of LDS) per instruction, lane l landing at byte 16 l of the slab, so the
// swizzle is applied on the global side. The buffer form takes the row offset in a scalar
// register and the lane offset in a 32-bit vector register, so the addressing costs no vector
// instructions.
template <bool kIsV>
__device__ __forceinline__ void tile_dma(__amdgpu_buffer_rsrc_t src, int tile_off, uint16_t* lds,
                                         int w, const DmaOffsets& d, int rb) {
  const int wave_off = tile_off + w * 32 * rb;
  uint16_t* wave_dst = lds + w * (32 * 128);
#pragma unroll
  for (int i = 0; i < 8; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(src, (lds_void*)(wave_dst + 4 * i * 128), 16,
                                             kIsV ? d.v : d.k[i & 3], wave_off + 4 * i * rb, 0,
                                             0);
}

// S^T tiles of one key block: sacc[jt] holds keys 32 jt .. 32 jt + 31 (rows) x the wave's 32
// queries; qf is the B operand (queries as columns) held in registers.
__device__ __forceinline__ void qk_block(const uint16_t* k_tile, const bf16x8 (&qf)[8], int l32,
                                         int h, f32x16 (&sacc)[4]) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[jt][r] = 0.f;
    const int kr = 32 * jt + l32;
    const uint16_t* krow = k_tile + kr * 128;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + k_swz(kr, 2 * s + h) * 8);
      sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[jt], 0, 0, 0);
    }
  }
}

// Key row (within its 128-key tile) of accumulator register r of sacc[jt] in lane half h: the
// 32x32 MFMA result layout puts row 8 (r / 4) + 4 h + r % 4 of the 32-row tile jt in register r.
__device__ __forceinline__ int sacc_key(int jt, int r, int h) {
  return 32 * jt + 8 * (r >> 2) + 4 * h + (r & 3);
}

// Plain (not DMA) copy of a partial tile: rows [0, valid) of `src` (128 bf16 per row, rows
// `stride` elements apart) into the swizzled LDS layout, rows [valid, 128) zero-filled. All 256
// threads of the workgroup take part; the caller synchronises before and after.
template <bool kIsV>
__device__ __forceinline__ void tile_load_partial(const uint16_t* src, int valid, uint16_t* lds,
                                                  int tid, int64_t stride) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int q = tid + 256 * i;  // 16-byte chunk of the tile
    const int row = q >> 4, lc = q & 15;
    const u32x4 v = row < valid
                        ? *reinterpret_cast<const u32x4*>(src + row * stride + lc * 8)
                        : u32x4{0u, 0u, 0u, 0u};
    const int pc = kIsV ? v_swz(row, lc) : k_swz(row, lc);
    *reinterpret_cast<u32x4*>(lds + row * 128 + pc * 8) = v;
  }
}

__device__ __forceinline__ int64_t clip64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

}  // namespace dbsp
