// Block mean pooling of K ([SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？",
// method overview, block partition bullet: the vectors inside each 128-token block are averaged;
// a partial last block, when lk is not a multiple of 128, averages the tokens it holds).
//
// One workgroup per key block of a (batch, head): up to 128 consecutive tokens of head_dim
// contiguous elements each, the tokens a fixed stride apart. Each of the 256 threads owns one 16-byte column chunk of
// 128 / (256 / chunks) rows, issues all of its loads before any arithmetic (rows past the end of
// a partial block are not read), sums in fp32, and the partial column sums meet in LDS. Output
// per block: the fp32 mean m split as hi = bf16(m) and lo = bf16(m - hi), in the tiled operand
// order of the scoring MFMAs (see ktile_offset). HBM-bound: every input byte is read once.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

// Pooled keys are stored in the operand order of the scoring MFMAs (16x16x32 bf16, B operand):
// key block n of a (batch, head) with nkb blocks sits in tile t = n / 16 at lane
// l = 16 * kq + (n % 16) of k step ks, where dim d = 32 ks + 8 kq + e. A tile is
// [ks][hi | lo][64 lanes][8] bf16 (D / 32 * 2 KiB), so one wave-wide 16-byte load per
// (ks, hi | lo) reads 1 KiB contiguously.
template <int D>
__device__ __forceinline__ int64_t ktile_offset(int64_t bh, int n, int ntiles, int d, int hl) {
  const int t = n >> 4, m = n & 15;
  const int ks = d >> 5, kq = (d >> 3) & 3, e = d & 7;
  return ((((bh * ntiles + t) * (D / 32) + ks) * 2 + hl) * 64 + 16 * kq + m) * 8 + e;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_blocks_kernel(const T* __restrict__ k, Strides ks,
                                                          int heads, uint16_t* __restrict__ kbar,
                                                          int nkb, int64_t lk) {
  constexpr int kVec = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  constexpr int kChunks = D / kVec;               // chunks per row
  constexpr int kRowsPerPass = 256 / kChunks;     // rows covered by one pass of the workgroup
  constexpr int kPasses = kBlock / kRowsPerPass;  // passes per block
  static_assert(kChunks * kRowsPerPass == 256 && kPasses * kRowsPerPass == kBlock, "shape");

  __shared__ float partial[kRowsPerPass][D + 1];

  const int64_t g = blockIdx.x;
  const int64_t bh = g / nkb;
  const int n = (int)(g - bh * nkb);
  const int64_t first = (int64_t)n * kBlock;
  const int valid = (int)(lk - first < kBlock ? lk - first : kBlock);  // 1 .. 128
  const T* src = k + token_offset(ks, bh, heads, first);
  const int64_t st = ks.t;  // elements between consecutive tokens
  const int t = threadIdx.x;
  const int chunk = t % kChunks;
  const int row0 = t / kChunks;

  u32x4 raw[kPasses];
  if (valid == kBlock) {  // uniform: a whole block, unguarded loads
#pragma unroll
    for (int p = 0; p < kPasses; ++p)
      raw[p] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(src + (int64_t)(row0 + p * kRowsPerPass) * st) + chunk);
  } else {
#pragma unroll
    for (int p = 0; p < kPasses; ++p) {
      const int row = row0 + p * kRowsPerPass;
      raw[p] = row < valid ? __builtin_nontemporal_load(
                                 reinterpret_cast<const u32x4*>(src + (int64_t)row * st) + chunk)
                           : u32x4{0u, 0u, 0u, 0u};
    }
  }

  float acc[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc[e] = 0.f;
#pragma unroll
  for (int p = 0; p < kPasses; ++p) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += __uint_as_float(raw[p][w] << 16);
        acc[2 * w + 1] += __uint_as_float(raw[p][w] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(raw[p][w]);
    }
  }
#pragma unroll
  for (int e = 0; e < kVec; ++e) partial[row0][chunk * kVec + e] = acc[e];
  __syncthreads();
  for (int col = t; col < D; col += 256) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < kRowsPerPass; ++r) s += partial[r][col];
    const float m = valid == kBlock ? s * (1.0f / kBlock) : s / (float)valid;
    const uint32_t hi = f32_to_bf16_bits(m);
    const uint16_t lo = (uint16_t)f32_to_bf16_bits(m - __uint_as_float(hi << 16));
    const int ntiles = (nkb + 15) >> 4;
    kbar[ktile_offset<D>(bh, n, ntiles, col, 0)] = (uint16_t)hi;
    kbar[ktile_offset<D>(bh, n, ntiles, col, 1)] = lo;
  }
}

hipError_t launch_pool(const void* k, const Strides& ks, int heads, uint16_t* kbar, int64_t bh,
                       int nkb, int64_t lk, int head_dim, bool bf16, hipStream_t stream) {
  dim3 grid((unsigned)(bh * nkb)), block(256);
  if (bf16 && head_dim == 128)
    pool_blocks_kernel<uint16_t, 128><<<grid, block, 0, stream>>>((const uint16_t*)k, ks, heads,
                                                                   kbar, nkb, lk);
  else if (bf16 && head_dim == 64)
    pool_blocks_kernel<uint16_t, 64><<<grid, block, 0, stream>>>((const uint16_t*)k, ks, heads,
                                                                  kbar, nkb, lk);
  else if (!bf16 && head_dim == 64)
    pool_blocks_kernel<float, 64><<<grid, block, 0, stream>>>((const float*)k, ks, heads, kbar,
                                                               nkb, lk);
  else if (!bf16 && head_dim == 128)
    pool_blocks_kernel<float, 128><<<grid, block, 0, stream>>>((const float*)k, ks, heads, kbar,
                                                                nkb, lk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dbsp
