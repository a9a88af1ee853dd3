// Block mean pooling of Q and K ([SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？",
// method overview, block partition bullet: the vectors inside each 128-token block are averaged).
//
// One launch pools every Q block and every K block. Workgroup g < nq_blocks reads Q block g,
// the rest read K blocks; a block is 128 consecutive rows of head_dim elements, contiguous in
// memory (32 KiB for bf16 x 128 or fp32 x 64). Each of the 256 threads owns one 16-byte column
// chunk of 128 / (256 / chunks) rows, issues all of its loads before any arithmetic, sums in
// fp32, and the partial column sums meet in LDS. Output: fp32 [blocks, head_dim] means.
// HBM-bound: every input byte is read exactly once.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

template <typename T, int D>
__global__ __launch_bounds__(256) void pool_blocks_kernel(const T* __restrict__ q,
                                                          const T* __restrict__ k,
                                                          float* __restrict__ qbar,
                                                          float* __restrict__ kbar,
                                                          int64_t nq_blocks) {
  constexpr int kVec = 16 / (int)sizeof(T);       // elements per 16-byte chunk
  constexpr int kChunks = D / kVec;               // chunks per row
  constexpr int kRowsPerPass = 256 / kChunks;     // rows covered by one pass of the workgroup
  constexpr int kPasses = kBlock / kRowsPerPass;  // passes per block
  static_assert(kChunks * kRowsPerPass == 256 && kPasses * kRowsPerPass == kBlock, "shape");

  __shared__ float partial[kRowsPerPass][D + 1];

  int64_t g = blockIdx.x;
  const T* src;
  float* dst;
  if (g < nq_blocks) {
    src = q + g * (int64_t)kBlock * D;
    dst = qbar + g * D;
  } else {
    g -= nq_blocks;
    src = k + g * (int64_t)kBlock * D;
    dst = kbar + g * D;
  }
  const int t = threadIdx.x;
  const int chunk = t % kChunks;
  const int row0 = t / kChunks;

  u32x4 raw[kPasses];
#pragma unroll
  for (int p = 0; p < kPasses; ++p)
    raw[p] = __builtin_nontemporal_load(
        reinterpret_cast<const u32x4*>(src + (int64_t)(row0 + p * kRowsPerPass) * D) + chunk);

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
    dst[col] = s * (1.0f / kBlock);
  }
}

hipError_t launch_pool(const void* q, const void* k, float* qbar, float* kbar, int64_t nq_blocks,
                       int64_t nk_blocks, int head_dim, bool bf16, hipStream_t stream) {
  dim3 grid((unsigned)(nq_blocks + nk_blocks)), block(256);
  if (bf16 && head_dim == 128)
    pool_blocks_kernel<uint16_t, 128><<<grid, block, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k, qbar, kbar, nq_blocks);
  else if (bf16 && head_dim == 64)
    pool_blocks_kernel<uint16_t, 64><<<grid, block, 0, stream>>>(
        (const uint16_t*)q, (const uint16_t*)k, qbar, kbar, nq_blocks);
  else if (!bf16 && head_dim == 64)
    pool_blocks_kernel<float, 64><<<grid, block, 0, stream>>>((const float*)q, (const float*)k,
                                                               qbar, kbar, nq_blocks);
  else if (!bf16 && head_dim == 128)
    pool_blocks_kernel<float, 128><<<grid, block, 0, stream>>>((const float*)q, (const float*)k,
                                                                qbar, kbar, nq_blocks);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dbsp
