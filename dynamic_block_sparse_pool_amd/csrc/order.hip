// Longest-first (LPT) order of the CSR rows for the attention launch, per (batch, head).
//
// In the cumulative-mass mode of [CalibAtt] "Accelerating Text-to-Video Generation with
// Calibrated Sparse Attention" (key design 1) every (head, query block) row keeps a different
// number of key blocks, so the attention workgroups of one launch have unequal work. Started in
// row order, long rows that begin late leave most of the GPU idle at the end of the launch;
// started longest first (the LPT list-scheduling rule), the last rows to start are the short
// ones. The heads keep their order, and only the rows of each head are sorted: the workgroups
// running together then still share one or two heads' K and V in the caches (a global sort
// would mix all heads and overflow the last-level cache). The order only changes which
// workgroup runs which row: every row's result is the same.
//
// A counting sort on the key (head, kept count): count rows per bucket bh * (nkb + 1) + (nkb -
// kept), exclusive scan of the buckets, then each row takes the next slot of its bucket. Rows of
// one head with equal counts land in an unspecified order (slots are taken with atomics). Up to
// kLptHeadBuckets buckets per head the sort runs in one launch with one workgroup per (batch,
// head) and the head's buckets in LDS (lpt_head_kernel); beyond that the buckets of all heads
// live in the caller's workspace and four launches count, scan and place.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

__device__ __forceinline__ int64_t row_bucket(const int32_t* row_ptr, int64_t col_capacity,
                                              int64_t r, int nqb, int nkb) {
  int64_t b = row_ptr[r], e = row_ptr[r + 1];
  b = b < 0 ? 0 : (b > col_capacity ? col_capacity : b);
  e = e < b ? b : (e > col_capacity ? col_capacity : e);
  const int64_t len = e - b;
  return (r / nqb) * (nkb + 1) + (nkb - (len < nkb ? len : nkb));
}

constexpr int kLptHeadBuckets = 8192;  // 32 KiB of LDS

// One workgroup per (batch, head) pair bh: its nqb rows, bucketed by nkb - kept count.
__global__ __launch_bounds__(1024) void lpt_head_kernel(const int32_t* __restrict__ row_ptr,
                                                        int64_t col_capacity, int nqb, int nkb,
                                                        int32_t* __restrict__ order) {
  extern __shared__ int32_t bucket[];  // nkb + 1 counts, then start slots
  __shared__ uint32_t wave_tot[16];
  const int nbk = nkb + 1;
  const int64_t base = (int64_t)blockIdx.x * nqb;  // the head's first row
  const int64_t key0 = (int64_t)blockIdx.x * nbk;   // row_bucket of the head's first bucket
  const int t = threadIdx.x;
  for (int i = t; i < nbk; i += 1024) bucket[i] = 0;
  __syncthreads();
  for (int i = t; i < nqb; i += 1024)
    atomicAdd(&bucket[row_bucket(row_ptr, col_capacity, base + i, nqb, nkb) - key0], 1);
  __syncthreads();
  // exclusive scan of the buckets: thread t owns buckets [per t, per t + per)
  const int per = (nbk + 1023) / 1024;
  const int b0 = t * per;
  uint32_t own = 0;
  for (int i = 0; i < per; ++i)
    if (b0 + i < nbk) own += (uint32_t)bucket[b0 + i];
  const uint32_t incl = wave_prefix_sum_u32(own);
  const int lane = t & 63, wave = t >> 6;
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  uint32_t run = incl - own;
  for (int i = 0; i < wave; ++i) run += wave_tot[i];
  for (int i = 0; i < per; ++i) {
    if (b0 + i < nbk) {
      const int32_t c = bucket[b0 + i];
      bucket[b0 + i] = (int32_t)run;
      run += (uint32_t)c;
    }
  }
  __syncthreads();
  for (int i = t; i < nqb; i += 1024) {
    const int32_t pos =
        atomicAdd(&bucket[row_bucket(row_ptr, col_capacity, base + i, nqb, nkb) - key0], 1);
    order[base + pos] = (int32_t)(base + i);
  }
}

__global__ __launch_bounds__(256) void lpt_zero_kernel(int32_t* counts, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) counts[i] = 0;
}

__global__ __launch_bounds__(256) void lpt_count_kernel(const int32_t* __restrict__ row_ptr,
                                                        int64_t col_capacity, int64_t rows,
                                                        int nqb, int nkb, int32_t* counts) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < rows) atomicAdd(&counts[row_bucket(row_ptr, col_capacity, r, nqb, nkb)], 1);
}

__global__ __launch_bounds__(256) void lpt_place_kernel(const int32_t* __restrict__ row_ptr,
                                                        int64_t col_capacity, int64_t rows,
                                                        int nqb, int nkb, int32_t* cursor,
                                                        int32_t* __restrict__ order) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r >= rows) return;
  const int32_t pos = atomicAdd(&cursor[row_bucket(row_ptr, col_capacity, r, nqb, nkb)], 1);
  order[pos] = (int32_t)r;
}

hipError_t launch_row_order_lpt(const int32_t* row_ptr, int64_t col_capacity, int64_t rows,
                                int nqb, int nkb, int32_t* order, int32_t* counts,
                                int32_t* cursor, hipStream_t stream) {
  const int64_t nb = (rows / nqb) * (int64_t)(nkb + 1);
  if (rows == 0) return hipSuccess;
  if (nkb + 1 <= kLptHeadBuckets) {
    lpt_head_kernel<<<(unsigned)(rows / nqb), 1024, (size_t)(nkb + 1) * sizeof(int32_t),
                      stream>>>(row_ptr, col_capacity, nqb, nkb, order);
    return hipGetLastError();
  }
  lpt_zero_kernel<<<(unsigned)((nb + 255) / 256), 256, 0, stream>>>(counts, nb);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const unsigned grid = (unsigned)((rows + 255) / 256);
  lpt_count_kernel<<<grid, 256, 0, stream>>>(row_ptr, col_capacity, rows, nqb, nkb, counts);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  if ((err = launch_exclusive_scan(counts, cursor, nb, stream)) != hipSuccess) return err;
  lpt_place_kernel<<<grid, 256, 0, stream>>>(row_ptr, col_capacity, rows, nqb, nkb, cursor,
                                             order);
  return hipGetLastError();
}

}  // namespace dbsp
