// Interval encoding of the skip list.
//
// Source: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
// key design 4: the mask of each query block is stored as the contiguous intervals of key
// blocks it needs, preloaded read-only before generation. These kernels convert between that
// encoding and the CSR the attention kernel reads:
//   csr_runs_kernel      one wave per row counts the maximal runs of consecutive blocks;
//   (per-row counts -> exclusive scan, shared with mass-mode selection)
//   csr_to_iv_kernel     one wave per row writes [start, end) of every run, pairing the k-th
//                        run start with the k-th run end in entry order;
//   iv_lengths_kernel    one wave per row sums its interval lengths;
//   iv_to_csr_kernel     one wave per row writes the blocks of its intervals in order.
// Entries outside [0, nkb) are skipped; an in-range CSR entry c continues the run of the entry
// before it when that entry is c - 1 (ascending CSRs, as this library writes them, encode
// exactly). Writes past a capacity are dropped (the host sizes capacities by the bound).
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

__device__ __forceinline__ void row_extent(const int32_t* row_ptr, int64_t row, int64_t cap,
                                           int64_t* beg, int64_t* end) {
  int64_t b = row_ptr[row], e = row_ptr[row + 1];
  b = b < 0 ? 0 : (b > cap ? cap : b);
  e = e < b ? b : (e > cap ? cap : e);
  *beg = b;
  *end = e;
}

// Entry e of a row starts (ends) a run: in range, and the entry before (after) it is not the
// in-range block just below (above). The neighbour has to be in range itself: an out-of-range
// -1 before block 0 (or nkb after block nkb - 1) continues nothing, so every chain of in-range
// entries that step by +1 has exactly one start (its first entry) and one stop (its last), and
// the k-th start and the k-th stop of a row always belong to the same run.
__device__ __forceinline__ void run_flags(const int32_t* col_idx, int64_t e, int64_t beg,
                                          int64_t end, int nkb, bool* start, bool* stop,
                                          int* c_out) {
  const bool live = e < end;
  const int c = live ? col_idx[e] : -1;
  const bool in = live && c >= 0 && c < nkb;
  const int prev = (live && e > beg) ? col_idx[e - 1] : -2;
  const int next = (live && e + 1 < end) ? col_idx[e + 1] : -2;
  *start = in && !(c > 0 && prev == c - 1);
  *stop = in && !(c + 1 < nkb && next == c + 1);
  *c_out = c;
}

__global__ __launch_bounds__(256) void csr_runs_kernel(const int32_t* __restrict__ row_ptr,
                                                       const int32_t* __restrict__ col_idx,
                                                       int64_t col_capacity, int nkb,
                                                       int64_t rows, int32_t* __restrict__ counts) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int64_t beg, end;
  row_extent(row_ptr, row, col_capacity, &beg, &end);
  int n = 0;
  for (int64_t e0 = beg; e0 < end; e0 += 64) {
    bool start, stop;
    int c;
    run_flags(col_idx, e0 + lane, beg, end, nkb, &start, &stop, &c);
    n += __popcll(ballot64(start));
  }
  if (lane == 0) counts[row] = n;
}

__global__ __launch_bounds__(256) void csr_to_iv_kernel(const int32_t* __restrict__ row_ptr,
                                                        const int32_t* __restrict__ col_idx,
                                                        int64_t col_capacity, int nkb,
                                                        int64_t rows,
                                                        const int32_t* __restrict__ iv_ptr,
                                                        int32_t* __restrict__ iv,
                                                        int64_t iv_capacity) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int64_t beg, end;
  row_extent(row_ptr, row, col_capacity, &beg, &end);
  int64_t ns = iv_ptr[row], ne = iv_ptr[row];
  for (int64_t e0 = beg; e0 < end; e0 += 64) {
    bool start, stop;
    int c;
    run_flags(col_idx, e0 + lane, beg, end, nkb, &start, &stop, &c);
    const uint64_t sm = ballot64(start), em = ballot64(stop);
    const int64_t ps = ns + mbcnt64(sm), pe = ne + mbcnt64(em);
    if (start && ps < iv_capacity) iv[2 * ps] = c;
    if (stop && pe < iv_capacity) iv[2 * pe + 1] = c + 1;
    ns += __popcll(sm);
    ne += __popcll(em);
  }
}

// Interval j of a row, clipped to [0, nkb) (an empty or reversed interval has length 0).
__device__ __forceinline__ void iv_clip(const int32_t* iv, int64_t j, int nkb, int* s, int* n) {
  int a = iv[2 * j], b = iv[2 * j + 1];
  a = a < 0 ? 0 : (a > nkb ? nkb : a);
  b = b < a ? a : (b > nkb ? nkb : b);
  *s = a;
  *n = b - a;
}

__global__ __launch_bounds__(256) void iv_lengths_kernel(const int32_t* __restrict__ iv_ptr,
                                                         const int32_t* __restrict__ iv,
                                                         int64_t iv_capacity, int nkb,
                                                         int64_t rows, int32_t* __restrict__ counts) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int64_t beg, end;
  row_extent(iv_ptr, row, iv_capacity, &beg, &end);
  int64_t total = 0;
  for (int64_t j = beg + lane; j < end; j += 64) {
    int s, n;
    iv_clip(iv, j, nkb, &s, &n);
    total += n;
  }
  total = wave_sum_u64((uint64_t)total);
  if (lane == 0) counts[row] = (int32_t)total;
}

__global__ __launch_bounds__(256) void iv_to_csr_kernel(const int32_t* __restrict__ iv_ptr,
                                                        const int32_t* __restrict__ iv,
                                                        int64_t iv_capacity, int nkb, int64_t rows,
                                                        const int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        int64_t col_capacity) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int64_t beg, end;
  row_extent(iv_ptr, row, iv_capacity, &beg, &end);
  int64_t out = row_ptr[row];
  for (int64_t j = beg; j < end; ++j) {
    int s, n;
    iv_clip(iv, j, nkb, &s, &n);
    for (int t = lane; t < n; t += 64)
      if (out + t < col_capacity) col_idx[out + t] = s + t;
    out += n;
  }
}

static hipError_t scan_rows(const int32_t* counts, int32_t* ptr, int64_t rows, hipStream_t stream) {
  SelectArgs a{};
  a.counts = const_cast<int32_t*>(counts);
  a.row_ptr = ptr;
  a.n_rows = rows;
  return launch_scan_counts(a, stream);
}

hipError_t launch_csr_to_intervals(const int32_t* row_ptr, const int32_t* col_idx,
                                   int64_t col_capacity, int nkb, int64_t rows, int32_t* iv_ptr,
                                   int32_t* iv, int64_t iv_capacity, int32_t* counts,
                                   hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + 3) / 4);
  csr_runs_kernel<<<grid, 256, 0, stream>>>(row_ptr, col_idx, col_capacity, nkb, rows, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if ((err = scan_rows(counts, iv_ptr, rows, stream)) != hipSuccess) return err;
  csr_to_iv_kernel<<<grid, 256, 0, stream>>>(row_ptr, col_idx, col_capacity, nkb, rows, iv_ptr, iv,
                                             iv_capacity);
  return hipGetLastError();
}

hipError_t launch_intervals_to_csr(const int32_t* iv_ptr, const int32_t* iv, int64_t iv_capacity,
                                   int nkb, int64_t rows, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, int32_t* counts, hipStream_t stream) {
  const unsigned grid = (unsigned)((rows + 3) / 4);
  iv_lengths_kernel<<<grid, 256, 0, stream>>>(iv_ptr, iv, iv_capacity, nkb, rows, counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if ((err = scan_rows(counts, row_ptr, rows, stream)) != hipSuccess) return err;
  iv_to_csr_kernel<<<grid, 256, 0, stream>>>(iv_ptr, iv, iv_capacity, nkb, rows, row_ptr, col_idx,
                                             col_capacity);
  return hipGetLastError();
}

}  // namespace dbsp
