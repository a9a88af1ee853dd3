// Cross-input vote of block masks into one static mask.
//
// Source: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
// key design 2, Eq. (8) and the description of Eq. (9): the binary masks chosen for every
// calibration input are averaged element-wise into a keep frequency, and a block is kept when
// that frequency is at least rho (the worked example: rho = 0.5 over 64 inputs keeps blocks
// chosen at least 32 times). The result is encoded once as a read-only skip list (key design 4)
// and reused for new inputs.
//
// vote_accumulate_kernel: one wave per CSR row adds 1 to counts[row][c] for every in-range entry
// of the row. Entries of one row are distinct (ascending CSR), so no two lanes touch the same
// counter and no atomics are needed; the counts are exact integers.
// vote_select_kernel: one wave per row keeps c when counts[row][c] / n >= rho, decided exactly
// as the sign of fma(-rho, n, count) (a single rounding of an exact difference cannot change
// its sign), and writes the kept bitmask and count in the mass-mode format; the CSR is then
// built by the same scan and fill as mass-mode selection.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

__global__ __launch_bounds__(256) void vote_accumulate_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    int64_t col_capacity, int nkb, int64_t rows, int32_t* __restrict__ counts) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int64_t beg = row_ptr[row], end = row_ptr[row + 1];
  beg = beg < 0 ? 0 : (beg > col_capacity ? col_capacity : beg);
  end = end < beg ? beg : (end > col_capacity ? col_capacity : end);
  for (int64_t e = beg + lane; e < end; e += 64) {
    const int c = col_idx[e];
    if (c >= 0 && c < nkb) counts[row * nkb + c] += 1;
  }
}

__global__ __launch_bounds__(256) void vote_select_kernel(const int32_t* __restrict__ counts,
                                                          double n_inputs, double rho,
                                                          SelectArgs a) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.n_rows) return;
  const int lane = threadIdx.x & 63;
  uint32_t cnt = 0;
  for (int e = 0; e < a.words; ++e) {
    const int c = e * 64 + lane;
    const bool keep = c < a.nkb && fma(-rho, n_inputs, (double)counts[row * a.nkb + c]) >= 0.0;
    const uint64_t km = ballot64(keep);
    if (lane == 0) a.masks[row * a.words + e] = km;
    cnt += (uint32_t)__popcll(km);
  }
  if (lane == 0) a.counts[row] = (int32_t)cnt;
}

hipError_t launch_vote_accumulate(const int32_t* row_ptr, const int32_t* col_idx,
                                  int64_t col_capacity, int nkb, int64_t rows, int32_t* counts,
                                  hipStream_t stream) {
  vote_accumulate_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(
      row_ptr, col_idx, col_capacity, nkb, rows, counts);
  return hipGetLastError();
}

hipError_t launch_vote_select(const int32_t* counts, int n_inputs, double rho, const SelectArgs& a,
                              hipStream_t stream) {
  vote_select_kernel<<<(unsigned)((a.n_rows + 3) / 4), 256, 0, stream>>>(counts, (double)n_inputs,
                                                                         rho, a);
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_counts_to_csr(a, stream);
}

}  // namespace dbsp
