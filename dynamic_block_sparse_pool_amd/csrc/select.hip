// Pooled block scores, clip-aware forced blocks, Top-K / cumulative-mass selection and the CSR
// skip list.
//
// Sources: [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", method overview
// (aggregated block scores, clip-aware dense segments, joint Top-K per head and query block,
// forward-only index); [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse
// Attention", key design 1 and Eq. (5) (shortest energy-sorted prefix reaching a threshold,
// restored to block order) and key design 4 (per-query-block skip list).
//
// score_select_kernel: one workgroup (4 waves) owns 16 consecutive query blocks of one
// (batch, head). Phase 1 computes S = qbar kbar^T * scale for its 16 rows against every key
// block with 16x16x32 bf16 MFMAs on a hi/lo split of the fp32 operands
// (x = hi + lo, hi = bf16(x), lo = bf16(x - hi); S ~ hi.hi + hi.lo + lo.hi, relative error
// near 2^-16 of |qbar||kbar|), and parks the 16 score rows in LDS. Phase 2 gives each wave
// four rows; a wave holds one row in registers (lane l, slot e -> key block 64 e + l) and
// finds the selection threshold by an MSB-first bitwise search over order-preserving uint32
// keys, using wave ballots (Top-K: counts) or 64-bit wave sums of fixed-point masses (mass).
// Keys above the threshold are kept, and keys equal to it in ascending block order until the
// count or mass is met: the same set a stable (value desc, index asc) sort prefix gives.
// Emitting kept flags slot by slot with mbcnt yields col_idx already ascending.
//
// Top-K rows all have |F| + K entries, so row_ptr is written in closed form. Mass rows vary:
// the kernel stores a per-row bitmask and count, scan_counts_kernel forms row_ptr, and
// fill_csr_kernel expands the bitmasks into col_idx.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

constexpr int kRowsPerWG = 16;
constexpr uint32_t kMassBits = 62;


__device__ __forceinline__ void split_bf16(const float* x, bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    __bf16 h = (__bf16)x[e];
    hi[e] = h;
    lo[e] = (__bf16)(x[e] - (float)h);
  }
}

// Exact floor(p * 2^62) for a non-negative finite float p < 2.
__device__ __forceinline__ uint64_t mass_units(float p) {
  uint32_t u = __float_as_uint(p);
  int ex = (int)((u >> 23) & 0xffu);
  if (ex == 0) return 0;  // zero or subnormal: below 2^-126, far below one unit
  uint64_t m = (uint64_t)((u & 0x7fffffu) | 0x800000u);
  int sh = ex - 150 + (int)kMassBits;  // p = m * 2^(ex - 150)
  if (sh >= 0) return m << sh;         // sh <= 40 for p < 2
  if (sh <= -64) return 0;
  return m >> (-sh);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

__device__ __forceinline__ bool is_forced(int c, const SelectArgs& a) {
  return (c >= a.t0 && c < a.t1) || (c >= a.e0 && c < a.e1);
}

template <int D, int MAXSLOTS>
__global__ __launch_bounds__(256) void score_select_kernel(SelectArgs a) {
  extern __shared__ float s_lds[];  // [kRowsPerWG][lds_stride]
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * kRowsPerWG;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nkb = a.nkb;

  // ---------------- phase 1: scores for 16 rows x all key blocks
  {
    constexpr int KSTEPS = D / 32;
    const int m = lane & 15;       // A row / B column inside the 16x16 tile
    const int kq = lane >> 4;      // which 8-wide k chunk of the 32
    bf16x8 qhi[KSTEPS], qlo[KSTEPS];
    {
      const int qi = row0 + m;
      const float* qrow = a.qbar + ((int64_t)bh * a.nqb + qi) * D;
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        float x[8];
        if (qi < a.nqb) {
          f32x4 v0 = *reinterpret_cast<const f32x4*>(qrow + ks * 32 + kq * 8);
          f32x4 v1 = *reinterpret_cast<const f32x4*>(qrow + ks * 32 + kq * 8 + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { x[e] = v0[e]; x[4 + e] = v1[e]; }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        split_bf16(x, qhi[ks], qlo[ks]);
      }
    }
    const int ntiles = (nkb + 15) >> 4;
    const float* kbase = a.kbar + (int64_t)bh * nkb * D;
    for (int t = wave; t < ntiles; t += 4) {
      const int n = t * 16 + m;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        float x[8];
        if (n < nkb) {
          const float* kr = kbase + (int64_t)n * D + ks * 32 + kq * 8;
          f32x4 v0 = *reinterpret_cast<const f32x4*>(kr);
          f32x4 v1 = *reinterpret_cast<const f32x4*>(kr + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) { x[e] = v0[e]; x[4 + e] = v1[e]; }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = 0.f;
        }
        bf16x8 khi, klo;
        split_bf16(x, khi, klo);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo[ks], khi, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[ks], klo, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[ks], khi, acc, 0, 0, 0);
      }
      if (n < nkb) {
#pragma unroll
        for (int r = 0; r < 4; ++r) s_lds[(kq * 4 + r) * a.lds_stride + n] = acc[r] * a.scale;
      }
    }
  }
  __syncthreads();

  // ---------------- phase 2: per-row selection, one wave per row
  const int slots = (nkb + 63) >> 6;
  for (int rr = wave; rr < kRowsPerWG; rr += 4) {
    const int qi = row0 + rr;
    if (qi >= a.nqb) break;
    const int64_t row = (int64_t)bh * a.nqb + qi;
    const float* srow = s_lds + rr * a.lds_stride;

    float val[MAXSLOTS];
    uint32_t key[MAXSLOTS];
#pragma unroll
    for (int e = 0; e < MAXSLOTS; ++e) {
      const int c = e * 64 + lane;
      val[e] = (e < slots && c < nkb) ? srow[c] : 0.f;
    }

    if (a.mode == 0) {
      // ---- Top-K
      if (a.scores_out) {
#pragma unroll
        for (int e = 0; e < MAXSLOTS; ++e) {
          const int c = e * 64 + lane;
          if (e < slots && c < nkb) a.scores_out[row * nkb + c] = val[e];
        }
      }
#pragma unroll
      for (int e = 0; e < MAXSLOTS; ++e) {
        const int c = e * 64 + lane;
        key[e] = (e < slots && c < nkb && !is_forced(c, a)) ? order_key(val[e]) : 0u;
      }
      const uint32_t kk = (uint32_t)a.kk;
      uint32_t T = 0;
      bool exact = false;
      if (kk > 0) {
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = T | (1u << bit);
          uint32_t cnt = 0;
#pragma unroll
          for (int e = 0; e < MAXSLOTS; ++e)
            if (e < slots) cnt += (uint32_t)__popcll(ballot64(key[e] >= cand));
          if (cnt >= kk) {
            T = cand;
            if (cnt == kk) { exact = true; break; }
          }
        }
      }
      uint32_t need = 0;  // how many keys equal to T are kept
      if (kk > 0 && !exact) {
        uint32_t gt = 0;
#pragma unroll
        for (int e = 0; e < MAXSLOTS; ++e)
          if (e < slots) gt += (uint32_t)__popcll(ballot64(key[e] > T));
        need = kk - gt;
      }
      int64_t out = row * (int64_t)a.per_row;
      uint32_t eq_seen = 0;
#pragma unroll
      for (int e = 0; e < MAXSLOTS; ++e) {
        if (e >= slots) continue;
        const int c = e * 64 + lane;
        const bool valid = c < nkb;
        bool keep = valid && is_forced(c, a);
        if (kk > 0) {
          if (exact) {
            keep = keep || key[e] >= T;
          } else {
            const bool eq = key[e] == T;
            const uint64_t eqm = ballot64(eq);
            keep = keep || key[e] > T || (eq && eq_seen + (uint32_t)mbcnt64(eqm) < need);
            eq_seen += (uint32_t)__popcll(eqm);
          }
        }
        const uint64_t km = ballot64(keep);
        const int64_t pos = out + mbcnt64(km);
        if (keep && pos < a.col_capacity) a.col_idx[pos] = c;
        out += __popcll(km);
      }
      if (lane == 0) {
        a.row_ptr[row] = (int32_t)(row * a.per_row);
        if (row == (int64_t)gridDim.y * a.nqb - 1) a.row_ptr[row + 1] = (int32_t)((row + 1) * a.per_row);
      }
    } else {
      // ---- cumulative mass over the softmax of the row
      float mx = -INFINITY;
#pragma unroll
      for (int e = 0; e < MAXSLOTS; ++e) {
        const int c = e * 64 + lane;
        if (e < slots && c < nkb) mx = fmaxf(mx, val[e]);
      }
      mx = wave_max_f32(mx);
      float part = 0.f;
#pragma unroll
      for (int e = 0; e < MAXSLOTS; ++e) {
        const int c = e * 64 + lane;
        val[e] = (e < slots && c < nkb) ? __expf(val[e] - mx) : 0.f;
        part += val[e];
      }
      const float inv = 1.0f / wave_sum_f32(part);
      uint64_t fsum = 0, csum = 0;
#pragma unroll
      for (int e = 0; e < MAXSLOTS; ++e) {
        const int c = e * 64 + lane;
        const bool valid = e < slots && c < nkb;
        const float p = val[e] * inv;
        val[e] = p;
        if (valid && a.scores_out) a.scores_out[row * nkb + c] = p;
        const bool f = valid && is_forced(c, a);
        key[e] = (valid && !f) ? order_key(p) : 0u;
        const uint64_t u = valid ? mass_units(p) : 0ull;
        if (f) fsum += u; else csum += u;
      }
      fsum = wave_sum_u64(fsum);
      csum = wave_sum_u64(csum);
      // mode: 0 keep forced only, 1 keep all, 2 threshold
      int how;
      uint64_t need_mass = 0;
      if (a.keep_all) how = 1;
      else if (fsum >= a.theta) how = 0;
      else {
        need_mass = a.theta - fsum;
        how = (csum < need_mass) ? 1 : 2;
      }
      uint32_t T = 0;
      uint64_t n_eq = 0;
      if (how == 2) {
        for (int bit = 31; bit >= 0; --bit) {
          const uint32_t cand = T | (1u << bit);
          uint64_t s = 0;
#pragma unroll
          for (int e = 0; e < MAXSLOTS; ++e)
            if (e < slots && key[e] >= cand) s += mass_units(val[e]);
          s = wave_sum_u64(s);
          if (s >= need_mass) T = cand;
        }
        uint64_t above = 0;
#pragma unroll
        for (int e = 0; e < MAXSLOTS; ++e)
          if (e < slots && key[e] > T) above += mass_units(val[e]);
        above = wave_sum_u64(above);
        const uint64_t uT = mass_units(key_to_float(T));  // > 0 by construction of T
        n_eq = (need_mass - above + uT - 1) / uT;
      }
      uint32_t cnt = 0;
      uint64_t eq_seen = 0;
      uint64_t* mrow = a.masks + row * a.words;
#pragma unroll
      for (int e = 0; e < MAXSLOTS; ++e) {
        if (e >= slots) continue;
        const int c = e * 64 + lane;
        const bool valid = c < nkb;
        bool keep;
        if (how == 1) keep = valid;
        else {
          keep = valid && is_forced(c, a);
          if (how == 2) {
            const bool eq = key[e] == T;
            const uint64_t eqm = ballot64(eq);
            keep = keep || key[e] > T || (eq && eq_seen + (uint64_t)mbcnt64(eqm) < n_eq);
            eq_seen += (uint64_t)__popcll(eqm);
          }
        }
        const uint64_t km = ballot64(keep);
        if (lane == 0) mrow[e] = km;
        cnt += (uint32_t)__popcll(km);
      }
      if (lane == 0) a.counts[row] = (int32_t)cnt;
    }
  }
}

// Exclusive prefix sum of the per-row counts into row_ptr (single workgroup of 1024 threads).
__global__ __launch_bounds__(1024) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ row_ptr,
                                                           int64_t rows) {
  __shared__ int64_t part[1024];
  const int t = threadIdx.x;
  const int64_t seg = (rows + 1023) / 1024;
  const int64_t b = t * seg;
  const int64_t e = (b + seg < rows) ? b + seg : rows;
  int64_t s = 0;
  for (int64_t i = b; i < e; ++i) s += counts[i];
  part[t] = s;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    int64_t v = (t >= off) ? part[t - off] : 0;
    __syncthreads();
    part[t] += v;
    __syncthreads();
  }
  int64_t run = part[t] - s;  // exclusive
  for (int64_t i = b; i < e; ++i) {
    row_ptr[i] = (int32_t)run;
    run += counts[i];
  }
  if (t == 1023) row_ptr[rows] = (int32_t)part[1023];
}

// Expand per-row bitmasks into ascending col_idx (one wave per row).
__global__ __launch_bounds__(256) void fill_csr_kernel(const uint64_t* __restrict__ masks,
                                                       const int32_t* __restrict__ row_ptr,
                                                       int32_t* __restrict__ col_idx,
                                                       int64_t rows, int words,
                                                       int64_t col_capacity) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  int64_t out = row_ptr[row];
  for (int e = 0; e < words; ++e) {
    const uint64_t w = masks[row * words + e];
    const bool keep = (w >> lane) & 1ull;
    const int64_t pos = out + mbcnt64(w);
    if (keep && pos < col_capacity) col_idx[pos] = e * 64 + lane;
    out += __popcll(w);
  }
}

template <int D>
static hipError_t launch_score_select_d(const SelectArgs& a, int64_t bh, hipStream_t stream) {
  dim3 grid((unsigned)((a.nqb + kRowsPerWG - 1) / kRowsPerWG), (unsigned)bh), block(256);
  size_t lds = (size_t)kRowsPerWG * a.lds_stride * sizeof(float);
  const int slots = (a.nkb + 63) / 64;
  if (slots <= 4)
    score_select_kernel<D, 4><<<grid, block, lds, stream>>>(a);
  else if (slots <= 8)
    score_select_kernel<D, 8><<<grid, block, lds, stream>>>(a);
  else if (slots <= 16)
    score_select_kernel<D, 16><<<grid, block, lds, stream>>>(a);
  else
    score_select_kernel<D, 32><<<grid, block, lds, stream>>>(a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, int64_t bh, int head_dim, hipStream_t stream) {
  hipError_t err;
  if (head_dim == 128) err = launch_score_select_d<128>(a, bh, stream);
  else if (head_dim == 64) err = launch_score_select_d<64>(a, bh, stream);
  else return hipErrorInvalidValue;
  if (err != hipSuccess || a.mode == 0) return err;
  const int64_t rows = bh * a.nqb;
  scan_counts_kernel<<<1, 1024, 0, stream>>>(a.counts, a.row_ptr, rows);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  fill_csr_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(a.masks, a.row_ptr, a.col_idx,
                                                                  rows, a.words, a.col_capacity);
  return hipGetLastError();
}

}  // namespace dbsp
