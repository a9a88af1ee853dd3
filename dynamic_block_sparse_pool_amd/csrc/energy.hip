// Token-level block energy and the retained attention mass of a block mask.
//
// Sources: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
// key design 1, Eq. (5): the energy of query block r and key block c is the attention
// probability mass between them, summed over the block's queries and keys and divided by the
// block size; every query-block row of E sums to 1. The page computes it with a custom kernel
// that never materialises the attention matrix. [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力
// 不能跨尺度复用？", Figures 3 and 4, report the retained mass of masks (the sum of E over the kept
// blocks).
//
// block_energy_bf16_kernel (bf16, head_dim 128): one workgroup of 4 waves per (batch, head,
// query block) row, wave w owning queries [32 w, 32 w + 32) with the same S^T = K Q^T tiling on
// 32x32x16 bf16 MFMAs as the attention kernel. Two sweeps over every key block of the head:
//   1. a running sum of exp2(s - m) per query against a lazily raised reference m, giving its
//      log-sum-exp (log2 units);
//   2. per key block, the sum of exp2(s - lse) over the block's 128 x 128 pairs: each lane adds
//      its 64 values, the wave adds its lanes in a fixed DPP order, and the four wave totals are
//      added in wave order and divided by 128 (deterministic, no atomics).
// K tiles are double-buffered in LDS: the DMA of the next block runs while this one is scored.
// Every row of a head walks the same blocks in the same order, so the K stream is shared
// through L2 by the workgroups of a head that run together.
//
// block_energy_f32_kernel (fp32, head_dim 64 or 128): one thread per query, K block in LDS,
// the same two sweeps with plain FMA arithmetic and a tree reduction per key block.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace dbsp {

// Step g of the 2 * n steps over the n whole key blocks (block g mod n) lives in LDS buffer
// g & 1. Waits for it, lets every wave finish the previous step, and starts the DMA of step g + 1
// into the other buffer (the final step re-fetches its own block: an unconditional issue keeps
// the compiler's DMA wait tracking exact).
__device__ __forceinline__ const uint16_t* energy_step_begin(int g, int n, uint16_t* k_lds,
                                                             __amdgpu_buffer_rsrc_t kbuf, int w,
                                                             const DmaOffsets& dmo) {
  constexpr int kTileBytes = kBlock * 128 * 2;
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  wg_barrier();
  const int gn = g + 1 < 2 * n ? g + 1 : g;
  const int cn = gn < n ? gn : gn - n;
  tile_dma<false>(kbuf, cn * kTileBytes, k_lds + ((g + 1) & 1) * (kBlock * 128), w, dmo, 256);
  return k_lds + (g & 1) * (kBlock * 128);
}

// The partial last key block (keys [0, klast) of it exist) goes through plain loads into LDS
// buffer `buf`, outside the DMA pipeline; keys past klast are masked to -inf.
__device__ __forceinline__ const uint16_t* energy_tail_tile(const uint16_t* ktail, int klast,
                                                            uint16_t* k_lds, int buf, int tid) {
  wait_lgkmcnt0();
  wg_barrier();  // every wave is done with buffer `buf`
  uint16_t* kt = k_lds + buf * (kBlock * 128);
  tile_load_partial<false>(ktail, klast, kt, tid, 128);
  __syncthreads();
  return kt;
}

__device__ __forceinline__ void mask_tail(f32x16 (&sacc)[4], int h, int klast) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (sacc_key(jt, r, h) >= klast) sacc[jt][r] = -INFINITY;
}

// Sweep 1 on one S^T tile: running sum per query of exp2(s - m_run) against a lazily raised
// reference m_run (log2 units). The tile's terms are added against the current reference
// first; the reference is kept while every lane's partial sum over the tile (64 terms) stays at
// or below kLseSumLimit, which bounds every term by it. Only when a tile breaks the bound, or the
// query has no finite reference yet, is the exact tile maximum taken, the reference raised to it,
// the running sum rescaled and the tile's terms recomputed: on the first tile and when the scores
// grow by more than about 2^10. lse = m_run + log2(sum) does not depend on the reference, so
// only the rounding differs from an eager update; the row maximum is not computed in the
// common case.
constexpr float kLseSumLimit = 65536.f;

__device__ __forceinline__ float lse_terms(const f32x16 (&sacc)[4], float scale_log2,
                                           float m_run) {
  // masked keys of a query with no finite reference yet give exp2(-inf) = 0, not NaN
  const float mneg = m_run == -INFINITY ? 0.f : -m_run;
  float ps = 0.f;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(fmaf(sacc[jt][r], scale_log2, mneg));
  return ps;
}

__device__ __forceinline__ void lse_update(const f32x16 (&sacc)[4], float scale_log2, float& m_run,
                                           float& l_run) {
  float ps = lse_terms(sacc, scale_log2, m_run);
  // !(x <= limit) is also true for NaN and +inf sums
  if (__ballot(m_run == -INFINITY || !(ps <= kLseSumLimit)) != 0ull) {
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[jt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // lanes l32 and l32 + 32 hold the same query
    const float m_new = fmaxf(m_run, mx * scale_log2);
    // exp2(-inf) = 0 for the first finite reference; -inf - -inf would be NaN
    l_run *= m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    m_run = m_new;
    ps = lse_terms(sacc, scale_log2, m_run);
  }
  l_run += ps;
}

// Sweep 2 on the S^T tile of key block c: the wave's probability total for c lands in lane
// c mod 64 of `acc`; every 64 blocks (and after the last one) the four wave totals are added in
// wave order, divided by the number of queries of the block, and written.
__device__ __forceinline__ void energy_update(const f32x16 (&sacc)[4], float scale_log2,
                                              float lse2, bool q_valid, int c, int nkb, int lane,
                                              int w, float (*part)[64], float& acc, float* erow,
                                              float qcount) {
  float ps = 0.f;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) ps += __builtin_amdgcn_exp2f(fmaf(sacc[jt][r], scale_log2, -lse2));
  const float t = wave_total_f32(q_valid ? ps : 0.f);
  acc = lane == (c & 63) ? t : acc;
  if ((c & 63) == 63 || c == nkb - 1) {  // uniform: flush 64 blocks (or the tail)
    part[w][lane] = acc;
    wait_lgkmcnt0();
    wg_barrier();
    const int cc = (c & ~63) + lane;
    if (w == 0 && cc <= c)
      erow[cc] = (((part[0][lane] + part[1][lane]) + part[2][lane]) + part[3][lane]) / qcount;
  }
}

__global__ __launch_bounds__(256, 2) void block_energy_bf16_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, int nqb, int nkb,
    int64_t lq, int64_t lk, float scale_log2, float* __restrict__ energy,
    float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[2 * kBlock * 128];
  __shared__ float part[4][64];

  const int64_t row = blockIdx.x;
  const int64_t bh = row / nqb;
  const int qb = (int)(row - bh * nqb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const __amdgpu_buffer_rsrc_t kbuf = raw_buffer(kg + bh * lk * 128, (uint32_t)(lk * 256));
  const DmaOffsets dmo = dma_offsets(lane, 256, 256);
  // whole key blocks go through the DMA pipeline; a partial last one is handled apart
  const int klast = (int)(lk - (int64_t)(nkb - 1) * kBlock);
  const bool has_tail = klast < kBlock;
  const int nfull = has_tail ? nkb - 1 : nkb;
  const uint16_t* ktail = kg + (bh * lk + (int64_t)(nkb - 1) * kBlock) * 128;
  const int qcount_i = (int)(lq - (int64_t)qb * kBlock < kBlock ? lq - (int64_t)qb * kBlock
                                                                : kBlock);
  const float qcount = (float)qcount_i;

  // Q^T as the B operand: lane (h, l32) holds query 32 w + l32, dims 16 s + 8 h .. +7; queries
  // past lq are zero and add nothing to the energies
  const int64_t qi = (int64_t)qb * kBlock + 32 * w + l32;
  const bool q_valid = qi < lq;
  const int64_t qtok = bh * lq + qi;
  bf16x8 qf[8];
  {
    const uint16_t* qr = qg + (q_valid ? qtok : bh * lq) * 128 + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
      qf[s] = q_valid ? v : bf16x8{};
    }
  }

  if (nfull > 0) tile_dma<false>(kbuf, 0, k_lds, w, dmo, 256);

  // sweep 1: log-sum-exp per query (lanes l32 and l32 + 32 hold halves of the same query)
  float m_run = -INFINITY, l_run = 0.f;
  for (int g = 0; g < nfull; ++g) {
    const uint16_t* kt = energy_step_begin(g, nfull, k_lds, kbuf, w, dmo);
    f32x16 sacc[4];
    qk_block(kt, qf, l32, h, sacc);
    lse_update(sacc, scale_log2, m_run, l_run);
  }
  if (has_tail) {  // the DMA in flight (block 0 of sweep 2) targets buffer nfull & 1
    const uint16_t* kt = energy_tail_tile(ktail, klast, k_lds, (nfull & 1) ^ 1, tid);
    f32x16 sacc[4];
    qk_block(kt, qf, l32, h, sacc);
    mask_tail(sacc, h, klast);
    lse_update(sacc, scale_log2, m_run, l_run);
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float lse2 = m_run + __log2f(l_tot);
  if (lse && h == 0 && q_valid) lse[qtok] = lse2 * 0.69314718055994531f;

  // sweep 2: block energies
  float* erow = energy + row * nkb;
  float acc = 0.f;
  for (int g = nfull; g < 2 * nfull; ++g) {
    const uint16_t* kt = energy_step_begin(g, nfull, k_lds, kbuf, w, dmo);
    f32x16 sacc[4];
    qk_block(kt, qf, l32, h, sacc);
    energy_update(sacc, scale_log2, lse2, q_valid, g - nfull, nkb, lane, w, part, acc, erow,
                  qcount);
  }
  if (has_tail) {  // the last step re-fetched its own block into buffer 0
    const uint16_t* kt = energy_tail_tile(ktail, klast, k_lds, 1, tid);
    f32x16 sacc[4];
    qk_block(kt, qf, l32, h, sacc);
    mask_tail(sacc, h, klast);
    energy_update(sacc, scale_log2, lse2, q_valid, nkb - 1, nkb, lane, w, part, acc, erow,
                  qcount);
  }
  wait_vmcnt<0>();
}

template <int D>
__global__ __launch_bounds__(128) void block_energy_f32_kernel(EnergyArgs a) {
  __shared__ float k_lds[kBlock][D];
  __shared__ float red[kBlock];
  const int64_t row = blockIdx.x;
  const int64_t bh = row / a.nqb;
  const int qb = (int)(row - bh * a.nqb);
  const int t = threadIdx.x;
  const int64_t qi = (int64_t)qb * kBlock + t;
  const bool q_valid = qi < a.lq;
  const int64_t qtok = bh * a.lq + (q_valid ? qi : 0);
  const int qcount = (int)(a.lq - (int64_t)qb * kBlock < kBlock ? a.lq - (int64_t)qb * kBlock
                                                                : kBlock);
  const float* qp = static_cast<const float*>(a.q) + qtok * D;
  const float* kp = static_cast<const float*>(a.k) + bh * a.lk * D;
  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = q_valid ? qp[d] : 0.f;

  float m_run = -INFINITY, l_run = 0.f, lse2 = 0.f;
  for (int g = 0; g < 2 * a.nkb; ++g) {
    const int c = g < a.nkb ? g : g - a.nkb;
    const int valid = (int)(a.lk - (int64_t)c * kBlock < kBlock ? a.lk - (int64_t)c * kBlock
                                                                : kBlock);
    const float* kb = kp + (int64_t)c * kBlock * D;
    for (int i = t; i < kBlock * D; i += kBlock) (&k_lds[0][0])[i] = i < valid * D ? kb[i] : 0.f;
    __syncthreads();
    if (g < a.nkb) {
      for (int j0 = 0; j0 < valid; j0 += 32) {  // chunks of 32 keys keep the scores in registers
        float s[32];
        float mx = -INFINITY;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          float dot = 0.f;
#pragma unroll
          for (int d = 0; d < D; ++d) dot = fmaf(qv[d], k_lds[j0 + j][d], dot);
          s[j] = j0 + j < valid ? dot * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, s[j]);
        }
        const float m_new = fmaxf(m_run, mx);
        float ps = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) ps += __builtin_amdgcn_exp2f(s[j] - m_new);
        l_run = l_run * __builtin_amdgcn_exp2f(m_run - m_new) + ps;
        m_run = m_new;
      }
      if (g == a.nkb - 1) {
        lse2 = m_run + __log2f(l_run);
        if (a.lse && q_valid) a.lse[qtok] = lse2 * 0.69314718055994531f;
      }
    } else {
      float ps = 0.f;
      for (int j = 0; j < valid; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(qv[d], k_lds[j][d], dot);
        ps += __builtin_amdgcn_exp2f(fmaf(dot, a.scale_log2, -lse2));
      }
      red[t] = q_valid ? ps : 0.f;
      __syncthreads();
      for (int off = kBlock / 2; off > 0; off >>= 1) {
        if (t < off) red[t] += red[t + off];
        __syncthreads();
      }
      if (t == 0) a.energy[row * a.nkb + c] = red[0] / (float)qcount;
    }
    __syncthreads();
  }
}

// Retained mass of a CSR mask: one wave per row adds the energies of the row's in-range entries
// in float64 (lane-strided partial sums, then a fixed butterfly order).
__global__ __launch_bounds__(256) void retained_mass_kernel(
    const float* __restrict__ energy, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int64_t col_capacity, int nkb, int64_t rows,
    double* __restrict__ mass) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int64_t beg = clip64(row_ptr[row], 0, col_capacity);
  const int64_t end = clip64(row_ptr[row + 1], beg, col_capacity);
  double s = 0.0;
  for (int64_t e = beg + lane; e < end; e += 64) {
    const int c = col_idx[e];
    if (c >= 0 && c < nkb) s += (double)energy[row * nkb + c];
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (lane == 0) mass[row] = s;
}

hipError_t launch_energy(const EnergyArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  const dim3 grid((unsigned)a.rows);
  if (bf16 && head_dim == 128)
    block_energy_bf16_kernel<<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.nqb, a.nkb, a.lq,
        a.lk, a.scale_log2, a.energy, a.lse);
  else if (!bf16 && head_dim == 64)
    block_energy_f32_kernel<64><<<grid, kBlock, 0, stream>>>(a);
  else if (!bf16 && head_dim == 128)
    block_energy_f32_kernel<128><<<grid, kBlock, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_retained_mass(const float* energy, const int32_t* row_ptr,
                                const int32_t* col_idx, int64_t col_capacity, int nkb,
                                int64_t rows, double* mass, hipStream_t stream) {
  retained_mass_kernel<<<(unsigned)((rows + 3) / 4), 256, 0, stream>>>(
      energy, row_ptr, col_idx, col_capacity, nkb, rows, mass);
  return hipGetLastError();
}

}  // namespace dbsp
