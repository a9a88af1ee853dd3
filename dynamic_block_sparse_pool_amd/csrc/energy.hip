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
// query block) row at a time, wave w owning queries [32 w, 32 w + 32) with the same S^T = K Q^T
// tiling on 32x32x16 bf16 MFMAs as the attention kernel, and one sweep over every key block of
// the head: per query it keeps a running sum of exp2(s - m) against a lazily raised reference m
// (its log-sum-exp at the end) and, per key block, log2 of the block's sum of exp2(s), which it
// parks in a workspace slot of its own; after the sweep the block energies are formed from those
// and the log-sum-exps (each lane adds two queries, the wave adds its lanes in a fixed DPP
// order: deterministic, no atomics). K tiles are double-buffered in LDS: the DMA of the next
// block runs while this one is scored. Every row of a head walks the same blocks in the same
// order, so the K stream is shared through L2 by the workgroups of a head that run together.
//
// block_energy_f32_kernel (fp32, head_dim 64 or 128): one thread per query, K block in LDS,
// two sweeps (log-sum-exp, then the block sums against it) with plain FMA arithmetic and a tree
// reduction per key block.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace dbsp {

// Step g over the n whole key blocks (block g) reads `cur`, whose DMA was issued one step
// earlier: waits for it, lets every wave finish the previous step (which read `next`), and
// starts the DMA of block g + 1 into `next` (the final step re-fetches its own block: an
// unconditional issue keeps the DMA wait tracking simple). `cur` and `next` are two separate
// LDS arrays chosen at compile time, so the compiler can tell the DMA into one from the reads of
// the other and leaves the prefetch in flight across the step's LDS reads.
__device__ __forceinline__ void energy_step_begin(int g, int n, uint16_t* next,
                                                  __amdgpu_buffer_rsrc_t kbuf, int w,
                                                  const DmaOffsets& dmo) {
  constexpr int kTileBytes = kBlock * 128 * 2;
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  wg_barrier();
  const int cn = g + 1 < n ? g + 1 : g;
  tile_dma<false>(kbuf, cn * kTileBytes, next, w, dmo, 256);
}

// The partial last key block (keys [0, klast) of it exist) goes through plain loads into LDS,
// outside the DMA pipeline, once every wave is done with the tile and the DMAs have landed;
// keys past klast are masked to -inf.
__device__ __forceinline__ void energy_tail_tile(const uint16_t* ktail, int klast,
                                                 uint16_t* tile, int tid) {
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  wg_barrier();
  tile_load_partial<false>(ktail, klast, tile, tid, 128);
  __syncthreads();
}

__device__ __forceinline__ void mask_tail(f32x16 (&sacc)[4], int h, int klast) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (sacc_key(jt, r, h) >= klast) sacc[jt][r] = -INFINITY;
}

// One S^T tile of the sweep: running sum per query of exp2(s - m_run) against a lazily raised
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

__device__ __forceinline__ float lse_update(const f32x16 (&sacc)[4], float scale_log2,
                                            float& m_run, float& l_run) {
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
  return ps;  // the lane's terms of this tile against the (possibly raised) m_run
}

// The query's log2-sum over one key block: lse_update on the block's S^T tile, then
// m_run + log2 of the block's terms (lanes l32 and l32 + 32 hold the two key halves of the same
// query and share m_run), i.e. log2 of the sum of exp2(s * scale_log2) over the block's keys,
// which does not depend on the reference. -inf when the query has no term in the block.
__device__ __forceinline__ float block_log2sum(const f32x16 (&sacc)[4], float scale_log2,
                                               float& m_run, float& l_run) {
  const float ps = lse_update(sacc, scale_log2, m_run, l_run);
  return m_run + __log2f(ps + __shfl_xor(ps, 32, 64));
}

// The A operands of d slice s (dims 16 s .. 16 s + 15) for the four 32-key sub-tiles of a K tile
// (the fragments qk_block reads for that slice).
__device__ __forceinline__ void read_k_slice(const uint16_t* k_tile, int s, int l32, int h,
                                             bf16x8 (&dst)[4]) {
#pragma unroll
  for (int jt = 0; jt < 4; ++jt) {
    const int kr = 32 * jt + l32;
    dst[jt] = *reinterpret_cast<const bf16x8*>(k_tile + kr * 128 + k_swz(kr, 2 * s + h) * 8);
  }
}

// qk_block with the d slices outermost: the four sub-tiles' MFMAs of one slice run back to back
// on the same Q fragment, as four independent accumulation chains, and the K fragments of slice
// s + 1 are read under the MFMAs of slice s (the scheduling fences keep that order). Each
// accumulator still adds its slices in ascending order, so the results equal qk_block's bit for
// bit.
__device__ __forceinline__ void qk_block_sd_outer(const uint16_t* k_tile,
                                                  const bf16x8 (&qf)[8], int l32, int h,
                                                  f32x16 (&sacc)[4]) {
  bf16x8 ka[2][4];
  read_k_slice(k_tile, 0, l32, h, ka[0]);
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[jt][r] = 0.f;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    if (s + 1 < 8) read_k_slice(k_tile, s + 1, l32, h, ka[(s + 1) & 1]);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
      sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[s & 1][jt], qf[s], sacc[jt], 0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One sweep per row. For each (batch, head, query block) row the workgroup walks every key
// block once; per query t and key block c it keeps b[c][t] = log2 sum over the block's keys of
// exp2(s * scale_log2) (block_log2sum) in its own slot of the workspace, and the running
// log-sum-exp of the query. Once the sweep ends, energy[row][c] = (1 / n) * sum over the block's
// queries of exp2(b[c][t] - lse_t): Eq. (5) with each query's probabilities summed per key
// block first. The dense Q K^T product is formed once (the two-pass alternative forms it twice:
// once for the log-sum-exp, once for the block sums against it).
//
// Persistent: gridDim.x workgroups (at most rows), workgroup g taking rows g, g + gridDim.x, ...,
// each owning the nkb * 128 floats at ws + g * nkb * 128, written during a row's sweep and read
// back by the same workgroup after it; rows run in the same order across the grid as a
// one-row-per-workgroup launch would dispatch them, so the workgroups of one XCD still sweep the
// same head's K together (through L2). The b values of block c are stored at the start of step
// c + 1, next to the DMA of block c + 2, so the step's vector-memory wait covers both.
// Per block, each lane adds 64 terms, the two halves of a query meet by a lane swap, and the
// energies add 128 queries in a fixed DPP order: results are bit-reproducible.
__global__ __launch_bounds__(256, 2) void block_energy_bf16_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg, int nqb, int nkb,
    int64_t lq, int64_t lk, int64_t rows, float scale_log2, float* __restrict__ energy,
    float* __restrict__ lse, float* __restrict__ ws) {
  __shared__ __attribute__((aligned(1024))) uint16_t k0[kBlock * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t k1[kBlock * 128];
  __shared__ float lse_s[kBlock];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int qoff = 32 * w + l32;
  const DmaOffsets dmo = dma_offsets(lane, 256, 256);
  // whole key blocks go through the DMA pipeline; a partial last one is handled apart
  const int klast = (int)(lk - (int64_t)(nkb - 1) * kBlock);
  const bool has_tail = klast < kBlock;
  const int nfull = has_tail ? nkb - 1 : nkb;
  float* __restrict__ slot = ws + (int64_t)blockIdx.x * nkb * kBlock;

  for (int64_t row = blockIdx.x; row < rows; row += gridDim.x) {
    const int64_t bh = row / nqb;
    const int qb = (int)(row - bh * nqb);
    const __amdgpu_buffer_rsrc_t kbuf = raw_buffer(kg + bh * lk * 128, (uint32_t)(lk * 256));
    const uint16_t* ktail = kg + (bh * lk + (int64_t)(nkb - 1) * kBlock) * 128;
    const int qcount_i = (int)(lq - (int64_t)qb * kBlock < kBlock ? lq - (int64_t)qb * kBlock
                                                                  : kBlock);

    // Q^T as the B operand: lane (h, l32) holds query 32 w + l32, dims 16 s + 8 h .. +7; queries
    // past lq are zero and their block sums are stored as -inf (no contribution)
    const int64_t qi = (int64_t)qb * kBlock + qoff;
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

    if (nfull > 0) tile_dma<false>(kbuf, 0, k0, w, dmo, 256);

    // step g: block g from k0 (g even) or k1 (g odd); its b goes out at step g + 1
    float m_run = -INFINITY, l_run = 0.f, b_prev = -INFINITY;
#define DBSP_ENERGY_STEP(G, CUR, NEXT)                                                        \
  do {                                                                                        \
    energy_step_begin((G), nfull, (NEXT), kbuf, w, dmo);                                      \
    if ((G) > 0 && h == 0) slot[(int64_t)((G) - 1) * kBlock + qoff] = b_prev;                 \
    f32x16 sacc[4];                                                                           \
    qk_block_sd_outer((CUR), qf, l32, h, sacc);                                               \
    const float b = block_log2sum(sacc, scale_log2, m_run, l_run);                            \
    b_prev = q_valid ? b : -INFINITY;                                                         \
  } while (0)
    int g = 0;
    for (; g + 1 < nfull; g += 2) {
      DBSP_ENERGY_STEP(g, k0, k1);
      DBSP_ENERGY_STEP(g + 1, k1, k0);
    }
    if (g < nfull) DBSP_ENERGY_STEP(g, k0, k1);
#undef DBSP_ENERGY_STEP
    if (nfull > 0 && h == 0) slot[(int64_t)(nfull - 1) * kBlock + qoff] = b_prev;
    if (has_tail) {
      energy_tail_tile(ktail, klast, k0, tid);
      f32x16 sacc[4];
      qk_block(k0, qf, l32, h, sacc);
      mask_tail(sacc, h, klast);
      const float b = block_log2sum(sacc, scale_log2, m_run, l_run);
      if (h == 0) slot[(int64_t)(nkb - 1) * kBlock + qoff] = q_valid ? b : -INFINITY;
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    const float lse2 = m_run + __log2f(l_tot);
    if (lse && h == 0 && q_valid) lse[qtok] = lse2 * 0.69314718055994531f;
    if (h == 0) lse_s[qoff] = lse2;
    wait_vmcnt<0>();  // the slot's stores (and the last re-fetch) complete
    wait_lgkmcnt0();
    wg_barrier();

    // energies: wave w takes key blocks [64 (4 i + w), + 64), eight blocks' loads in flight;
    // lane j of the wave ends up with block base + j and the wave stores 64 energies at once
    const float la = lse_s[2 * lane], lb = lse_s[2 * lane + 1];
    const float inv_q = 1.0f / (float)qcount_i;
    float* erow = energy + row * nkb;
    for (int base = 64 * w; base < nkb; base += 256) {
      float mine = 0.f;
      for (int j0 = 0; j0 < 64; j0 += 8) {
        f32x2 bv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int c = base + j0 + j;  // wave-uniform
          bv[j] = c < nkb ? *reinterpret_cast<const f32x2*>(slot + (int64_t)c * kBlock + 2 * lane)
                          : f32x2{-INFINITY, -INFINITY};
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float e = __builtin_amdgcn_exp2f(bv[j][0] - la) + __builtin_amdgcn_exp2f(bv[j][1] - lb);
          const float t = wave_total_f32(e);
          mine = lane == j0 + j ? t : mine;
        }
      }
      if (base + lane < nkb) erow[base + lane] = mine * inv_q;
    }
    wg_barrier();  // lse_s and the slot belong to the next row
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
  if (bf16 && head_dim == 128) {
    if (a.slots < 1 || a.slots > a.rows || !a.ws) return hipErrorInvalidValue;
    block_energy_bf16_kernel<<<dim3((unsigned)a.slots), 256, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k), a.nqb, a.nkb, a.lq,
        a.lk, a.rows, a.scale_log2, a.energy, a.lse, a.ws);
  }
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
