// Forward block-sparse attention over the kept key blocks of every (batch, head, query block).
//
// Sources: [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", method overview,
// FastFlex bullet (the selected blocks run through a forward-only sparse attention path);
// [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention", key
// design 4 (the kernel walks a read-only per-query-block list of key blocks and skips the rest).
//
// attn_fwd_bf16_kernel (bf16, head_dim 128): one workgroup of 4 waves per CSR row (one query
// block of 128 tokens); wave w owns queries [32 w, 32 w + 32). Per kept key block:
//   * K [128 x 128] and V [128 x 128] are copied to LDS (XOR-swizzled against bank conflicts);
//   * S^T = K Q^T on 32x32x16 bf16 MFMAs: Q^T is the B operand, held in registers for the
//     whole row; the result leaves every lane with one query column and 64 key rows, so the
//     row max needs one cross-half exchange;
//   * an fp32 online softmax in the exp2 domain (the log2(e) factor folded into the scale)
//     whose exponent reference is raised lazily, only when a block exceeds it by 2^8;
//   * O^T += V^T P^T: the probabilities go straight from the S^T accumulators (as bf16) into
//     the B operand, and V^T comes from LDS through ds_read_tr16_b64, which transposes 4x16-bit
//     groups across each 16-lane block on the read (the K-index order is matched to the
//     accumulator layout of S^T).
// Epilogue: O = O^T / l, written in fp32 or bf16, and lse = ln 2 * (m + log2 l).
//
// attn_fwd_f32_kernel (fp32, head_dim 64 or 128): plain FMA arithmetic, one thread per query,
// K and V blocks staged in LDS, online softmax in chunks of 32 keys.
#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace dbsp {

constexpr int kListCap = 2048;  // kept-block indices staged in LDS per window
constexpr float kRescaleSlack = 8.0f;  // lazy online-softmax rescale threshold, log2 units

// Copy the in-range entries of col_idx[*pos, end) into list in their original order, 256
// entries per pass (wave w takes the w-th 64), stopping before a pass that could overflow
// kListCap. Advances *pos past the entries consumed and returns how many were kept. Entries
// equal to `tail` (the partial last key block, or -1) are left out of the list and recorded in
// *tail_seen instead. All four waves take part; the results are visible to all of them on return.
__device__ __forceinline__ int stage_list(const int32_t* __restrict__ col_idx, int64_t* pos,
                                          int64_t end, int nkb, int tail, int* list,
                                          int* wave_cnt, int* tail_seen, int tid) {
  const int lane = tid & 63, w = tid >> 6;
  int total = 0;
  int64_t p = *pos;
  while (p < end && total + 256 <= kListCap) {
    const int64_t e = p + 64 * w + lane;
    const int c = e < end ? col_idx[e] : -1;
    const bool is_tail = c == tail && tail >= 0;
    const bool ok = c >= 0 && c < nkb && !is_tail;
    const uint64_t m = __ballot(ok);
    const uint64_t tm = __ballot(is_tail);
    if (lane == 0) {
      wave_cnt[w] = __popcll(m);
      if (tm) *tail_seen = 1;
    }
    __syncthreads();
    int before = total;
    for (int i = 0; i < w; ++i) before += wave_cnt[i];
    if (ok) list[before + mbcnt64(m)] = c;
    total += wave_cnt[0] + wave_cnt[1] + wave_cnt[2] + wave_cnt[3];
    p += 256;
    __syncthreads();
  }
  *pos = p < end ? p : end;
  return total;
}

// Online softmax of one key tile for the lane's query column (lanes l32 and l32 + 32 share it),
// exp2 domain. The exponent reference m_run is raised only when this tile's maximum exceeds it
// by more than kRescaleSlack (log2 units), so probabilities stay below 2^kRescaleSlack and the
// rescale of O and l is skipped for most tiles. Softmax is invariant to the reference, and l and
// O stay consistent with the same m_run, so only rounding differs. Produces the probabilities
// as bf16 B operands of the P V product (pf[s] = keys 16 s .. 16 s + 15 in accumulator order).
__device__ __forceinline__ void softmax_tile(const f32x16 (&sacc)[4], float scale_log2,
                                             float& m_run, float& l_run, f32x16 (&oacc)[4],
                                             bf16x8 (&pf)[8]) {
  float mx = -INFINITY;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[jt][r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
  if (__ballot(mx * scale_log2 > m_run + kRescaleSlack) != 0ull) {
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);  // 0 on the first tile
    l_run *= alpha;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nt][r] *= alpha;
    m_run = m_new;
  }
  float psum = 0.f;
#pragma unroll
  for (int jt = 0; jt < 4; ++jt)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = __builtin_amdgcn_exp2f(fmaf(sacc[jt][r], scale_log2, -m_run));
      psum += p;
      pf[2 * jt + (r >> 3)][r & 7] = (__bf16)p;
    }
  l_run += psum;
}

// O^T += V^T P^T over one key tile; k step s covers keys 16 s .. 16 s + 15 in the accumulator
// order of S^T, and V^T comes from the swizzled V tile through transposing LDS reads.
__device__ __forceinline__ void pv_tile(const uint16_t* v_lds, const bf16x8 (&pf)[8], int h,
                                        int tr_row, int tr_col, f32x16 (&oacc)[4]) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const int jb = 16 * s + 4 * h + tr_row;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int col = 32 * nt + tr_col;
      const int off_lo = jb * 128 + v_swz(jb, col >> 3) * 8 + (col & 7);
      const int off_hi = (jb + 8) * 128 + v_swz(jb + 8, col >> 3) * 8 + (col & 7);
      // whole-vector casts only: __builtin_bit_cast of a vector element reads element 0
      // whatever the index with this compiler, which loses the upper dword of each read
      const u32x2 lo = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_lds + off_lo)));
      const u32x2 hi = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_lds + off_hi)));
      const u32x4 w4 = {lo[0], lo[1], hi[0], hi[1]};
      oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w4), pf[s],
                                                         oacc[nt], 0, 0, 0);
    }
  }
}

// Pointers are separate __restrict__ parameters and the kept-block indices are staged in LDS:
// a vector load of an index inside the pipelined loop would need a vector-memory wait that
// drains the K/V prefetch. A partial last key block (lk not a multiple of 128) is kept out of
// the DMA pipeline and processed once at the end from plain, bounds-checked loads with its
// missing keys masked (kTail variant only: the extra code raises register pressure in the main
// loop, so whole-block shapes run the variant without it); queries past lq are computed on
// zeros and not stored. kDenseRows: K and V rows are 128 contiguous bf16 (256 bytes apart, the
// common layout), which turns the DMA's row offsets into constants the compiler keeps in
// precomputed scalar registers; other strides take the variant with run-time row offsets.
template <bool kTail, bool kDenseRows>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ qg, const uint16_t* __restrict__ kg,
    const uint16_t* __restrict__ vg, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ col_idx, int64_t col_capacity, int nqb, int nkb, int64_t lq,
    int64_t lk, int heads, Strides qs, Strides ks, Strides vs, Strides os, float scale_log2,
    void* __restrict__ o, int o_bf16, float* __restrict__ lse) {
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[kBlock * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[kBlock * 128];
  __shared__ int list[kListCap];
  __shared__ int wave_cnt[8];

  const int64_t row = blockIdx.x;
  const int64_t bh = row / nqb;
  const int qb = (int)(row - bh * nqb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, held in a scalar register
  const int h = lane >> 5;
  const int l32 = lane & 31;
  // the partial last key block, if any, and the keys it holds
  const int klast = (int)(lk - (int64_t)(nkb - 1) * kBlock);
  const int tail = kTail ? nkb - 1 : -1;

  // K and V of this (batch, head): lk rows of 128 bf16, rbk / rbv bytes apart (256 when
  // contiguous); the DMA reads whole blocks only, within (lk - 1) rows + 256 bytes
  const int rbk = kDenseRows ? 256 : (int)(ks.t * 2), rbv = kDenseRows ? 256 : (int)(vs.t * 2);
  const uint16_t* kh = kg + token_offset(ks, bh, heads, 0);
  const uint16_t* vh = vg + token_offset(vs, bh, heads, 0);
  const __amdgpu_buffer_rsrc_t kbuf = raw_buffer(kh, (uint32_t)((lk - 1) * rbk + 256));
  const __amdgpu_buffer_rsrc_t vbuf = raw_buffer(vh, (uint32_t)((lk - 1) * rbv + 256));
  const DmaOffsets dmo = dma_offsets(lane, rbk, rbv);
  const int kTileK = kBlock * rbk, kTileV = kBlock * rbv;  // bytes between key blocks

  // Q^T as the B operand of S^T = K Q^T: lane (h, l32) holds query 32 w + l32, dims 16 s + 8 h .. +7
  const int64_t qi = (int64_t)qb * kBlock + 32 * w + l32;  // query within the (batch, head)
  const bool q_valid = qi < lq;
  const int64_t qtok = bh * lq + qi;                       // lse index (contiguous)
  bf16x8 qf[8];
  {
    const uint16_t* qr = qg + token_offset(qs, bh, heads, q_valid ? qi : 0) + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
      qf[s] = q_valid ? v : bf16x8{};
    }
  }

  int64_t pos = clip64(row_ptr[row], 0, col_capacity);
  const int64_t end = clip64(row_ptr[row + 1], pos, col_capacity);
  if (tid == 0) wave_cnt[4] = 0;  // the tail block was listed
  __syncthreads();

  f32x16 oacc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  while (pos < end) {
    const int n = stage_list(col_idx, &pos, end, nkb, tail, list, wave_cnt, wave_cnt + 4, tid);
    if (n == 0) continue;
    {
      const int cb = __builtin_amdgcn_readfirstlane(list[0]);
      tile_dma<false>(kbuf, cb * kTileK, k_lds, w, dmo, rbk);
      tile_dma<true>(vbuf, cb * kTileV, v_lds, w, dmo, rbv);
    }
    for (int i = 0; i < n; ++i) {
      const bool more = i + 1 < n;

      // K(i) landed in every wave's part (V(i) may still be in flight)
      wait_vmcnt<8>();
      wg_barrier();

      // S^T tiles: sacc[jt] covers keys 32 jt .. 32 jt + 31 (rows) x this wave's 32 queries
      f32x16 sacc[4];
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[jt][r] = 0.f;
        const int kr = 32 * jt + l32;
        const uint16_t* krow = k_lds + kr * 128;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const bf16x8 ka = *reinterpret_cast<const bf16x8*>(krow + k_swz(kr, 2 * s + h) * 8);
          sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[jt], 0, 0, 0);
        }
      }
      // the prefetch is unconditional (the last iteration re-fetches its own block): a
      // conditional DMA makes the compiler's wait bookkeeping drain all pending DMAs
      const int cb_next = __builtin_amdgcn_readfirstlane(list[more ? i + 1 : i]);
      wait_lgkmcnt0();
      wg_barrier();  // every wave is done reading K(i)
      tile_dma<false>(kbuf, cb_next * kTileK, k_lds, w, dmo, rbk);

      bf16x8 pf[8];
      softmax_tile(sacc, scale_log2, m_run, l_run, oacc, pf);

      // V(i) landed (the K prefetch just issued may still be in flight)
      wait_vmcnt<8>();
      wg_barrier();

      // O^T += V^T P^T (written out here rather than through pv_tile: the same code behind a
      // call made the compiler's LDS-DMA wait tracking add a drain of the K prefetch)
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const int jb = 16 * s + 4 * h + tr_row;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int col = 32 * nt + tr_col;
          const int off_lo = jb * 128 + v_swz(jb, col >> 3) * 8 + (col & 7);
          const int off_hi = (jb + 8) * 128 + v_swz(jb + 8, col >> 3) * 8 + (col & 7);
          const u32x2 lo = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_lds + off_lo)));
          const u32x2 hi = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(v_lds + off_hi)));
          const u32x4 w4 = {lo[0], lo[1], hi[0], hi[1]};
          oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w4),
                                                             pf[s], oacc[nt], 0, 0, 0);
        }
      }
      wait_lgkmcnt0();
      wg_barrier();  // every wave is done reading V(i)
      tile_dma<true>(vbuf, cb_next * kTileV, v_lds, w, dmo, rbv);
    }
    wait_vmcnt<0>();
  }

  if (kTail && wave_cnt[4]) {  // uniform: the partial last key block is kept for this row
    wait_vmcnt<0>();
    wait_lgkmcnt0();
    wg_barrier();  // every wave's DMAs have landed and every wave is done with the tiles
    const int64_t tok = (int64_t)tail * kBlock;
    // opaque copy of the thread index: keeps the copy's address arithmetic inside this block
    // (hoisted above the main loop it would hold registers through it)
    int t_opaque = tid;
    asm volatile("" : "+v"(t_opaque));
    tile_load_partial<false>(kh + tok * ks.t, klast, k_lds, t_opaque, ks.t);
    tile_load_partial<true>(vh + tok * vs.t, klast, v_lds, t_opaque, vs.t);
    __syncthreads();
    // tile bases offset by an opaque zero, so that the reads below do not share (and keep live
    // through the main loop) the loop's precomputed LDS addresses
    int zero = 0;
    asm volatile("" : "+v"(zero));
    const uint16_t* kt = k_lds + zero;
    const uint16_t* vt = v_lds + zero;
    f32x16 sacc[4];
    qk_block(kt, qf, l32, h, sacc);
    // opaque copies for the mask too: the 64 comparisons would otherwise be hoisted as well
    int h_opaque = h, klast_opaque = klast;
    asm volatile("" : "+v"(h_opaque), "+s"(klast_opaque));
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (sacc_key(jt, r, h_opaque) >= klast_opaque) sacc[jt][r] = -INFINITY;
    bf16x8 pf[8];
    softmax_tile(sacc, scale_log2, m_run, l_run, oacc, pf);
    pv_tile(vt, pf, h, tr_row, tr_col, oacc);
  }

  // epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (!q_valid) return;
  const int64_t otok = token_offset(os, bh, heads, qi);
  if (o_bf16) {
    uint16_t* orow = static_cast<uint16_t*>(o) + otok;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n0 = 32 * nt + 8 * g + 4 * h;
        u32x2 pk;
        pk[0] = f32_to_bf16_bits(oacc[nt][4 * g] * inv) |
                (f32_to_bf16_bits(oacc[nt][4 * g + 1] * inv) << 16);
        pk[1] = f32_to_bf16_bits(oacc[nt][4 * g + 2] * inv) |
                (f32_to_bf16_bits(oacc[nt][4 * g + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + n0) = pk;
      }
  } else {
    float* orow = static_cast<float*>(o) + otok;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n0 = 32 * nt + 8 * g + 4 * h;
        f32x4 ov;
#pragma unroll
        for (int e = 0; e < 4; ++e) ov[e] = oacc[nt][4 * g + e] * inv;
        *reinterpret_cast<f32x4*>(orow + n0) = ov;
      }
  }
  if (lse && h == 0)
    lse[qtok] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(AttnArgs a) {
  __shared__ float k_lds[kBlock][D];
  __shared__ float v_lds[kBlock][D];
  const int64_t row = blockIdx.x;
  const int64_t bh = row / a.nqb;
  const int qb = (int)(row - bh * a.nqb);
  const int t = threadIdx.x;
  const int64_t qi = (int64_t)qb * kBlock + t;
  const bool q_valid = qi < a.lq;
  const int64_t qtok = bh * a.lq + (q_valid ? qi : 0);  // lse index (contiguous)
  const float* qp = static_cast<const float*>(a.q) + token_offset(a.qs, bh, a.heads, q_valid ? qi : 0);
  const float* kp = static_cast<const float*>(a.k) + token_offset(a.ks, bh, a.heads, 0);
  const float* vp = static_cast<const float*>(a.v) + token_offset(a.vs, bh, a.heads, 0);

  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = q_valid ? qp[d] : 0.f;
  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  int64_t beg = a.row_ptr[row], end = a.row_ptr[row + 1];
  beg = clip64(beg, 0, a.col_capacity);
  end = clip64(end, beg, a.col_capacity);
  for (int64_t it = beg; it < end; ++it) {
    const int cb = a.col_idx[it];
    if (cb < 0 || cb >= a.nkb) continue;
    // keys held by this block (the last one may be partial); missing rows are zero-filled and
    // skipped below
    const int valid = (int)(a.lk - (int64_t)cb * kBlock < kBlock ? a.lk - (int64_t)cb * kBlock
                                                                 : kBlock);
    const float* kb = kp + (int64_t)cb * kBlock * a.ks.t;
    const float* vb = vp + (int64_t)cb * kBlock * a.vs.t;
    for (int i = t; i < kBlock * D; i += 128) {
      const int r = i / D, col = i - (i / D) * D;
      const bool in = r < valid;
      (&k_lds[0][0])[i] = in ? kb[r * a.ks.t + col] : 0.f;
      (&v_lds[0][0])[i] = in ? vb[r * a.vs.t + col] : 0.f;
    }
    __syncthreads();
    for (int j0 = 0; j0 < valid; j0 += 32) {
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
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[j] - m_new);
        l_run += p;
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(p, v_lds[j0 + j][d], acc[d]);
      }
      m_run = m_new;
    }
    __syncthreads();
  }
  if (!q_valid) return;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  const int64_t otok = token_offset(a.os, bh, a.heads, qi);
  if (a.o_bf16) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + otok;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = (uint16_t)f32_to_bf16_bits(acc[d] * inv);
  } else {
    float* orow = static_cast<float*>(a.o) + otok;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  }
  if (a.lse) a.lse[qtok] = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
}

hipError_t launch_attn(const AttnArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  dim3 grid((unsigned)a.rows);
  if (bf16 && head_dim == 128) {
    const bool tail = a.lk % kBlock != 0, dense = a.ks.t == 128 && a.vs.t == 128;
    auto* kern = tail ? (dense ? attn_fwd_bf16_kernel<true, true>
                               : attn_fwd_bf16_kernel<true, false>)
                      : (dense ? attn_fwd_bf16_kernel<false, true>
                               : attn_fwd_bf16_kernel<false, false>);
    kern<<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t*>(a.q), static_cast<const uint16_t*>(a.k),
        static_cast<const uint16_t*>(a.v), a.row_ptr, a.col_idx, a.col_capacity, a.nqb, a.nkb,
        a.lq, a.lk, a.heads, a.qs, a.ks, a.vs, a.os, a.scale_log2, a.o, a.o_bf16, a.lse);
  } else if (!bf16 && head_dim == 64)
    attn_fwd_f32_kernel<64><<<grid, 128, 0, stream>>>(a);
  else if (!bf16 && head_dim == 128)
    attn_fwd_f32_kernel<128><<<grid, 128, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dbsp
