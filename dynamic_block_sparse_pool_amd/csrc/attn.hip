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
//   * the block is processed in four sub-tiles of 32 keys; S^T = K Q^T on 32x32x16 bf16 MFMAs
//     (Q^T is the B operand, held in registers for the whole row) leaves every lane with one
//     query column and 16 keys of the sub-tile;
//   * the sub-tiles are software-pipelined: the softmax of sub-tile u runs next to the QK
//     MFMAs of u + 1 and the PV MFMAs of u - 1, so the vector ALU and the matrix cores of a
//     wave overlap;
//   * an fp32 online softmax in the exp2 domain (the log2(e) factor folded into the scale)
//     whose reference is raised lazily: probabilities are formed against the current reference
//     first, and only a sub-tile whose partial row sums break a bound takes its exact maximum
//     and rescales O and l, so the row maximum is not computed in the common case;
//   * O^T += V^T P^T: the probabilities go straight from the S^T accumulators (as bf16) into
//     the B operand, and V^T comes from LDS through ds_read_tr16_b64, which transposes 4x16-bit
//     groups across each 16-lane block on the read (the K-index order is matched to the
//     accumulator layout of S^T).
// Epilogue: O = O^T / l, written in fp32 or bf16, and lse = ln 2 * (m + log2 l).
//
// attn_fwd_f32_kernel (fp32, head_dim 64 or 128): plain FMA arithmetic, four lanes per query
// (a quarter of the head dimension each), K and V blocks staged in LDS, online softmax in
// chunks of 32 keys.
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "tile.hpp"

namespace dbsp {

constexpr int kListCap = 2048;  // kept-block indices staged in LDS per window

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

// Work unit of the bf16 kernel: a sub-tile of 32 keys x the wave's 32 queries. In the
// accumulator order of S^T, register r of lane half h holds key sacc_key(jt, r, h) of the block
// for sub-tile jt; the P operand of 16-key step j of the sub-tile takes registers 8 j .. 8 j + 7,
// and V^T is read in the same order.

// Per-lane byte offsets of a wave's LDS reads within a tile. The XOR swizzles make the offset
// of each 16-byte K chunk step (and of each V column tile) depend on the lane, so those are
// held in registers; rows further down (other sub-tiles, steps and halves) differ by constants
// and go into the instructions' offset fields.
struct LdsOff {
  int k[8];  // K row l32 (sub-tile 0), chunk step sd
  int v[4];  // V^T rows 4 h + tr_row (sub-tile 0, step 0, low half), column tile nt
};

__device__ __forceinline__ LdsOff lds_offsets(int l32, int h, int tr_row, int tr_col) {
  LdsOff o;
#pragma unroll
  for (int sd = 0; sd < 8; ++sd) o.k[sd] = 2 * (l32 * 128 + k_swz(l32, 2 * sd + h) * 8);
  const int jb = 4 * h + tr_row;  // jb & 3 == tr_row for every row read below
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int col = 32 * nt + tr_col;
    o.v[nt] = 2 * (jb * 128 + v_swz(jb, col >> 3) * 8 + (col & 7));
  }
  return o;
}

// A copy of the offsets that the compiler cannot see through, taken once per block: the
// tile-base additions then stay next to their reads instead of being hoisted out of the loop
// for every sub-tile, where they would hold registers for the whole row.
__device__ __forceinline__ LdsOff lds_opaque(const LdsOff& in) {
  LdsOff o = in;
#pragma unroll
  for (int i = 0; i < 8; ++i) asm volatile("" : "+v"(o.k[i]));
#pragma unroll
  for (int i = 0; i < 4; ++i) asm volatile("" : "+v"(o.v[i]));
  return o;
}

// S^T of sub-tile jt of the K tile at kt x the wave's queries: 32 keys x 32 queries.
__device__ __forceinline__ void qk_sub(const uint16_t* kt, const LdsOff& lo,
                                       const bf16x8 (&qf)[8], int jt, f32x16& s) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
  for (int sd = 0; sd < 8; ++sd) {
    // sub-tile jt: 32 rows (8 KiB) further; k_swz depends on the row only modulo 16
    const bf16x8 ka = *reinterpret_cast<const bf16x8*>(
        reinterpret_cast<const char*>(kt) + lo.k[sd] + jt * 8192);
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[sd], s, 0, 0, 0);
  }
}

// O^T += V^T P^T over sub-tile jt of the V tile at vt (V^T through transposing LDS reads of the
// swizzled tile).
__device__ __forceinline__ void pv_sub(const uint16_t* vt, const LdsOff& lo,
                                       const bf16x8 (&pf)[2], int jt, f32x16 (&oacc)[4]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    // rows 32 jt + 16 j further (8 KiB per sub-tile, 4 KiB per step), high half 8 rows more;
    // v_swz depends on the row only modulo 4
    const int row_off = jt * 8192 + j * 4096;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const char* base = reinterpret_cast<const char*>(vt) + lo.v[nt] + row_off;
      // whole-vector casts only: __builtin_bit_cast of a vector element reads element 0
      // whatever the index with this compiler, which loses the upper dword of each read
      const u32x2 lov = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base)));
      const u32x2 hiv = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(base + 2048)));
      const u32x4 w4 = {lov[0], lov[1], hiv[0], hiv[1]};
      oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, w4), pf[j],
                                                         oacc[nt], 0, 0, 0);
    }
  }
}

// Online softmax in the exp2 domain with a lazily raised reference. P = exp2(S scale_log2 -
// m_run) is computed against the current reference m_run first; the reference is kept as long
// as every lane's partial row sum over a sub-tile (16 probabilities) stays at or below
// kSumLimit, which bounds every probability by it (fp32 O and l and bf16 P have ample range for
// that). Only when a sub-tile breaks the bound, or the query has no finite reference yet, is
// the exact sub-tile maximum taken, the reference raised to it, O and l rescaled and P
// recomputed: on a query's first sub-tile and when its scores grow by more than about 2^12.
// The row maximum is therefore never computed in the common case. Softmax does not depend on
// the reference, and O and l always share it, so only the rounding differs from an eager
// update. A query whose keys so far are all masked keeps m_run = -inf (O and l stay zero).
constexpr float kSumLimit = 65536.f;

// P of one sub-tile against the current reference, as bf16 B operands (pf[j] = keys
// 16 j .. 16 j + 15 of the sub-tile in accumulator order), and the lane's partial row sum.
__device__ __forceinline__ void softmax_sub(const f32x16& s, float scale_log2, float m_run,
                                            bf16x8 (&pf)[2], float& psum) {
  // masked keys of a query with no finite reference yet give exp2(-inf) = 0, not NaN
  const float mneg = m_run == -INFINITY ? 0.f : -m_run;
#pragma unroll
  for (int r = 0; r < 16; ++r)
    pf[r >> 3][r & 7] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[r], scale_log2, mneg));
  // row sum of the bf16 probabilities that the PV product uses, two per v_dot2 (exact products
  // by 1, fp32 accumulation): O is then normalised by the sum of its own weights
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
  const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const u32x4 pw = __builtin_bit_cast(u32x4, pf[j]);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t dw = pw[i];  // a scalar copy: bit_cast of a vector element misreads
      sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, dw), ones, sum, false);
    }
  }
  psum = sum;
}

// Accept the sub-tile's probabilities or, when a lane breaks the bound (see above), raise the
// reference to the exact maximum, rescale O and l, and recompute them; then add the row sum.
__device__ __forceinline__ void settle_sub(const f32x16& s, float scale_log2, float& m_run,
                                           float& l_run, f32x16 (&oacc)[4], bf16x8 (&pf)[2],
                                           float& psum) {
  // !(x <= limit) is also true for NaN and +inf sums
  if (__ballot(m_run == -INFINITY || !(psum <= kSumLimit)) != 0ull) {
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));  // lanes l32 and l32 + 32 hold the same query
    const float m_new = fmaxf(m_run, mx * scale_log2);
    // exp2(-inf) = 0 for the first finite reference; -inf - -inf would be NaN
    const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
    l_run *= alpha;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nt][r] *= alpha;
    m_run = m_new;
    softmax_sub(s, scale_log2, m_run, pf, psum);
  }
  l_run += psum;
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
    void* __restrict__ o, int o_bf16, float* __restrict__ lse,
    const int32_t* __restrict__ row_order, int64_t rows) {
  __shared__ __attribute__((aligned(1024))) uint16_t k_lds[kBlock * 128];
  __shared__ __attribute__((aligned(1024))) uint16_t v_lds[kBlock * 128];
  __shared__ int list[kListCap];
  __shared__ int wave_cnt[8];

  // the row of this workgroup (uniform): an entry of row_order outside [0, rows) does nothing
  const int64_t row = row_order ? (int64_t)row_order[blockIdx.x] : (int64_t)blockIdx.x;
  if (row < 0 || row >= rows) return;
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
  const LdsOff loff = lds_offsets(l32, h, tr_row, tr_col);

  while (pos < end) {
    const int n = stage_list(col_idx, &pos, end, nkb, tail, list, wave_cnt, wave_cnt + 4, tid);
    if (n == 0) continue;
    {
      const int cb = __builtin_amdgcn_readfirstlane(list[0]);
      tile_dma<false>(kbuf, cb * kTileK, k_lds, w, dmo, rbk);
      tile_dma<true>(vbuf, cb * kTileV, v_lds, w, dmo, rbv);
    }
    // block i of the window; the last one (kLast) issues no prefetch, so no DMA is in flight
    // when the window ends (an unconditional prefetch would re-fetch a block for nothing, and a
    // conditional one makes the compiler's wait bookkeeping drain all pending DMAs)
    auto block = [&](int i, auto last) {
      constexpr bool kLast = decltype(last)::value;
      // K(i) landed in every wave's part (V(i) may still be in flight)
      wait_vmcnt<8>();
      wg_barrier();
      const LdsOff lo = lds_opaque(loff);

      // sub-tiles u = 0 .. 3 of the block: the softmax of u runs next to the QK MFMAs of u + 1
      // and the PV MFMAs of u - 1
      f32x16 sa, sb;
      bf16x8 pfa[2], pfb[2];
      float psum;
      qk_sub(k_lds, lo, qf, 0, sa);
      softmax_sub(sa, scale_log2, m_run, pfa, psum);
      qk_sub(k_lds, lo, qf, 1, sb);
      settle_sub(sa, scale_log2, m_run, l_run, oacc, pfa, psum);

      // V(i) landed (nothing else is in flight)
      wait_vmcnt<0>();
      wg_barrier();
      softmax_sub(sb, scale_log2, m_run, pfb, psum);
      qk_sub(k_lds, lo, qf, 2, sa);
      pv_sub(v_lds, lo, pfa, 0, oacc);
      settle_sub(sb, scale_log2, m_run, l_run, oacc, pfb, psum);

      softmax_sub(sa, scale_log2, m_run, pfa, psum);
      qk_sub(k_lds, lo, qf, 3, sb);
      pv_sub(v_lds, lo, pfb, 1, oacc);
      settle_sub(sa, scale_log2, m_run, l_run, oacc, pfa, psum);

      int cb_next = 0;
      if (!kLast) {
        cb_next = __builtin_amdgcn_readfirstlane(list[i + 1]);
        wait_lgkmcnt0();
        wg_barrier();  // every wave is done reading K(i)
        tile_dma<false>(kbuf, cb_next * kTileK, k_lds, w, dmo, rbk);
      }

      softmax_sub(sb, scale_log2, m_run, pfb, psum);
      pv_sub(v_lds, lo, pfa, 2, oacc);
      settle_sub(sb, scale_log2, m_run, l_run, oacc, pfb, psum);
      pv_sub(v_lds, lo, pfb, 3, oacc);

      if (!kLast) {
        wait_lgkmcnt0();
        wg_barrier();  // every wave is done reading V(i)
        tile_dma<true>(vbuf, cb_next * kTileV, v_lds, w, dmo, rbv);
      }
    };
    for (int i = 0; i + 1 < n; ++i) block(i, std::false_type{});
    block(n - 1, std::true_type{});
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
    const LdsOff lo = lds_opaque(loff);
    // opaque copies for the mask too: the comparisons would otherwise be hoisted above the loop
    int h_opaque = h, klast_opaque = klast;
    asm volatile("" : "+v"(h_opaque), "+s"(klast_opaque));
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      f32x16 s;
      qk_sub(k_lds, lo, qf, jt, s);
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (sacc_key(jt, r, h_opaque) >= klast_opaque) s[r] = -INFINITY;
      bf16x8 pf[2];
      float psum;
      softmax_sub(s, scale_log2, m_run, pf, psum);
      settle_sub(s, scale_log2, m_run, l_run, oacc, pf, psum);
      pv_sub(v_lds, lo, pf, jt, oacc);
    }
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

// fp32 path: one workgroup of 512 threads per CSR row. Each query of the block is served by a
// quad of consecutive lanes; lane `part` of the quad holds dims [part * D / 4, (part + 1) * D / 4)
// of the query and of its output accumulator. A key's logit is the sum of the four partial dot
// products (two quad shuffles, the same bits in all four lanes), so the softmax state (m, l) is
// replicated in the quad and each lane updates its quarter of O.
template <int D>
__global__ __launch_bounds__(512) void attn_fwd_f32_kernel(AttnArgs a) {
  constexpr int kPart = D / 4;   // dims per lane
  constexpr int kVecs = kPart / 4;
  __shared__ __attribute__((aligned(16))) float k_lds[kBlock * D];
  __shared__ __attribute__((aligned(16))) float v_lds[kBlock * D];
  // the row of this workgroup (uniform): an entry of row_order outside [0, rows) does nothing
  const int64_t row = a.row_order ? (int64_t)a.row_order[blockIdx.x] : (int64_t)blockIdx.x;
  if (row < 0 || row >= a.rows) return;
  const int64_t bh = row / a.nqb;
  const int qb = (int)(row - bh * a.nqb);
  const int t = threadIdx.x;
  const int part = t & 3;
  const int64_t qi = (int64_t)qb * kBlock + (t >> 2);
  const bool q_valid = qi < a.lq;
  const int64_t qtok = bh * a.lq + (q_valid ? qi : 0);  // lse index (contiguous)
  const float* qp = static_cast<const float*>(a.q) +
                    token_offset(a.qs, bh, a.heads, q_valid ? qi : 0) + part * kPart;
  const float* kp = static_cast<const float*>(a.k) + token_offset(a.ks, bh, a.heads, 0);
  const float* vp = static_cast<const float*>(a.v) + token_offset(a.vs, bh, a.heads, 0);

  float qv[kPart], acc[kPart];
#pragma unroll
  for (int c = 0; c < kVecs; ++c) {
    const f32x4 x = q_valid ? *reinterpret_cast<const f32x4*>(qp + 4 * c) : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < 4; ++e) qv[4 * c + e] = x[e];
  }
#pragma unroll
  for (int d = 0; d < kPart; ++d) acc[d] = 0.f;
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
    for (int i = t; i < kBlock * D / 4; i += 512) {
      const int r = i / (D / 4), c4 = i - r * (D / 4);
      const bool in = r < valid;
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      reinterpret_cast<f32x4*>(k_lds)[i] =
          in ? *reinterpret_cast<const f32x4*>(kb + r * a.ks.t + 4 * c4) : z;
      reinterpret_cast<f32x4*>(v_lds)[i] =
          in ? *reinterpret_cast<const f32x4*>(vb + r * a.vs.t + 4 * c4) : z;
    }
    __syncthreads();
    for (int j0 = 0; j0 < valid; j0 += 32) {
      float s[32];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float* kr = k_lds + (j0 + j) * D + part * kPart;
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < kVecs; ++c) {
          const f32x4 kk = *reinterpret_cast<const f32x4*>(kr + 4 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) dot = fmaf(qv[4 * c + e], kk[e], dot);
        }
        dot += __shfl_xor(dot, 1, 64);
        dot += __shfl_xor(dot, 2, 64);
        s[j] = j0 + j < valid ? dot * a.scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int d = 0; d < kPart; ++d) acc[d] *= alpha;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float p = __builtin_amdgcn_exp2f(s[j] - m_new);
        l_run += p;
        const float* vr = v_lds + (j0 + j) * D + part * kPart;
#pragma unroll
        for (int c = 0; c < kVecs; ++c) {
          const f32x4 vv = *reinterpret_cast<const f32x4*>(vr + 4 * c);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[4 * c + e] = fmaf(p, vv[e], acc[4 * c + e]);
        }
      }
      m_run = m_new;
    }
    __syncthreads();
  }
  if (!q_valid) return;
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  const int64_t otok = token_offset(a.os, bh, a.heads, qi) + part * kPart;
  if (a.o_bf16) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + otok;
#pragma unroll
    for (int d = 0; d < kPart; ++d) orow[d] = (uint16_t)f32_to_bf16_bits(acc[d] * inv);
  } else {
    float* orow = static_cast<float*>(a.o) + otok;
#pragma unroll
    for (int c = 0; c < kVecs; ++c) {
      f32x4 ov;
#pragma unroll
      for (int e = 0; e < 4; ++e) ov[e] = acc[4 * c + e] * inv;
      *reinterpret_cast<f32x4*>(orow + 4 * c) = ov;
    }
  }
  if (a.lse && part == 0)
    a.lse[qtok] = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
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
        a.lq, a.lk, a.heads, a.qs, a.ks, a.vs, a.os, a.scale_log2, a.o, a.o_bf16, a.lse,
        a.row_order, a.rows);
  } else if (!bf16 && head_dim == 64)
    attn_fwd_f32_kernel<64><<<grid, 512, 0, stream>>>(a);
  else if (!bf16 && head_dim == 128)
    attn_fwd_f32_kernel<128><<<grid, 512, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dbsp
