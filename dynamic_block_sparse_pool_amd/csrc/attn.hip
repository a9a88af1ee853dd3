// Forward block-sparse attention over the kept key blocks of every (batch, head, query block).
//
// Sources: [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", method overview,
// FastFlex bullet (the selected blocks run through a forward-only sparse attention path);
// [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention", key
// design 4 (the kernel walks a read-only per-query-block list of key blocks and skips the rest).
//
// attn_fwd_bf16_kernel (bf16, head_dim 128): one workgroup of 4 waves per CSR row (one query
// block of 128 tokens); wave w owns queries [32 w, 32 w + 32). Per kept key block:
//   * K [128 x 128] and V [128 x 128] are copied to LDS (rows padded against bank conflicts);
//   * S^T = K Q^T on 32x32x16 bf16 MFMAs: Q^T is the B operand, held in registers for the
//     whole row; the result leaves every lane with one query column and 64 key rows, so the
//     row max needs one cross-half exchange;
//   * an fp32 online softmax in the exp2 domain (the log2(e) factor folded into the scale);
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

namespace dbsp {

constexpr int kKStride = 136;  // bf16 per K row in LDS (272 B: 16 consecutive rows hit distinct banks)
constexpr int kVStride = 160;  // bf16 per V row in LDS (320 B: transpose reads are conflict free)


__device__ __forceinline__ int64_t clip64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__global__ __launch_bounds__(256, 2) void attn_fwd_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t k_lds[kBlock * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t v_lds[kBlock * kVStride];

  const int64_t row = blockIdx.x;
  const int64_t bh = row / a.nqb;
  const int qb = (int)(row - bh * a.nqb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int h = lane >> 5;
  const int l32 = lane & 31;
  const int64_t lq = (int64_t)a.nqb * kBlock;
  const int64_t lk = (int64_t)a.nkb * kBlock;

  const uint16_t* qp = static_cast<const uint16_t*>(a.q);
  const uint16_t* kp = static_cast<const uint16_t*>(a.k) + bh * lk * 128;
  const uint16_t* vp = static_cast<const uint16_t*>(a.v) + bh * lk * 128;

  // Q^T as the B operand of S^T = K Q^T: lane (h, l32) holds query 32 w + l32, dims 16 s + 8 h .. +7
  const int64_t qtok = bh * lq + (int64_t)qb * kBlock + 32 * w + l32;
  bf16x8 qf[8];
  {
    const uint16_t* qr = qp + qtok * 128 + 8 * h;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(qr + 16 * s);
  }

  int64_t beg = a.row_ptr[row], end = a.row_ptr[row + 1];
  beg = clip64(beg, 0, a.col_capacity);
  end = clip64(end, beg, a.col_capacity);

  f32x16 oacc[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[nt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  // per-thread coordinates for the cooperative K / V copies: 8 passes of 16 rows x 16 chunks
  const int cp_row = tid >> 4;
  const int cp_chunk = tid & 15;
  // per-lane coordinates for the transposed V reads
  const int tr_row = (lane & 15) >> 2;
  const int tr_col = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  for (int64_t it = beg; it < end; ++it) {
    const int cb = a.col_idx[it];
    if (cb < 0 || cb >= a.nkb) continue;
    const uint16_t* kb = kp + (int64_t)cb * kBlock * 128;
    const uint16_t* vb = vp + (int64_t)cb * kBlock * 128;
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = cp_row + 16 * p;
      kr[p] = load_u32x4(kb + r * 128 + cp_chunk * 8);
      vr[p] = load_u32x4(vb + r * 128 + cp_chunk * 8);
    }
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = cp_row + 16 * p;
      *reinterpret_cast<u32x4*>(k_lds + r * kKStride + cp_chunk * 8) = kr[p];
      *reinterpret_cast<u32x4*>(v_lds + r * kVStride + cp_chunk * 8) = vr[p];
    }
    __syncthreads();

    // S^T tiles: sacc[jt] covers keys 32 jt .. 32 jt + 31 (rows) x this wave's 32 queries
    f32x16 sacc[4];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[jt][r] = 0.f;
      const uint16_t* kr0 = k_lds + (32 * jt + l32) * kKStride + 8 * h;
#pragma unroll
      for (int s = 0; s < 8; ++s) {
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kr0 + 16 * s);
        sacc[jt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[s], sacc[jt], 0, 0, 0);
      }
    }

    // online softmax for query column l32 (lanes l32 and l32 + 32 share it)
    float mx = -INFINITY;
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[jt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
    float psum = 0.f;
    bf16x8 pf[8];
#pragma unroll
    for (int jt = 0; jt < 4; ++jt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(sacc[jt][r], a.scale_log2, -m_new));
        psum += p;
        pf[2 * jt + (r >> 3)][r & 7] = (__bf16)p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[nt][r] *= alpha;

    // O^T += V^T P^T; k step s covers keys 16 s .. 16 s + 15 in the accumulator order of S^T
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int jb = 16 * s + 4 * h + tr_row;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int col = 32 * nt + tr_col;
        // whole-vector casts only: an element-wise rebuild of these results has been seen to
        // lose the upper dword of each read in the generated code
        const u32x2 lo = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(v_lds + jb * kVStride + col)));
        const u32x2 hi = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(v_lds + (jb + 8) * kVStride + col)));
        const u32x4 w4 = {lo[0], lo[1], hi[0], hi[1]};
        const bf16x8 va = __builtin_bit_cast(bf16x8, w4);
        oacc[nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[s], oacc[nt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // epilogue
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = l_tot > 0.f ? 1.0f / l_tot : 0.f;
  if (a.o_bf16) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + qtok * 128;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n0 = 32 * nt + 8 * g + 4 * h;
        u32x2 pk;
        pk[0] = f32_to_bf16_bits(oacc[nt][4 * g] * inv) | (f32_to_bf16_bits(oacc[nt][4 * g + 1] * inv) << 16);
        pk[1] = f32_to_bf16_bits(oacc[nt][4 * g + 2] * inv) | (f32_to_bf16_bits(oacc[nt][4 * g + 3] * inv) << 16);
        *reinterpret_cast<u32x2*>(orow + n0) = pk;
      }
  } else {
    float* orow = static_cast<float*>(a.o) + qtok * 128;
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
  if (a.lse && h == 0)
    a.lse[qtok] = l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.69314718055994531f : -INFINITY;
}

template <int D>
__global__ __launch_bounds__(128) void attn_fwd_f32_kernel(AttnArgs a) {
  __shared__ float k_lds[kBlock][D];
  __shared__ float v_lds[kBlock][D];
  const int64_t row = blockIdx.x;
  const int64_t bh = row / a.nqb;
  const int qb = (int)(row - bh * a.nqb);
  const int t = threadIdx.x;
  const int64_t lq = (int64_t)a.nqb * kBlock;
  const int64_t lk = (int64_t)a.nkb * kBlock;
  const int64_t qtok = bh * lq + (int64_t)qb * kBlock + t;
  const float* qp = static_cast<const float*>(a.q) + qtok * D;
  const float* kp = static_cast<const float*>(a.k) + bh * lk * D;
  const float* vp = static_cast<const float*>(a.v) + bh * lk * D;

  float qv[D];
#pragma unroll
  for (int d = 0; d < D; ++d) qv[d] = qp[d];
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
    const float* kb = kp + (int64_t)cb * kBlock * D;
    const float* vb = vp + (int64_t)cb * kBlock * D;
    for (int i = t; i < kBlock * D; i += 128) {
      (&k_lds[0][0])[i] = kb[i];
      (&v_lds[0][0])[i] = vb[i];
    }
    __syncthreads();
    for (int j0 = 0; j0 < kBlock; j0 += 32) {
      float s[32];
      float mx = -INFINITY;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        float dot = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) dot = fmaf(qv[d], k_lds[j0 + j][d], dot);
        s[j] = dot * a.scale_log2;
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
  const float inv = l_run > 0.f ? 1.0f / l_run : 0.f;
  if (a.o_bf16) {
    uint16_t* orow = static_cast<uint16_t*>(a.o) + qtok * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = (uint16_t)f32_to_bf16_bits(acc[d] * inv);
  } else {
    float* orow = static_cast<float*>(a.o) + qtok * D;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv;
  }
  if (a.lse) a.lse[qtok] = l_run > 0.f ? (m_run + __log2f(l_run)) * 0.69314718055994531f : -INFINITY;
}

hipError_t launch_attn(const AttnArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  dim3 grid((unsigned)a.rows);
  if (bf16 && head_dim == 128)
    attn_fwd_bf16_kernel<<<grid, 256, 0, stream>>>(a);
  else if (!bf16 && head_dim == 64)
    attn_fwd_f32_kernel<64><<<grid, 128, 0, stream>>>(a);
  else if (!bf16 && head_dim == 128)
    attn_fwd_f32_kernel<128><<<grid, 128, 0, stream>>>(a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace dbsp
