// Anchor-row path of spatially repeating heads.
//
// Source: [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention",
// key design 3 (spatial repetition: k equally spaced anchor rows per frame, default 5) and key
// design 4 (repeating heads run ordinary attention on the reduced query set and broadcast the
// outputs to the nearest spatial rows). A frame has H spatial rows of W query tokens; the query
// sequence is frames x H x W tokens followed by trailing tokens that belong to no frame.
//
// Anchors are the centres of k equal bands of the H rows, a_j = floor((2 j + 1) H / (2 k)); a
// row takes its nearest anchor (ties to the lower one) at the same column; trailing tokens
// attend as themselves.
//
// The path is three kernels around the block-sparse attention kernel:
//   anchor_gather_kernel    packs the anchor rows' queries (then the trailing ones) into a
//                           contiguous [BH, La_pad, d] buffer, zero-padded to a block multiple;
//   dense_csr_kernel        a CSR keeping every key block for every packed query block;
//   attention               the hot path's attention kernel on the packed queries;
//   anchor_broadcast_kernel writes each query token's output (and lse) from its anchor's.
// The broadcast copies bits, so every row equals its anchor row's output exactly.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

__device__ __forceinline__ int anchor_row(int j, int rows, int k) {
  return (int)(((int64_t)(2 * j + 1) * rows) / (2 * k));
}

// Index j of the anchor nearest to row r (ties to the lower j). The anchors are increasing, so
// the nearest one is the band index or a neighbour of it; a short scan keeps it obviously exact.
__device__ __forceinline__ int nearest_anchor_of(int r, int rows, int k) {
  int best = 0, best_d = abs(r - anchor_row(0, rows, k));
  for (int j = 1; j < k; ++j) {
    const int d = abs(r - anchor_row(j, rows, k));
    if (d < best_d) {
      best = j;
      best_d = d;
    }
  }
  return best;
}

// Source query token of packed position t (t < La), see the file comment.
__device__ __forceinline__ int64_t anchor_source(int64_t t, const AnchorGeom& g) {
  const int64_t per_frame = (int64_t)g.n_anchors * g.width;
  const int64_t anchored = (int64_t)g.frames * per_frame;
  if (t >= anchored) return (int64_t)g.frames * g.rows * g.width + (t - anchored);
  const int64_t f = t / per_frame;
  const int64_t rem = t - f * per_frame;
  const int j = (int)(rem / g.width);
  const int64_t c = rem - (int64_t)j * g.width;
  return (f * g.rows + anchor_row(j, g.rows, g.n_anchors)) * g.width + c;
}

// One thread per 16-byte chunk of a packed query row.
__global__ __launch_bounds__(256) void anchor_gather_kernel(const char* __restrict__ q,
                                                            char* __restrict__ qa, AnchorGeom g,
                                                            int row_bytes, int64_t n_chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int per_row = row_bytes / 16;
  const int64_t row = i / per_row;  // bh * la_pad + t
  const int part = (int)(i - row * per_row);
  const int64_t bh = row / g.la_pad;
  const int64_t t = row - bh * g.la_pad;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (t < g.la) {
    const int64_t src = bh * g.lq + anchor_source(t, g);
    v = *reinterpret_cast<const u32x4*>(q + src * row_bytes + part * 16);
  }
  *reinterpret_cast<u32x4*>(qa + row * row_bytes + part * 16) = v;
}

__global__ __launch_bounds__(256) void dense_csr_kernel(int32_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        int64_t rows, int nkb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (int64_t r = i; r <= rows; r += (int64_t)gridDim.x * 256) row_ptr[r] = (int32_t)(r * nkb);
  const int64_t n = rows * nkb;
  for (int64_t e = i; e < n; e += (int64_t)gridDim.x * 256) col_idx[e] = (int32_t)(e % nkb);
}

// One thread per 16-byte chunk of an output row (and the lse of the row's token).
__global__ __launch_bounds__(256) void anchor_broadcast_kernel(const char* __restrict__ oa,
                                                               const float* __restrict__ lse_a,
                                                               char* __restrict__ o,
                                                               float* __restrict__ lse,
                                                               AnchorGeom g, int row_bytes,
                                                               int64_t n_chunks) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n_chunks) return;
  const int per_row = row_bytes / 16;
  const int64_t row = i / per_row;  // bh * lq + t
  const int part = (int)(i - row * per_row);
  const int64_t bh = row / g.lq;
  const int64_t t = row - bh * g.lq;
  const int64_t video = (int64_t)g.frames * g.rows * g.width;
  int64_t src;
  if (t >= video) {
    src = (int64_t)g.frames * g.n_anchors * g.width + (t - video);
  } else {
    const int64_t per_frame = (int64_t)g.rows * g.width;
    const int64_t f = t / per_frame;
    const int64_t rem = t - f * per_frame;
    const int r = (int)(rem / g.width);
    const int64_t c = rem - (int64_t)r * g.width;
    src = (f * g.n_anchors + nearest_anchor_of(r, g.rows, g.n_anchors)) * g.width + c;
  }
  const int64_t srow = bh * g.la_pad + src;
  *reinterpret_cast<u32x4*>(o + row * row_bytes + part * 16) =
      *reinterpret_cast<const u32x4*>(oa + srow * row_bytes + part * 16);
  if (lse && part == 0) lse[row] = lse_a[srow];
}

hipError_t launch_anchor(const AnchorArgs& a, int head_dim, bool bf16, hipStream_t stream) {
  const AnchorGeom& g = a.geom;
  const int q_row_bytes = head_dim * (bf16 ? 2 : 4);
  const int o_row_bytes = head_dim * (a.o_bf16 ? 2 : 4);
  const int64_t gather_chunks = a.bh * g.la_pad * (q_row_bytes / 16);
  anchor_gather_kernel<<<(unsigned)((gather_chunks + 255) / 256), 256, 0, stream>>>(
      static_cast<const char*>(a.q), static_cast<char*>(a.qa), g, q_row_bytes, gather_chunks);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int64_t rows_a = a.bh * (g.la_pad / kBlock);
  const int64_t csr_items = rows_a * a.nkb > rows_a + 1 ? rows_a * a.nkb : rows_a + 1;
  const int64_t csr_want = (csr_items + 255) / 256;
  const unsigned csr_blocks = (unsigned)(csr_want < 65536 ? csr_want : 65536);
  dense_csr_kernel<<<csr_blocks, 256, 0, stream>>>(a.row_ptr, a.col_idx, rows_a, a.nkb);
  if ((err = hipGetLastError()) != hipSuccess) return err;
  AttnArgs at{};
  at.q = a.qa;
  at.k = a.k;
  at.v = a.v;
  at.row_ptr = a.row_ptr;
  at.col_idx = a.col_idx;
  at.col_capacity = rows_a * a.nkb;
  at.nqb = (int)(g.la_pad / kBlock);
  at.nkb = a.nkb;
  at.lq = g.la_pad;
  at.lk = a.lk;
  // every buffer is contiguous per (batch, head) pair bh, so the pairs act as one batch axis
  at.heads = 1;
  at.qs = Strides{g.la_pad * head_dim, 0, head_dim};
  at.ks = Strides{a.lk * head_dim, 0, head_dim};
  at.vs = at.ks;
  at.os = at.qs;
  at.rows = rows_a;
  at.scale_log2 = a.scale_log2;
  at.o = a.oa;
  at.o_bf16 = a.o_bf16;
  at.lse = a.lse_a;
  if ((err = launch_attn(at, head_dim, bf16, stream)) != hipSuccess) return err;
  const int64_t out_chunks = a.bh * g.lq * (o_row_bytes / 16);
  anchor_broadcast_kernel<<<(unsigned)((out_chunks + 255) / 256), 256, 0, stream>>>(
      static_cast<const char*>(a.oa), a.lse_a, static_cast<char*>(a.o), a.lse, g, o_row_bytes,
      out_chunks);
  return hipGetLastError();
}

}  // namespace dbsp
