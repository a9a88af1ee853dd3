// Launch interface between the host API (api.hip) and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dbsp {

// Element strides of a [batch, heads, tokens, head_dim] view (the innermost dimension is
// contiguous). Contiguous tensors have {heads * L * d, L * d, d}; a [batch, L, heads, d] tensor
// seen head-major has {L * heads * d, d, heads * d}.
struct Strides {
  int64_t b, h, t;
};

// Element offset of token t of (batch, head) pair bh = b * heads + h.
__host__ __device__ __forceinline__ int64_t token_offset(const Strides& s, int64_t bh, int heads,
                                                         int64_t t) {
  return (bh / heads) * s.b + (bh % heads) * s.h + t * s.t;
}

// Largest forced set passed as a bitmask in the kernel arguments: one bit per key block.
constexpr int kMaxForcedWords = 32;  // 2048 key blocks

struct SelectArgs {
  const void* q;           // queries (bf16 or fp32), pooled in the kernel
  Strides qs;              // ... laid out with these strides
  int heads;               // H, to split the (batch, head) index
  const uint16_t* ksplit;  // pooled keys as bf16 hi | lo in MFMA tile order (workspace):
                           // [BH][ceil(nkb / 16)][D / 32][hi | lo][64 lanes][8]
  int nqb, nkb;
  int64_t lq, lk;      // tokens per (batch, head); the last block may be partial
  float scale;         // score scale
  int t0, t1, e0, e1;  // forced key-block ranges [t0, t1) and [e0, e1) ...
  int forced_by_words; // ... or, when set, the forced blocks are the set bits of forced_words
  uint64_t forced_words[kMaxForcedWords];
  int mode;            // 0 Top-K, 1 mass
  int kk;              // Top-K: candidates kept per row
  int per_row;         // Top-K: entries per row (forced + kk)
  uint64_t theta;      // mass: ceil(tau * 2^62)
  int keep_all;        // mass: tau >= 1
  int32_t* row_ptr;
  int32_t* col_idx;
  int64_t col_capacity;
  float* scores_out;   // nullable [rows, nkb]
  int32_t* counts;     // mass: [rows] (workspace)
  uint64_t* masks;     // mass: [rows, words] (workspace)
  int words;           // mass: ceil(nkb / 64)
  int lds_stride;      // floats per score row in LDS
  int64_t n_rows;      // batch * heads * nqb
};

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  Strides qs, ks, vs, os;  // element strides of Q, K, V and O
  const int32_t* row_ptr;
  const int32_t* col_idx;
  int64_t col_capacity;
  int heads, nqb, nkb;
  int64_t lq, lk;    // tokens per (batch, head); the last block may be partial
  int64_t rows;
  float scale_log2;  // softmax_scale * log2(e)
  void* o;
  int o_bf16;
  float* lse;
  const int32_t* row_order;  // nullable: workgroup b processes row row_order[b] (else row b)
};

struct EnergyArgs {
  const void* q;
  const void* k;
  int nqb, nkb;
  int64_t lq, lk;    // tokens per (batch, head); the last block may be partial
  int64_t rows;
  float scale_log2;  // softmax_scale * log2(e)
  float* energy;     // [rows, nkb]
  float* lse;        // nullable [rows * 128]
  float* ws;         // bf16 path: slots * nkb * 128 floats (per-query block log2-sums)
  int64_t slots;     // bf16 path: persistent workgroups, 1 .. rows
};

// Workgroups of the one-sweep bf16 energy kernel that a full workspace provides for: two per
// compute unit of a 256-CU device.
constexpr int64_t kEnergySlots = 512;

// Query geometry of the anchor-row path: frames x rows x width tokens, then trailing tokens.
struct AnchorGeom {
  int frames, rows, width, n_anchors;
  int64_t lq;      // query tokens per (batch, head)
  int64_t la;      // packed queries: frames * n_anchors * width + (lq - frames * rows * width)
  int64_t la_pad;  // la rounded up to a block multiple
};

struct AnchorArgs {
  const void* q;
  const void* k;
  const void* v;
  void* qa;          // workspace: packed queries [bh, la_pad, d], input dtype
  void* oa;          // workspace: packed outputs [bh, la_pad, d], output dtype
  float* lse_a;      // workspace: [bh, la_pad]
  int32_t* row_ptr;  // workspace: dense CSR over the packed query blocks
  int32_t* col_idx;
  int64_t bh;
  int nkb;
  int64_t lk;        // key tokens per (batch, head)
  float scale_log2;
  void* o;
  int o_bf16;
  float* lse;        // nullable [bh, lq]
  AnchorGeom geom;
};

// Pooled keys of every (batch, head): bh heads of lk tokens each, nkb = ceil(lk / 128) blocks.
hipError_t launch_pool(const void* k, const Strides& ks, int heads, uint16_t* ksplit, int64_t bh,
                       int nkb, int64_t lk, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_select(const SelectArgs& a, int64_t bh, int head_dim, bool bf16,
                         hipStream_t stream);
hipError_t launch_attn(const AttnArgs& a, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_energy(const EnergyArgs& a, int head_dim, bool bf16, hipStream_t stream);
hipError_t launch_retained_mass(const float* energy, const int32_t* row_ptr,
                                const int32_t* col_idx, int64_t col_capacity, int nkb,
                                int64_t rows, double* mass, hipStream_t stream);
hipError_t launch_select_energy(const SelectArgs& a, const float* energy, hipStream_t stream);
// row_ptr / col_idx from the per-row counts and kept bitmasks in a.counts / a.masks
hipError_t launch_counts_to_csr(const SelectArgs& a, hipStream_t stream);
// a.row_ptr = exclusive prefix of a.counts over a.n_rows rows (row_ptr[n_rows] = total)
hipError_t launch_scan_counts(const SelectArgs& a, hipStream_t stream);
// out[0 .. n] = exclusive prefix of counts[0 .. n) (out[n] = total); counts 256-byte aligned
hipError_t launch_exclusive_scan(const int32_t* counts, int32_t* out, int64_t n,
                                 hipStream_t stream);
hipError_t launch_csr_to_intervals(const int32_t* row_ptr, const int32_t* col_idx,
                                   int64_t col_capacity, int nkb, int64_t rows, int32_t* iv_ptr,
                                   int32_t* iv, int64_t iv_capacity, int32_t* counts,
                                   hipStream_t stream);
hipError_t launch_intervals_to_csr(const int32_t* iv_ptr, const int32_t* iv, int64_t iv_capacity,
                                   int nkb, int64_t rows, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, int32_t* counts, hipStream_t stream);
hipError_t launch_vote_accumulate(const int32_t* row_ptr, const int32_t* col_idx,
                                  int64_t col_capacity, int nkb, int64_t rows, int32_t* counts,
                                  hipStream_t stream);
hipError_t launch_anchor(const AnchorArgs& a, int head_dim, bool bf16, hipStream_t stream);
// order = the rows of each (batch, head) sorted by kept count, longest first, heads in order.
// Workspace: nb = (rows / nqb) * (nkb + 1) bucket counts (256-byte aligned), then nb + 1 cursors.
hipError_t launch_row_order_lpt(const int32_t* row_ptr, int64_t col_capacity, int64_t rows,
                                int nqb, int nkb, int32_t* order, int32_t* counts,
                                int32_t* cursor, hipStream_t stream);
hipError_t launch_vote_select(const int32_t* counts, int n_inputs, double rho, const SelectArgs& a,
                              hipStream_t stream);

}  // namespace dbsp
