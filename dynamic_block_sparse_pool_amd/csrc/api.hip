// Host side of the C ABI declared in include/dbsp.h: argument validation (pure host code, runs
// before any HIP call), workspace and nnz sizing, and kernel launches.
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "../../include/dbsp.h"
#include "common.hpp"

#include "kernels.hpp"

namespace {

constexpr int32_t kVersion = 110;  // 0.1.1: token-level energy, retained mass, energy selection
// bf16 attention addresses a head's K and V with 32-bit byte offsets (block index x 32 KiB)
constexpr int32_t kMaxBf16KeyBlocks = 65535;

bool shape_ok(const dbsp_dims* d) {
  if (!d) return false;
  if (d->batch <= 0 || d->heads <= 0 || d->lq <= 0 || d->lk <= 0) return false;
  if (d->dtype != DBSP_F32 && d->dtype != DBSP_BF16) return false;
  if (d->head_dim <= 0) return false;
  return true;
}

// Blocks per sequence: a length that is not a multiple of 128 ends in a partial block.
int32_t nqb_of(const dbsp_dims* d) { return (d->lq + DBSP_BLOCK - 1) / DBSP_BLOCK; }
int32_t nkb_of(const dbsp_dims* d) { return (d->lk + DBSP_BLOCK - 1) / DBSP_BLOCK; }

bool dtype_supported(const dbsp_dims* d) {
  if (d->dtype == DBSP_BF16) return d->head_dim == 128 || d->head_dim == 64;
  return d->head_dim == 64 || d->head_dim == 128;
}

bool attn_supported(const dbsp_dims* d) {
  if (d->dtype == DBSP_BF16) return d->head_dim == 128;
  return d->head_dim == 64 || d->head_dim == 128;
}

int64_t rows_of(const dbsp_dims* d) {
  return (int64_t)d->batch * d->heads * nqb_of(d);
}

// Validates the two forced ranges against nkb; returns the forced count or -1.
int32_t forced_count(int32_t nkb, dbsp_range t, dbsp_range e) {
  const dbsp_range r[2] = {t, e};
  for (int i = 0; i < 2; ++i)
    if (r[i].begin < 0 || r[i].begin > r[i].end || r[i].end > nkb) return -1;
  const bool both = t.begin < t.end && e.begin < e.end;
  if (both && t.begin < e.end && e.begin < t.end) return -1;  // overlap
  return (t.end - t.begin) + (e.end - e.begin);
}

// The forced key blocks of a call: two ranges, or an explicit list held as a bitmask.
struct ForcedSet {
  bool by_words = false;
  dbsp_range t{0, 0}, e{0, 0};
  uint64_t words[dbsp::kMaxForcedWords] = {};
  int32_t count = 0;
};

int32_t forced_from_ranges(int32_t nkb, dbsp_range t, dbsp_range e, ForcedSet* f) {
  const int32_t n = forced_count(nkb, t, e);
  if (n < 0) return DBSP_ERR_INVALID_ARG;
  f->by_words = false;
  f->t = t;
  f->e = e;
  f->count = n;
  return DBSP_OK;
}

// Indices must lie in [0, nkb) and be distinct; nkb above the bitmask size is unsupported.
int32_t forced_from_list(int32_t nkb, const int32_t* list, int32_t n, ForcedSet* f) {
  if (n < 0 || (n > 0 && !list)) return DBSP_ERR_INVALID_ARG;
  if (nkb > 64 * dbsp::kMaxForcedWords) return DBSP_ERR_UNSUPPORTED;
  ForcedSet r;
  r.by_words = true;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t c = list[i];
    if (c < 0 || c >= nkb) return DBSP_ERR_INVALID_ARG;
    uint64_t& w = r.words[c >> 6];
    const uint64_t bit = 1ull << (c & 63);
    if (w & bit) return DBSP_ERR_INVALID_ARG;  // duplicate
    w |= bit;
  }
  r.count = n;
  *f = r;
  return DBSP_OK;
}

int32_t topk_k_f(const dbsp_dims* d, double density, const ForcedSet& fs, int32_t override_k,
                 int32_t* k_out) {
  if (!shape_ok(d) || !k_out) return DBSP_ERR_INVALID_ARG;
  const int32_t nkb = nkb_of(d);
  const int32_t ncand = nkb - fs.count;
  int64_t k;
  if (override_k >= 0) {
    if (override_k > ncand) return DBSP_ERR_INVALID_ARG;
    k = override_k;
  } else {
    if (!(density >= 0.0 && density <= 1.0)) return DBSP_ERR_INVALID_ARG;  // also rejects NaN
    k = (int64_t)ceil(density * (double)ncand);
    if (k > ncand) k = ncand;
  }
  *k_out = (int32_t)k;
  return DBSP_OK;
}

int32_t topk_k(const dbsp_dims* d, double density, dbsp_range t, dbsp_range e, int32_t override_k,
               int32_t* k_out) {
  if (!shape_ok(d) || !k_out) return DBSP_ERR_INVALID_ARG;
  ForcedSet fs;
  const int32_t st = forced_from_ranges(nkb_of(d), t, e, &fs);
  if (st != DBSP_OK) return st;
  return topk_k_f(d, density, fs, override_k, k_out);
}

int32_t nnz_bound_f(const dbsp_dims* d, int32_t mode, double param, const ForcedSet& fs,
                    int32_t override_k, int64_t* out) {
  if (!shape_ok(d) || !out) return DBSP_ERR_INVALID_ARG;
  const int32_t nkb = nkb_of(d);
  if (mode == DBSP_TOPK) {
    int32_t k;
    const int32_t st = topk_k_f(d, param, fs, override_k, &k);
    if (st != DBSP_OK) return st;
    *out = rows_of(d) * (int64_t)(fs.count + k);
    return DBSP_OK;
  }
  if (mode == DBSP_MASS) {
    if (!(param > 0.0 && param <= 1.0)) return DBSP_ERR_INVALID_ARG;
    *out = rows_of(d) * (int64_t)nkb;
    return DBSP_OK;
  }
  return DBSP_ERR_INVALID_ARG;
}

int32_t nnz_bound(const dbsp_dims* d, int32_t mode, double param, dbsp_range t, dbsp_range e,
                  int32_t override_k, int64_t* out) {
  if (!shape_ok(d) || !out) return DBSP_ERR_INVALID_ARG;
  ForcedSet fs;
  const int32_t st = forced_from_ranges(nkb_of(d), t, e, &fs);
  if (st != DBSP_OK) return st;
  return nnz_bound_f(d, mode, param, fs, override_k, out);
}

void apply_forced(const ForcedSet& fs, dbsp::SelectArgs* a) {
  a->t0 = fs.t.begin;
  a->t1 = fs.t.end;
  a->e0 = fs.e.begin;
  a->e1 = fs.e.end;
  a->forced_by_words = fs.by_words ? 1 : 0;
  for (int i = 0; i < dbsp::kMaxForcedWords; ++i) a->forced_words[i] = fs.words[i];
}

uint64_t align256(uint64_t x) { return (x + 255) & ~(uint64_t)255; }

// Floats per score row in LDS: at least nkb, rounded to 16, and congruent to 16 or 48 modulo 64
// so that the four rows an MFMA output spans fall in distinct banks.
int score_lds_stride(int nkb) {
  int s = (nkb + 15) & ~15;
  while ((s & 63) != 16 && (s & 63) != 48) s += 16;
  return s;
}

struct WorkspaceLayout {
  uint64_t qbar, kbar, counts, masks, total;
};

WorkspaceLayout layout_of(const dbsp_dims* d, int32_t mode) {
  WorkspaceLayout w{};
  const uint64_t bh = (uint64_t)d->batch * d->heads;
  const uint64_t nqb = nqb_of(d), nkb = nkb_of(d);
  uint64_t off = 0;
  // pooled keys, each stored as bf16 hi and lo halves (2 x head_dim x 2 bytes); the pooled
  // queries never leave the selection kernel
  w.qbar = off;
  w.kbar = off;  // tiles of 16 key blocks (the last one padded)
  off = align256(off + bh * ((nkb + 15) / 16) * 16 * d->head_dim * 2 * sizeof(uint16_t));
  if (mode == DBSP_MASS) {
    w.counts = off;
    off = align256(off + bh * nqb * sizeof(int32_t));
    w.masks = off;
    off = align256(off + bh * nqb * ((nkb + 63) / 64) * sizeof(uint64_t));
  }
  w.total = off;
  return w;
}

// Anchor-row path: validated geometry and workspace layout.
struct AnchorLayout {
  dbsp::AnchorGeom g;
  uint64_t qa, oa, lse_a, row_ptr, col_idx, total;
};

int32_t anchor_layout(const dbsp_dims* d, int32_t frames, int32_t rows, int32_t width,
                      int32_t n_anchors, int32_t o_dtype, AnchorLayout* out) {
  if (!shape_ok(d) || frames < 1 || rows < 1 || width < 1 || n_anchors < 1 || n_anchors > rows)
    return DBSP_ERR_INVALID_ARG;
  if (o_dtype != DBSP_F32 && o_dtype != DBSP_BF16) return DBSP_ERR_INVALID_ARG;
  const int64_t video = (int64_t)frames * rows * width;
  if (video > d->lq) return DBSP_ERR_INVALID_ARG;
  AnchorLayout l{};
  l.g.frames = frames;
  l.g.rows = rows;
  l.g.width = width;
  l.g.n_anchors = n_anchors;
  l.g.lq = d->lq;
  l.g.la = (int64_t)frames * n_anchors * width + (d->lq - video);
  l.g.la_pad = (l.g.la + DBSP_BLOCK - 1) / DBSP_BLOCK * DBSP_BLOCK;
  const uint64_t bh = (uint64_t)d->batch * d->heads;
  const uint64_t in_elt = d->dtype == DBSP_BF16 ? 2 : 4, out_elt = o_dtype == DBSP_BF16 ? 2 : 4;
  const uint64_t rows_a = bh * (uint64_t)(l.g.la_pad / DBSP_BLOCK);
  const uint64_t nkb = nkb_of(d);
  if (rows_a * nkb > (uint64_t)INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  uint64_t off = 0;
  l.qa = off;
  off = align256(off + bh * l.g.la_pad * d->head_dim * in_elt);
  l.oa = off;
  off = align256(off + bh * l.g.la_pad * d->head_dim * out_elt);
  l.lse_a = off;
  off = align256(off + bh * l.g.la_pad * sizeof(float));
  l.row_ptr = off;
  off = align256(off + (rows_a + 1) * sizeof(int32_t));
  l.col_idx = off;
  off = align256(off + rows_a * nkb * sizeof(int32_t));
  l.total = off;
  *out = l;
  return DBSP_OK;
}

// Workspace of one persistent workgroup of the bf16 energy kernel: a float per (key block,
// query of a block).
uint64_t energy_slot_bytes(const dbsp_dims* dims) {
  return (uint64_t)nkb_of(dims) * dbsp::kBlock * sizeof(float);
}

// dbsp_select_energy: per-row counts and kept bitmasks only.
WorkspaceLayout energy_select_layout(const dbsp_dims* d) {
  WorkspaceLayout w{};
  const uint64_t rows = (uint64_t)rows_of(d), nkb = nkb_of(d);
  w.counts = 0;
  w.masks = align256(rows * sizeof(int32_t));
  w.total = align256(w.masks + rows * ((nkb + 63) / 64) * sizeof(uint64_t));
  return w;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Strides of a contiguous [batch, heads, len, head_dim] tensor.
dbsp::Strides contiguous(const dbsp_dims* d, int64_t len) {
  return dbsp::Strides{(int64_t)d->heads * len * d->head_dim, len * d->head_dim,
                       (int64_t)d->head_dim};
}

// Caller strides: non-negative, every row 16-byte aligned (as the base pointer must be), and
// for written tensors rows that do not overlap within a head.
bool strides_ok(const dbsp_strides* s, const dbsp_dims* d, bool written) {
  if (!s) return false;
  const int64_t elt = d->dtype == DBSP_BF16 ? 2 : 4;
  if (s->batch < 0 || s->head < 0 || s->token < 0) return false;
  if ((s->batch * elt) % 16 || (s->head * elt) % 16 || (s->token * elt) % 16) return false;
  if (written && s->token < d->head_dim) return false;
  return true;
}

dbsp::Strides to_strides(const dbsp_strides* s) {
  return dbsp::Strides{s->batch, s->head, s->token};
}

// Device scratch of dbsp_sparse_select_noalloc, for callers that cannot allocate: one copy of
// this array per GPU, created when the library's code object is loaded on that GPU and held
// until the process ends. In host code the name is only a stand-in for the symbol: the device
// address of each GPU's copy comes from hipGetSymbolAddress, called once per device with that
// device current, and only that address is ever handed to kernels.
__device__ __align__(256) unsigned char scratch[DBSP_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// The current device's copy of `scratch` (looked up on the first call on that device).
int32_t noalloc_scratch(void* stream, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices)
    return DBSP_ERR_HIP;
  if (stream) {  // the stream must run on the current device, whose copy is looked up
    int sdev = -1;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev) != hipSuccess)
      return DBSP_ERR_HIP;
    if (sdev != dev) return DBSP_ERR_INVALID_ARG;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DBSP_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DBSP_OK;
}

}  // namespace

extern "C" {

int32_t dbsp_version(void) { return kVersion; }

const char* dbsp_status_string(int32_t status) {
  switch (status) {
    case DBSP_OK: return "ok";
    case DBSP_ERR_INVALID_ARG: return "invalid argument";
    case DBSP_ERR_UNSUPPORTED: return "unsupported shape or type";
    case DBSP_ERR_CAPACITY: return "col_idx capacity below the nnz bound";
    case DBSP_ERR_WORKSPACE: return "workspace missing or too small";
    case DBSP_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

int32_t dbsp_topk_budget(const dbsp_dims* dims, double density, dbsp_range text_blocks,
                         dbsp_range dense_extra_blocks, int32_t topk_override, int32_t* k_out) {
  return topk_k(dims, density, text_blocks, dense_extra_blocks, topk_override, k_out);
}

int32_t dbsp_select_nnz_bound_list(const dbsp_dims* dims, int32_t mode, double density_or_mass,
                                   const int32_t* forced_blocks, int32_t n_forced,
                                   int32_t topk_override, int64_t* nnz_bound_out) {
  if (!shape_ok(dims) || !nnz_bound_out) return DBSP_ERR_INVALID_ARG;
  ForcedSet fs;
  const int32_t st = forced_from_list(nkb_of(dims), forced_blocks, n_forced, &fs);
  if (st != DBSP_OK) return st;
  return nnz_bound_f(dims, mode, density_or_mass, fs, topk_override, nnz_bound_out);
}

int32_t dbsp_select_nnz_bound(const dbsp_dims* dims, int32_t mode, double density_or_mass,
                              dbsp_range text_blocks, dbsp_range dense_extra_blocks,
                              int32_t topk_override, int64_t* nnz_bound_out) {
  return nnz_bound(dims, mode, density_or_mass, text_blocks, dense_extra_blocks, topk_override,
                   nnz_bound_out);
}

int32_t dbsp_select_workspace_bytes(const dbsp_dims* dims, int32_t mode, uint64_t* bytes) {
  if (!shape_ok(dims) || !bytes || (mode != DBSP_TOPK && mode != DBSP_MASS))
    return DBSP_ERR_INVALID_ARG;
  *bytes = layout_of(dims, mode).total;
  return DBSP_OK;
}

static int32_t sparse_select_impl(const void* q, const void* k, const dbsp_dims* dims,
                                  const dbsp_strides* q_strides, const dbsp_strides* k_strides,
                                  const ForcedSet* fs_in, dbsp_range text_blocks,
                                  dbsp_range dense_extra_blocks, int32_t mode,
                                  double density_or_mass, int32_t topk_override, float score_scale,
                                  int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                  float* scores_out, void* workspace, uint64_t workspace_bytes,
                                  void* stream) {
  if (!shape_ok(dims) || !q || !k || !row_ptr || !col_idx) return DBSP_ERR_INVALID_ARG;
  if (mode != DBSP_TOPK && mode != DBSP_MASS) return DBSP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k)) return DBSP_ERR_INVALID_ARG;
  if (!(isfinite(score_scale))) return DBSP_ERR_INVALID_ARG;
  if (!dtype_supported(dims)) return DBSP_ERR_UNSUPPORTED;
  if ((q_strides && !strides_ok(q_strides, dims, false)) ||
      (k_strides && !strides_ok(k_strides, dims, false)))
    return DBSP_ERR_INVALID_ARG;
  const int32_t nkb = nkb_of(dims);
  const int32_t nqb = nqb_of(dims);
  if (nkb > DBSP_MAX_KEY_BLOCKS) return DBSP_ERR_UNSUPPORTED;
  const dbsp::Strides qs = q_strides ? to_strides(q_strides) : contiguous(dims, dims->lq);
  const dbsp::Strides ks = k_strides ? to_strides(k_strides) : contiguous(dims, dims->lk);
  ForcedSet fs;
  if (fs_in) {
    fs = *fs_in;
  } else {
    const int32_t st = forced_from_ranges(nkb, text_blocks, dense_extra_blocks, &fs);
    if (st != DBSP_OK) return st;
  }
  int64_t bound;
  int32_t st = nnz_bound_f(dims, mode, density_or_mass, fs, topk_override, &bound);
  if (st != DBSP_OK) return st;
  if (bound > INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  if (col_capacity < bound) return DBSP_ERR_CAPACITY;
  const WorkspaceLayout wl = layout_of(dims, mode);
  if (!workspace || workspace_bytes < wl.total || ((uintptr_t)workspace & 255u))
    return DBSP_ERR_WORKSPACE;

  char* ws = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t bh = (int64_t)dims->batch * dims->heads;
  uint16_t* ksplit = reinterpret_cast<uint16_t*>(ws + wl.kbar);
  const bool bf16 = dims->dtype == DBSP_BF16;
  if (dbsp::launch_pool(k, ks, dims->heads, ksplit, bh, nkb, dims->lk, dims->head_dim, bf16, s) !=
      hipSuccess)
    return DBSP_ERR_HIP;

  dbsp::SelectArgs a{};
  a.q = q;
  a.qs = qs;
  a.heads = dims->heads;
  a.ksplit = ksplit;
  a.nqb = nqb;
  a.nkb = nkb;
  a.lq = dims->lq;
  a.lk = dims->lk;
  a.scale = score_scale > 0.f ? score_scale : (float)(1.0 / sqrt((double)dims->head_dim));
  apply_forced(fs, &a);
  a.mode = mode;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_capacity = col_capacity;
  a.scores_out = scores_out;
  a.lds_stride = score_lds_stride(nkb);
  a.n_rows = bh * nqb;
  if (mode == DBSP_TOPK) {
    int32_t kk;
    topk_k_f(dims, density_or_mass, fs, topk_override, &kk);
    a.kk = kk;
    a.per_row = fs.count + kk;
  } else {
    a.keep_all = density_or_mass >= 1.0;
    a.theta = (uint64_t)ceil(density_or_mass * 4611686018427387904.0);  // tau * 2^62
    a.counts = reinterpret_cast<int32_t*>(ws + wl.counts);
    a.masks = reinterpret_cast<uint64_t*>(ws + wl.masks);
    a.words = (nkb + 63) / 64;
  }
  if (dbsp::launch_select(a, bh, dims->head_dim, bf16, s) != hipSuccess) return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_sparse_select(const void* q, const void* k, const dbsp_dims* dims,
                           dbsp_range text_blocks, dbsp_range dense_extra_blocks, int32_t mode,
                           double density_or_mass, int32_t topk_override, float score_scale,
                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                           float* scores_out, void* workspace, uint64_t workspace_bytes,
                           void* stream) {
  return sparse_select_impl(q, k, dims, nullptr, nullptr, nullptr, text_blocks,
                            dense_extra_blocks, mode, density_or_mass, topk_override, score_scale,
                            row_ptr, col_idx, col_capacity, scores_out, workspace,
                            workspace_bytes, stream);
}

int32_t dbsp_sparse_select_noalloc(const void* q, const void* k, const dbsp_dims* dims,
                                   dbsp_range text_blocks, dbsp_range dense_extra_blocks,
                                   int32_t mode, double density_or_mass, int32_t topk_override,
                                   float score_scale, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, float* scores_out, void* stream) {
  // the size check comes first, so a shape too large for the static scratch is refused before
  // anything touches the GPU
  if (!shape_ok(dims) || (mode != DBSP_TOPK && mode != DBSP_MASS)) return DBSP_ERR_INVALID_ARG;
  if (layout_of(dims, mode).total > (uint64_t)DBSP_NOALLOC_SCRATCH_BYTES)
    return DBSP_ERR_WORKSPACE;
  void* ws = nullptr;
  const int32_t st = noalloc_scratch(stream, &ws);
  if (st != DBSP_OK) return st;
  return sparse_select_impl(q, k, dims, nullptr, nullptr, nullptr, text_blocks,
                            dense_extra_blocks, mode, density_or_mass, topk_override, score_scale,
                            row_ptr, col_idx, col_capacity, scores_out, ws,
                            (uint64_t)DBSP_NOALLOC_SCRATCH_BYTES, stream);
}

int32_t dbsp_sparse_select_strided(const void* q, const dbsp_strides* q_strides, const void* k,
                                   const dbsp_strides* k_strides, const dbsp_dims* dims,
                                   dbsp_range text_blocks, dbsp_range dense_extra_blocks,
                                   int32_t mode, double density_or_mass, int32_t topk_override,
                                   float score_scale, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, float* scores_out, void* workspace,
                                   uint64_t workspace_bytes, void* stream) {
  if (!q_strides || !k_strides) return DBSP_ERR_INVALID_ARG;
  return sparse_select_impl(q, k, dims, q_strides, k_strides, nullptr, text_blocks,
                            dense_extra_blocks, mode, density_or_mass, topk_override, score_scale,
                            row_ptr, col_idx, col_capacity, scores_out, workspace,
                            workspace_bytes, stream);
}

int32_t dbsp_sparse_select_list(const void* q, const void* k, const dbsp_dims* dims,
                                const int32_t* forced_blocks, int32_t n_forced, int32_t mode,
                                double density_or_mass, int32_t topk_override, float score_scale,
                                int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                float* scores_out, void* workspace, uint64_t workspace_bytes,
                                void* stream) {
  if (!shape_ok(dims)) return DBSP_ERR_INVALID_ARG;
  ForcedSet fs;
  const int32_t st = forced_from_list(nkb_of(dims), forced_blocks, n_forced, &fs);
  if (st != DBSP_OK) return st;
  return sparse_select_impl(q, k, dims, nullptr, nullptr, &fs, dbsp_range{0, 0},
                            dbsp_range{0, 0}, mode,
                            density_or_mass, topk_override, score_scale, row_ptr, col_idx,
                            col_capacity, scores_out, workspace, workspace_bytes, stream);
}

static int32_t attn_impl(const void* q, const dbsp_strides* q_strides, const void* k,
                         const dbsp_strides* k_strides, const void* v,
                         const dbsp_strides* v_strides, const dbsp_dims* dims,
                         const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                         float softmax_scale, void* o, const dbsp_strides* o_strides,
                         int32_t o_dtype, float* lse_out, const int32_t* row_order,
                         void* stream) {
  if (!shape_ok(dims) || !q || !k || !v || !row_ptr || !o) return DBSP_ERR_INVALID_ARG;
  if (col_capacity < 0 || (col_capacity > 0 && !col_idx)) return DBSP_ERR_INVALID_ARG;
  if (o_dtype != DBSP_F32 && o_dtype != DBSP_BF16) return DBSP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return DBSP_ERR_INVALID_ARG;
  if (!(isfinite(softmax_scale))) return DBSP_ERR_INVALID_ARG;
  if ((q_strides && !strides_ok(q_strides, dims, false)) ||
      (k_strides && !strides_ok(k_strides, dims, false)) ||
      (v_strides && !strides_ok(v_strides, dims, false)))
    return DBSP_ERR_INVALID_ARG;
  if (o_strides) {
    // O is written in o_dtype: rows must hold head_dim elements and stay 16-byte aligned
    dbsp_dims od = *dims;
    od.dtype = o_dtype;
    if (!strides_ok(o_strides, &od, true)) return DBSP_ERR_INVALID_ARG;
  }
  if (!attn_supported(dims)) return DBSP_ERR_UNSUPPORTED;
  const dbsp::Strides ks = k_strides ? to_strides(k_strides) : contiguous(dims, dims->lk);
  const dbsp::Strides vs = v_strides ? to_strides(v_strides) : contiguous(dims, dims->lk);
  if (dims->dtype == DBSP_BF16) {
    if (nkb_of(dims) > kMaxBf16KeyBlocks) return DBSP_ERR_UNSUPPORTED;
    // a head's K and V are addressed with 32-bit byte offsets
    const int64_t span = ((int64_t)nkb_of(dims) * DBSP_BLOCK) * 2;
    if (span * ks.t > INT32_MAX || span * vs.t > INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  }
  const float scale = softmax_scale > 0.f ? softmax_scale
                                          : (float)(1.0 / sqrt((double)dims->head_dim));
  dbsp::AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.qs = q_strides ? to_strides(q_strides) : contiguous(dims, dims->lq);
  a.ks = ks;
  a.vs = vs;
  a.os = o_strides ? to_strides(o_strides) : contiguous(dims, dims->lq);
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_capacity = col_capacity;
  a.heads = dims->heads;
  a.nqb = nqb_of(dims);
  a.nkb = nkb_of(dims);
  a.lq = dims->lq;
  a.lk = dims->lk;
  a.rows = rows_of(dims);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o = o;
  a.o_bf16 = o_dtype == DBSP_BF16;
  a.lse = lse_out;
  a.row_order = row_order;
  if (dbsp::launch_attn(a, dims->head_dim, dims->dtype == DBSP_BF16,
                        static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_sparse_attn_fwd(const void* q, const void* k, const void* v, const dbsp_dims* dims,
                             const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                             float softmax_scale, void* o, int32_t o_dtype, float* lse_out,
                             void* stream) {
  return attn_impl(q, nullptr, k, nullptr, v, nullptr, dims, row_ptr, col_idx, col_capacity,
                   softmax_scale, o, nullptr, o_dtype, lse_out, nullptr, stream);
}

int32_t dbsp_sparse_attn_fwd_ordered(const void* q, const void* k, const void* v,
                                     const dbsp_dims* dims, const int32_t* row_ptr,
                                     const int32_t* col_idx, int64_t col_capacity,
                                     float softmax_scale, void* o, int32_t o_dtype,
                                     float* lse_out, const int32_t* row_order, void* stream) {
  if (!row_order) return DBSP_ERR_INVALID_ARG;
  return attn_impl(q, nullptr, k, nullptr, v, nullptr, dims, row_ptr, col_idx, col_capacity,
                   softmax_scale, o, nullptr, o_dtype, lse_out, row_order, stream);
}

int32_t dbsp_row_order_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes) {
  if (!shape_ok(dims) || !bytes) return DBSP_ERR_INVALID_ARG;
  // one int32 count per (batch, head, kept count) bucket (256-byte aligned), then one cursor per
  // bucket and the total
  const uint64_t nb = (uint64_t)dims->batch * (uint64_t)dims->heads * ((uint64_t)nkb_of(dims) + 1);
  *bytes = ((4 * nb + 255) & ~(uint64_t)255) + 4 * (nb + 1);
  return DBSP_OK;
}

int32_t dbsp_row_order_lpt(const int32_t* row_ptr, const dbsp_dims* dims, int64_t col_capacity,
                           int32_t* order, void* workspace, uint64_t workspace_bytes,
                           void* stream) {
  if (!shape_ok(dims) || !row_ptr || !order || col_capacity < 0) return DBSP_ERR_INVALID_ARG;
  if (rows_of(dims) > INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  uint64_t need = 0;
  dbsp_row_order_workspace_bytes(dims, &need);
  if (!workspace || workspace_bytes < need || ((uintptr_t)workspace & 255))
    return DBSP_ERR_WORKSPACE;
  const uint64_t nb = (uint64_t)dims->batch * (uint64_t)dims->heads * ((uint64_t)nkb_of(dims) + 1);
  int32_t* counts = static_cast<int32_t*>(workspace);
  int32_t* cursor = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) +
                                               ((4 * nb + 255) & ~(uint64_t)255));
  if (dbsp::launch_row_order_lpt(row_ptr, col_capacity, rows_of(dims), nqb_of(dims),
                                 nkb_of(dims), order, counts, cursor,
                                 static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_sparse_attn_fwd_strided(const void* q, const dbsp_strides* q_strides, const void* k,
                                     const dbsp_strides* k_strides, const void* v,
                                     const dbsp_strides* v_strides, const dbsp_dims* dims,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_capacity, float softmax_scale, void* o,
                                     const dbsp_strides* o_strides, int32_t o_dtype,
                                     float* lse_out, void* stream) {
  if (!q_strides || !k_strides || !v_strides || !o_strides) return DBSP_ERR_INVALID_ARG;
  return attn_impl(q, q_strides, k, k_strides, v, v_strides, dims, row_ptr, col_idx,
                   col_capacity, softmax_scale, o, o_strides, o_dtype, lse_out, nullptr, stream);
}

int32_t dbsp_block_energy_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes) {
  if (!shape_ok(dims) || !bytes) return DBSP_ERR_INVALID_ARG;
  if (!attn_supported(dims) || nkb_of(dims) > DBSP_MAX_KEY_BLOCKS) return DBSP_ERR_UNSUPPORTED;
  const int64_t rows = rows_of(dims);
  *bytes = dims->dtype == DBSP_BF16
               ? (uint64_t)std::min<int64_t>(rows, dbsp::kEnergySlots) * energy_slot_bytes(dims)
               : 0;
  return DBSP_OK;
}

int32_t dbsp_block_energy(const void* q, const void* k, const dbsp_dims* dims, float softmax_scale,
                          float* energy, float* lse_out, void* workspace,
                          uint64_t workspace_bytes, void* stream) {
  if (!shape_ok(dims) || !q || !k || !energy) return DBSP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || ((uintptr_t)energy & 3u) || ((uintptr_t)lse_out & 3u))
    return DBSP_ERR_INVALID_ARG;
  if (!(isfinite(softmax_scale))) return DBSP_ERR_INVALID_ARG;
  if (!attn_supported(dims)) return DBSP_ERR_UNSUPPORTED;
  if (nkb_of(dims) > DBSP_MAX_KEY_BLOCKS) return DBSP_ERR_UNSUPPORTED;
  const float scale = softmax_scale > 0.f ? softmax_scale
                                          : (float)(1.0 / sqrt((double)dims->head_dim));
  dbsp::EnergyArgs a{};
  a.q = q;
  a.k = k;
  a.nqb = nqb_of(dims);
  a.nkb = nkb_of(dims);
  a.lq = dims->lq;
  a.lk = dims->lk;
  a.rows = rows_of(dims);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.energy = energy;
  a.lse = lse_out;
  if (dims->dtype == DBSP_BF16) {  // one slot per persistent workgroup, as many as fit
    const uint64_t per_slot = energy_slot_bytes(dims);
    a.slots = std::min<int64_t>(std::min<int64_t>(a.rows, dbsp::kEnergySlots),
                                (int64_t)std::min<uint64_t>(workspace_bytes / per_slot, INT64_MAX));
    if (!workspace || a.slots < 1 || ((uintptr_t)workspace & 255u)) return DBSP_ERR_WORKSPACE;
    a.ws = static_cast<float*>(workspace);
  }
  if (dbsp::launch_energy(a, dims->head_dim, dims->dtype == DBSP_BF16,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_retained_mass(const float* energy, const dbsp_dims* dims, const int32_t* row_ptr,
                           const int32_t* col_idx, int64_t col_capacity, double* mass,
                           void* stream) {
  if (!shape_ok(dims) || !energy || !row_ptr || !mass) return DBSP_ERR_INVALID_ARG;
  if (col_capacity < 0 || (col_capacity > 0 && !col_idx)) return DBSP_ERR_INVALID_ARG;
  if (dbsp::launch_retained_mass(energy, row_ptr, col_idx, col_capacity, nkb_of(dims),
                                 rows_of(dims), mass, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_select_energy_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes) {
  if (!shape_ok(dims) || !bytes) return DBSP_ERR_INVALID_ARG;
  *bytes = energy_select_layout(dims).total;
  return DBSP_OK;
}

int32_t dbsp_select_energy(const float* energy, const dbsp_dims* dims, dbsp_range text_blocks,
                           dbsp_range dense_extra_blocks, double mass, int32_t* row_ptr,
                           int32_t* col_idx, int64_t col_capacity, void* workspace,
                           uint64_t workspace_bytes, void* stream) {
  if (!shape_ok(dims) || !energy || !row_ptr || !col_idx) return DBSP_ERR_INVALID_ARG;
  const int32_t nkb = nkb_of(dims);
  if (nkb > DBSP_MAX_KEY_BLOCKS) return DBSP_ERR_UNSUPPORTED;
  int64_t bound;
  const int32_t st = nnz_bound(dims, DBSP_MASS, mass, text_blocks, dense_extra_blocks, -1, &bound);
  if (st != DBSP_OK) return st;
  if (bound > INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  if (col_capacity < bound) return DBSP_ERR_CAPACITY;
  const WorkspaceLayout wl = energy_select_layout(dims);
  if (!workspace || workspace_bytes < wl.total || ((uintptr_t)workspace & 255u))
    return DBSP_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  dbsp::SelectArgs a{};
  a.nqb = nqb_of(dims);
  a.nkb = nkb;
  ForcedSet fs;
  forced_from_ranges(nkb, text_blocks, dense_extra_blocks, &fs);  // validated by nnz_bound
  apply_forced(fs, &a);
  a.mode = DBSP_MASS;
  a.keep_all = mass >= 1.0;
  a.theta = (uint64_t)ceil(mass * 4611686018427387904.0);  // tau * 2^62
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_capacity = col_capacity;
  a.counts = reinterpret_cast<int32_t*>(ws + wl.counts);
  a.masks = reinterpret_cast<uint64_t*>(ws + wl.masks);
  a.words = (nkb + 63) / 64;
  a.n_rows = rows_of(dims);
  if (dbsp::launch_select_energy(a, energy, static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_vote_accumulate(const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                             const dbsp_dims* dims, int32_t* counts, void* stream) {
  if (!shape_ok(dims) || !row_ptr || !counts) return DBSP_ERR_INVALID_ARG;
  if (col_capacity < 0 || (col_capacity > 0 && !col_idx)) return DBSP_ERR_INVALID_ARG;
  if (dbsp::launch_vote_accumulate(row_ptr, col_idx, col_capacity, nkb_of(dims),
                                   rows_of(dims), counts, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_vote_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes) {
  if (!shape_ok(dims) || !bytes) return DBSP_ERR_INVALID_ARG;
  *bytes = energy_select_layout(dims).total;
  return DBSP_OK;
}

int32_t dbsp_vote_select(const int32_t* counts, const dbsp_dims* dims, int32_t n_inputs, double rho,
                         int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                         void* workspace, uint64_t workspace_bytes, void* stream) {
  if (!shape_ok(dims) || !counts || !row_ptr || !col_idx) return DBSP_ERR_INVALID_ARG;
  if (n_inputs < 1 || !(rho >= 0.0 && rho <= 1.0)) return DBSP_ERR_INVALID_ARG;  // rejects NaN
  const int32_t nkb = nkb_of(dims);
  if (nkb > DBSP_MAX_KEY_BLOCKS) return DBSP_ERR_UNSUPPORTED;
  const int64_t bound = rows_of(dims) * (int64_t)nkb;
  if (bound > INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  if (col_capacity < bound) return DBSP_ERR_CAPACITY;
  const WorkspaceLayout wl = energy_select_layout(dims);
  if (!workspace || workspace_bytes < wl.total || ((uintptr_t)workspace & 255u))
    return DBSP_ERR_WORKSPACE;
  char* ws = static_cast<char*>(workspace);
  dbsp::SelectArgs a{};
  a.nqb = nqb_of(dims);
  a.nkb = nkb;
  a.row_ptr = row_ptr;
  a.col_idx = col_idx;
  a.col_capacity = col_capacity;
  a.counts = reinterpret_cast<int32_t*>(ws + wl.counts);
  a.masks = reinterpret_cast<uint64_t*>(ws + wl.masks);
  a.words = (nkb + 63) / 64;
  a.n_rows = rows_of(dims);
  if (dbsp::launch_vote_select(counts, n_inputs, rho, a, static_cast<hipStream_t>(stream)) !=
      hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_anchor_workspace_bytes(const dbsp_dims* dims, int32_t frames, int32_t rows_per_frame,
                                    int32_t row_width, int32_t n_anchors, int32_t o_dtype,
                                    uint64_t* bytes) {
  if (!bytes) return DBSP_ERR_INVALID_ARG;
  AnchorLayout l;
  const int32_t st = anchor_layout(dims, frames, rows_per_frame, row_width, n_anchors, o_dtype, &l);
  if (st != DBSP_OK) return st;
  *bytes = l.total;
  return DBSP_OK;
}

int32_t dbsp_anchor_attn_fwd(const void* q, const void* k, const void* v, const dbsp_dims* dims,
                             int32_t frames, int32_t rows_per_frame, int32_t row_width,
                             int32_t n_anchors, float softmax_scale, void* o, int32_t o_dtype,
                             float* lse_out, void* workspace, uint64_t workspace_bytes,
                             void* stream) {
  if (!shape_ok(dims) || !q || !k || !v || !o) return DBSP_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) ||
      ((uintptr_t)lse_out & 3u))
    return DBSP_ERR_INVALID_ARG;
  if (!(isfinite(softmax_scale))) return DBSP_ERR_INVALID_ARG;
  AnchorLayout l;
  const int32_t st = anchor_layout(dims, frames, rows_per_frame, row_width, n_anchors, o_dtype, &l);
  if (st != DBSP_OK) return st;
  if (!attn_supported(dims)) return DBSP_ERR_UNSUPPORTED;
  if (dims->dtype == DBSP_BF16 && nkb_of(dims) > kMaxBf16KeyBlocks)
    return DBSP_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < l.total || ((uintptr_t)workspace & 255u))
    return DBSP_ERR_WORKSPACE;
  const float scale = softmax_scale > 0.f ? softmax_scale
                                          : (float)(1.0 / sqrt((double)dims->head_dim));
  char* ws = static_cast<char*>(workspace);
  dbsp::AnchorArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.qa = ws + l.qa;
  a.oa = ws + l.oa;
  a.lse_a = reinterpret_cast<float*>(ws + l.lse_a);
  a.row_ptr = reinterpret_cast<int32_t*>(ws + l.row_ptr);
  a.col_idx = reinterpret_cast<int32_t*>(ws + l.col_idx);
  a.bh = (int64_t)dims->batch * dims->heads;
  a.nkb = nkb_of(dims);
  a.lk = dims->lk;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.o = o;
  a.o_bf16 = o_dtype == DBSP_BF16;
  a.lse = lse_out;
  a.geom = l.g;
  if (dbsp::launch_anchor(a, dims->head_dim, dims->dtype == DBSP_BF16,
                          static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_skiplist_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes) {
  if (!shape_ok(dims) || !bytes) return DBSP_ERR_INVALID_ARG;
  *bytes = align256((uint64_t)rows_of(dims) * sizeof(int32_t));
  return DBSP_OK;
}

int32_t dbsp_csr_to_intervals(const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_capacity, const dbsp_dims* dims, int32_t* iv_ptr,
                              int32_t* iv, int64_t iv_capacity, void* workspace,
                              uint64_t workspace_bytes, void* stream) {
  if (!shape_ok(dims) || !row_ptr || !iv_ptr || !iv) return DBSP_ERR_INVALID_ARG;
  if (col_capacity < 0 || (col_capacity > 0 && !col_idx) || iv_capacity < 0)
    return DBSP_ERR_INVALID_ARG;
  const int64_t nkb = nkb_of(dims);
  // a row holds at most ceil(nkb / 2) maximal runs of in-range blocks
  if (iv_capacity < rows_of(dims) * ((nkb + 1) / 2)) return DBSP_ERR_CAPACITY;
  if (!workspace || workspace_bytes < (uint64_t)rows_of(dims) * sizeof(int32_t) ||
      ((uintptr_t)workspace & 255u))
    return DBSP_ERR_WORKSPACE;
  if (dbsp::launch_csr_to_intervals(row_ptr, col_idx, col_capacity, (int)nkb, rows_of(dims),
                                    iv_ptr, iv, iv_capacity, static_cast<int32_t*>(workspace),
                                    static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

int32_t dbsp_intervals_to_csr(const int32_t* iv_ptr, const int32_t* iv, int64_t iv_capacity,
                              const dbsp_dims* dims, int32_t* row_ptr, int32_t* col_idx,
                              int64_t col_capacity, void* workspace, uint64_t workspace_bytes,
                              void* stream) {
  if (!shape_ok(dims) || !iv_ptr || !row_ptr || !col_idx) return DBSP_ERR_INVALID_ARG;
  if (iv_capacity < 0 || (iv_capacity > 0 && !iv) || col_capacity < 0)
    return DBSP_ERR_INVALID_ARG;
  const int64_t nkb = nkb_of(dims);
  const int64_t bound = rows_of(dims) * nkb;  // disjoint intervals of a row cover at most nkb
  if (bound > INT32_MAX) return DBSP_ERR_UNSUPPORTED;
  if (col_capacity < bound) return DBSP_ERR_CAPACITY;
  if (!workspace || workspace_bytes < (uint64_t)rows_of(dims) * sizeof(int32_t) ||
      ((uintptr_t)workspace & 255u))
    return DBSP_ERR_WORKSPACE;
  if (dbsp::launch_intervals_to_csr(iv_ptr, iv, iv_capacity, (int)nkb, rows_of(dims), row_ptr,
                                    col_idx, col_capacity, static_cast<int32_t*>(workspace),
                                    static_cast<hipStream_t>(stream)) != hipSuccess)
    return DBSP_ERR_HIP;
  return DBSP_OK;
}

}  // extern "C"
