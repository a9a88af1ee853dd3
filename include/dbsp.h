/*
 * dbsp.h - C ABI of libdbsp.so: per-head dynamic block-sparse attention on gfx950 (MI355X).
 *
 * The hot path is two calls:
 *
 *   dbsp_sparse_select    Q, K -> for every (batch, head, query block) the key blocks to attend,
 *                         as a forward-only CSR skip list.
 *   dbsp_sparse_attn_fwd  Q, K, V, CSR -> O (and optionally the log-sum-exp), attending only
 *                         to the tokens of the kept key blocks.
 *
 * Beside it, the token-level quantities the pages measure masks with:
 *
 *   dbsp_block_energy     Q, K -> the token-level energy of every (query block, key block) pair.
 *   dbsp_retained_mass    energy, CSR -> the attention mass each row's mask keeps.
 *   dbsp_select_energy    energy -> a CSR by the cumulative-mass rule on token-level energies.
 *   dbsp_vote_accumulate, dbsp_vote_select
 *                         masks of several calibration inputs -> one static CSR by vote.
 *   dbsp_anchor_attn_fwd  the alternative path of spatially repeating heads: attention for a few
 *                         anchor rows per frame, broadcast to the nearest rows.
 *   dbsp_csr_to_intervals, dbsp_intervals_to_csr
 *                         the skip list as contiguous key-block intervals, and back.
 *
 * What the calls compute follows two pages:
 *   [SparSTAR] "SparSTAR: Sparse Attention for SpaceTime AutoRegressive Video Synthesis", in the
 *       pchao.org digest titled "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", section
 *       "方法概览" (method overview): 128-token blocks, mean-pooled Q and K per block, a pooled
 *       compatibility score per block pair, clip-aware dense segments (text; in the first clip
 *       also the image pyramid), a joint Top-K over the remaining key blocks, per-head masks,
 *       and a forward-only sparse attention path that builds no backward index.
 *   [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse Attention"
 *       (papernotes.org), key design 1 with Eq. (5) (block energy; keep the shortest prefix of
 *       the energy-sorted row that reaches a threshold, restored to the original order) and
 *       key design 4 (a read-only per-query-block list of key blocks consumed by the kernel).
 *
 * Conventions shared by every call
 *   Layout     Q is [batch, heads, lq, head_dim]; K and V are [batch, heads, lk, head_dim];
 *              all contiguous row-major and 16-byte aligned (the *_strided calls take other
 *              layouts, e.g. [batch, L, heads, head_dim]). lq, lk >= 1.
 *              Block i of a sequence is tokens [128 i, min(128 i + 128, L)): a length that is
 *              not a multiple of 128 ends in a partial block, which pools to the mean of the
 *              tokens it holds and contributes only those tokens to attention and energies
 *              (queries past the end are not written). There are ceil(L / 128) blocks; every
 *              "lk / 128" below means that count.
 *   Rows       CSR row r = (b * heads + h) * (lq / 128) + i for batch b, head h, query block i.
 *              col_idx of a row lists key-block indices in strictly ascending order.
 *   Types      dtype DBSP_BF16 (head_dim 128) or DBSP_F32 (head_dim 64 or 128).
 *   Memory     The caller allocates every buffer (inputs, outputs, CSR, workspace) in device
 *              memory. The library allocates nothing, frees nothing, keeps no state between
 *              calls and never writes its inputs. Calls on different streams with disjoint
 *              output and workspace buffers may overlap. (The one exception is
 *              dbsp_sparse_select_noalloc, whose scratch is a static device array per GPU.)
 *   Streams    `stream` is a hipStream_t (NULL = the null stream). Calls enqueue work and return
 *              without waiting for it. nnz is left on the device in row_ptr[rows].
 *   Errors     Every argument check runs on the host before anything is launched; a negative
 *              status is returned and no output is touched. DBSP_ERR_HIP reports a failed
 *              launch. Non-finite input values are not checked: masks and outputs are then
 *              unspecified. Kernels never read or write outside the buffers described here,
 *              even for malformed CSR contents (out-of-range column entries are skipped and row
 *              extents are clipped to col_capacity).
 */
#ifndef DBSP_H
#define DBSP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DBSP_BLOCK 128          /* tokens per block ([SparSTAR] method overview)          */
#define DBSP_MAX_KEY_BLOCKS 2048 /* largest lk / 128 supported by dbsp_sparse_select        */

enum {
  DBSP_OK = 0,
  DBSP_ERR_INVALID_ARG = -1, /* null pointer, bad shape, range or parameter                  */
  DBSP_ERR_UNSUPPORTED = -2, /* valid request this build does not implement                  */
  DBSP_ERR_CAPACITY = -3,    /* col_capacity below the bound from dbsp_select_nnz_bound      */
  DBSP_ERR_WORKSPACE = -4,   /* workspace missing or smaller than dbsp_select_workspace_bytes */
  DBSP_ERR_HIP = -5          /* a HIP launch failed                                          */
};

enum { DBSP_F32 = 0, DBSP_BF16 = 1 };  /* element types                                      */
enum { DBSP_TOPK = 0, DBSP_MASS = 1 }; /* selection rules                                    */

/* Half-open range [begin, end) of key-block indices; empty when begin == end. */
typedef struct dbsp_range {
  int32_t begin;
  int32_t end;
} dbsp_range;

/* Problem shape. dtype is DBSP_F32 or DBSP_BF16 and applies to Q, K and V. */
typedef struct dbsp_dims {
  int32_t batch;
  int32_t heads;
  int32_t lq;
  int32_t lk;
  int32_t head_dim;
  int32_t dtype;
} dbsp_dims;

/* Element strides of a [batch, heads, tokens, head_dim] view whose head_dim elements are
 * contiguous: token (b, h, t) starts at element b * batch + h * head + t * token. Contiguous
 * tensors are {heads * L * head_dim, L * head_dim, head_dim}; a [batch, L, heads, head_dim]
 * tensor is {L * heads * head_dim, head_dim, heads * head_dim}. Used by the *_strided calls. */
typedef struct {
  int64_t batch;
  int64_t head;
  int64_t token;
} dbsp_strides;

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t dbsp_version(void);

/* Human-readable text for a status code; never NULL, static storage. */
const char* dbsp_status_string(int32_t status);

/*
 * Number of kept key blocks per row in Top-K mode for a given density: the forced blocks plus
 * K = min(|C|, ceil(density * |C|)) candidates, |C| = lk / 128 minus the forced count
 * ([SparSTAR] decreasing density schedule: a density is the kept fraction of the blocks that
 * are not forced). topk_override >= 0 replaces K (must be <= |C|). Host only.
 * Writes K to *k_out. Returns DBSP_ERR_INVALID_ARG for a density outside [0, 1], bad ranges or
 * an override above |C|.
 */
int32_t dbsp_topk_budget(const dbsp_dims* dims, double density, dbsp_range text_blocks,
                         dbsp_range dense_extra_blocks, int32_t topk_override, int32_t* k_out);

/*
 * Upper bound on nnz for dbsp_sparse_select: exact (rows * (forced + K)) in DBSP_TOPK mode and
 * rows * (lk / 128) in DBSP_MASS mode. col_idx must hold at least this many entries. Host only.
 */
int32_t dbsp_select_nnz_bound(const dbsp_dims* dims, int32_t mode, double density_or_mass,
                              dbsp_range text_blocks, dbsp_range dense_extra_blocks,
                              int32_t topk_override, int64_t* nnz_bound);

/* Bytes of device workspace dbsp_sparse_select needs for this shape and mode. Host only. */
int32_t dbsp_select_workspace_bytes(const dbsp_dims* dims, int32_t mode, uint64_t* bytes);

/*
 * Selection ([SparSTAR] method overview; [CalibAtt] key design 1).
 *
 * For every (batch, head):
 *   1. qbar_i = mean of the 128 query vectors of block i; kbar_c likewise for key block c.
 *   2. S_ic = (qbar_i . kbar_c) * score_scale (score_scale <= 0 means 1 / sqrt(head_dim)).
 *   3. F = text_blocks U dense_extra_blocks is kept in every row (clip-aware retention: text
 *      always; in the first clip also the image-pyramid range; pass an empty range otherwise).
 *   4a. DBSP_TOPK: keep K more blocks of C = (all \ F) with the largest S_ic; K comes from
 *       density_or_mass in [0, 1] as in dbsp_topk_budget. Equal scores go to the lower block
 *       index; -0.0 equals +0.0.
 *   4b. DBSP_MASS: p_ic = softmax over all key blocks c of S_ic (fp32). With fixed-point masses
 *       u = floor(p * 2^62) and threshold ceil(tau * 2^62), tau = density_or_mass in (0, 1]:
 *       F counts first, then candidates are added in (p descending, index ascending) order
 *       until the sum reaches the threshold; if it never does, every block is kept; tau = 1
 *       keeps every block.
 *   5. row_ptr [rows + 1] (int32, device) receives the exclusive prefix of the per-row counts;
 *      col_idx [col_capacity] (int32, device) the kept blocks of each row, ascending.
 *
 * scores_out, if not NULL, is a device float32 [rows, lk / 128] buffer that receives the exact
 * values the selection compared: S in Top-K mode and p in mass mode.
 * workspace must be device memory of at least dbsp_select_workspace_bytes bytes, 256-byte
 * aligned; its contents on entry do not matter.
 * Limits: lk / 128 <= DBSP_MAX_KEY_BLOCKS; the nnz bound must fit in int32.
 */
int32_t dbsp_sparse_select(const void* q, const void* k, const dbsp_dims* dims,
                           dbsp_range text_blocks, dbsp_range dense_extra_blocks, int32_t mode,
                           double density_or_mass, int32_t topk_override, float score_scale,
                           int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                           float* scores_out, void* workspace, uint64_t workspace_bytes,
                           void* stream);

/*
 * dbsp_sparse_select with the forced set F given as an explicit list of key-block indices
 * instead of two ranges (the pages' forced segments are contiguous; a list covers any other
 * layout of conditioning blocks). forced_blocks is HOST memory holding n_forced distinct
 * indices in [0, lk / 128), in any order; it is read before the call returns (the set travels
 * to the kernels in their launch arguments, so nothing is copied to the device). Everything
 * else is as dbsp_sparse_select with F = the listed blocks.
 * Errors: DBSP_ERR_INVALID_ARG for a negative count, a NULL list with n_forced > 0, an index out
 * of range or a duplicate; otherwise as dbsp_sparse_select.
 */
int32_t dbsp_sparse_select_list(const void* q, const void* k, const dbsp_dims* dims,
                                const int32_t* forced_blocks, int32_t n_forced, int32_t mode,
                                double density_or_mass, int32_t topk_override, float score_scale,
                                int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                                float* scores_out, void* workspace, uint64_t workspace_bytes,
                                void* stream);

/*
 * dbsp_sparse_select without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc). It allocates nothing and frees nothing: its scratch (the pooled keys; in
 * DBSP_MASS mode also per-row counts and bitmasks) lives in a static device array of
 * DBSP_NOALLOC_SCRATCH_BYTES bytes, one copy per GPU, held from the library's first use on that
 * GPU until the process ends; its address is looked up once per device on the first call.
 * Every argument and result is as dbsp_sparse_select; the caller still passes the CSR and
 * scores_out buffers. No scratch content needs to be zero on entry; each call leaves its own.
 * Calls that overlap in time on one GPU (different streams or host threads) share that
 * scratch and race: serialise them, or use dbsp_sparse_select with a workspace per stream.
 * The stream must belong to the current device (NULL = the null stream of the current device).
 * Errors: as dbsp_sparse_select, plus DBSP_ERR_WORKSPACE when the shape needs more scratch than
 * DBSP_NOALLOC_SCRATCH_BYTES (dbsp_select_workspace_bytes gives the need; it is checked before
 * any GPU work), DBSP_ERR_INVALID_ARG for a stream of another device, DBSP_ERR_HIP when the
 * scratch address cannot be looked up.
 */
#define DBSP_NOALLOC_SCRATCH_BYTES (32u << 20) /* 32 MiB per GPU                             */
int32_t dbsp_sparse_select_noalloc(const void* q, const void* k, const dbsp_dims* dims,
                                   dbsp_range text_blocks, dbsp_range dense_extra_blocks,
                                   int32_t mode, double density_or_mass, int32_t topk_override,
                                   float score_scale, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, float* scores_out, void* stream);

/*
 * dbsp_sparse_select on strided Q and K views (dbsp_strides, in elements of the input dtype):
 * for example [batch, L, heads, head_dim] tensors, or K shared by all heads of a batch entry
 * (head stride 0). Strides must be non-negative with every token row 16-byte aligned.
 * Everything else is as dbsp_sparse_select. Errors: DBSP_ERR_INVALID_ARG for NULL or bad
 * strides; otherwise as dbsp_sparse_select.
 */
int32_t dbsp_sparse_select_strided(const void* q, const dbsp_strides* q_strides, const void* k,
                                   const dbsp_strides* k_strides, const dbsp_dims* dims,
                                   dbsp_range text_blocks, dbsp_range dense_extra_blocks,
                                   int32_t mode, double density_or_mass, int32_t topk_override,
                                   float score_scale, int32_t* row_ptr, int32_t* col_idx,
                                   int64_t col_capacity, float* scores_out, void* workspace,
                                   uint64_t workspace_bytes, void* stream);

/* dbsp_select_nnz_bound for a forced list (host memory, as dbsp_sparse_select_list). */
int32_t dbsp_select_nnz_bound_list(const dbsp_dims* dims, int32_t mode, double density_or_mass,
                                   const int32_t* forced_blocks, int32_t n_forced,
                                   int32_t topk_override, int64_t* nnz_bound_out);

/*
 * Block-sparse attention, forward only ([SparSTAR] FastFlex bullet; [CalibAtt] key design 4).
 *
 * For each CSR row r = (b, h, i) and each query t of block i:
 *   o_t   = sum over tokens j of the kept key blocks of softmax_j(q_t . k_j * softmax_scale) v_j
 *   lse_t = log(sum over the same j of exp(q_t . k_j * softmax_scale))
 * with softmax_scale <= 0 meaning 1 / sqrt(head_dim), no causal mask, and O = 0, lse = -inf
 * for a row with no kept block. Arithmetic: bf16 inputs use bf16 matrix-core products with
 * float32 accumulation and a float32 online softmax (probabilities rounded to bf16 before the
 * value product); float32 inputs use float32 throughout.
 *
 * row_ptr [rows + 1] and col_idx are device int32 arrays as produced by dbsp_sparse_select (or
 * any CSR with ascending or unordered in-range entries); entries outside [0, lk / 128) are
 * skipped and row extents are clipped to [0, col_capacity).
 * o is [batch, heads, lq, head_dim] in o_dtype (DBSP_F32 or DBSP_BF16, round to nearest even).
 * lse_out, if not NULL, is float32 [batch, heads, lq].
 * Limits: bf16 inputs need lk / 128 <= 65535 (a head's K and V are addressed with 32-bit byte
 * offsets); DBSP_ERR_UNSUPPORTED otherwise.
 */
int32_t dbsp_sparse_attn_fwd(const void* q, const void* k, const void* v, const dbsp_dims* dims,
                             const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                             float softmax_scale, void* o, int32_t o_dtype, float* lse_out,
                             void* stream);

/*
 * dbsp_sparse_attn_fwd on strided Q, K, V and O views (dbsp_strides in elements: Q, K, V in the
 * input dtype, O in o_dtype). Strides must be non-negative with every token row 16-byte
 * aligned; O's token stride must be at least head_dim (rows of different heads or batch
 * entries must not overlap either; that is not checked). lse_out stays contiguous
 * [batch, heads, lq]. bf16 inputs also need (lk rounded up to 128) * token stride * 2 bytes
 * below 2^31 for K and V. Errors as dbsp_sparse_attn_fwd, plus DBSP_ERR_INVALID_ARG for NULL
 * or bad strides.
 */
int32_t dbsp_sparse_attn_fwd_strided(const void* q, const dbsp_strides* q_strides, const void* k,
                                     const dbsp_strides* k_strides, const void* v,
                                     const dbsp_strides* v_strides, const dbsp_dims* dims,
                                     const int32_t* row_ptr, const int32_t* col_idx,
                                     int64_t col_capacity, float softmax_scale, void* o,
                                     const dbsp_strides* o_strides, int32_t o_dtype,
                                     float* lse_out, void* stream);

/*
 * dbsp_sparse_attn_fwd with workgroup b processing row row_order[b] instead of row b, e.g. the
 * longest-first order of dbsp_row_order_lpt. The order only decides which rows start first; each
 * row's O and lse are the same as without it. row_order: device int32 [rows]; it should be a
 * permutation of [0, rows): entries outside [0, rows) are skipped (their rows are not written)
 * and a repeated entry computes its row twice. DBSP_ERR_INVALID_ARG for a NULL row_order, else
 * as dbsp_sparse_attn_fwd.
 */
int32_t dbsp_sparse_attn_fwd_ordered(const void* q, const void* k, const void* v,
                                     const dbsp_dims* dims, const int32_t* row_ptr,
                                     const int32_t* col_idx, int64_t col_capacity,
                                     float softmax_scale, void* o, int32_t o_dtype,
                                     float* lse_out, const int32_t* row_order, void* stream);

/*
 * Longest-first (LPT) row order for the attention launch, per head. With the cumulative-mass
 * selection ([CalibAtt] key design 1) rows keep different numbers of key blocks; starting the
 * longest rows first keeps a long row from starting last and leaving the GPU idle at the end.
 *
 * order (device int32 [rows], written) = the CSR rows in (batch, head) order, and within each
 * (batch, head) sorted by kept count (row extents clipped to [0, col_capacity) as in
 * dbsp_sparse_attn_fwd), longest first; rows of one head with equal counts appear in an
 * unspecified order (the result is a permutation either way). Heads are not mixed, so the rows
 * running together share one or two heads' K and V in the caches. workspace: device memory of
 * at least dbsp_row_order_workspace_bytes bytes (about 8 bytes per (batch, head, kept count)),
 * 256-byte aligned, overwritten. Enqueued on stream.
 * Errors: DBSP_ERR_INVALID_ARG (NULL row_ptr / order, negative col_capacity, bad dims),
 * DBSP_ERR_WORKSPACE, DBSP_ERR_UNSUPPORTED (more than 2^31 - 1 rows), DBSP_ERR_HIP.
 */
int32_t dbsp_row_order_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes);
int32_t dbsp_row_order_lpt(const int32_t* row_ptr, const dbsp_dims* dims, int64_t col_capacity,
                           int32_t* order, void* workspace, uint64_t workspace_bytes,
                           void* stream);

/*
 * Token-level block energy ([CalibAtt] key design 1, Eq. (5)).
 *
 * For each row r = (b, h, i) and each key block c of the same (b, h):
 *   energy[r][c] = (1 / n_i) * sum over queries t of block i and keys j of block c of P_tj,
 *   n_i = the number of queries block i holds (128 unless it is a partial last block),
 *   P_tj = softmax over ALL lk keys of (q_t . k_j * softmax_scale)
 * so each row sums to 1 (up to rounding). softmax_scale <= 0 means 1 / sqrt(head_dim). The
 * attention matrix is never stored. bf16: one pass over the keys per row, keeping per query its
 * log-sum-exp and, per key block, the log of that block's sum of exponentials (in the
 * workspace); the energies follow from the two once the pass ends. float32: two passes
 * (log-sum-exp per query, then the block sums against it), no workspace. Arithmetic as
 * dbsp_sparse_attn_fwd (bf16 matrix-core products with float32 accumulation; float32 for
 * float32 inputs); sums add in a fixed order, so results are bit-reproducible.
 *
 * q, k: as for dbsp_sparse_attn_fwd (no V). energy: device float32 [rows, lk / 128].
 * lse_out, if not NULL: device float32 [batch, heads, lq], the natural-log log-sum-exp of each
 * query over all keys.
 * workspace: device memory, 256-byte aligned, contents ignored and overwritten; bf16 inputs
 * need at least lk / 128 * 512 bytes (one workgroup's slot; more slots run more workgroups at
 * once, up to the size dbsp_block_energy_workspace_bytes reports, min(rows, 512) slots); float32
 * inputs need none (NULL and 0 accepted). Calls that share a workspace must not overlap.
 * Cost: 2 * 128 * 128 * head_dim FLOP per (row, key block) pair for bf16 (the dense QK^T
 * product once), twice that for float32.
 * Errors: DBSP_ERR_INVALID_ARG for null or misaligned pointers, a bad shape or a non-finite
 * scale; DBSP_ERR_UNSUPPORTED for other dtype / head_dim pairs or lk / 128 > DBSP_MAX_KEY_BLOCKS;
 * DBSP_ERR_WORKSPACE for a missing, misaligned or too small workspace (bf16).
 */
int32_t dbsp_block_energy_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes);
int32_t dbsp_block_energy(const void* q, const void* k, const dbsp_dims* dims, float softmax_scale,
                          float* energy, float* lse_out, void* workspace,
                          uint64_t workspace_bytes, void* stream);

/*
 * Retained attention mass of a block mask ([SparSTAR] Figures 3 and 4 report it per scale and
 * clip): mass[r] = sum over the in-range entries c of CSR row r of energy[r][c], added in float64.
 * energy: device float32 [rows, lk / 128] (from dbsp_block_energy); row_ptr / col_idx /
 * col_capacity as for dbsp_sparse_attn_fwd (entries outside [0, lk / 128) skipped, extents
 * clipped); mass: device float64 [rows]. Duplicate entries count twice.
 * Errors: DBSP_ERR_INVALID_ARG for null pointers, a bad shape or a negative capacity.
 */
int32_t dbsp_retained_mass(const float* energy, const dbsp_dims* dims, const int32_t* row_ptr,
                           const int32_t* col_idx, int64_t col_capacity, double* mass,
                           void* stream);

/*
 * Token-level mass-mode selection: the cumulative-mass rule of dbsp_sparse_select's DBSP_MASS
 * mode ([CalibAtt] key design 1: keep the shortest prefix of the energy-sorted row that reaches
 * the threshold, back in index order) applied to given block probabilities, such as the token-level
 * energies of dbsp_block_energy, instead of the pooled-score softmax. Step 4b of
 * dbsp_sparse_select with p_ic = energy[r][c] (fixed-point masses floor(p * 2^62), forced
 * blocks first, ties to the lower index, keep all if the row never reaches tau, tau = 1 keeps
 * all); step 5 for the output. energy: device float32 [rows, lk / 128], values in [0, 1]
 * and each row summing to at most 2 (any row of probabilities, rounding included, does: the
 * fixed-point row sums are then below 2^63 and exact in 64 bits; rows above that bound are not
 * checked and give an unspecified mask, never an access outside the buffers).
 * workspace: at least dbsp_select_energy_workspace_bytes bytes of device memory, 256-byte
 * aligned. The nnz bound is rows * (lk / 128) (dbsp_select_nnz_bound in DBSP_MASS mode).
 * Errors: as dbsp_sparse_select (ranges, tau in (0, 1], capacity, workspace); DBSP_ERR_UNSUPPORTED
 * for lk / 128 > DBSP_MAX_KEY_BLOCKS or an nnz bound above INT32_MAX.
 */
int32_t dbsp_select_energy(const float* energy, const dbsp_dims* dims, dbsp_range text_blocks,
                           dbsp_range dense_extra_blocks, double mass, int32_t* row_ptr,
                           int32_t* col_idx, int64_t col_capacity, void* workspace,
                           uint64_t workspace_bytes, void* stream);

/* Workspace bytes dbsp_select_energy needs for dims (per-row counts and kept bitmasks). */
int32_t dbsp_select_energy_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes);

/*
 * Cross-input vote ([CalibAtt] key design 2, Eq. (8) and the description of Eq. (9)): the masks
 * chosen for each calibration input are averaged element-wise and a block is kept when its keep
 * frequency is at least rho; the result is one static CSR reused for new inputs (key design 4).
 *
 * dbsp_vote_accumulate adds one input's mask: counts[r][c] += 1 for every in-range entry c of
 * CSR row r (row_ptr / col_idx / col_capacity as for dbsp_sparse_attn_fwd; entries of a row
 * must be distinct, as every CSR this library writes is). counts: device int32 [rows, lk / 128],
 * zero-filled by the caller before the first input. Calls on one counts buffer must not overlap.
 *
 * dbsp_vote_select writes the CSR of {(r, c) : counts[r][c] / n_inputs >= rho}, the comparison
 * exact on the rational count / n_inputs against the double rho, in [0, 1]; rows ascending as
 * in dbsp_sparse_select step 5. The nnz bound is rows * (lk / 128); workspace: at least
 * dbsp_vote_workspace_bytes bytes, 256-byte aligned. The page's worked example: rho = 0.5 with
 * 64 inputs keeps the blocks counted 32 times or more.
 * Errors: DBSP_ERR_INVALID_ARG for null pointers, a bad shape, n_inputs < 1 or rho outside
 * [0, 1]; DBSP_ERR_CAPACITY, DBSP_ERR_WORKSPACE and DBSP_ERR_UNSUPPORTED as dbsp_select_energy.
 */
int32_t dbsp_vote_accumulate(const int32_t* row_ptr, const int32_t* col_idx, int64_t col_capacity,
                             const dbsp_dims* dims, int32_t* counts, void* stream);
int32_t dbsp_vote_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes);
int32_t dbsp_vote_select(const int32_t* counts, const dbsp_dims* dims, int32_t n_inputs, double rho,
                         int32_t* row_ptr, int32_t* col_idx, int64_t col_capacity,
                         void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * Interval skip list ([CalibAtt] key design 4: the mask of each query block is stored as the
 * contiguous intervals of key blocks it needs, loaded read-only before generation).
 *
 * dbsp_csr_to_intervals encodes a CSR (as written by dbsp_sparse_select, dbsp_select_energy or
 * dbsp_vote_select: ascending, distinct entries) as maximal runs: iv_ptr [rows + 1] (device
 * int32, exclusive prefix of the run counts) and iv [n_runs][2] (device int32 pairs
 * [start, end) of key blocks, ascending). Entries outside [0, lk / 128) are skipped.
 * iv_capacity (pairs) must be at least rows * ceil((lk / 128) / 2), the most runs a mask can
 * have.
 * dbsp_intervals_to_csr decodes intervals (clipped to [0, lk / 128); those of a row must not
 * overlap) into row_ptr / col_idx; col_capacity must be at least rows * (lk / 128).
 * Both take a workspace of at least dbsp_skiplist_workspace_bytes (per-row counts), 256-byte
 * aligned. Errors: DBSP_ERR_INVALID_ARG for null pointers, a bad shape or a negative
 * capacity; DBSP_ERR_CAPACITY below the bounds above; DBSP_ERR_WORKSPACE.
 */
int32_t dbsp_skiplist_workspace_bytes(const dbsp_dims* dims, uint64_t* bytes);
int32_t dbsp_csr_to_intervals(const int32_t* row_ptr, const int32_t* col_idx,
                              int64_t col_capacity, const dbsp_dims* dims, int32_t* iv_ptr,
                              int32_t* iv, int64_t iv_capacity, void* workspace,
                              uint64_t workspace_bytes, void* stream);
int32_t dbsp_intervals_to_csr(const int32_t* iv_ptr, const int32_t* iv, int64_t iv_capacity,
                              const dbsp_dims* dims, int32_t* row_ptr, int32_t* col_idx,
                              int64_t col_capacity, void* workspace, uint64_t workspace_bytes,
                              void* stream);

/*
 * Anchor-row attention for spatially repeating heads ([CalibAtt] key design 3, spatial
 * repetition, and key design 4, the repeating-head execution path).
 *
 * The query sequence of each (batch, head) is `frames` frames of `rows_per_frame` spatial rows
 * of `row_width` tokens (token (f, r, c) at f * rows_per_frame * row_width + r * row_width + c),
 * followed by lq - frames * rows_per_frame * row_width trailing tokens in no frame. Per frame,
 * the n_anchors anchor rows a_j = floor((2 j + 1) * rows_per_frame / (2 * n_anchors)) attend to
 * all lk keys (dense softmax attention, arithmetic as dbsp_sparse_attn_fwd); every row r of the
 * frame takes the output of its nearest anchor row (smallest |r - a_j|, ties to the lower j) at
 * the same column, bit for bit; trailing tokens attend as themselves. The page's default is 5
 * anchors per frame (for a Wan 720p latent frame: 45 rows of 80 tokens).
 *
 * o: [batch, heads, lq, head_dim] in o_dtype; lse_out (nullable): float32 [batch, heads, lq],
 * each token's being its anchor's. workspace: at least dbsp_anchor_workspace_bytes for the same
 * arguments, 256-byte aligned (packed anchor queries and outputs and a dense CSR of the packed
 * query blocks).
 * Errors: DBSP_ERR_INVALID_ARG for null or misaligned pointers, a bad shape, frames, rows or
 * width < 1, n_anchors outside [1, rows_per_frame], a geometry longer than lq or a non-finite
 * scale; DBSP_ERR_UNSUPPORTED as dbsp_sparse_attn_fwd, or when the packed CSR would exceed
 * INT32_MAX entries; DBSP_ERR_WORKSPACE for a missing, small or misaligned workspace.
 */
int32_t dbsp_anchor_workspace_bytes(const dbsp_dims* dims, int32_t frames, int32_t rows_per_frame,
                                    int32_t row_width, int32_t n_anchors, int32_t o_dtype,
                                    uint64_t* bytes);
int32_t dbsp_anchor_attn_fwd(const void* q, const void* k, const void* v, const dbsp_dims* dims,
                             int32_t frames, int32_t rows_per_frame, int32_t row_width,
                             int32_t n_anchors, float softmax_scale, void* o, int32_t o_dtype,
                             float* lse_out, void* workspace, uint64_t workspace_bytes,
                             void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DBSP_H */
