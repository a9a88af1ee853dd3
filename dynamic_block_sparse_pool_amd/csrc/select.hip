// Pooled block scores, clip-aware forced blocks, Top-K / cumulative-mass selection and the CSR
// skip list.
//
// Sources: [SparSTAR] "SparSTAR：为什么视频自回归的稀疏注意力不能跨尺度复用？", method overview
// (aggregated block scores, clip-aware dense segments, joint Top-K per head and query block,
// forward-only index); [CalibAtt] "Accelerating Text-to-Video Generation with Calibrated Sparse
// Attention", key design 1 and Eq. (5) (shortest energy-sorted prefix reaching a threshold,
// restored to block order) and key design 4 (per-query-block skip list).
//
// score_select_kernel: one workgroup (8 waves) owns a tile of 16 (or, in the last generation
// of workgroups, 8) consecutive query blocks of one (batch, head); see select_tiling.
//   Phase 0 mean-pools the tile's query blocks straight from Q (the pooling kernel handles the
//   keys, which every workgroup of the head needs before it can score). Streaming Q here lets
//   the query traffic overlap the latency-bound scoring and selection of other workgroups.
//   Phase 1 computes S = qbar kbar^T * scale for the tile's rows against every key block with
//   16x16x32 bf16 MFMAs on the hi/lo split of the pooled vectors written by the pooling kernel
//   (x = hi + lo; S ~ hi.hi + hi.lo + lo.hi accumulated in fp32, relative error near 2^-16 of
//   |qbar||kbar|). Pooled keys arrive in MFMA operand order, so each operand load is one
//   contiguous 1 KiB read per wave. Each wave walks key tiles of 16 with the next tile's
//   operands in flight, and parks the scores in LDS.
//   Phase 2 gives each wave up to two rows. A wave holds one row in registers (lane l, slot e -> key
//   block 64 e + l), maps scores to order-preserving uint32 keys and finds the selection
//   threshold T most significant bits first: in Top-K mode by radix select on bytes with a
//   per-wave LDS histogram (stopping when a bucket holds exactly the remaining count), in mass
//   mode by radix search on bytes with a per-wave LDS histogram of 64-bit fixed-point masses,
//   starting at the first byte where the smallest and largest candidate keys differ (T lies
//   between them). Keys above T are kept, and keys
//   equal to T in ascending block order until the count (Top-K) or mass (mass mode) is met:
//   the same set as the prefix of a stable (value desc, index asc) sort. Kept flags are
//   emitted slot by slot with mbcnt, so col_idx comes out ascending.
// Top-K rows all have |F| + K entries, so row_ptr is written in closed form. Mass rows vary:
// the kernel stores a per-row bitmask and count, scan_counts_kernel forms row_ptr, and
// fill_csr_kernel expands the bitmasks into col_idx.
#include "common.hpp"
#include "kernels.hpp"

namespace dbsp {

constexpr int kRowsPerWG = 16;
constexpr int kWaves = 8;
constexpr uint32_t kMassBits = 62;

// Exact floor(p * 2^62) for a non-negative finite float p < 2.
__device__ __forceinline__ uint64_t mass_units(float p) {
  const uint32_t u = __float_as_uint(p);
  const int ex = (int)((u >> 23) & 0xffu);
  if (ex == 0) return 0;  // zero or subnormal: below 2^-126, far below one unit
  const uint64_t m = (uint64_t)((u & 0x7fffffu) | 0x800000u);
  const int sh = ex - 150 + (int)kMassBits;  // p = m * 2^(ex - 150)
  if (sh >= 0) return m << sh;               // sh <= 40 for p < 2
  if (sh <= -64) return 0;
  return m >> (-sh);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7fffffffu) : ~key;
  return __uint_as_float(u);
}

// Callers pass 0 <= c < nkb <= 2048, so the word index is in range; it is uniform across a
// wave (c = 64 e + lane), so the word comes from the kernel arguments through a scalar load.
__device__ __forceinline__ bool is_forced(int c, const SelectArgs& a) {
  const bool in_ranges = (c >= a.t0 && c < a.t1) || (c >= a.e0 && c < a.e1);
  const bool in_words = (a.forced_words[c >> 6] >> (c & 63)) & 1ull;
  return a.forced_by_words ? in_words : in_ranges;
}

// The threshold lies between the smallest and largest candidate key, so it shares their
// common high bits: start from those bits and return the highest bit still to decide (-1 when
// the two keys are equal).
__device__ __forceinline__ int search_start(uint32_t kmin, uint32_t kmax, uint32_t* T) {
  const uint32_t diff = kmin ^ kmax;
  if (diff == 0) {
    *T = kmin;
    return -1;
  }
  const int hb = 31 - __builtin_clz(diff);
  *T = hb == 31 ? 0u : (kmax & ~((2u << hb) - 1u));
  return hb;
}

// Phase 0: wave w mean-pools query blocks row0 + 2 w and row0 + 2 w + 1 of this (batch, head)
// straight from Q, those below row_end (the tile's end). A token row is kChunks 16-byte chunks; lane l sums chunk l % kChunks of
// every (64 / kChunks)-th token of both blocks, with 16 loads in flight per lane (8 per block),
// and the means are stored as bf16 hi | lo in qlds [16][2][D], the form the scoring MFMAs read.
template <typename T, int D>
__device__ __forceinline__ void pool_q_rows(const SelectArgs& a, uint16_t* qlds, int bh, int row0,
                                            int row_end, int lane, int wave) {
  constexpr int kVec = 16 / (int)sizeof(T);
  constexpr int kChunks = D / kVec;
  constexpr int kRowsPerLoad = 64 / kChunks;
  constexpr int kLoads = kBlock / kRowsPerLoad;
  constexpr int kBatch = 8;
  static_assert(kLoads % kBatch == 0, "batching");
  const int chunk = lane % kChunks;
  const int r0 = lane / kChunks;
  const int rr0 = 2 * wave;
  const bool live0 = row0 + rr0 < row_end, live1 = row0 + rr0 + 1 < row_end;
  if (!live0) return;
  const int64_t first0 = (int64_t)(row0 + rr0) * kBlock;  // first token of block rr0
  const int64_t st = a.qs.t;                                // elements between tokens
  const T* src0 = static_cast<const T*>(a.q) + token_offset(a.qs, bh, a.heads, first0) +
                  (int64_t)r0 * st + chunk * kVec;
  // the second block is only read when it exists; otherwise the first is read twice
  const T* src1 = live1 ? src0 + (int64_t)kBlock * st : src0;
  // tokens held by each block (a partial last block holds fewer than 128; rows past it are
  // not read)
  const int valid0 = (int)(a.lq - first0 < kBlock ? a.lq - first0 : kBlock);
  const int64_t first1 = first0 + kBlock;
  const int valid1 = live1 ? (int)(a.lq - first1 < kBlock ? a.lq - first1 : kBlock) : valid0;
  float acc0[kVec], acc1[kVec];
#pragma unroll
  for (int e = 0; e < kVec; ++e) acc0[e] = acc1[e] = 0.f;
  auto add = [](float* acc, const u32x4& raw) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        acc[2 * w] += __uint_as_float(raw[w] << 16);
        acc[2 * w + 1] += __uint_as_float(raw[w] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int w = 0; w < 4; ++w) acc[w] += __uint_as_float(raw[w]);
    }
  };
  if (valid0 == kBlock && valid1 == kBlock) {  // uniform: whole blocks, unguarded loads
#pragma unroll 1
    for (int b = 0; b < kLoads; b += kBatch) {
      u32x4 raw0[kBatch], raw1[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t off = (int64_t)(b + i) * kRowsPerLoad * st;
        raw0[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src0 + off));
        raw1[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src1 + off));
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        add(acc0, raw0[i]);
        add(acc1, raw1[i]);
      }
    }
  } else {  // a partial last block: rows past its end are not read
#pragma unroll 1
    for (int b = 0; b < kLoads; b += kBatch) {
      u32x4 raw0[kBatch], raw1[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int row = (b + i) * kRowsPerLoad + r0;
        const int64_t off = (int64_t)(b + i) * kRowsPerLoad * st;
        raw0[i] = row < valid0
                      ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src0 + off))
                      : u32x4{0u, 0u, 0u, 0u};
        raw1[i] = row < valid1
                      ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src1 + off))
                      : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        add(acc0, raw0[i]);
        add(acc1, raw1[i]);
      }
    }
  }
#pragma unroll
  for (int off = kChunks; off < 64; off <<= 1)
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
      acc0[e] += __shfl_xor(acc0[e], off, 64);
      acc1[e] += __shfl_xor(acc1[e], off, 64);
    }
  if (lane < kChunks) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      if (j == 1 && !live1) break;
      const float* acc = j == 0 ? acc0 : acc1;
      const int valid = j == 0 ? valid0 : valid1;
      uint16_t* dst = qlds + (rr0 + j) * 2 * D + chunk * kVec;
#pragma unroll
      for (int e = 0; e < kVec; ++e) {
        const float m = valid == kBlock ? acc[e] * (1.0f / kBlock) : acc[e] / (float)valid;
        const uint32_t hi = f32_to_bf16_bits(m);
        dst[e] = (uint16_t)hi;
        dst[D + e] = (uint16_t)f32_to_bf16_bits(m - __uint_as_float(hi << 16));
      }
    }
  }
}

template <int D>
__device__ __forceinline__ void score_phase(const SelectArgs& a, float* s_lds,
                                            const uint16_t* qlds, int bh, int row0, int row_end,
                                            int lane, int wave) {
  constexpr int KSTEPS = D / 32;
  const int nkb = a.nkb;
  const int m = lane & 15;   // A row / B column inside the 16x16 tile
  const int kq = lane >> 4;  // which 8-wide k chunk of the 32
  bf16x8 qhi[KSTEPS], qlo[KSTEPS];
  {
    const bool live = row0 + m < row_end;
    const uint16_t* qrow = qlds + m * 2 * D;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      qhi[ks] = *reinterpret_cast<const bf16x8*>(qrow + ks * 32 + kq * 8);
      qlo[ks] = *reinterpret_cast<const bf16x8*>(qrow + D + ks * 32 + kq * 8);
      if (!live) {
        qhi[ks] = bf16x8{};
        qlo[ks] = bf16x8{};
      }
    }
  }
  const int ntiles = (nkb + 15) >> 4;
  // tiled operand order written by the pooling kernel: [tile][ks][hi | lo][64 lanes][8]
  const uint16_t* kbase = a.ksplit + (int64_t)bh * ntiles * KSTEPS * 2 * 512 + lane * 8;
  bf16x8 khi[KSTEPS], klo[KSTEPS];
  auto load_tile = [&](int t) {
    const uint16_t* kr = kbase + (int64_t)t * KSTEPS * 2 * 512;
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      khi[ks] = *reinterpret_cast<const bf16x8*>(kr + (2 * ks) * 512);
      klo[ks] = *reinterpret_cast<const bf16x8*>(kr + (2 * ks + 1) * 512);
    }
  };
  int t = wave;
  if (t < ntiles) load_tile(t);
  for (; t < ntiles; t += kWaves) {
    bf16x8 chi[KSTEPS], clo[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      chi[ks] = khi[ks];
      clo[ks] = klo[ks];
    }
    if (t + kWaves < ntiles) load_tile(t + kWaves);  // next tile in flight during the MFMAs
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo[ks], chi[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[ks], clo[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi[ks], chi[ks], acc, 0, 0, 0);
    }
    const int n = t * 16 + m;
    if (n < nkb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) s_lds[(kq * 4 + r) * a.lds_stride + n] = acc[r] * a.scale;
    }
  }
}

// Radix step of the Top-K threshold search. Among the candidate keys that share the already
// decided high bits `prefix` (bits above shift + 8), count them per 8-bit digit at bits
// [shift, shift + 8) in the wave's LDS histogram, then find the largest digit d for which at
// least `need` keys have digit >= d. Returns d and, via *above, how many keys have a larger
// digit and, via *bucket, how many have digit d. `hist` is this wave's 256-entry histogram;
// all calls are wave-uniform.
template <int S>
__device__ __forceinline__ int radix_digit(const uint32_t (&key)[S], uint32_t prefix, int shift,
                                           uint32_t need, uint32_t* hist, int lane,
                                           uint32_t* above, uint32_t* bucket) {
  *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_wave_barrier();
  const int hs = shift + 8;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const uint32_t k = key[e];
    const bool in = k != 0u && (hs >= 32 || (k >> hs) == (prefix >> hs));
    if (in) __hip_atomic_fetch_add(hist + ((k >> shift) & 0xffu), 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WAVEFRONT);
  }
  __builtin_amdgcn_wave_barrier();
  // lane l reads the four digits 4 (63 - l) .. 4 (63 - l) + 3, so lanes run from the highest
  // digits down and an inclusive prefix sum over lanes counts keys with digit >= 4 (63 - l)
  const int g = 63 - lane;
  const u32x4 b = *reinterpret_cast<const u32x4*>(hist + 4 * g);
  const uint32_t t = b[0] + b[1] + b[2] + b[3];
  const uint32_t suf = wave_prefix_sum_u32(t);
  const uint32_t hi = suf - t;  // keys with a digit above 4 g + 3
  const bool here = hi < need && suf >= need;
  const uint64_t m = ballot64(here);
  const int src = (int)__builtin_ctzll(m);  // exactly one lane holds the crossing digit
  int d;
  uint32_t a, n;
  if (hi + b[3] >= need) { d = 3; a = hi; n = b[3]; }
  else if (hi + b[3] + b[2] >= need) { d = 2; a = hi + b[3]; n = b[2]; }
  else if (hi + b[3] + b[2] + b[1] >= need) { d = 1; a = hi + b[3] + b[2]; n = b[1]; }
  else { d = 0; a = hi + b[3] + b[2] + b[1]; n = b[0]; }
  d = (int)lane_u32((uint32_t)(4 * g + d), src);
  *above = lane_u32(a, src);
  *bucket = lane_u32(n, src);
  return d;
}

// The top-byte step of the Top-K threshold search without LDS atomics. Candidate keys of a row
// tend to share one to three top bytes (sign and high exponent bits), which makes a 256-bin
// histogram of them collide on a few bins. Walking down from the largest top byte present, count
// the keys with that byte by ballots until the running count reaches `need`: the same digit,
// count above and bucket size as radix_digit at shift 24. Gives up (returns false) after
// kTopWalk bytes, leaving the histogram to decide.
constexpr int kTopWalk = 4;

template <int S>
__device__ __forceinline__ bool top_byte_walk(const uint32_t (&key)[S], uint32_t need, int* digit,
                                              uint32_t* above, uint32_t* bucket) {
  uint32_t acc = 0;
  uint32_t bound = 257;  // digits below this are still to visit (+1 encoding: 0 = none)
#pragma unroll 1
  for (int it = 0; it < kTopWalk; ++it) {
    uint32_t mx = 0;
#pragma unroll
    for (int e = 0; e < S; ++e) {
      const uint32_t d1 = (key[e] >> 24) + 1u;
      if (key[e] != 0u && d1 < bound) mx = mx > d1 ? mx : d1;
    }
    mx = wave_max_u32_dpp(mx);
    if (mx == 0u) return false;  // no candidate left (cannot happen while need <= candidates)
    const uint32_t d = mx - 1u;
    uint32_t cnt = 0;
#pragma unroll
    for (int e = 0; e < S; ++e)
      cnt += (uint32_t)__popcll(ballot64(key[e] != 0u && (key[e] >> 24) == d));
    if (acc + cnt >= need) {
      *digit = (int)d;
      *above = acc;
      *bucket = cnt;
      return true;
    }
    acc += cnt;
    bound = mx;
  }
  return false;
}

// Top-K selection of one row held as S slots per lane; writes col_idx and (lane 0) row_ptr.
// The K-th largest candidate key T is found one byte at a time, most significant first
// (radix select; the top byte by top_byte_walk when it settles within kTopWalk steps); a byte
// whose bucket holds exactly the remaining count ends the search early. All ballots and shuffles
// sit in wave-uniform control flow.
template <int S>
__device__ __forceinline__ void select_topk_row(const SelectArgs& a, const float* srow,
                                                int64_t row, int lane, uint32_t* hist) {
  const int nkb = a.nkb;
  float val[S];
  uint32_t key[S];
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    const bool valid = c < nkb;
    val[e] = valid ? srow[c] : 0.f;
    key[e] = (valid && !is_forced(c, a)) ? order_key(val[e]) : 0u;  // 0: not a candidate
  }
  if (a.scores_out) {
#pragma unroll
    for (int e = 0; e < S; ++e) {
      const int c = e * 64 + lane;
      if (c < nkb) a.scores_out[row * nkb + c] = val[e];
    }
  }
  const uint32_t kk = (uint32_t)a.kk;
  uint32_t T = 0;     // threshold key (its decided high bytes)
  uint32_t need = kk; // candidates still to take among keys matching T's decided bytes
  bool exact = true;  // true: keep exactly the candidate keys whose decided bytes >= T's
  int low = 0;        // bits of T below this are undecided (exact) or zero (tie case)
  if (kk > 0) {
    exact = false;
    for (int shift = 24; shift >= 0; shift -= 8) {
      uint32_t above, cnt_d;
      int d;
      if (shift != 24 || !top_byte_walk<S>(key, need, &d, &above, &cnt_d))
        d = radix_digit<S>(key, T, shift, need, hist, lane, &above, &cnt_d);
      T |= (uint32_t)d << shift;
      need -= above;
      low = shift;
      if (cnt_d == need) {  // the whole bucket is taken
        exact = true;
        break;
      }
    }
  }
  // exact: keep keys whose bits >= low compare >= T's; otherwise keep keys > T and the first
  // `need` keys equal to T in ascending block order.
  int64_t out = row * (int64_t)a.per_row;
  uint32_t eq_seen = 0;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    const bool valid = c < nkb;
    const bool candidate = key[e] != 0u && kk > 0;
    const uint32_t kh = low >= 32 ? 0u : (key[e] >> low);
    const uint32_t th = low >= 32 ? 0u : (T >> low);
    const bool eq = candidate && !exact && key[e] == T;
    const uint64_t eqm = ballot64(eq);
    const bool take = candidate && (exact ? kh >= th
                                          : (key[e] > T || (eq && eq_seen + (uint32_t)mbcnt64(eqm) < need)));
    eq_seen += (uint32_t)__popcll(eqm);
    const bool keep = (valid && is_forced(c, a)) || take;
    const uint64_t km = ballot64(keep);
    const int64_t pos = out + mbcnt64(km);
    if (keep && pos < a.col_capacity) a.col_idx[pos] = c;
    out += __popcll(km);
  }
  if (lane == 0) {
    a.row_ptr[row] = (int32_t)(row * a.per_row);
    if (row == (int64_t)a.n_rows - 1) a.row_ptr[row + 1] = (int32_t)((row + 1) * a.per_row);
  }
}

// Radix step of the mass threshold search. Among the candidate keys that share the already
// decided high bits `prefix` (bits above shift + 8), add their fixed-point masses per 8-bit
// digit at bits [shift, shift + 8) in the wave's LDS histogram (256 x 64-bit), then find the
// largest digit d whose keys, together with the keys of larger digits, carry at least `need`.
// Returns d and, via *above, the mass of the larger digits. All calls are wave-uniform, and
// the histogram holds at least `need` in total.
template <int S>
__device__ __forceinline__ int radix_mass_digit(const uint32_t (&key)[S], const uint64_t (&u)[S],
                                                uint32_t prefix, int shift, uint64_t need,
                                                uint64_t* hist, int lane, uint64_t* above) {
  *reinterpret_cast<u32x4*>(hist + 4 * lane) = u32x4{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4*>(hist + 4 * lane + 2) = u32x4{0u, 0u, 0u, 0u};
  __builtin_amdgcn_wave_barrier();
  const int hs = shift + 8;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const uint32_t k = key[e];
    const bool in = k != 0u && u[e] != 0ull && (hs >= 32 || (k >> hs) == (prefix >> hs));
    if (in) __hip_atomic_fetch_add(hist + ((k >> shift) & 0xffu), u[e], __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WAVEFRONT);
  }
  __builtin_amdgcn_wave_barrier();
  // lane l reads the four digits 4 (63 - l) .. 4 (63 - l) + 3, so lanes run from the highest
  // digits down and an inclusive prefix sum over lanes gives the mass of digits >= 4 (63 - l)
  const int g = 63 - lane;
  const uint64_t b0 = hist[4 * g], b1 = hist[4 * g + 1], b2 = hist[4 * g + 2],
                 b3 = hist[4 * g + 3];
  const uint64_t t = b0 + b1 + b2 + b3;
  const uint64_t suf = wave_prefix_sum_u64(t);
  const uint64_t hi = suf - t;  // mass of the digits above 4 g + 3
  const uint64_t m = ballot64(hi < need && suf >= need);
  // exactly one lane holds the crossing digit when the histogram holds `need`; an empty ballot
  // (only possible for rows outside the documented input range) falls back to lane 0
  const int src = m ? (int)__builtin_ctzll(m) : 0;
  int d;
  uint64_t a;
  if (hi + b3 >= need) { d = 3; a = hi; }
  else if (hi + b3 + b2 >= need) { d = 2; a = hi + b3; }
  else if (hi + b3 + b2 + b1 >= need) { d = 1; a = hi + b3 + b2; }
  else { d = 0; a = hi + b3 + b2 + b1; }
  d = (int)lane_u32((uint32_t)(4 * g + d), src);
  *above = ((uint64_t)lane_u32((uint32_t)(a >> 32), src) << 32) | lane_u32((uint32_t)a, src);
  return d;
}

// Cumulative-mass selection of one row from its block probabilities p (slot e of lane l is key
// block 64 e + l; entries past nkb are ignored); writes the kept bitmask words and count. The
// key T of the block that completes the prefix is found a byte at a time (radix_mass_digit),
// starting below the high bytes every candidate key shares. `hist` is this wave's 256-entry
// 64-bit LDS histogram.
template <int S>
__device__ __forceinline__ void select_mass_probs(const SelectArgs& a, const float (&prob)[S],
                                                  int64_t row, int lane, uint64_t* hist) {
  const int nkb = a.nkb;
  uint64_t u[S];
  uint32_t key[S];
  uint64_t fsum = 0, csum = 0;
  uint32_t kmin = 0xffffffffu, kmax = 0u;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    const bool valid = c < nkb;
    const float p = prob[e];
    const bool f = valid && is_forced(c, a);
    u[e] = valid ? mass_units(p) : 0ull;
    key[e] = (valid && !f) ? order_key(p) : 0u;
    if (f) fsum += u[e];
    else csum += u[e];
    if (key[e] != 0u) {
      kmin = min(kmin, key[e]);
      kmax = max(kmax, key[e]);
    }
  }
  fsum = wave_total_u64(fsum);
  csum = wave_total_u64(csum);
  // how: 0 keep forced only, 1 keep all, 2 threshold
  int how;
  uint64_t need_mass = 0;
  if (a.keep_all) {
    how = 1;
  } else if (fsum >= a.theta) {
    how = 0;
  } else {
    need_mass = a.theta - fsum;
    how = (csum < need_mass) ? 1 : 2;
  }
  uint32_t T = 0;
  uint64_t n_eq = 0;
  if (how == 2) {
    kmin = wave_min_dpp(kmin);
    kmax = wave_max_u32_dpp(kmax);
    // every candidate key shares the bits above the highest bit where kmin and kmax differ;
    // the search starts at the byte holding that bit. `need` is the mass still to collect
    // among the keys that match T's decided bytes.
    uint64_t need = need_mass;
    const int hb = search_start(kmin, kmax, &T);
    for (int shift = hb < 0 ? -8 : (hb / 8) * 8; shift >= 0; shift -= 8) {
      uint64_t ab;
      const int d = radix_mass_digit<S>(key, u, T, shift, need, hist, lane, &ab);
      T = (T & ~(0xffu << shift)) | ((uint32_t)d << shift);
      need -= ab;
    }
    // T is the key of a candidate whose mass completes the prefix, so uT > 0; the candidates
    // above T carry need_mass - need. (uT == 0 only for rows outside the documented range,
    // whose 64-bit sums wrapped: such a row keeps no block equal to T instead of dividing by 0.)
    const uint64_t uT = mass_units(key_to_float(T));
    n_eq = uT ? (need + uT - 1) / uT : 0;
  }
  uint32_t cnt = 0;
  uint64_t eq_seen = 0;
  uint64_t* mrow = a.masks + row * a.words;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    const bool valid = c < nkb;
    const bool eq = how == 2 && key[e] != 0u && key[e] == T;
    const uint64_t eqm = ballot64(eq);
    bool keep;
    if (how == 1) {
      keep = valid;
    } else {
      keep = valid && is_forced(c, a);
      if (how == 2)
        keep = keep || (key[e] != 0u && key[e] > T) ||
               (eq && eq_seen + (uint64_t)mbcnt64(eqm) < n_eq);
    }
    eq_seen += (uint64_t)__popcll(eqm);
    const uint64_t km = ballot64(keep);
    if (lane == 0 && e < a.words) mrow[e] = km;
    cnt += (uint32_t)__popcll(km);
  }
  if (lane == 0) a.counts[row] = (int32_t)cnt;
}

// Pooled-score mass mode: p = softmax over the row's scores (written to scores_out when given),
// then the cumulative-mass selection.
template <int S>
__device__ __forceinline__ void select_mass_row(const SelectArgs& a, const float* srow,
                                                int64_t row, int lane, uint64_t* hist) {
  const int nkb = a.nkb;
  float val[S];
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    val[e] = c < nkb ? srow[c] : -INFINITY;
    mx = fmaxf(mx, val[e]);
  }
  mx = wave_max_dpp(mx);
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    val[e] = c < nkb ? __expf(val[e] - mx) : 0.f;
    part += val[e];
  }
  const float inv = 1.0f / wave_total_f32(part);
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    val[e] *= inv;
    if (c < nkb && a.scores_out) a.scores_out[row * nkb + c] = val[e];
  }
  select_mass_probs<S>(a, val, row, lane, hist);
}

// Work items of the scoring and selection kernel. Each (batch, head) is cut into nbig tiles of
// kRowsPerWG query blocks from its start and nsmall tiles of kSmallRows blocks for the rest. The
// kernel holds 2 workgroups per CU, kSlotsPerXcd on each XCD, and a workgroup's time grows with
// its tile, so the split follows how full the last generation of long tiles would be: when all
// of an XCD's long tiles fit in one generation, every tile is short (twice as many workgroups in
// flight); when the last generation would be at most half full, its rows go into short tiles
// spread over the slots; otherwise only the rows past a head's last whole long tile are short.
constexpr int kSmallRows = 8;
constexpr int64_t kSlotsPerXcd = 64;
struct SelectTiling {
  int nbig, nsmall;
};
__host__ __device__ inline SelectTiling select_tiling(int64_t n_heads, int nqb) {
  const int64_t nh = (n_heads + 7) / 8;  // heads of the fullest XCD
  const int64_t t16 = nh * ((nqb + kRowsPerWG - 1) / kRowsPerWG);
  const int64_t partial = t16 % kSlotsPerXcd;
  int small_rows;
  if (t16 <= kSlotsPerXcd) {
    small_rows = nqb;
  } else if (partial == 0 || partial > kSlotsPerXcd / 2) {
    small_rows = nqb % kRowsPerWG;
  } else {
    const int64_t per_head = (partial * kRowsPerWG + nh - 1) / nh;
    const int64_t rounded = (per_head + kSmallRows - 1) / kSmallRows * kSmallRows;
    small_rows = rounded < (int64_t)nqb ? (int)rounded : nqb;
  }
  const int nbig = (nqb - small_rows) / kRowsPerWG;
  const int rest = nqb - nbig * kRowsPerWG;
  return {nbig, (rest + kSmallRows - 1) / kSmallRows};
}
// Workgroups are dealt to the 8 XCDs round-robin by id, so id b runs on XCD b % 8. XCD x takes
// the heads [x n / 8, (x + 1) n / 8): first all their long tiles, head after head, then all their
// short ones, so each XCD keeps the pooled keys of the heads it is on
// (2 * nkb * head_dim * 2 bytes each) in its own L2.
__host__ __device__ inline int64_t xcd_head_begin(int64_t n_heads, int x) { return n_heads * x / 8; }

inline int64_t select_items_per_xcd(int64_t n_heads, int nqb) {
  const SelectTiling t = select_tiling(n_heads, nqb);
  int64_t m = 0;
  for (int x = 0; x < 8; ++x) {
    const int64_t nh = xcd_head_begin(n_heads, x + 1) - xcd_head_begin(n_heads, x);
    m = nh * (t.nbig + t.nsmall) > m ? nh * (t.nbig + t.nsmall) : m;
  }
  return m;
}

// This workgroup's tile: (batch, head) bh and query blocks [row0, row_end). False: no tile.
__device__ __forceinline__ bool select_work_item(int64_t n_heads, int nqb, int* bh, int* row0,
                                                 int* row_end) {
  const int x = (int)(blockIdx.x % 8);
  const int64_t i = blockIdx.x / 8;
  const SelectTiling t = select_tiling(n_heads, nqb);
  const int64_t h0 = xcd_head_begin(n_heads, x);
  const int64_t nh = xcd_head_begin(n_heads, x + 1) - h0;
  const int64_t nb = nh * t.nbig;
  if (i < nb) {
    *bh = (int)(h0 + i / t.nbig);
    *row0 = (int)(i % t.nbig) * kRowsPerWG;
    *row_end = *row0 + kRowsPerWG;
    return true;
  }
  const int64_t j = i - nb;
  if (j >= nh * t.nsmall) return false;
  *bh = (int)(h0 + j / t.nsmall);
  *row0 = t.nbig * kRowsPerWG + (int)(j % t.nsmall) * kSmallRows;
  *row_end = *row0 + kSmallRows < nqb ? *row0 + kSmallRows : nqb;
  return true;
}

template <typename T, int D, int S, int MODE>
__global__ __launch_bounds__(64 * kWaves) void score_select_kernel(SelectArgs a, int n_heads) {
  // [kRowsPerWG][lds_stride] scores, then an area holding first the pooled queries (phases 0-1)
  // and then one 256-bin histogram per wave (phase 2: 8 KiB of 32-bit counts in Top-K mode,
  // 16 KiB of 64-bit masses in mass mode)
  extern __shared__ float s_lds[];
  int bh, row0, row_end;
  if (!select_work_item(n_heads, a.nqb, &bh, &row0, &row_end)) return;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;

  uint16_t* qlds = reinterpret_cast<uint16_t*>(s_lds + kRowsPerWG * a.lds_stride);
  pool_q_rows<T, D>(a, qlds, bh, row0, row_end, lane, wave);
  __syncthreads();
  score_phase<D>(a, s_lds, qlds, bh, row0, row_end, lane, wave);
  __syncthreads();

  for (int rr = wave; rr < kRowsPerWG; rr += kWaves) {
    const int qi = row0 + rr;
    if (qi >= row_end) break;
    const int64_t row = (int64_t)bh * a.nqb + qi;
    const float* srow = s_lds + rr * a.lds_stride;
    if (MODE == 0)
      select_topk_row<S>(a, srow, row, lane,
                         reinterpret_cast<uint32_t*>(s_lds + kRowsPerWG * a.lds_stride) + 256 * wave);
    else
      select_mass_row<S>(a, srow, row, lane,
                         reinterpret_cast<uint64_t*>(s_lds + kRowsPerWG * a.lds_stride) + 256 * wave);
  }
}

// Exclusive prefix sum of the per-row counts into row_ptr (one workgroup of 1024 threads).
// Passes of 1024 kPer rows: thread t takes rows kPer t .. kPer t + kPer - 1 of the pass (all
// loads issued first, 16 bytes at a time), adds them, the 1024 thread totals are scanned (DPP
// wave scans, then the 16 wave totals), and every thread writes its kPer exclusive prefixes
// (16 bytes at a time when row_ptr allows). The launch picks kPer so that most row counts take
// one pass. Counts are small (at most 2048 per row), so int32 prefixes suffice: the host rejects
// an nnz bound above INT32_MAX.
template <int kPer>
__global__ __launch_bounds__(1024) void scan_counts_kernel(const int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ row_ptr,
                                                           int64_t rows) {
  static_assert(kPer % 4 == 0, "whole 16-byte groups");
  constexpr int64_t kPass = 1024 * kPer;
  __shared__ uint32_t wave_tot[16];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const bool vec_out = (reinterpret_cast<uintptr_t>(row_ptr) & 15u) == 0;
  uint32_t carry = 0;  // sum of all earlier passes
  for (int64_t base = 0; base < rows; base += kPass) {
    const int64_t r0 = base + (int64_t)t * kPer;
    const bool whole = r0 + kPer <= rows;
    int32_t c[kPer];
    if (whole) {  // kPer * 4 contiguous bytes per thread (counts is 256-byte aligned)
#pragma unroll
      for (int g = 0; g < kPer / 4; ++g) {
        const u32x4 a = load_u32x4(counts + r0 + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) c[4 * g + i] = (int32_t)a[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) c[i] = r0 + i < rows ? counts[r0 + i] : 0;
    }
    uint32_t own = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) own += (uint32_t)c[i];
    const uint32_t incl = wave_prefix_sum_u32(own);  // within the wave
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    uint32_t before = carry;
    for (int i = 0; i < wave; ++i) before += wave_tot[i];
    uint32_t pass_total = 0;
    for (int i = 0; i < 16; ++i) pass_total += wave_tot[i];
    uint32_t run = before + incl - own;  // exclusive prefix of this thread's first row
    if (whole && vec_out) {
#pragma unroll
      for (int g = 0; g < kPer / 4; ++g) {
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          o[i] = run;
          run += (uint32_t)c[4 * g + i];
        }
        *reinterpret_cast<u32x4*>(row_ptr + r0 + 4 * g) = o;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kPer; ++i) {
        if (r0 + i < rows) row_ptr[r0 + i] = (int32_t)run;
        run += (uint32_t)c[i];
      }
    }
    carry += pass_total;
    __syncthreads();  // wave_tot is rewritten by the next pass
  }
  if (t == 0) row_ptr[rows] = (int32_t)carry;
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
  // the row's words in one load (lane e holds word e; words <= 32), then read back per word
  const uint64_t mine = lane < words ? masks[row * words + lane] : 0ull;
  for (int e = 0; e < words; ++e) {
    const uint64_t w = ((uint64_t)__builtin_amdgcn_readlane((int)(mine >> 32), e) << 32) |
                       (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mine, e);
    const bool keep = (w >> lane) & 1ull;
    const int64_t pos = out + mbcnt64(w);
    if (keep && pos < col_capacity) col_idx[pos] = e * 64 + lane;
    out += __popcll(w);
  }
}

// Token-level mass mode: the block probabilities of each row are given (block energies, one
// row per wave, four rows per workgroup).
template <int S>
__global__ __launch_bounds__(256) void select_energy_kernel(SelectArgs a, const float* energy) {
  __shared__ __attribute__((aligned(16))) uint64_t hist[4][256];
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.n_rows) return;
  const int lane = threadIdx.x & 63;
  float p[S];
#pragma unroll
  for (int e = 0; e < S; ++e) {
    const int c = e * 64 + lane;
    p[e] = c < a.nkb ? energy[row * a.nkb + c] : 0.f;
  }
  select_mass_probs<S>(a, p, row, lane, hist[threadIdx.x >> 6]);
}

hipError_t launch_exclusive_scan(const int32_t* counts, int32_t* out, int64_t n,
                                 hipStream_t stream) {
  if (n <= 1024 * 8)
    scan_counts_kernel<8><<<1, 1024, 0, stream>>>(counts, out, n);
  else if (n <= 1024 * 16)
    scan_counts_kernel<16><<<1, 1024, 0, stream>>>(counts, out, n);
  else
    scan_counts_kernel<32><<<1, 1024, 0, stream>>>(counts, out, n);
  return hipGetLastError();
}

hipError_t launch_scan_counts(const SelectArgs& a, hipStream_t stream) {
  return launch_exclusive_scan(a.counts, a.row_ptr, a.n_rows, stream);
}

hipError_t launch_counts_to_csr(const SelectArgs& a, hipStream_t stream) {
  hipError_t err = launch_scan_counts(a, stream);
  if (err != hipSuccess) return err;
  fill_csr_kernel<<<(unsigned)((a.n_rows + 3) / 4), 256, 0, stream>>>(
      a.masks, a.row_ptr, a.col_idx, a.n_rows, a.words, a.col_capacity);
  return hipGetLastError();
}

static hipError_t launch_select_energy_rows(const SelectArgs& a, const float* energy,
                                            hipStream_t stream) {
  const dim3 grid((unsigned)((a.n_rows + 3) / 4));
  const int slots = (a.nkb + 63) / 64;
#define DBSP_SLOTS(N)                                              \
  if (slots <= N) {                                                \
    select_energy_kernel<N><<<grid, 256, 0, stream>>>(a, energy);  \
    return hipGetLastError();                                      \
  }
  DBSP_SLOTS(1) DBSP_SLOTS(2) DBSP_SLOTS(4) DBSP_SLOTS(6) DBSP_SLOTS(8) DBSP_SLOTS(10)
  DBSP_SLOTS(12) DBSP_SLOTS(16) DBSP_SLOTS(20) DBSP_SLOTS(24) DBSP_SLOTS(28) DBSP_SLOTS(32)
#undef DBSP_SLOTS
  return hipErrorInvalidValue;
}

hipError_t launch_select_energy(const SelectArgs& a, const float* energy, hipStream_t stream) {
  const hipError_t err = launch_select_energy_rows(a, energy, stream);
  if (err != hipSuccess) return err;
  return launch_counts_to_csr(a, stream);
}

template <typename T, int D, int MODE>
static hipError_t launch_score_select_dm(const SelectArgs& a, int64_t bh, hipStream_t stream) {
  const dim3 grid((unsigned)(8 * select_items_per_xcd(bh, a.nqb)));
  const dim3 block(64 * kWaves);
  // the area after the scores holds the pooled queries (8 KiB at most), then one histogram per
  // wave: 256 x 32-bit (Top-K) or 256 x 64-bit (mass)
  const size_t lds = (size_t)kRowsPerWG * a.lds_stride * sizeof(float) + (MODE == 0 ? 8192 : 16384);
  const int slots = (a.nkb + 63) / 64;
#define DBSP_SLOTS(N)                                                               \
  if (slots <= N) {                                                                 \
    score_select_kernel<T, D, N, MODE><<<grid, block, lds, stream>>>(a, (int)bh);               \
    return hipGetLastError();                                                       \
  }
  DBSP_SLOTS(1) DBSP_SLOTS(2) DBSP_SLOTS(4) DBSP_SLOTS(6) DBSP_SLOTS(8) DBSP_SLOTS(10)
  DBSP_SLOTS(12) DBSP_SLOTS(16) DBSP_SLOTS(20) DBSP_SLOTS(24) DBSP_SLOTS(28) DBSP_SLOTS(32)
#undef DBSP_SLOTS
  return hipErrorInvalidValue;
}

hipError_t launch_select(const SelectArgs& a, int64_t bh, int head_dim, bool bf16,
                         hipStream_t stream) {
  hipError_t err;
  if (bf16 && head_dim == 128)
    err = a.mode == 0 ? launch_score_select_dm<uint16_t, 128, 0>(a, bh, stream)
                      : launch_score_select_dm<uint16_t, 128, 1>(a, bh, stream);
  else if (bf16 && head_dim == 64)
    err = a.mode == 0 ? launch_score_select_dm<uint16_t, 64, 0>(a, bh, stream)
                      : launch_score_select_dm<uint16_t, 64, 1>(a, bh, stream);
  else if (!bf16 && head_dim == 128)
    err = a.mode == 0 ? launch_score_select_dm<float, 128, 0>(a, bh, stream)
                      : launch_score_select_dm<float, 128, 1>(a, bh, stream);
  else if (!bf16 && head_dim == 64)
    err = a.mode == 0 ? launch_score_select_dm<float, 64, 0>(a, bh, stream)
                      : launch_score_select_dm<float, 64, 1>(a, bh, stream);
  else
    return hipErrorInvalidValue;
  if (err != hipSuccess || a.mode == 0) return err;
  return launch_counts_to_csr(a, stream);
}

}  // namespace dbsp
