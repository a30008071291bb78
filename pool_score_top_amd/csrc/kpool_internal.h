// Internal declarations shared by the HIP translation units of libkpool.
// Device helpers live here; each kernel is launched from the file that
// defines it through a host launcher declared below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kpool {

// ----------------------------------------------------------------------------
// Launch planning data for the score kernel.  A "segment" is the part of one
// sequence that falls in the current row chunk; it is cut into row tiles of
// kTileRows rows that never straddle a sequence (each tile shares one set of
// pooled keys).  Segments travel by value in the kernel arguments.
// ----------------------------------------------------------------------------
constexpr int kMaxSegs = 32;

struct SegList {
  int32_t nseg;
  int32_t tile_start[kMaxSegs + 1];  // prefix of row tiles per segment
  int32_t row_lo[kMaxSegs];          // first global row of the segment
  int32_t row_hi[kMaxSegs];          // one past the last global row
  int32_t seq_start[kMaxSegs];       // global row of the sequence's token 0
  int32_t pool_base[kMaxSegs];       // first pooled-key row of the sequence
  int32_t pool_count[kMaxSegs];      // pools of the sequence (caps every row's visible count)
};

// ----------------------------------------------------------------------------
// Host launchers (each returns hipGetLastError() after the launch).
// ----------------------------------------------------------------------------
hipError_t launch_pool_keys(const uint16_t *k, const int32_t *cu_seqlens, const int32_t *cu_pools,
                            int32_t nseq, int32_t D, int32_t kpool, int64_t P_tot, uint16_t *kp,
                            hipStream_t stream);

hipError_t launch_pool_keys_gated(const uint16_t *k, const uint16_t *g, const float *ape,
                                  const int32_t *cu_seqlens, const int32_t *cu_pools, int32_t nseq,
                                  int32_t D, int32_t kpool, int64_t P_tot, uint16_t *kp,
                                  hipStream_t stream);

// true if (H, D) has a compiled score kernel
bool score_supported(int H, int D);
int score_tile_rows();
// Score workgroups the device runs at once (CUs x workgroups per CU), 0 if unknown.
int score_slots(int H, int D, int device);
// Scores of the chunk's rows go to out[(row - chunk_row0) * ld + pool]; the max of each
// 16-pool group of a row (over its visible pools) to gmax[(row - chunk_row0) * ldg + pool/16].
constexpr int kGroup = 16;
hipError_t launch_score(int H, int D, const uint16_t *q, const uint16_t *kp, const float *w,
                        float scale, int32_t kpool, const SegList &segs, int32_t ntiles,
                        int32_t npseg, int32_t pseg_pools, int64_t chunk_row0, int64_t ld,
                        float *out, int64_t ldg, float *gmax, hipStream_t stream);

constexpr int kTopkMaxBudget = 2048;
// Rows [row0, row0 + nrows) of `scores` (row r at scores + r*ld).  The number
// of ranked entries of row r is n_valid[r] if n_valid is not null, else
// (t / kpool + 1) for the row's sequence-local position t (global row
// grow0 + r looked up in cu_seqlens), capped at L / kpool for a sequence of L
// tokens in tail mode (full pools only).
// With gmax (the score kernel's 16-pool group maxima, row pitch ldg) the selection reads
// the group maxima first and then only the groups that can hold a winner; without it
// every row is read in full.
hipError_t launch_topk(const float *scores, int64_t ld, int64_t nrows, const int32_t *n_valid,
                       const int32_t *cu_seqlens, int32_t nseq, int64_t grow0, int32_t kpool,
                       bool tail, int32_t budget, int32_t *out, const float *gmax, int64_t ldg,
                       hipStream_t stream);

hipError_t launch_scores_copy(const float *ws, int64_t ld, int64_t nrows, const int32_t *cu_seqlens,
                              int32_t nseq, int64_t grow0, int32_t kpool, bool tail, float *dst,
                              int64_t dst_ld, hipStream_t stream);

// tail: full pools only, and kpool - 1 tail slots after a row's budget*kpool expanded ones
hipError_t launch_expand(const int32_t *pool_ids, const int32_t *cu_seqlens, int32_t nseq,
                         int32_t kpool, bool tail, int64_t q_lo, int64_t nrows, int32_t budget,
                         int32_t *token_ids, hipStream_t stream);

// ----------------------------------------------------------------------------
// Device helpers
// ----------------------------------------------------------------------------
#if defined(__HIPCC__)

// Pools visible to the row at sequence-local position t of a sequence of L tokens:
// p*kpool <= t, and in tail mode (full pools only) p < L / kpool.
__device__ inline int64_t visible_count(int64_t t, int64_t L, int kpool, bool tail) {
  const int64_t n = t / kpool + 1;
  return tail ? min(n, L / kpool) : n;
}

// Index of the sequence holding global row `row`: the largest s < nseq with
// cu[s] <= row (empty sequences are skipped because their start repeats).
__device__ inline int find_seq(const int32_t *__restrict__ cu, int nseq, int64_t row) {
  int lo = 0, hi = nseq;  // answer in [lo, hi)
  while (hi - lo > 1) {
    int mid = (lo + hi) >> 1;
    if (cu[mid] <= row) lo = mid; else hi = mid;
  }
  return lo;
}

// fp32 -> order-preserving uint32: larger key = larger value.  -0.0 is folded
// onto +0.0 first, and every NaN maps to 0, below -inf (whose key is
// 0x007FFFFF), so NaN is never ranked above a number.
__device__ inline uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

#endif

}  // namespace kpool
