/*
 * kpool.h - C ABI of the MI355X (gfx950) k-pool DSA indexer selection.
 *
 * The selection a DSA indexer makes for each query row (pages: Atlas
 * inference docs, spark_model/layers/glm5next_dsa/tp.rs, module doc "Why the
 * indexer is REPLICATED, not sharded"; Megatron-LM PR #8299, sections
 * "Mechanism" and "Change"):
 *
 *   1. pool the keys over kpool consecutive tokens            kpool_pool_keys
 *   2. score every causally visible pool of row i as
 *        S[i,p] = sum_h w[i,h] * relu(scale * <q[i,h,:], kp[p,:]>)
 *      and keep the best `budget` pools, higher score first and the
 *      smaller pool index on equal scores                     kpool_score_topk
 *   3. expand the kept pools to token ids p*kpool + j and drop the tokens
 *      that come after the row                                kpool_expand
 *
 * Conventions shared by every entry point
 *   - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *     allocates no device memory, keeps no pointer after it returns and never
 *     synchronises: all work is enqueued on `stream` (a hipStream_t; NULL is
 *     the default stream).  Results are ready when the stream reaches them.
 *   - bf16 tensors are passed as their uint16_t bit patterns.  Tensors are
 *     row-major and contiguous; q, kp, k and w must be 16-byte aligned.
 *   - Packed variable-length batches ("THD") are described by cu_seqlens:
 *     sequence s holds the global rows [cu_seqlens[s], cu_seqlens[s+1]).
 *     Positions, pool ids and token ids are SEQUENCE-LOCAL: row i of
 *     sequence s sits at t = i - cu_seqlens[s], and sees the pools p with
 *     p*kpool <= t.  A single sequence is nseq = 1, cu_seqlens = {0, T}.
 *     `cu_seqlens_host` is a host copy used to validate and plan launches;
 *     `cu_seqlens_dev` / `cu_pools_dev` hold the same arrays on the device.
 *   - Every entry point validates its arguments before it launches anything
 *     and returns KPOOL_OK (0) or a negative kpool_status; the reason is then
 *     in kpool_last_error() (thread-local).  Nothing is thrown across the ABI.
 *     Launch failures map to KPOOL_EHIP; faults that happen while a kernel
 *     runs surface at the caller's next synchronisation.
 *   - Every setting is an argument: there is no process-wide switch.  Calls on
 *     one stream are ordered.  The library's only lasting state is, per caller
 *     stream that asked for the chunk overlap (KPOOL_FLAG_OVERLAP), one helper
 *     stream (default priority) with two events, created on first use and kept
 *     until the process ends; the helper joins back into the caller's stream
 *     before the call returns, so results are ordered on the caller's stream as
 *     usual.  Calls on different caller streams use different helpers.  Besides
 *     that, per device and once: the number of score workgroups the device runs
 *     at once (an occupancy query, used to plan launches) and, for
 *     kpool_score_topk_noalloc, its static scratch array's device address.  The
 *     optional profiler below is per host thread.
 */
#ifndef KPOOL_H
#define KPOOL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KPOOL_OK = 0,
  KPOOL_EINVAL = -1,       /* bad argument: range, size, pointer, alignment */
  KPOOL_EUNSUPPORTED = -2, /* head count / head dim not compiled in */
  KPOOL_EWORKSPACE = -3,   /* workspace smaller than one score row */
  KPOOL_EHIP = -4          /* a HIP launch or runtime call failed */
} kpool_status;

/* Message for the last non-OK return on this thread ("" if none). */
const char *kpool_last_error(void);

/* ABI version (major*100 + minor): 300. */
int kpool_version(void);

/* Tail mode (flags bit of kpool_count_pools, kpool_pool_keys(_gated),
 * kpool_score_topk(_noalloc) and kpool_expand; pass the same choice to all of
 * them).  Megatron-LM PR #8299 "Change" names a "tail append" between pool
 * expansion and mask filtering but does not define it; this library's reading:
 * a sequence of L tokens has only its L / kpool full pools (the pool count of
 * the Atlas tp.rs module doc, seq / kpool), and its remaining L mod kpool
 * tokens, the tail, are appended to every row's expanded token ids and filtered
 * causally like them.  Without the flag a trailing partial pool is a pool of its
 * own and there is no tail. */
#define KPOOL_FLAG_TAIL 2u

/* Pool bookkeeping on the host (Atlas tp.rs module doc: a sequence of L
 * tokens has L/kpool pools).
 *   flags            0: ceil(L / kpool) pools, a trailing partial pool kept;
 *                    KPOOL_FLAG_TAIL: floor(L / kpool), full pools only
 *   cu_pools_host[s] = sum over s' < s of the pool counts, [nseq + 1] (nullable)
 *   *max_pools_out   = the largest pool count of one sequence (nullable)
 * Returns the total pool count P_tot (>= 0) or a negative kpool_status. */
int64_t kpool_count_pools(const int32_t *cu_seqlens_host, int32_t nseq, int32_t kpool,
                          uint32_t flags, int32_t *cu_pools_host, int32_t *max_pools_out);

/* Step 1 - pooled keys (Megatron-LM PR #8299 "Mechanism": rows score the
 * pooled keys).  For pool p of sequence s, with n = min(kpool, L_s - p*kpool):
 *   kp[cu_pools[s] + p, d] = bf16_rne( fp32( (sum_j k[cu_seqlens[s] + p*kpool + j, d]) / n ) )
 * where the sum is taken in fp32 in token order starting from +0.
 *   k   bf16 [T, D]  one key per token (the indexer's key projection has no head axis)
 *   kp  bf16 [P_tot, D] output, P_tot from kpool_count_pools with the same flags
 *   flags 0 or KPOOL_FLAG_TAIL (full pools only; cu_pools_dev must count the same way)
 * D must be a multiple of 8 (<= 1024); kpool >= 1. */
int kpool_pool_keys(const uint16_t *k, const int32_t *cu_seqlens_host,
                    const int32_t *cu_seqlens_dev, const int32_t *cu_pools_dev,
                    int32_t nseq, int32_t D, int32_t kpool, uint32_t flags, uint16_t *kp,
                    void *stream);

/* Step 1, gated variant - the GLM-5.3 indexer's k-pool compression (Atlas inference
 * docs, glm5next_dsa/tp.rs: the shard plan's indexer tensors include a compression
 * gate [index_head_dim, hidden] and a slot embedding [index_kpool, index_head_dim];
 * Megatron-LM PR #8299 "Mechanism": gate scores are an input of the op).  The pages
 * give no formula; this library's reading, for pool p of sequence s with tokens
 * t_j = cu_seqlens[s] + p*kpool + j, j < n = min(kpool, L_s - p*kpool), and each dim d:
 *   z_j = g[t_j, d] + ape[j, d],  m = max_j z_j,  e_j = exp(z_j - m)
 *   kp[cu_pools[s] + p, d] = bf16_rne( (sum_j e_j * k[t_j, d]) / (sum_j e_j) )
 * in fp64, rounded once to bf16 (sums in slot order; a trailing partial pool uses
 * ape[0 .. n-1]).
 *   k    bf16 [T, D]      keys
 *   g    bf16 [T, D]      gate scores (the gate projection's output per token and dim)
 *   ape  fp32 [kpool, D]  slot embeddings
 *   kp   bf16 [P_tot, D]  output, laid out as for kpool_pool_keys
 * flags: 0 or KPOOL_FLAG_TAIL, as for kpool_pool_keys.
 * k, g, ape and kp must be 16-byte aligned; D a multiple of 8 (<= 1024); kpool >= 1.
 * Inputs must be finite. */
int kpool_pool_keys_gated(const uint16_t *k, const uint16_t *g, const float *ape,
                          const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                          const int32_t *cu_pools_dev, int32_t nseq, int32_t D, int32_t kpool,
                          uint32_t flags, uint16_t *kp, void *stream);

/* Workspace for kpool_score_topk over rows [q_lo, q_hi): per query row of a
 * chunk, one fp32 score row at a pitch of max_pools rounded up to 64 plus one
 * fp32 maximum per 16 pools of it; the score rows of one chunk are capped at
 * 2 GiB (Megatron-LM PR #8299 "Change": the chunked score path caps its score
 * buffer at 2 GiB per chunk).  With nbuf = 2 the size covers two such chunk
 * buffers when the range needs more than one chunk (for KPOOL_FLAG_OVERLAP:
 * two chunks are then in flight, up to 2 x 2 GiB of scores); with nbuf = 1, one.
 * Returns 0 for an empty range or an nbuf other than 1 or 2. */
size_t kpool_workspace_bytes(int64_t q_lo, int64_t q_hi, int32_t max_pools, int32_t nbuf);

/* Flags of kpool_score_topk. */
#define KPOOL_FLAG_OVERLAP 1u /* two chunk buffers, chunks alternating between two streams */

/* The chunk plan kpool_score_topk follows for a sequence of at most max_pools pools
 * (per kpool_count_pools with the same tail flag), a workspace of workspace_bytes and
 * these flags: returns the rows per chunk (> 0; each chunk's fp32 scores at most
 * 2 GiB) and writes the number of chunk buffers (1, or 2 with KPOOL_FLAG_OVERLAP and
 * room for two rows) to *nbuf_out (nullable).  Returns a negative kpool_status for
 * max_pools < 1, unknown flags, or a workspace smaller than one row. */
int64_t kpool_chunk_rows(int32_t max_pools, size_t workspace_bytes, uint32_t flags,
                         int32_t *nbuf_out);

/* Step 2 - score and select, for the global rows [q_lo, q_hi).
 * (Megatron-LM PR #8299 "Change": one rank's contiguous slice of query rows
 * goes through the chunked score/top-k path; per row the result equals the
 * unsliced one.  Atlas tp.rs module doc: the score formula and tie-break.)
 *   q        bf16 [T, H, D]    index queries
 *   kp       bf16 [P_tot, D]   pooled keys from kpool_pool_keys
 *   w        fp32 [T, H]       per-row head weights (any sign)
 *   scale    > 0, usually 1/sqrt(D)
 *   budget   pools kept per row, 1..2048 (index_topk / kpool; 2048 for the per-token
 *            indexer, kpool = 1)
 *   workspace, workspace_bytes: device scratch of at least one row
 *            (kpool_workspace_bytes(q_lo, q_lo + 1, max_pools, 1)).  Each chunk
 *            has as many rows as the 2 GiB score cap and its buffer allow.
 *            Contents are scratch on return.
 *   flags    KPOOL_FLAG_OVERLAP and/or KPOOL_FLAG_TAIL.  Without OVERLAP: one
 *            chunk buffer; every launch on the caller's stream, one after the other
 *            (each kernel runs alone, which per-kernel timing needs).  With
 *            KPOOL_FLAG_OVERLAP: a workspace of two rows or more is split into two
 *            chunk buffers, and consecutive chunks alternate between the caller's
 *            stream and its helper stream, so one chunk's selection runs beside the
 *            next chunk's scoring; each buffer keeps the 2 GiB cap.  Results are
 *            bitwise the same either way.  KPOOL_FLAG_TAIL: full pools only (kp
 *            pooled with the same flag), so a row sees min(t / kpool + 1, L / kpool)
 *            pools.  Unknown bits return KPOOL_EINVAL.
 *   pool_ids int32 [q_hi - q_lo, budget] output: sequence-local pool ids,
 *            best first by (score desc, pool asc), -1 after the visible pools
 *            run out.  -0.0 ranks equal to +0.0; NaN ranks below -inf.  q, kp and
 *            w must be finite (the score's ReLU does not propagate NaN).
 *   scores_out NULLABLE fp32 [q_hi - q_lo, max_pools] (max_pools of
 *            kpool_count_pools with the same tail flag): the fp32 scores the
 *            selection ranked, -inf where the pool is not visible.
 * Supported (H, D): (4, 16) and (32, 128).  q_lo == q_hi is a no-op.
 * Sizes: one sequence's pooled keys must stay below 4 GiB (fewer than 2^24 pools
 * at D = 128) and one fp32 score row within 2 GiB; larger returns
 * KPOOL_EUNSUPPORTED. */
int kpool_score_topk(const uint16_t *q, const uint16_t *kp, const float *w,
                     const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                     int32_t nseq, int32_t H, int32_t D, int32_t kpool, float scale,
                     int64_t q_lo, int64_t q_hi, int32_t budget,
                     void *workspace, size_t workspace_bytes, uint32_t flags,
                     int32_t *pool_ids, float *scores_out, void *stream);

/* kpool_score_topk for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, and harnesses that forbid hipMalloc.  Same
 * arguments and results as kpool_score_topk (flags: KPOOL_FLAG_TAIL as there;
 * KPOOL_FLAG_OVERLAP has no effect here) but without a workspace argument: the workspace is a
 * static device array of KPOOL_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library:
 * each GPU the library runs on holds its own copy until the process ends.  The call
 * allocates nothing (no hipMalloc / hipFree, no stream or event creation; the profiler
 * is bypassed); its chunks, as many rows each as one 64 MiB workspace holds, run on
 * `stream` one after the other.
 *   - A sequence whose score row (its pools rounded up to 64, plus one maximum per
 *     16 of them, 4 bytes each) exceeds the scratch, i.e. more than about 15.79M
 *     pools, returns KPOOL_EWORKSPACE with a message saying so.
 *   - All calls on one GPU share that GPU's array, which keeps the last call's
 *     contents (nothing in it needs clearing between calls).  Calls that overlap on
 *     one GPU (different streams or host threads at once) race on it: order them. */
#define KPOOL_NOALLOC_SCRATCH_BYTES (64u << 20)
int kpool_score_topk_noalloc(const uint16_t *q, const uint16_t *kp, const float *w,
                             const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                             int32_t nseq, int32_t H, int32_t D, int32_t kpool, float scale,
                             int64_t q_lo, int64_t q_hi, int32_t budget, uint32_t flags,
                             int32_t *pool_ids, float *scores_out, void *stream);

/* Step 3 - expansion and causal filter (Megatron-LM PR #8299 "Change": pool
 * expansion and mask filtering run after the pool ids are known).
 *   token_ids[i - q_lo, b*kpool + j] = p*kpool + j   if p = pool_ids[i - q_lo, b] >= 0
 *                                                    and p*kpool + j <= t(i)
 *                                    = -1            otherwise
 *   flags 0 or KPOOL_FLAG_TAIL.  Tail mode appends kpool - 1 slots per row: with
 *   a = (L / kpool) * kpool for the row's sequence of L tokens,
 *   token_ids[i - q_lo, budget*kpool + j] = a + j if a + j < L and a + j <= t(i), else -1.
 *   pool_ids  int32 [q_hi - q_lo, budget];
 *   token_ids int32 [q_hi - q_lo, budget*kpool (+ kpool - 1 in tail mode)], 16-byte
 *   aligned when kpool = 4 without tail mode. */
int kpool_expand(const int32_t *pool_ids, const int32_t *cu_seqlens_host,
                 const int32_t *cu_seqlens_dev, int32_t nseq, int32_t kpool,
                 int64_t q_lo, int64_t q_hi, int32_t budget, uint32_t flags,
                 int32_t *token_ids, void *stream);

/* The selection step alone, over caller-provided fp32 scores (the second
 * half of the chunk loop, exposed so it can be checked on its own).
 *   scores   fp32 [rows, ld], ld % 4 == 0, 16-byte aligned
 *   n_valid  int32 [rows] device: row r ranks scores[r, 0 .. n_valid[r]),
 *            0 <= n_valid[r] <= ld (a value outside is clamped to that range: a
 *            negative count selects nothing, one past ld ranks the whole row)
 *   budget   1..2048, as for kpool_score_topk
 *   pool_ids int32 [rows, budget]: same ordering and padding as kpool_score_topk */
int kpool_topk(const float *scores, int64_t ld, const int32_t *n_valid, int64_t rows,
               int32_t budget, int32_t *pool_ids, void *stream);

/* Optional per-kernel device timing, per host thread.  While enabled on a
 * thread, every launch that thread's calls make is bracketed by HIP events on
 * its stream.  kpool_profile_collect waits for the events the calling thread
 * recorded, adds each kernel kind's elapsed time (ms) and launch count into
 * ms[kind] / launches[kind] (arrays of KPOOL_PROFILE_KINDS) and forgets them.
 * Other threads' records and switches are untouched.  Event spans of
 * overlapped chunks (KPOOL_FLAG_OVERLAP) include whatever else the GPU runs
 * meanwhile; time kernels with flags = 0. */
#define KPOOL_PROFILE_KINDS 5 /* 0 pool_keys, 1 score, 2 topk, 3 expand, 4 scores_out copy */
int kpool_profile_enable(int on);
int kpool_profile_collect(double *ms, int64_t *launches);

#ifdef __cplusplus
}
#endif

#endif /* KPOOL_H */
