// C ABI of libkpool: argument validation, chunk planning and launches.
//
// Pages: Megatron-LM PR #8299, "Change" -- a contiguous range of query rows is
// scored and selected through a chunk loop whose fp32 score buffer is capped
// at 2 GiB per chunk; the selections are int32 pool ids; expansion and mask
// filtering follow.  This file is that loop for one GPU: [q_lo, q_hi) is the
// one-GPU form of a rank's query slice.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <map>
#include <memory>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/kpool.h"
#include "kpool_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char *fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return KPOOL_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

constexpr int64_t kChunkCapBytes = int64_t(1) << 31;  // 2 GiB of fp32 scores per chunk
#ifndef KPOOL_POOL_SEG_MAX
#define KPOOL_POOL_SEG_MAX 16384
#endif
#ifndef KPOOL_SCORE_TARGET_WGS
#define KPOOL_SCORE_TARGET_WGS 1024
#endif
constexpr int kPoolSegMax = KPOOL_POOL_SEG_MAX;  // pools per score workgroup (max, multiple of 64)

int64_t pitch_of(int32_t max_pools) { return (int64_t)(max_pools + 63) / 64 * 64; }

// cu_seqlens_host: nseq >= 1 entries + 1, starts at 0, non-decreasing.
int check_cu(const int32_t *cu, int32_t nseq, const char *fn) {
  if (!cu) return fail(KPOOL_EINVAL, "%s: cu_seqlens_host is null", fn);
  if (nseq < 1) return fail(KPOOL_EINVAL, "%s: nseq must be >= 1 (got %d)", fn, nseq);
  if (cu[0] != 0) return fail(KPOOL_EINVAL, "%s: cu_seqlens[0] must be 0 (got %d)", fn, cu[0]);
  for (int32_t s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s])
      return fail(KPOOL_EINVAL, "%s: cu_seqlens must be non-decreasing (cu[%d]=%d > cu[%d]=%d)",
                  fn, s, cu[s], s + 1, cu[s + 1]);
  return KPOOL_OK;
}

// ---------------------------------------------------------------------------
// Optional per-kernel timing with HIP events on the launch stream.  The switch
// and the records are per host thread, so one thread's profiling never sees or
// changes another thread's launches.
// ---------------------------------------------------------------------------
struct ProfRec {
  int kind;
  hipEvent_t a, b;
};
thread_local bool g_prof_on = false;
thread_local std::vector<ProfRec> g_prof;

template <class F>
hipError_t timed(int kind, hipStream_t stream, F &&launch) {
  if (!g_prof_on) return launch();
  ProfRec rec{kind, nullptr, nullptr};
  hipError_t e = hipEventCreate(&rec.a);
  if (e == hipSuccess) e = hipEventCreate(&rec.b);
  if (e == hipSuccess) e = hipEventRecord(rec.a, stream);
  if (e == hipSuccess) e = launch();
  if (e == hipSuccess) e = hipEventRecord(rec.b, stream);
  if (e == hipSuccess) {
    g_prof.push_back(rec);
  } else {  // (the launch's own error is returned; the record is dropped)
    if (rec.a) (void)hipEventDestroy(rec.a);
    if (rec.b) (void)hipEventDestroy(rec.b);
  }
  return e;
}

template <class F>
hipError_t timed_if(bool profile, int kind, hipStream_t stream, F &&launch) {
  return profile ? timed(kind, stream, launch) : launch();
}

int hip_fail(const char *fn, hipError_t e) {
  return fail(KPOOL_EHIP, "%s: HIP error %d (%s)", fn, (int)e, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// Helper streams for the two-buffer chunk loop: one per caller stream (so calls
// on independent caller streams never queue behind each other), each with its
// own fork/join events and lock.  Created on first use (default priority,
// non-blocking) on the caller stream's device and kept until the process ends.
// ---------------------------------------------------------------------------
struct Aux {
  std::mutex mu;  // held while a call enqueues on this helper
  hipStream_t helper = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_aux_mu;  // guards the map only
std::map<std::pair<int, hipStream_t>, std::unique_ptr<Aux>> g_aux;

hipError_t get_aux(hipStream_t stream, Aux **out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> guard(g_aux_mu);
  std::unique_ptr<Aux> &slot = g_aux[{dev, stream}];
  if (!slot) {
    std::unique_ptr<Aux> a(new Aux);
    int cur = 0;
    e = hipGetDevice(&cur);
    const bool switched = e == hipSuccess && cur != dev;
    if (switched) e = hipSetDevice(dev);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&a->helper, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&a->fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&a->join, hipEventDisableTiming);
    if (e != hipSuccess) {  // a partly made helper is released; the next call retries
      if (a->join) (void)hipEventDestroy(a->join);
      if (a->fork) (void)hipEventDestroy(a->fork);
      if (a->helper) (void)hipStreamDestroy(a->helper);
    }
    if (switched) (void)hipSetDevice(cur);
    if (e != hipSuccess) {
      g_aux.erase({dev, stream});
      return e;
    }
    slot = std::move(a);
  }
  *out = slot.get();
  return hipSuccess;
}

// ---------------------------------------------------------------------------
// Static scratch for kpool_score_topk_noalloc: the chunk workspace of callers that
// cannot allocate device memory.  Every GPU the library runs on holds its own copy
// until the process ends.  In host code `scratch` is only a host-side stand-in for the
// symbol; the device address comes from hipGetSymbolAddress, taken once per device
// with that device current, and only that address is handed to kernels.  Nothing in it
// has to start at zero: each chunk's score kernel writes every score and group maximum
// that the chunk's selection then reads.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = KPOOL_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_ptr(hipStream_t stream, void **out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    const bool switched = e == hipSuccess && cur != dev;
    if (switched) e = hipSetDevice(dev);
    void *p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (switched) (void)hipSetDevice(cur);
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

// Per row of a chunk the workspace holds ld fp32 scores and ld/16 fp32 group maxima.
int64_t ws_row_bytes(int64_t ld) { return (ld + ld / kpool::kGroup) * 4; }

// The chunk plan of the loop: the number of chunk buffers and the rows per chunk for a
// score pitch ld and a workspace of the given size (at least one row).
struct ChunkPlan {
  int nbuf;
  int64_t rows;
};
ChunkPlan plan_chunks(int64_t ld, size_t workspace_bytes, bool overlap) {
  const int64_t row_bytes = ws_row_bytes(ld);
  const int nbuf = (overlap && (int64_t)workspace_bytes >= 2 * row_bytes) ? 2 : 1;
  const int64_t rows = std::max<int64_t>(
      1, std::min<int64_t>(kChunkCapBytes / (ld * 4), (int64_t)workspace_bytes / nbuf / row_bytes));
  return {nbuf, rows};
}
// The chunk loop behind kpool_score_topk and kpool_score_topk_noalloc.  With
// use_scratch, the workspace is this device's static scratch array (resolved after the
// arguments are validated), chunks run on the caller's stream one after the other and
// the profiler is bypassed, so the call creates and allocates nothing.
int score_topk_impl(const char *fn, const uint16_t *q, const uint16_t *kp, const float *w,
                    const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev, int32_t nseq,
                    int32_t H, int32_t D, int32_t kpool, float scale, int64_t q_lo, int64_t q_hi,
                    int32_t budget, void *workspace, size_t workspace_bytes, uint32_t flags,
                    bool use_scratch, int32_t *pool_ids, float *scores_out, void *stream) {
  int rc = check_cu(cu_seqlens_host, nseq, fn);
  if (rc) return rc;
  const int64_t T = cu_seqlens_host[nseq];
  if (kpool < 1) return fail(KPOOL_EINVAL, "%s: kpool must be >= 1 (got %d)", fn, kpool);
  if (budget < 1 || budget > kpool::kTopkMaxBudget)
    return fail(KPOOL_EINVAL, "%s: budget must be in [1, %d] (got %d)", fn, kpool::kTopkMaxBudget, budget);
  if (!(scale > 0.0f) || !isfinite(scale)) return fail(KPOOL_EINVAL, "%s: scale must be finite and > 0", fn);
  if (q_lo < 0 || q_lo > q_hi || q_hi > T)
    return fail(KPOOL_EINVAL, "%s: need 0 <= q_lo <= q_hi <= T (q_lo=%lld q_hi=%lld T=%lld)", fn,
                (long long)q_lo, (long long)q_hi, (long long)T);
  if (!kpool::score_supported(H, D))
    return fail(KPOOL_EUNSUPPORTED, "%s: (H=%d, D=%d) not compiled; supported (4,16) and (32,128)", fn, H, D);
  constexpr uint32_t kKnown = KPOOL_FLAG_OVERLAP | KPOOL_FLAG_TAIL;
  if (flags & ~kKnown) return fail(KPOOL_EINVAL, "%s: unknown flags 0x%x", fn, flags & ~kKnown);
  const bool tail = flags & KPOOL_FLAG_TAIL;
  if (q_lo == q_hi) return ok();
  std::vector<int32_t> cu_pools(nseq + 1);
  int32_t max_pools = 0;
  kpool_count_pools(cu_seqlens_host, nseq, kpool, tail ? KPOOL_FLAG_TAIL : 0u, cu_pools.data(),
                    &max_pools);
  // (kp may be null only when there is no pool to read)
  if (!q || (!kp && max_pools > 0) || !w || !cu_seqlens_dev || !pool_ids)
    return fail(KPOOL_EINVAL, "%s: null pointer", fn);
  if (!aligned16(q) || !aligned16(kp) || !aligned16(w))
    return fail(KPOOL_EINVAL, "%s: q, kp and w must be 16-byte aligned", fn);
  // The score kernel addresses one sequence's pooled keys and one chunk's score rows
  // with 32-bit byte offsets: a sequence's keys must stay below 4 GiB (16M pools at
  // D = 128) and one score row within the 2 GiB chunk cap.
  if ((int64_t)max_pools * D * 2 > (int64_t)0xFFFFFFFF || pitch_of(max_pools) * 4 > kChunkCapBytes)
    return fail(KPOOL_EUNSUPPORTED, "%s: a sequence of %d pools is beyond the supported size", fn,
                max_pools);
  hipStream_t st = (hipStream_t)stream;
  if (max_pools == 0) {
    // No sequence has a pool (tail mode, every sequence shorter than kpool): nothing to
    // score.  The selection kernel reads no score of a row without visible pools and
    // writes its ids as -1; scores_out has no columns.
    hipError_t e = timed_if(!use_scratch, 2, st, [&] {
      return kpool::launch_topk(nullptr, 0, q_hi - q_lo, nullptr, cu_seqlens_dev, nseq, q_lo, kpool,
                                tail, budget, pool_ids, nullptr, 0, st);
    });
    if (e != hipSuccess) return hip_fail(fn, e);
    return ok();
  }
  const int64_t ld = pitch_of(max_pools);
  const int64_t ldg = ld / kpool::kGroup;
  const int64_t row_bytes = ws_row_bytes(ld);
  if (use_scratch) {
    if (row_bytes > (int64_t)kScratchBytes)
      return fail(KPOOL_EWORKSPACE,
                  "%s: one score row needs %lld bytes, beyond the %lld-byte static scratch (a "
                  "sequence of %d pools; at most %lld pools fit)", fn, (long long)row_bytes,
                  (long long)kScratchBytes, max_pools, (long long)(kScratchBytes / 4 * 16 / 17));
    hipError_t e = scratch_ptr(st, &workspace);
    if (e != hipSuccess) return hip_fail(fn, e);
    workspace_bytes = kScratchBytes;
    flags &= ~(uint32_t)KPOOL_FLAG_OVERLAP;
  }
  if (!workspace || (int64_t)workspace_bytes < row_bytes)
    return fail(KPOOL_EWORKSPACE, "%s: workspace must hold one score row (%lld bytes), got %zu", fn,
                (long long)row_bytes, workspace_bytes);
  if (!aligned16(workspace)) return fail(KPOOL_EINVAL, "%s: workspace must be 16-byte aligned", fn);
  // With KPOOL_FLAG_OVERLAP and a workspace of at least two rows, two chunk buffers:
  // chunks then alternate between the caller's stream and a helper stream, so one
  // chunk's selection and the next chunk's scoring overlap instead of draining the GPU
  // between launches.  Each buffer's fp32 score rows stay within the 2 GiB cap.
  const ChunkPlan plan = plan_chunks(ld, workspace_bytes, flags & KPOOL_FLAG_OVERLAP);
  const int nbuf = plan.nbuf;
  const int64_t chunk_rows = plan.rows;
  const int64_t nchunks = (q_hi - q_lo + chunk_rows - 1) / chunk_rows;
  float *ws_buf[2], *gws_buf[2];
  for (int b = 0; b < 2; ++b) {
    ws_buf[b] = (float *)((char *)workspace + (b % nbuf) * chunk_rows * row_bytes);
    gws_buf[b] = ws_buf[b] + chunk_rows * ld;  // group maxima follow the score rows
  }
  const int tile_rows = kpool::score_tile_rows();
  // score workgroups the device runs at once, for the segment plan below (0: unknown)
  int slots = 0;
  {
    int dev = 0;
    if ((st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev)) == hipSuccess)
      slots = kpool::score_slots(H, D, dev);
  }

  // score + select of rows [c0, c1) into one buffer, on one stream
  auto enqueue_chunk = [&](int64_t c0, int64_t c1, float *ws, float *gws, hipStream_t cs) -> hipError_t {
    // sequences overlapping [c0, c1): one segment each, cut into row tiles
    struct Seg { int32_t lo, hi, start, pool_base, pool_count; };
    std::vector<Seg> segs;
    int s = (int)(std::upper_bound(cu_seqlens_host, cu_seqlens_host + nseq + 1, (int32_t)c0) -
                  cu_seqlens_host) - 1;
    for (; s < nseq && cu_seqlens_host[s] < c1; ++s) {
      const int64_t lo = std::max<int64_t>(c0, cu_seqlens_host[s]);
      const int64_t hi = std::min<int64_t>(c1, cu_seqlens_host[s + 1]);
      if (lo < hi)
        segs.push_back({(int32_t)lo, (int32_t)hi, cu_seqlens_host[s], cu_pools[s],
                        cu_pools[s + 1] - cu_pools[s]});
    }
    for (size_t g0 = 0; g0 < segs.size(); g0 += kpool::kMaxSegs) {
      kpool::SegList L{};
      int32_t ntiles = 0, max_npv = 0;
      for (size_t g = g0; g < std::min(segs.size(), g0 + kpool::kMaxSegs); ++g) {
        const Seg &sg = segs[g];
        const int j = L.nseg++;
        L.tile_start[j] = ntiles;
        L.row_lo[j] = sg.lo;
        L.row_hi[j] = sg.hi;
        L.seq_start[j] = sg.start;
        L.pool_base[j] = sg.pool_base;
        L.pool_count[j] = sg.pool_count;
        ntiles += (sg.hi - sg.lo + tile_rows - 1) / tile_rows;
        max_npv = std::max<int32_t>(max_npv, std::min((sg.hi - 1 - sg.start) / kpool + 1, sg.pool_count));
      }
      L.tile_start[L.nseg] = ntiles;
      // No row of these sequences sees a pool (tail mode: each is shorter than kpool), so
      // there is nothing to score; the selection writes their ids as -1 without reading
      // scores, and the scores_out copy writes -inf.  (A zero-segment launch would have
      // an empty grid.)
      if (max_npv == 0) continue;
      // Pool segments per tile: at most KPOOL_SCORE_TARGET_WGS workgroups per launch (4 per
      // CU), segments of 64..kPoolSegMax pools; fewer, longer workgroups reload q less
      // often.  Among the segment counts from that target down to the fewest the size cap
      // allows, take the one whose rounds of workgroups over the device's slots, each as
      // long as one segment, cover the tiles soonest: a last round that is nearly empty
      // costs a whole segment's time.  Ties keep more segments.
      auto seg_pools = [&](int64_t ns) {
        const int64_t ps = (max_npv + ns - 1) / ns;
        return std::min<int64_t>(kPoolSegMax, std::max<int64_t>(64, (ps + 63) / 64 * 64));
      };
      const int64_t want_segs =
          std::max<int64_t>(1, (KPOOL_SCORE_TARGET_WGS + ntiles - 1) / ntiles);
      const int64_t min_segs = std::max<int64_t>(1, (max_npv + kPoolSegMax - 1) / kPoolSegMax);
      int64_t pseg = seg_pools(want_segs);
      if (slots > 0) {
        int64_t best = -1;
        for (int64_t ns = std::max(want_segs, min_segs); ns >= min_segs; --ns) {
          const int64_t ps = seg_pools(ns);
          const int64_t nwg = (int64_t)ntiles * ((max_npv + ps - 1) / ps);
          const int64_t cost = (nwg + slots - 1) / slots * ps;
          if (best < 0 || cost < best) {
            best = cost;
            pseg = ps;
          }
        }
      }
      const int32_t npseg = (int32_t)((max_npv + pseg - 1) / pseg);
      hipError_t e = timed_if(!use_scratch, 1, cs, [&] {
        return kpool::launch_score(H, D, q, kp, w, scale, kpool, L, ntiles, npseg, (int32_t)pseg,
                                   c0, ld, ws, ldg, gws, cs);
      });
      if (e != hipSuccess) return e;
    }
    hipError_t e = timed_if(!use_scratch, 2, cs, [&] {
      return kpool::launch_topk(ws, ld, c1 - c0, nullptr, cu_seqlens_dev, nseq, c0, kpool, tail, budget,
                                pool_ids + (c0 - q_lo) * budget, gws, ldg, cs);
    });
    if (e != hipSuccess) return e;
    if (scores_out) {
      e = timed_if(!use_scratch, 4, cs, [&] {
        return kpool::launch_scores_copy(ws, ld, c1 - c0, cu_seqlens_dev, nseq, c0, kpool, tail,
                                         scores_out + (c0 - q_lo) * max_pools, max_pools, cs);
      });
    }
    return e;
  };

  if (nbuf == 1 || nchunks == 1) {
    for (int64_t c0 = q_lo; c0 < q_hi; c0 += chunk_rows) {
      hipError_t e = enqueue_chunk(c0, std::min(q_hi, c0 + chunk_rows), ws_buf[0], gws_buf[0], st);
      if (e != hipSuccess) return hip_fail(fn, e);
    }
    return ok();
  }
  // chunk c goes to buffer c % 2 on stream c % 2; chunk c + 2 reuses the buffer after
  // chunk c's selection because both sit on the same stream
  Aux *aux = nullptr;
  hipError_t e = get_aux(st, &aux);
  if (e != hipSuccess) return hip_fail(fn, e);
  std::lock_guard<std::mutex> guard(aux->mu);
  hipStream_t streams[2] = {st, aux->helper};
  e = hipEventRecord(aux->fork, st);
  if (e == hipSuccess) e = hipStreamWaitEvent(aux->helper, aux->fork, 0);
  if (e != hipSuccess) return hip_fail(fn, e);
  hipError_t first_err = hipSuccess;
  int64_t c = 0;
  for (int64_t c0 = q_lo; c0 < q_hi && first_err == hipSuccess; c0 += chunk_rows, ++c)
    first_err = enqueue_chunk(c0, std::min(q_hi, c0 + chunk_rows), ws_buf[c & 1], gws_buf[c & 1],
                              streams[c & 1]);
  // join: the caller's stream waits for the helper whatever happened above
  e = hipEventRecord(aux->join, aux->helper);
  if (e == hipSuccess) e = hipStreamWaitEvent(st, aux->join, 0);
  if (first_err != hipSuccess) return hip_fail(fn, first_err);
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

}  // namespace

extern "C" {

const char *kpool_last_error(void) { return g_err.c_str(); }

int kpool_version(void) { return 300; }

int64_t kpool_count_pools(const int32_t *cu_seqlens_host, int32_t nseq, int32_t kpool,
                          uint32_t flags, int32_t *cu_pools_host, int32_t *max_pools_out) {
  int rc = check_cu(cu_seqlens_host, nseq, "kpool_count_pools");
  if (rc) return rc;
  if (kpool < 1) return fail(KPOOL_EINVAL, "kpool_count_pools: kpool must be >= 1 (got %d)", kpool);
  if (flags & ~(uint32_t)KPOOL_FLAG_TAIL)
    return fail(KPOOL_EINVAL, "kpool_count_pools: unknown flags 0x%x", flags);
  const bool tail = flags & KPOOL_FLAG_TAIL;
  int64_t tot = 0;
  int32_t mx = 0;
  if (cu_pools_host) cu_pools_host[0] = 0;
  for (int32_t s = 0; s < nseq; ++s) {
    const int64_t L = (int64_t)cu_seqlens_host[s + 1] - cu_seqlens_host[s];
    const int64_t np = tail ? L / kpool : (L + kpool - 1) / kpool;
    tot += np;
    mx = std::max<int32_t>(mx, (int32_t)np);
    if (cu_pools_host) cu_pools_host[s + 1] = (int32_t)tot;
  }
  if (max_pools_out) *max_pools_out = mx;
  ok();
  return tot;
}

int kpool_pool_keys(const uint16_t *k, const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                    const int32_t *cu_pools_dev, int32_t nseq, int32_t D, int32_t kpool, uint32_t flags,
                    uint16_t *kp, void *stream) {
  const char *fn = "kpool_pool_keys";
  int rc = check_cu(cu_seqlens_host, nseq, fn);
  if (rc) return rc;
  if (kpool < 1) return fail(KPOOL_EINVAL, "%s: kpool must be >= 1 (got %d)", fn, kpool);
  if (D < 8 || D > 1024 || D % 8) return fail(KPOOL_EINVAL, "%s: D must be a multiple of 8 in [8, 1024] (got %d)", fn, D);
  const int64_t P_tot = kpool_count_pools(cu_seqlens_host, nseq, kpool, flags, nullptr, nullptr);
  if (P_tot < 0) return (int)P_tot;
  if (P_tot == 0) return ok();
  if (!k || !kp || !cu_seqlens_dev || !cu_pools_dev) return fail(KPOOL_EINVAL, "%s: null pointer", fn);
  if (!aligned16(k) || !aligned16(kp)) return fail(KPOOL_EINVAL, "%s: k and kp must be 16-byte aligned", fn);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(0, st, [&] {
    return kpool::launch_pool_keys(k, cu_seqlens_dev, cu_pools_dev, nseq, D, kpool, P_tot, kp, st);
  });
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

size_t kpool_workspace_bytes(int64_t q_lo, int64_t q_hi, int32_t max_pools, int32_t nbuf) {
  if (q_hi <= q_lo || max_pools <= 0 || (nbuf != 1 && nbuf != 2)) return 0;
  const int64_t ld = pitch_of(max_pools);
  const int64_t cap_rows = std::max<int64_t>(1, kChunkCapBytes / (ld * 4));
  // nbuf full chunk buffers when the rows need more than one chunk
  return (size_t)(std::min<int64_t>(q_hi - q_lo, nbuf * cap_rows) * ws_row_bytes(ld));
}

int64_t kpool_chunk_rows(int32_t max_pools, size_t workspace_bytes, uint32_t flags,
                         int32_t *nbuf_out) {
  if (max_pools <= 0) return fail(KPOOL_EINVAL, "kpool_chunk_rows: max_pools must be >= 1");
  if (flags & ~(uint32_t)(KPOOL_FLAG_OVERLAP | KPOOL_FLAG_TAIL))
    return fail(KPOOL_EINVAL, "kpool_chunk_rows: unknown flags 0x%x", flags);
  const int64_t ld = pitch_of(max_pools);
  if ((int64_t)workspace_bytes < ws_row_bytes(ld))
    return fail(KPOOL_EWORKSPACE, "kpool_chunk_rows: workspace smaller than one score row");
  const ChunkPlan plan = plan_chunks(ld, workspace_bytes, flags & KPOOL_FLAG_OVERLAP);
  if (nbuf_out) *nbuf_out = plan.nbuf;
  ok();
  return plan.rows;
}

int kpool_score_topk(const uint16_t *q, const uint16_t *kp, const float *w,
                     const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev, int32_t nseq,
                     int32_t H, int32_t D, int32_t kpool, float scale, int64_t q_lo, int64_t q_hi,
                     int32_t budget, void *workspace, size_t workspace_bytes, uint32_t flags,
                     int32_t *pool_ids, float *scores_out, void *stream) {
  return score_topk_impl("kpool_score_topk", q, kp, w, cu_seqlens_host, cu_seqlens_dev, nseq, H, D,
                         kpool, scale, q_lo, q_hi, budget, workspace, workspace_bytes, flags, false,
                         pool_ids, scores_out, stream);
}

int kpool_score_topk_noalloc(const uint16_t *q, const uint16_t *kp, const float *w,
                             const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                             int32_t nseq, int32_t H, int32_t D, int32_t kpool, float scale,
                             int64_t q_lo, int64_t q_hi, int32_t budget, uint32_t flags,
                             int32_t *pool_ids, float *scores_out, void *stream) {
  return score_topk_impl("kpool_score_topk_noalloc", q, kp, w, cu_seqlens_host, cu_seqlens_dev, nseq,
                         H, D, kpool, scale, q_lo, q_hi, budget, nullptr, 0, flags, true, pool_ids,
                         scores_out, stream);
}

int kpool_pool_keys_gated(const uint16_t *k, const uint16_t *g, const float *ape,
                          const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                          const int32_t *cu_pools_dev, int32_t nseq, int32_t D, int32_t kpool,
                          uint32_t flags, uint16_t *kp, void *stream) {
  const char *fn = "kpool_pool_keys_gated";
  int rc = check_cu(cu_seqlens_host, nseq, fn);
  if (rc) return rc;
  if (kpool < 1) return fail(KPOOL_EINVAL, "%s: kpool must be >= 1 (got %d)", fn, kpool);
  if (D < 8 || D > 1024 || D % 8) return fail(KPOOL_EINVAL, "%s: D must be a multiple of 8 in [8, 1024] (got %d)", fn, D);
  const int64_t P_tot = kpool_count_pools(cu_seqlens_host, nseq, kpool, flags, nullptr, nullptr);
  if (P_tot < 0) return (int)P_tot;
  if (P_tot == 0) return ok();
  if (!k || !g || !ape || !kp || !cu_seqlens_dev || !cu_pools_dev) return fail(KPOOL_EINVAL, "%s: null pointer", fn);
  if (!aligned16(k) || !aligned16(g) || !aligned16(ape) || !aligned16(kp))
    return fail(KPOOL_EINVAL, "%s: k, g, ape and kp must be 16-byte aligned", fn);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(0, st, [&] {
    return kpool::launch_pool_keys_gated(k, g, ape, cu_seqlens_dev, cu_pools_dev, nseq, D, kpool,
                                         P_tot, kp, st);
  });
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int kpool_expand(const int32_t *pool_ids, const int32_t *cu_seqlens_host, const int32_t *cu_seqlens_dev,
                 int32_t nseq, int32_t kpool, int64_t q_lo, int64_t q_hi, int32_t budget,
                 uint32_t flags, int32_t *token_ids, void *stream) {
  const char *fn = "kpool_expand";
  int rc = check_cu(cu_seqlens_host, nseq, fn);
  if (rc) return rc;
  const int64_t T = cu_seqlens_host[nseq];
  if (kpool < 1) return fail(KPOOL_EINVAL, "%s: kpool must be >= 1 (got %d)", fn, kpool);
  if (budget < 1) return fail(KPOOL_EINVAL, "%s: budget must be >= 1 (got %d)", fn, budget);
  if (flags & ~(uint32_t)KPOOL_FLAG_TAIL) return fail(KPOOL_EINVAL, "%s: unknown flags 0x%x", fn, flags);
  const bool tail = flags & KPOOL_FLAG_TAIL;
  if (q_lo < 0 || q_lo > q_hi || q_hi > T)
    return fail(KPOOL_EINVAL, "%s: need 0 <= q_lo <= q_hi <= T", fn);
  if (q_lo == q_hi) return ok();
  if (!pool_ids || !token_ids || !cu_seqlens_dev) return fail(KPOOL_EINVAL, "%s: null pointer", fn);
  if (kpool == 4 && !tail && !aligned16(token_ids))
    return fail(KPOOL_EINVAL, "%s: token_ids must be 16-byte aligned", fn);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(3, st, [&] {
    return kpool::launch_expand(pool_ids, cu_seqlens_dev, nseq, kpool, tail, q_lo, q_hi - q_lo, budget,
                                token_ids, st);
  });
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int kpool_topk(const float *scores, int64_t ld, const int32_t *n_valid, int64_t rows, int32_t budget,
               int32_t *pool_ids, void *stream) {
  const char *fn = "kpool_topk";
  if (rows < 0) return fail(KPOOL_EINVAL, "%s: rows must be >= 0", fn);
  if (budget < 1 || budget > kpool::kTopkMaxBudget)
    return fail(KPOOL_EINVAL, "%s: budget must be in [1, %d] (got %d)", fn, kpool::kTopkMaxBudget, budget);
  if (ld < 0 || ld % 4) return fail(KPOOL_EINVAL, "%s: ld must be a non-negative multiple of 4", fn);
  if (rows == 0) return ok();
  if (!scores || !n_valid || !pool_ids) return fail(KPOOL_EINVAL, "%s: null pointer", fn);
  if (!aligned16(scores)) return fail(KPOOL_EINVAL, "%s: scores must be 16-byte aligned", fn);
  if (rows > 0x7FFFFFFF) return fail(KPOOL_EINVAL, "%s: too many rows", fn);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(2, st, [&] {
    return kpool::launch_topk(scores, ld, rows, n_valid, nullptr, 0, 0, 1, false, budget, pool_ids,
                              nullptr, 0, st);
  });
  if (e != hipSuccess) return hip_fail(fn, e);
  return ok();
}

int kpool_profile_enable(int on) {
  g_prof_on = on != 0;
  return ok();
}

int kpool_profile_collect(double *ms, int64_t *launches) {
  int rc = KPOOL_OK;
  for (ProfRec &r : g_prof) {
    float t = 0.0f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
    if (e != hipSuccess && rc == KPOOL_OK) rc = hip_fail("kpool_profile_collect", e);
    if (ms) ms[r.kind] += t;
    if (launches) launches[r.kind] += 1;
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  g_prof.clear();
  if (rc == KPOOL_OK) ok();
  return rc;
}

}  // extern "C"
