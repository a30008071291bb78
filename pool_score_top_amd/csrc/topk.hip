// Per-row top-k over fp32 score rows with the deterministic tie-break.
//
// Pages: Atlas inference glm5next_dsa/tp.rs module doc (the selection keeps
// the higher score and, on equal scores, the smaller pool index, because a
// library top-k leaves tie order undefined); Megatron-LM PR #8299 "Change"
// (int32 pool ids, budget = index_topk / kpool pools per row).
//
// Each element is ranked by the 64-bit key (order_key(score) << 32 | ~index):
// a larger key is better, and keys are unique, so "the best `budget` keys" is
// exactly the selection.  One workgroup owns one row, and several of them share
// a CU, so their memory latencies overlap.  Three instances, by budget: 256
// threads with NMAX = 4 maxima per thread up to 512, 512 threads with NMAX = 4 up
// to 1024, and 512 threads with NMAX = 8 up to 2048.
//
//   pass 1  (HBM)   every thread keeps NMAX maxima over disjoint parts of its
//                   elements (or, for long rows, of its 16-pool group maxima,
//                   written by the score kernel; the first round of those is
//                   requested before the row's length is known).  In each wave
//                   the ceil(budget/waves)-th largest of its 64*NMAX maxima is
//                   found by a binary search on a ballot count; the minimum L
//                   over the waves is a lower bound on the budget-th best key (at
//                   least budget distinct elements reach it).
//   pass 2  (L2)    elements with key >= L (for long rows: only inside the
//                   groups whose max reaches L) are appended to an LDS candidate
//                   list with one atomic per wave per step.  For iid scores the
//                   list holds about 0.7 x (number of maxima) entries, whatever
//                   the row length.
//   cut             when the list is longer than budget and that would double
//                   the sort, a radix select over the LDS list keeps exactly the
//                   best `budget` keys.
//   sort            bitonic sort of the candidates (descending 64-bit keys) with
//                   each thread holding consecutive keys: short distances inside
//                   a thread, then lane shuffles, then LDS; the first `budget`
//                   are written.
//   fallback        if the list overflows (heavy ties), an exact radix select
//                   over the 64-bit keys (8-bit digits, re-reading the row)
//                   finds the budget-th key and collects exactly budget
//                   elements, which are then sorted the same way.
// Rows with no more than `budget` elements keep them all: their keys go straight into
// the list and are sorted, with no bound, append or cut.  Unused output slots are -1.
#include <type_traits>

#include "kpool_internal.h"

namespace kpool {
namespace {

constexpr uint32_t kNegInfKey = 0x007FFFFFu;  // order_key(-inf)

// Three instances, by budget:
//   small   budgets up to 512:   256 threads, NMAX 4 (1024 maxima), lists of 1280;
//   medium  budgets up to 1024:  512 threads, NMAX 4 (2048 maxima), lists of 2560;
//   large   budgets up to 2048:  512 threads, NMAX 8 (4096 maxima), lists of 4096.
// Each way a wave's bound is at most its median maximum, so at most about ln 2 x
// (number of maxima) candidates are expected, plus the spread of the minimum over
// waves (iid rows of 16k-131k pools at budget 512: about 775 candidates in about 740
// groups, at most 930 and 880 over 200 rows).  The top-k is latency-bound, so the
// instances are sized for rows in flight: the small one's lists (16.4 KB of LDS) and
// rounds of 8 group maxima or 4 score pieces per thread (54 VGPRs) let eight rows
// share a CU, the limit of eight waves per SIMD; the medium one's (31 KB) four rows of
// 8 waves; the large one's (49 KB) three.  (Before the medium instance, budgets
// 513-1024 ran on the large one: 27.3 vs 19.3 ms of top-k per 512k step at budget
// 1024.)  A row that overflows a list takes the exact path, so the caps bound speed,
// not results.
template <int I>
struct Inst;
// small: budgets up to 512
template <>
struct Inst<0> {
  static constexpr int kNmax = 4, kThreads = 256, kCand = 1280, kMaxBudget = 512;
};
// medium: budgets 513 .. 1024
template <>
struct Inst<1> {
  static constexpr int kNmax = 4, kThreads = 512, kCand = 2560, kMaxBudget = 1024;
};
// large: budgets 1025 .. 2048
template <>
struct Inst<2> {
  static constexpr int kNmax = 8, kThreads = 512, kCand = 4096, kMaxBudget = kTopkMaxBudget;
};
template <int I>
struct Cfg {
  static constexpr int kNmax = Inst<I>::kNmax;
  static constexpr int kThreads = Inst<I>::kThreads;
  static constexpr int kWaves = kThreads / 64;
  static constexpr int kRound = 8;   // group maxima per thread per round
  static constexpr int kPieces = 4;  // 16-byte score pieces per thread per round
  static constexpr int kCand = Inst<I>::kCand;   // candidate keys in LDS
  static constexpr int kGroups = kCand;          // candidate 16-pool groups
  static constexpr int kMaxBudget = Inst<I>::kMaxBudget;
  static_assert(kNmax == 4 || kNmax == 8, "maxima per thread");
  // the cut gathers `budget` keys into the group list's space
  static_assert(kGroups / 2 >= kMaxBudget, "cut buffer");
  // a list longer than the budget's sort size is cut first, so sorts span at most
  // max(budget, that size) <= 4 kThreads keys
  static_assert(kMaxBudget <= 4 * kThreads && 4 * kThreads <= kCand, "sort sizes");
};

__device__ inline uint64_t compose(uint32_t okey, uint32_t idx) {
  return ((uint64_t)okey << 32) | (uint64_t)(~idx);
}
// Candidates are appended as (float bits << 32 | ~index) and turned into keys once
// the list is complete, where it is dense.
__device__ inline uint64_t compose_raw(float x, uint32_t idx) {
  return ((uint64_t)__float_as_uint(x) << 32) | (uint64_t)(~idx);
}
__device__ inline uint64_t raw_to_key(uint64_t r) {
  return ((uint64_t)order_key(__uint_as_float((uint32_t)(r >> 32))) << 32) | (r & 0xFFFFFFFFull);
}

// The float whose order key is k, for k = 0 (a NaN) or a key of a non-NaN value
// (k >= order_key(-inf)); with it, order_key(x) >= k reads as x >= key_float(k)
// for every non-NaN x when k != 0, and NaN (key 0) never passes.
__device__ inline float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// The rank-th largest (1-based, duplicates counted) of the wave's 64*NMAX values: the
// largest t with at least `rank` values >= t, found by a binary search over t's bits
// from the top (t = the bits decided so far with this bit set; keep the bit if enough
// values reach t).  One compare per value and bit, against a wave-uniform threshold;
// the counts are ballots.  The result is wave-uniform.
template <int NMAX>
__device__ inline uint32_t wave_kth_desc(const uint32_t (&x)[NMAX], int rank) {
  uint32_t v = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    const uint32_t t = v | (1u << b);
    int cnt = 0;
#pragma unroll
    for (int i = 0; i < NMAX; ++i) cnt += __popcll(__ballot(x[i] >= t));
    if (cnt >= rank) v = t;
  }
  return v;
}

// The value of lane (lane ^ D), D a power of two below 64, with D known at compile
// time: quad permutations for 1 and 2 (DPP), a fixed-pattern swizzle within 32 lanes for
// 4 to 16, and for 32 the half-wave swap (permlane32_swap(x, x) gives [x.lo, x.lo] and
// [x.hi, x.hi]).  No lane address is computed, and a stage's exchanges of all its keys
// are issued before the first is waited for.  (Measured against a generic lane
// permute: the selection is 2.4% faster at budget 512 and 5% at budget 2048; DPP or the
// 16-lane swap for distances 8 and 16, or swizzles for 1 and 2, were slower.)
template <int D>
__device__ inline uint32_t lanes_xor(uint32_t x) {
  if constexpr (D == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xB1, 0xF, 0xF, false);
  else if constexpr (D == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4E, 0xF, 0xF, false);
  else if constexpr (D < 32) return (uint32_t)__builtin_amdgcn_ds_swizzle((int)x, 0x1F | (D << 10));
  else {
    const auto z = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    return (__lane_id() & 32) ? z[0] : z[1];
  }
}
template <int D>
__device__ inline uint64_t lanes_xor_u64(uint64_t v) {
  return ((uint64_t)lanes_xor<D>((uint32_t)(v >> 32)) << 32) | lanes_xor<D>((uint32_t)v);
}
// The compare-exchange stages of one bitonic merge step k at lane distances D, D/2, ..
// 1 (distance j = D*M keys, those with j <= k/2).
template <int D, int M>
__device__ inline void lane_stages(uint64_t (&v)[M], int k, int tid, int e0) {
  if constexpr (D >= 1) {
    if (D * M <= (k >> 1)) {
      const bool lower = (tid & D) == 0;
      const bool desc = (e0 & k) == 0;
      uint64_t p[M];
#pragma unroll
      for (int m = 0; m < M; ++m) p[m] = lanes_xor_u64<D>(v[m]);
#pragma unroll
      for (int m = 0; m < M; ++m) v[m] = ((p[m] > v[m]) == (lower == desc)) ? p[m] : v[m];
    }
    lane_stages<D / 2, M>(v, k, tid, e0);
  }
}

// Bitonic sort (descending) of kThreads*M keys in a blocked layout: thread t holds
// elements t*M .. t*M + M-1 in v[0..M-1].  Compare-exchange distances j < M stay in a
// thread's registers, M <= j < 64M are lane shuffles within a wave, and only larger
// ones go through LDS (buf: kThreads*M keys, laid out m-major so that every LDS access
// of a wave is to consecutive keys).  Small distances are the most frequent stages of a
// bitonic sort, so most of them cost no communication.
template <int M, int kThreads>
__device__ void block_sort_desc(uint64_t (&v)[M], uint64_t *buf, int tid) {
  constexpr int N = kThreads * M;
  const int e0 = tid * M;
#pragma unroll 1
  for (int k = 2; k <= N; k <<= 1) {
    // distances through LDS
#pragma unroll 1
    for (int j = k >> 1; j >= 64 * M; j >>= 1) {
      const int d = j / M;
      __syncthreads();
#pragma unroll
      for (int m = 0; m < M; ++m) buf[m * kThreads + tid] = v[m];
      __syncthreads();
      const bool lower = (tid & d) == 0;
      const bool desc = (e0 & k) == 0;
#pragma unroll
      for (int m = 0; m < M; ++m) {
        const uint64_t p = buf[m * kThreads + (tid ^ d)];
        v[m] = ((p > v[m]) == (lower == desc)) ? p : v[m];  // larger kept when lower == desc
      }
    }
    // distances across lanes of one wave (larger kept when lower == desc)
    lane_stages<32, M>(v, k, tid, e0);
    // distances inside a thread
#pragma unroll
    for (int j = M / 2; j > 0; j >>= 1) {
      if (j < k) {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          if ((m & j) == 0) {
            const bool desc = ((e0 + m) & k) == 0;
            const uint64_t a = v[m], b = v[m | j];
            const bool sw = (a < b) == desc;  // (keys are unique; equal padding zeros need no swap)
            v[m] = sw ? b : a;
            v[m | j] = sw ? a : b;
          }
        }
      }
    }
  }
}

template <int M, int kThreads>
__device__ void sort_and_write(uint64_t *cand, uint32_t count, int budget, int32_t *orow, int tid) {
  uint64_t v[M];
  // the starting order is free: read the list m-major (consecutive keys per wave access)
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const uint32_t i = m * kThreads + tid;
    v[m] = i < count ? cand[i] : 0ull;  // 0 is below every real key
  }
  block_sort_desc<M, kThreads>(v, cand, tid);
#pragma unroll
  for (int m = 0; m < M; ++m) {
    const int i = tid * M + m;
    if (i < budget) orow[i] = (v[m] != 0ull) ? (int32_t)(~(uint32_t)v[m]) : -1;
  }
  // output slots past the sort size: the row has fewer candidates than that
  for (int i = M * kThreads + tid; i < budget; i += kThreads) orow[i] = -1;
}

template <int I>
struct Smem {
  uint64_t cand[Cfg<I>::kCand];
  uint32_t glist[Cfg<I>::kGroups];
  uint32_t hist[256];
  uint32_t wave_bound[Cfg<I>::kWaves];
  uint32_t wave_max[Cfg<I>::kWaves];
  uint64_t prefix;
  uint32_t count;
  uint32_t gcount;
  uint32_t scount;
  int32_t pbits;
  int32_t krem;
  int32_t done;
};

// Wave-aggregated append: lanes with c (0 .. 2^BITS - 1) items reserve c consecutive
// slots of *counter with one LDS atomic per wave; returns this lane's first slot.
template <int BITS>
__device__ inline uint32_t wave_reserve(uint32_t c, uint32_t *counter, int lane) {
  uint64_t b[BITS];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i) {
    b[i] = __ballot(c & (1u << i));
    tot += (uint32_t)__popcll(b[i]) << i;
  }
  if (tot == 0) return 0;
  uint32_t pre = 0;
#pragma unroll
  for (int i = 0; i < BITS; ++i)
    pre += __builtin_amdgcn_mbcnt_hi((uint32_t)(b[i] >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)b[i], 0u)) << i;
  uint32_t base = 0;
  if (lane == 0) base = atomicAdd(counter, tot);
  return __builtin_amdgcn_readfirstlane(base) + pre;  // every lane is active here
}

// One radix-select step, run by one whole wave: hist holds the 256 counts of the next
// 8-bit digit among the keys that match the current prefix.  From the top digit down,
// find the digit at which the running count reaches krem, and leave the narrowed state
// (prefix, pbits, krem, done) in sm.  Lane L looks after digits 255-4L .. 252-4L.
template <class SM>
__device__ inline void next_digit(SM &sm, uint64_t prefix, int pbits, int krem, int lane) {
  uint32_t c[4];
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[i] = sm.hist[255 - 4 * lane - i];
    tot += c[i];
  }
  // inclusive prefix over lanes, i.e. over digits from the top: within each 16-lane row
  // by shifted adds (DPP row_shr, lanes shifted in from outside the row read 0), then the
  // totals of the rows before
  uint32_t incl = tot;
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x111, 0xF, 0xF, false);  // row_shr:1
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x112, 0xF, 0xF, false);  // row_shr:2
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x114, 0xF, 0xF, false);  // row_shr:4
  incl += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x118, 0xF, 0xF, false);  // row_shr:8
  {
    const uint32_t r0 = __builtin_amdgcn_readlane(incl, 15), r1 = __builtin_amdgcn_readlane(incl, 31),
                   r2 = __builtin_amdgcn_readlane(incl, 47);
    const int row = lane >> 4;
    incl += (row >= 1 ? r0 : 0u) + (row >= 2 ? r1 : 0u) + (row >= 3 ? r2 : 0u);
  }
  const uint32_t excl = incl - tot;
  // the digits hold at least krem keys in all, so some lane reaches it
  const uint64_t hit = __ballot(incl >= (uint32_t)krem);
  if (lane == __ffsll((unsigned long long)hit) - 1) {
    uint32_t cum = excl;
    int i = 0;
    for (; i < 3; ++i) {
      if (cum + c[i] >= (uint32_t)krem) break;
      cum += c[i];
    }
    const int rem = krem - (int)cum;
    sm.krem = rem;
    sm.prefix = (prefix << 8) | (uint64_t)(255 - 4 * lane - i);
    sm.pbits = pbits + 8;
    sm.done = (c[i] == (uint32_t)rem) ? 1 : 0;
  }
}

// Append the elements of one float4 piece at `base` whose key reaches the bound
// (take_all: the bound is key 0, which every element reaches; otherwise the test is
// x >= bf in floats, see key_float), in raw form.  (Positions are 32-bit: a row
// holds fewer than 2^31 elements.)
template <int I>
__device__ inline void append_piece(const float4 x, int32_t base, int32_t n, bool take_all, float bf,
                                    Smem<I> &sm, int lane) {
  constexpr int kCandCap = Cfg<I>::kCand;
  const float xs[4] = {x.x, x.y, x.z, x.w};
  // One ballot per element slot: the wave's selected elements of slot e go to
  // consecutive positions after those of slots 0 .. e-1 (the list's order is free).
  bool sel[4];
  uint64_t msk[4];
  uint32_t off[4], tot = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // (bitwise, so that each test stays a lane mask)
    sel[e] = (base + e < n) & (take_all | (xs[e] >= bf));
    msk[e] = __ballot(sel[e]);
    off[e] = tot;
    tot += (uint32_t)__popcll(msk[e]);
  }
  if (tot == 0) return;  // wave-uniform
  uint32_t wbase = 0;
  if (lane == 0) wbase = atomicAdd(&sm.count, tot);
  wbase = __builtin_amdgcn_readfirstlane(wbase);  // every lane is active here
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (sel[e]) {
      const uint32_t pos = wbase + off[e] +
          __builtin_amdgcn_mbcnt_hi((uint32_t)(msk[e] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk[e], 0u));
      if (pos < (uint32_t)kCandCap) sm.cand[pos] = compose_raw(xs[e], (uint32_t)(base + e));
    }
  }
}

// GMAX: the score kernel's per-row maxima of 16-pool groups are available (row pitch
// ldg).  For long rows the bound then comes from the group maxima, and only the
// groups whose max reaches it are read.
template <bool GMAX, int I>
__global__ __launch_bounds__(Cfg<I>::kThreads) void topk_kernel(const float *__restrict__ scores, int64_t ld,
                                                        const int32_t *__restrict__ n_valid,
                                                        const int32_t *__restrict__ cu_seqlens,
                                                        int nseq, int64_t grow0, int kpool,
                                                        bool tail, int budget,
                                                        int32_t *__restrict__ out,
                                                        const float *__restrict__ gmax,
                                                        int64_t ldg) {
  constexpr int NMAX = Cfg<I>::kNmax;
  constexpr int kThreads = Cfg<I>::kThreads;
  constexpr int kWavesT = Cfg<I>::kWaves;
  constexpr int kRound = Cfg<I>::kRound;
  constexpr int kPieces = Cfg<I>::kPieces;
  constexpr int kCandCap = Cfg<I>::kCand;
  constexpr int kGroupCap = Cfg<I>::kGroups;
  static_assert(kRound % NMAX == 0, "group maxima per round");
  __shared__ Smem<I> sm;
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const float *row = scores + r * ld;
  const float *grow = GMAX ? gmax + r * ldg : nullptr;
  // Pass 1's first round of group maxima is requested before the row's length is known
  // (its lookup below is a dependent load, and a launch's rows all start at once):
  // indices are clamped to the row pitch, so the loads stay in the buffer, and those
  // past the row's groups are masked in pass 1.  Only when the pitch admits the group
  // path, which needs at least NMAX*kThreads groups, so that short rows do not pay.
  // (1.1% of the selection time at kpool 1, 0.3% at 512k tokens.)
  const bool early = GMAX && ldg >= (int64_t)NMAX * kThreads;
  float v0[kRound];
  if (early) {
#pragma unroll
    for (int j = 0; j < kRound; ++j) v0[j] = grow[min<int64_t>(tid + j * kThreads, ldg - 1)];
  }
  int64_t n;
  if (n_valid) {
    n = min<int64_t>(max<int64_t>(n_valid[r], 0), ld);
  } else {
    const int64_t i = grow0 + r;
    const int s = find_seq(cu_seqlens, nseq, i);
    n = visible_count(i - cu_seqlens[s], cu_seqlens[s + 1] - cu_seqlens[s], kpool, tail);
  }
  const int64_t ng = (n + kGroup - 1) / kGroup;  // 16-pool groups of the row
  // Group maxima are used when each of a thread's NMAX maxima covers at least one of
  // them (so every wave contributes 64*NMAX real maxima); shorter rows are read in full.
  // (n <= ld, so ng <= ldg: the group path implies `early`.)
  const bool use_groups = GMAX && n > budget && ng >= (int64_t)NMAX * kThreads;
  int32_t *orow = out + r * (int64_t)budget;
  if (tid == 0) {
    sm.count = 0;
    sm.gcount = 0;
    sm.scount = 0;
  }

  // A row with at most `budget` visible pools keeps all of them: their keys go straight
  // into the list (element i in slot i) and are sorted; there is nothing to bound or cut.
  if (n <= budget) {
    const int32_t n32 = (int32_t)n;  // <= budget <= 4 kThreads <= the list's capacity
    for (int32_t i = tid; i < n32; i += kThreads) sm.cand[i] = compose(order_key(row[i]), (uint32_t)i);
    __syncthreads();
    if (n32 <= kThreads) sort_and_write<1, kThreads>(sm.cand, (uint32_t)n32, budget, orow, tid);
    else if (n32 <= 2 * kThreads) sort_and_write<2, kThreads>(sm.cand, (uint32_t)n32, budget, orow, tid);
    else sort_and_write<4, kThreads>(sm.cand, (uint32_t)n32, budget, orow, tid);
    return;  // (n is the same for the whole workgroup)
  }

  // ---- pass 1: lower bound on the budget-th best key ----------------------
  // NMAX maxima per thread over disjoint parts of the row (its elements, or its
  // groups' maxima, which are elements too), so any budget of them are distinct
  // elements.
  uint32_t bound = 0, rowmax = 0xFFFFFFFFu;
  if (n > budget) {
    // The maxima are taken in the float domain (fmaxf skips NaN, and order_key is
    // monotonic on the rest, -0 and +0 sharing a key), then turned into keys; a slot
    // that saw only NaNs stays NaN, key 0.
    float fmx[NMAX];
#pragma unroll
    for (int i = 0; i < NMAX; ++i) fmx[i] = __uint_as_float(0x7FC00000u);
    if (use_groups) {
      // rounds of kRound independent loads per thread; item j goes to maximum j % NMAX;
      // round 0 was loaded early
#pragma unroll
      for (int j = 0; j < kRound; ++j)
        if (tid + j * kThreads < ng) fmx[j % NMAX] = fmaxf(fmx[j % NMAX], v0[j]);
      for (int64_t gb = (int64_t)kThreads * kRound; gb < ng; gb += (int64_t)kThreads * kRound) {
        float v[kRound];
#pragma unroll
        for (int j = 0; j < kRound; ++j)
          v[j] = grow[min(gb + tid + (int64_t)j * kThreads, ng - 1)];
#pragma unroll
        for (int j = 0; j < kRound; ++j)
          if (gb + tid + (int64_t)j * kThreads < ng) fmx[j % NMAX] = fmaxf(fmx[j % NMAX], v[j]);
      }
    } else {
      // NMAX/4 float4 pieces per thread per step; element e of piece q goes to
      // maximum 4q + e
      constexpr int NP = NMAX / 4;
      for (int64_t wbase = (int64_t)wave * 256 * NP; wbase < n; wbase += (int64_t)kThreads * 4 * NP) {
#pragma unroll
        for (int q = 0; q < NP; ++q) {
          const int64_t base = wbase + 256 * q + 4 * lane;
          if (base < n) {
            const float4 x = *reinterpret_cast<const float4 *>(row + base);
            const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (base + e < n) fmx[4 * q + e] = fmaxf(fmx[4 * q + e], xs[e]);
          }
        }
      }
    }
    uint32_t tmax[NMAX];
    uint32_t lm = 0;  // the row's best key: every element is at most one of these maxima
#pragma unroll
    for (int i = 0; i < NMAX; ++i) {
      tmax[i] = order_key(fmx[i]);
      lm = max(lm, tmax[i]);
      // A group max must not exceed the best key actually in its group.  The score
      // kernel's max skips NaN (key 0), so a group of NaNs reports -inf: count it as
      // key 0 here.  (Pass 2 and the row's best key keep -inf, an upper bound for such
      // a group.)
      if (use_groups && tmax[i] == kNegInfKey) tmax[i] = 0;
    }
    const int rank = (budget + kWavesT - 1) / kWavesT;  // 1..64*NMAX
    const uint32_t wb = wave_kth_desc<NMAX>(tmax, rank);
    // the wave's best key: a butterfly over compile-time lane distances
    lm = max(lm, lanes_xor<32>(lm));
    lm = max(lm, lanes_xor<16>(lm));
    lm = max(lm, lanes_xor<8>(lm));
    lm = max(lm, lanes_xor<4>(lm));
    lm = max(lm, lanes_xor<2>(lm));
    lm = max(lm, lanes_xor<1>(lm));
    if (lane == 0) {
      sm.wave_bound[wave] = wb;
      sm.wave_max[wave] = lm;
    }
    __syncthreads();
    bound = sm.wave_bound[0];
    rowmax = sm.wave_max[0];
#pragma unroll
    for (int w = 1; w < kWavesT; ++w) {
      bound = min(bound, sm.wave_bound[w]);
      rowmax = max(rowmax, sm.wave_max[w]);
    }
  }
  __syncthreads();
  // the bound as a float test (key 0 takes every element, NaN included)
  const bool take_all = bound == 0;
  const float bf = key_float(bound);

  // ---- pass 2: gather candidates with key >= bound ------------------------
  if (use_groups) {
    // groups whose max reaches the bound (uniform trip count; loads issued per round).
    // One ballot per load slot j: the wave's selected groups of slot j go to
    // consecutive positions after those of slots 0 .. j-1.  (Group indices are
    // 32-bit: a row has fewer than 2^27 groups.)
    const int32_t ng32 = (int32_t)ng;
    for (int32_t gb = 0; gb < ng32; gb += kThreads * kRound) {
      float v[kRound];
#pragma unroll
      // (the row's last read of its group maxima: non-temporal)
      for (int j = 0; j < kRound; ++j) v[j] = __builtin_nontemporal_load(grow + min(gb + tid + j * kThreads, ng32 - 1));
      bool sel[kRound];
      uint64_t msk[kRound];
      uint32_t off[kRound], tot = 0;
#pragma unroll
      for (int j = 0; j < kRound; ++j) {
        sel[j] = (gb + tid + j * kThreads < ng32) & (take_all | (v[j] >= bf));
        msk[j] = __ballot(sel[j]);
        off[j] = tot;
        tot += (uint32_t)__popcll(msk[j]);
      }
      if (tot == 0) continue;  // wave-uniform
      uint32_t wbase = 0;
      if (lane == 0) wbase = atomicAdd(&sm.gcount, tot);
      wbase = __builtin_amdgcn_readfirstlane(wbase);  // every lane is active here
#pragma unroll
      for (int j = 0; j < kRound; ++j) {
        if (sel[j]) {
          const uint32_t pos = wbase + off[j] +
              __builtin_amdgcn_mbcnt_hi((uint32_t)(msk[j] >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)msk[j], 0u));
          if (pos < (uint32_t)kGroupCap) sm.glist[pos] = (uint32_t)(gb + tid + j * kThreads);
        }
      }
    }
    __syncthreads();
    const uint32_t gcount = sm.gcount;
    if (gcount > (uint32_t)kGroupCap) {
      if (tid == 0) sm.count = kCandCap + 1;  // too many groups: exact fallback below
    } else {
      // four threads per group, one float4 each; rounds of kPieces loads per thread.  The
      // loads are non-temporal: each score piece is read once, and the group maxima of
      // the rows still to come should stay cached.
      typedef float f32x4 __attribute__((ext_vector_type(4)));
      const int32_t n32 = (int32_t)n;
      const int32_t npieces = 4 * (int32_t)gcount;
      for (int32_t pb = 0; pb < npieces; pb += kThreads * kPieces) {
        float4 x[kPieces];
        int32_t base[kPieces];
#pragma unroll
        for (int j = 0; j < kPieces; ++j) {
          const int32_t i = pb + tid + j * kThreads;
          base[j] = i < npieces ? (int32_t)sm.glist[i >> 2] * kGroup + (i & 3) * 4 : n32;
          const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(row + (base[j] < n32 ? base[j] : 0)));
          x[j] = make_float4(t.x, t.y, t.z, t.w);
        }
#pragma unroll
        for (int j = 0; j < kPieces; ++j) append_piece(x[j], base[j], n32, take_all, bf, sm, lane);
      }
    }
  } else {
    const int32_t n32 = (int32_t)n;
    for (int32_t wbase = wave * 256; wbase < n32; wbase += kThreads * 4) {
      const int32_t base = wbase + 4 * lane;
      const float4 x = base < n32 ? *reinterpret_cast<const float4 *>(row + base)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
      append_piece(x, base, n32, take_all, bf, sm, lane);
    }
  }
  __syncthreads();
  uint32_t count = sm.count;

  // ---- fallback: exact radix select when the candidate list overflowed ----
  if (count > (uint32_t)kCandCap) {
    uint64_t prefix = 0;
    int pbits = 0;
    int krem = budget;
    // keys are unique, so the bin holds exactly krem keys after at most 8 digits
    for (int pass = 0; pass < 8; ++pass) {
      if (tid < 256) sm.hist[tid] = 0;
      __syncthreads();
      for (int64_t base = 4 * (int64_t)tid; base < n; base += kThreads * 4) {
        const float4 x = *reinterpret_cast<const float4 *>(row + base);
        const float xs[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (base + e < n) {
            const uint64_t ck = compose(order_key(xs[e]), (uint32_t)(base + e));
            if (pbits == 0 || (ck >> (64 - pbits)) == prefix)
              atomicAdd(&sm.hist[(uint32_t)(ck >> (56 - pbits)) & 255u], 1u);
          }
        }
      }
      __syncthreads();
      if (wave == 0) next_digit(sm, prefix, pbits, krem, lane);
      if (tid == 0) sm.count = 0;
      __syncthreads();
      prefix = sm.prefix;
      pbits = sm.pbits;
      krem = sm.krem;
      if (sm.done) break;
    }
    // exactly `budget` keys have their top pbits >= prefix
    for (int64_t wbase = (int64_t)wave * 256; wbase < n; wbase += kThreads * 4) {
      const int64_t base = wbase + 4 * lane;
      uint64_t cks[4] = {0, 0, 0, 0};
      float xs[4] = {0.f, 0.f, 0.f, 0.f};
      bool sel[4] = {false, false, false, false};
      uint32_t c = 0;
      if (base < n) {
        const float4 x = *reinterpret_cast<const float4 *>(row + base);
        xs[0] = x.x;
        xs[1] = x.y;
        xs[2] = x.z;
        xs[3] = x.w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          cks[e] = compose(order_key(xs[e]), (uint32_t)(base + e));
          sel[e] = (base + e < n) && ((pbits >= 64 ? cks[e] : (cks[e] >> (64 - pbits))) >= prefix);
          c += sel[e] ? 1u : 0u;
        }
      }
      uint32_t pos = wave_reserve<3>(c, &sm.count, lane);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (sel[e]) {
          if (pos < (uint32_t)kCandCap) sm.cand[pos] = compose_raw(xs[e], (uint32_t)(base + e));
          ++pos;
        }
      }
    }
    __syncthreads();
    count = min(sm.count, (uint32_t)kCandCap);
  }
  // raw entries -> keys
  for (uint32_t i = tid; i < count; i += kThreads) sm.cand[i] = raw_to_key(sm.cand[i]);
  __syncthreads();

  // ---- exact cut to `budget` keys when that shrinks the sort ----------------
  // A radix select over the LDS list (8-bit digits of the unique 64-bit keys, usually
  // settled within a few digits) finds the budget-th key; the keys at or above it are
  // gathered into the spare group-list space and only those are sorted.
  auto sort_class = [](uint32_t x) { return x <= kThreads ? 1 : x <= 2 * kThreads ? 2 : x <= 4 * kThreads ? 4 : 8; };
  uint64_t *list = sm.cand;
  if (count > (uint32_t)budget && sort_class(count) > sort_class((uint32_t)budget)) {
    // Every candidate's top 32 key bits lie in [bound, rowmax], so all of them share
    // the leading bits common to those two: the digits inside that prefix are skipped
    // (for rows of similar scores the first one or two, whose histograms would put
    // every key into one bin).
    const int common = bound == rowmax ? 32 : __builtin_clz(bound ^ rowmax);
    int pbits = common / 8 * 8;
    uint64_t prefix = pbits ? ((uint64_t)rowmax >> (32 - pbits)) : 0ull;
    int krem = budget;
    for (int pass = 0; pass < 8; ++pass) {
      if (tid < 256) sm.hist[tid] = 0;
      __syncthreads();
      for (uint32_t i = tid; i < count; i += kThreads) {
        const uint64_t ck = sm.cand[i];
        if (pbits == 0 || (ck >> (64 - pbits)) == prefix)
          atomicAdd(&sm.hist[(uint32_t)(ck >> (56 - pbits)) & 255u], 1u);
      }
      __syncthreads();
      if (wave == 0) next_digit(sm, prefix, pbits, krem, lane);
      __syncthreads();
      prefix = sm.prefix;
      pbits = sm.pbits;
      krem = sm.krem;
      if (sm.done) break;
    }
    // exactly `budget` keys have their top pbits >= prefix (pbits >= 8 here)
    uint64_t *sel = reinterpret_cast<uint64_t *>(sm.glist);  // holds kGroupCap/2 >= budget keys
    for (uint32_t i0 = 0; i0 < count; i0 += kThreads) {
      const uint32_t i = i0 + tid;
      const uint64_t ck = i < count ? sm.cand[i] : 0ull;
      const bool take = i < count && (ck >> (64 - pbits)) >= prefix;
      const uint32_t pos = wave_reserve<1>(take ? 1u : 0u, &sm.scount, lane);
      if (take) sel[pos] = ck;
    }
    __syncthreads();
    list = sel;
    count = (uint32_t)budget;
  }

  // The sort covers the list in the smallest sort size that holds it (at most 4 kThreads
  // keys: a list in a larger sort class than the budget was cut to the budget above, and
  // budgets are at most 4 kThreads); a short row's slots past it are written as -1.
  if (count <= (uint32_t)kThreads) sort_and_write<1, kThreads>(list, count, budget, orow, tid);
  else if (count <= 2u * kThreads) sort_and_write<2, kThreads>(list, count, budget, orow, tid);
  else sort_and_write<4, kThreads>(list, count, budget, orow, tid);
}

// scores_out rows: the chunk buffer's visible scores, -inf elsewhere
__global__ __launch_bounds__(256) void scores_copy_kernel(const float *__restrict__ ws, int64_t ld,
                                                          const int32_t *__restrict__ cu_seqlens,
                                                          int nseq, int64_t grow0, int kpool,
                                                          bool tail, float *__restrict__ dst,
                                                          int64_t dst_ld) {
  const int64_t r = blockIdx.x;
  const int64_t i = grow0 + r;
  const int s = find_seq(cu_seqlens, nseq, i);
  const int64_t n = visible_count(i - cu_seqlens[s], cu_seqlens[s + 1] - cu_seqlens[s], kpool, tail);
  const float ninf = __uint_as_float(0xFF800000u);
  for (int64_t p = threadIdx.x; p < dst_ld; p += blockDim.x)
    dst[r * dst_ld + p] = p < n ? ws[r * ld + p] : ninf;
}

}  // namespace

template <bool GMAX, int I>
static void launch_topk_inst(const float *scores, int64_t ld, int64_t nrows, const int32_t *n_valid,
                             const int32_t *cu_seqlens, int32_t nseq, int64_t grow0, int32_t kpool,
                             bool tail, int32_t budget, int32_t *out, const float *gmax, int64_t ldg,
                             hipStream_t stream) {
  hipLaunchKernelGGL((topk_kernel<GMAX, I>), dim3((unsigned)nrows), dim3(Cfg<I>::kThreads), 0,
                     stream, scores, ld, n_valid, cu_seqlens, nseq, grow0, kpool, tail, budget, out,
                     gmax, ldg);
}

hipError_t launch_topk(const float *scores, int64_t ld, int64_t nrows, const int32_t *n_valid,
                       const int32_t *cu_seqlens, int32_t nseq, int64_t grow0, int32_t kpool,
                       bool tail, int32_t budget, int32_t *out, const float *gmax, int64_t ldg,
                       hipStream_t stream) {
  if (nrows <= 0) return hipSuccess;
  if (budget > kTopkMaxBudget) return hipErrorInvalidValue;
  // larger budgets need more maxima per row for a tight bound, and longer lists
  const int inst = budget <= Cfg<0>::kMaxBudget ? 0 : budget <= Cfg<1>::kMaxBudget ? 1 : 2;
  auto go = [&](auto gm, auto ic) {
    launch_topk_inst<decltype(gm)::value, decltype(ic)::value>(scores, ld, nrows, n_valid, cu_seqlens,
                                                               nseq, grow0, kpool, tail, budget, out,
                                                               gmax, ldg, stream);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  if (gmax) {
    if (inst == 0) go(T_{}, std::integral_constant<int, 0>{});
    else if (inst == 1) go(T_{}, std::integral_constant<int, 1>{});
    else go(T_{}, std::integral_constant<int, 2>{});
  } else {
    if (inst == 0) go(F_{}, std::integral_constant<int, 0>{});
    else if (inst == 1) go(F_{}, std::integral_constant<int, 1>{});
    else go(F_{}, std::integral_constant<int, 2>{});
  }
  return hipGetLastError();
}

hipError_t launch_scores_copy(const float *ws, int64_t ld, int64_t nrows, const int32_t *cu_seqlens,
                              int32_t nseq, int64_t grow0, int32_t kpool, bool tail, float *dst,
                              int64_t dst_ld, hipStream_t stream) {
  if (nrows <= 0) return hipSuccess;
  hipLaunchKernelGGL(scores_copy_kernel, dim3((unsigned)nrows), dim3(256), 0, stream, ws, ld,
                     cu_seqlens, nseq, grow0, kpool, tail, dst, dst_ld);
  return hipGetLastError();
}

}  // namespace kpool
