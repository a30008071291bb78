// Expansion and causal filter: pool id -> kpool token ids, -1 past the row.
//
// Pages: Megatron-LM PR #8299, "Change" (after the pool ids are known, pools
// are expanded to their tokens and the result is mask-filtered) and
// "Alternatives considered" (the expanded form is kpool times the pool-id
// payload).  Keeping a filtered slot in place as -1 and int32 token ids are
// this library's reading.
//
// Tail mode (a reading of the pages' "tail append", named between expansion and mask
// filtering in the same passage): the sequence's L mod kpool tokens after its last
// full pool are appended after a row's budget*kpool slots, in kpool - 1 more slots,
// and filtered like the rest (-1 where absent or after the row).
//
// HBM-bound: workgroups stride over rows (one sequence lookup per row), threads over
// a row's slots.  kpool == 4: each slot is one 16-byte store; kpool == 1 with 16-byte
// aligned rows: 4 slots per thread through 16-byte loads and stores; any other kpool
// whose rows hold a multiple of 4 slots (16-byte aligned output): 4 consecutive slots
// per thread and one 16-byte store; otherwise one token per thread and iteration.
#include "kpool_internal.h"

namespace kpool {
namespace {

constexpr int kExpandThreads = 256;
constexpr int kExpandMaxBlocks = 65536;

__global__ __launch_bounds__(kExpandThreads) void expand_kernel(const int32_t *__restrict__ pool_ids,
                                                                const int32_t *__restrict__ cu_seqlens,
                                                                int nseq, int kpool, bool tail,
                                                                int64_t q_lo, int64_t nrows,
                                                                int budget, bool vec, bool vec4,
                                                                int32_t *__restrict__ tok) {
  const int ntail = tail ? kpool - 1 : 0;
  const int64_t width = (int64_t)budget * kpool + ntail;
  for (int64_t r = blockIdx.x; r < nrows; r += gridDim.x) {
    const int64_t i = q_lo + r;
    const int s = find_seq(cu_seqlens, nseq, i);
    const int64_t t = i - cu_seqlens[s];
    const int32_t *prow = pool_ids + r * budget;
    int32_t *orow = tok + r * width;
    if (tail) {  // rows of odd width: one slot per thread, then the tail
      const int64_t L = cu_seqlens[s + 1] - cu_seqlens[s];
      const int64_t a = L / kpool * kpool;  // the tail's first token
      for (int64_t e = threadIdx.x; e < width; e += kExpandThreads) {
        int64_t tk;
        bool ok;
        if (e < (int64_t)budget * kpool) {
          const int32_t p = prow[e / kpool];
          tk = (int64_t)p * kpool + e % kpool;
          ok = p >= 0;
        } else {
          tk = a + (e - (int64_t)budget * kpool);
          ok = tk < L;
        }
        orow[e] = (ok && tk <= t) ? (int32_t)tk : -1;
      }
      continue;
    }
    // The 16-byte token-id stores are non-temporal: the output is written once and not
    // read again on the path.
    typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
    if (kpool == 4) {
      for (int j = threadIdx.x; j < budget; j += kExpandThreads) {
        const int32_t p = prow[j];
        int32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t tk = (int64_t)p * 4 + k;
          v[k] = (p >= 0 && tk <= t) ? (int32_t)tk : -1;
        }
        const i32x4 o = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<i32x4 *>(orow + 4 * j));
      }
    } else if (kpool == 1 && vec) {
      for (int j = threadIdx.x; j < budget / 4; j += kExpandThreads) {
        const int4 p = reinterpret_cast<const int4 *>(prow)[j];
        auto f = [&](int32_t q) { return (q >= 0 && q <= t) ? q : -1; };
        const i32x4 o = {f(p.x), f(p.y), f(p.z), f(p.w)};
        __builtin_nontemporal_store(o, reinterpret_cast<i32x4 *>(orow) + j);
      }
    } else if (vec4) {
      // any other kpool with rows of a multiple of 4 slots: 4 consecutive slots per thread
      // (slot e holds token (e / kpool) * kpool-th pool's e % kpool), one 16-byte store
      const int64_t n4 = (int64_t)budget * kpool / 4;
      for (int64_t e4 = threadIdx.x; e4 < n4; e4 += kExpandThreads) {
        int32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int64_t e = 4 * e4 + k;
          const int32_t p = prow[e / kpool];
          const int64_t tk = (int64_t)p * kpool + e % kpool;
          v[k] = (p >= 0 && tk <= t) ? (int32_t)tk : -1;
        }
        const i32x4 o = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(o, reinterpret_cast<i32x4 *>(orow) + e4);
      }
    } else {
      const int64_t n = (int64_t)budget * kpool;
      for (int64_t e = threadIdx.x; e < n; e += kExpandThreads) {
        const int32_t p = prow[e / kpool];
        const int64_t tk = (int64_t)p * kpool + e % kpool;
        orow[e] = (p >= 0 && tk <= t) ? (int32_t)tk : -1;
      }
    }
  }
}

}  // namespace

hipError_t launch_expand(const int32_t *pool_ids, const int32_t *cu_seqlens, int32_t nseq,
                         int32_t kpool, bool tail, int64_t q_lo, int64_t nrows, int32_t budget,
                         int32_t *token_ids, hipStream_t stream) {
  if (nrows <= 0) return hipSuccess;
  const bool vec = budget % 4 == 0 && ((uintptr_t)pool_ids % 16) == 0 && ((uintptr_t)token_ids % 16) == 0;
  // rows of budget * kpool slots start 16-byte aligned when that count is a multiple of 4
  const bool vec4 = ((int64_t)budget * kpool) % 4 == 0 && ((uintptr_t)token_ids % 16) == 0;
  const unsigned blocks = (unsigned)(nrows < kExpandMaxBlocks ? nrows : kExpandMaxBlocks);
  hipLaunchKernelGGL(expand_kernel, dim3(blocks), dim3(kExpandThreads), 0, stream, pool_ids,
                     cu_seqlens, nseq, kpool, tail, q_lo, nrows, budget, vec, vec4, token_ids);
  return hipGetLastError();
}

}  // namespace kpool
