// Expansion and causal filter: pool id -> kpool token ids, -1 past the row.
//
// Pages: Megatron-LM PR #8299, "Change" (after the pool ids are known, pools
// are expanded to their tokens and the result is mask-filtered) and
// "Alternatives considered" (the expanded form is kpool times the pool-id
// payload).  Keeping a filtered slot in place as -1 and int32 token ids are
// this library's reading.
//
// HBM-write-bound: one thread per (row, slot) reads one int32 and writes
// kpool int32 (one 16-byte store when kpool == 4).
#include "kpool_internal.h"

namespace kpool {
namespace {

__global__ __launch_bounds__(256) void expand_kernel(const int32_t *__restrict__ pool_ids,
                                                     const int32_t *__restrict__ cu_seqlens,
                                                     int nseq, int kpool, int64_t q_lo,
                                                     int64_t nrows, int budget,
                                                     int32_t *__restrict__ tok) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= nrows * budget) return;
  const int64_t r = gid / budget;
  const int64_t i = q_lo + r;
  const int s = find_seq(cu_seqlens, nseq, i);
  const int64_t t = i - cu_seqlens[s];
  const int32_t p = pool_ids[gid];
  int32_t *o = tok + gid * kpool;
  if (kpool == 4) {
    int32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t tk = (int64_t)p * 4 + j;
      v[j] = (p >= 0 && tk <= t) ? (int32_t)tk : -1;
    }
    *reinterpret_cast<int4 *>(o) = make_int4(v[0], v[1], v[2], v[3]);
  } else {
    for (int j = 0; j < kpool; ++j) {
      const int64_t tk = (int64_t)p * kpool + j;
      o[j] = (p >= 0 && tk <= t) ? (int32_t)tk : -1;
    }
  }
}

}  // namespace

hipError_t launch_expand(const int32_t *pool_ids, const int32_t *cu_seqlens, int32_t nseq,
                         int32_t kpool, int64_t q_lo, int64_t nrows, int32_t budget,
                         int32_t *token_ids, hipStream_t stream) {
  const int64_t n = nrows * budget;
  if (n <= 0) return hipSuccess;
  const int block = 256;
  hipLaunchKernelGGL(expand_kernel, dim3((unsigned)((n + block - 1) / block)), dim3(block), 0,
                     stream, pool_ids, cu_seqlens, nseq, kpool, q_lo, nrows, budget, token_ids);
  return hipGetLastError();
}

}  // namespace kpool
