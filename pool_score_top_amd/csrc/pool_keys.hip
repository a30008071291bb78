// Pooled keys: kp[pool] = bf16_rne(fp32 mean of the pool's kpool keys).
//
// Pages: Megatron-LM PR #8299, "Mechanism" (each query row scores the pooled
// keys); Atlas inference glm5next_dsa/tp.rs module doc (pools are kpool
// consecutive tokens, seq/kpool of them).  Mean pooling with an fp32 sum in
// token order from +0, an fp32 divide and a bf16 round-to-nearest-even result
// is this library's reading of the pooling operator.
//
// HBM-bound: each thread owns one 16-byte slice (8 dims) of one pool, reads the
// kpool matching key slices (the pool's keys are contiguous rows, so a wave
// reads one contiguous span) and writes 16 bytes.
#include "kpool_internal.h"

namespace kpool {
namespace {

__device__ inline uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ __launch_bounds__(256) void pool_keys_kernel(const uint16_t *__restrict__ k,
                                                        const int32_t *__restrict__ cu_seqlens,
                                                        const int32_t *__restrict__ cu_pools,
                                                        int nseq, int D, int kpool, int64_t P_tot,
                                                        uint16_t *__restrict__ kp) {
  const int slices = D >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t pool = gid / slices;
  if (pool >= P_tot) return;
  const int slice = (int)(gid - pool * slices);
  const int s = find_seq(cu_pools, nseq, pool);
  const int64_t p = pool - cu_pools[s];
  const int64_t start = cu_seqlens[s];
  const int64_t len = cu_seqlens[s + 1] - start;
  const int n = (int)min<int64_t>(kpool, len - p * kpool);

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.0f;
  const uint16_t *src = k + (start + p * kpool) * D + slice * 8;
  for (int j = 0; j < n; ++j) {
    const uint4 v = *reinterpret_cast<const uint4 *>(src + (int64_t)j * D);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = acc[2 * e] + __uint_as_float(wv[e] << 16);
      acc[2 * e + 1] = acc[2 * e + 1] + __uint_as_float(wv[e] & 0xFFFF0000u);
    }
  }
  const float fn = (float)n;
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = bf16_rne(__fdiv_rn(acc[2 * e], fn));
    const uint32_t hi = bf16_rne(__fdiv_rn(acc[2 * e + 1], fn));
    o[e] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4 *>(kp + pool * D + slice * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_pool_keys(const uint16_t *k, const int32_t *cu_seqlens, const int32_t *cu_pools,
                            int32_t nseq, int32_t D, int32_t kpool, int64_t P_tot, uint16_t *kp,
                            hipStream_t stream) {
  const int64_t threads = P_tot * (D / 8);
  const int block = 256;
  const int64_t grid = (threads + block - 1) / block;
  hipLaunchKernelGGL(pool_keys_kernel, dim3((unsigned)grid), dim3(block), 0, stream, k, cu_seqlens,
                     cu_pools, nseq, D, kpool, P_tot, kp);
  return hipGetLastError();
}

}  // namespace kpool
