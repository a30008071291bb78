// Pooled keys: kp[pool] = bf16_rne(fp32 mean of the pool's kpool keys).
//
// Pages: Megatron-LM PR #8299, "Mechanism" (each query row scores the pooled
// keys); Atlas inference glm5next_dsa/tp.rs module doc (pools are kpool
// consecutive tokens, seq/kpool of them).  Mean pooling with an fp32 sum in
// token order from +0, an fp32 divide and a bf16 round-to-nearest-even result
// is this library's reading of the pooling operator.
//
// The gated variant (the GLM-5.3 indexer's k-pool compression: a gate and a slot
// embedding, named by the Atlas inference docs, glm5next_dsa/tp.rs, indexer tensors
// of the shard plan; gate scores are an op input, Megatron-LM PR #8299 "Mechanism";
// the formula is this library's reading) weights the pool's keys per dim by a
// softmax over the slots of gate score + slot embedding, in fp64.
//
// HBM-bound: each thread owns one 16-byte slice (8 dims) of one pool, reads the
// kpool matching key slices (the pool's keys are contiguous rows, so a wave
// reads one contiguous span; the gated variant also the gate-score slices) and
// writes 16 bytes.
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

// bf16 bits of the fp64 value x rounded once to nearest (ties to even): the quantum is
// 2^(e-7) for 2^e <= |x| < 2^(e+1) and 2^-133 below the smallest normal bf16, rint rounds
// half to even, and the result (8 significant bits) is exact in fp32.
__device__ inline uint16_t bf16_rne_f64(double x) {
  double r;
  if (fabs(x) < 0x1p-126) {
    r = rint(x * 0x1p133) * 0x1p-133;
  } else {
    const int e = ilogb(x);
    r = ldexp(rint(ldexp(x, 7 - e)), e - 7);
  }
  return (uint16_t)(__float_as_uint((float)r) >> 16);
}

// Gated pooling of one (pool, 8-dim slice): per dim, z_j = g[t_j] + ape[j],
// m = max_j z_j, e_j = exp(z_j - m), kp = bf16((sum_j e_j k[t_j]) / (sum_j e_j)), with the
// sums in slot order (fma for the weighted keys).  The arithmetic is fp64: the kernel is
// HBM-bound (a few exp per 16 bytes read), and in fp64 the one rounding to bf16 is that of
// the exact value except within about 1e-14 of a rounding midpoint, where fp32 would pick
// the other neighbour for about one key element in 20000.  Two passes over the slots
// (the max, then the sums) re-read the gate slices, which the first pass has just brought
// into the cache.
__global__ __launch_bounds__(256) void pool_keys_gated_kernel(
    const uint16_t *__restrict__ k, const uint16_t *__restrict__ g, const float *__restrict__ ape,
    const int32_t *__restrict__ cu_seqlens, const int32_t *__restrict__ cu_pools, int nseq, int D,
    int kpool, int64_t P_tot, uint16_t *__restrict__ kp) {
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
  const int64_t off = (start + p * kpool) * D + slice * 8;
  const uint16_t *ksrc = k + off;
  const uint16_t *gsrc = g + off;
  const float *asrc = ape + slice * 8;

  // z of slot j, 8 dims: the bf16 gate score plus the fp32 slot embedding (exact in fp64)
  auto load_z = [&](int j, double (&z)[8]) {
    const uint4 gv = *reinterpret_cast<const uint4 *>(gsrc + (int64_t)j * D);
    const float4 a0 = *reinterpret_cast<const float4 *>(asrc + (int64_t)j * D);
    const float4 a1 = *reinterpret_cast<const float4 *>(asrc + (int64_t)j * D + 4);
    const uint32_t w[4] = {gv.x, gv.y, gv.z, gv.w};
    const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      z[2 * e] = (double)__uint_as_float(w[e] << 16) + (double)a[2 * e];
      z[2 * e + 1] = (double)__uint_as_float(w[e] & 0xFFFF0000u) + (double)a[2 * e + 1];
    }
  };
  double m[8], z[8];
  load_z(0, m);
  for (int j = 1; j < n; ++j) {
    load_z(j, z);
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = fmax(m[e], z[e]);
  }
  double den[8], num[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) den[e] = num[e] = 0.0;
  for (int j = 0; j < n; ++j) {
    load_z(j, z);
    const uint4 v = *reinterpret_cast<const uint4 *>(ksrc + (int64_t)j * D);
    const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double e0 = exp(z[2 * e] - m[2 * e]);
      const double e1 = exp(z[2 * e + 1] - m[2 * e + 1]);
      den[2 * e] += e0;
      den[2 * e + 1] += e1;
      num[2 * e] = fma(e0, (double)__uint_as_float(wv[e] << 16), num[2 * e]);
      num[2 * e + 1] = fma(e1, (double)__uint_as_float(wv[e] & 0xFFFF0000u), num[2 * e + 1]);
    }
  }
  uint32_t o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const uint32_t lo = bf16_rne_f64(num[2 * e] / den[2 * e]);
    const uint32_t hi = bf16_rne_f64(num[2 * e + 1] / den[2 * e + 1]);
    o[e] = lo | (hi << 16);
  }
  *reinterpret_cast<uint4 *>(kp + pool * D + slice * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_pool_keys_gated(const uint16_t *k, const uint16_t *g, const float *ape,
                                  const int32_t *cu_seqlens, const int32_t *cu_pools, int32_t nseq,
                                  int32_t D, int32_t kpool, int64_t P_tot, uint16_t *kp,
                                  hipStream_t stream) {
  const int64_t threads = P_tot * (D / 8);
  const int block = 256;
  const int64_t grid = (threads + block - 1) / block;
  hipLaunchKernelGGL(pool_keys_gated_kernel, dim3((unsigned)grid), dim3(block), 0, stream, k, g, ape,
                     cu_seqlens, cu_pools, nseq, D, kpool, P_tot, kp);
  return hipGetLastError();
}

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
