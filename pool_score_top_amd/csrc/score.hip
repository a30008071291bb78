// Score kernel: S[i,p] = sum_h w[i,h] * relu(scale * <q[i,h,:], kp[p,:]>) for
// the pools p visible to row i, written as fp32 into a row-chunk buffer.
//
// Pages: Atlas inference glm5next_dsa/tp.rs module doc "Why the indexer is
// REPLICATED, not sharded" (the head-weighted ReLU sum that forms the score);
// Megatron-LM PR #8299 "Mechanism" (every query row scores the pooled keys;
// the full work is the [queries, pools] score matrix) and "Test plan"
// (causal mask, packed varlen bounds).
//
// The dense contraction is [rows*H, D] x [D, pools] on the bf16 MFMA pipe:
//   * MFMA v_mfma_f32_16x16x32_bf16 with M = 16 heads of ONE row, N = 16 pools,
//     K = 32 of the head dim.  One lane then holds 4 heads x 1 pool of the
//     output, so the ReLU/weight/head-sum epilogue stays in registers and the
//     remaining cross-lane sum over the 4 lane groups is two swap steps
//     (permlane16 / permlane32) shared by 4 rows at once.
//   * A workgroup owns a tile of 32 rows of one sequence (8 waves x 4 rows); the
//     rows' q fragments and scale*w live in VGPRs for the whole kernel.  It
//     walks one segment of the pool axis, staging 64 pooled keys at a time
//     through double-buffered LDS (one barrier per stage), so each pooled key
//     fetched from L2 feeds 32 rows x 32 heads of MFMA work.
//   * Causal skipping: a tile only visits pools visible to its last row, and a
//     wave skips 16-pool sub-tiles beyond its own last row.  Scores are stored
//     only for visible (row, pool) pairs; the selection reads nothing else.
//   * The head dim is split across the 4 lane groups as contiguous runs of
//     D/4 (a fixed permutation of K applied to q and kp alike), so every lane
//     reads 16-byte contiguous pieces.
//   * Score bits depend only on (row, pool): each row has its own MFMA chain,
//     every pool column is reduced the same way, and the head sum runs in one
//     fixed order, so tiling, chunking and row-range splits cannot change them.
//   Arithmetic: bf16 x bf16 products accumulated by the MFMA in fp32; the
//   epilogue forms relu(dot) * (scale * w[h]) in fp32 (scale > 0, so this is
//   the same quantity as w * relu(scale * dot)) and sums the heads in fp32.
#include "kpool_internal.h"

namespace kpool {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;
constexpr int kRowsPerWave = 4;  // the 4-row swap reduction needs exactly 4
constexpr int kTileRows = kWaves * kRowsPerWave;
constexpr int kStagePools = 64;
constexpr int kSub = 16;

template <int H, int D>
struct Shape {
  static constexpr int MB = (H + 15) / 16;        // 16-head M blocks per row
  static constexpr int DP = (D + 31) / 32 * 32;   // head dim padded to the K step
  static constexpr int KS = DP / 32;              // K steps per dot product
  static constexpr int KG = DP / 4;               // contiguous dims per lane group
  static constexpr int PITCH = DP * 2 + 16;       // LDS bytes per pooled key (+16: bank skew)
  static constexpr int STAGE_BYTES = kStagePools * PITCH;
  static constexpr int CHUNKS = kStagePools * DP / 8;  // 16-byte pieces per stage
  static constexpr int CPT = (CHUNKS + kWaves * 64 - 1) / (kWaves * 64);  // pieces per thread
};

// permlane16_swap(a, b) gives a' = [a.g0, b.g0, a.g2, b.g2] and b' = [a.g1, b.g1, a.g3, b.g3]
// (g = 16-lane group), so a' + b' holds (a.g0+a.g1, b.g0+b.g1, a.g2+a.g3, b.g2+b.g3).
__device__ inline float swap16_sum(float a, float b) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int H, int D>
__global__ __launch_bounds__(kWaves * 64) void score_kernel(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ kp, const float *__restrict__ w,
    float scale, int kpool, SegList segs, int npseg, int pseg_pools, int64_t chunk_row0,
    int64_t ld, float *__restrict__ out) {
  using S = Shape<H, D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  const int tile = blockIdx.x / npseg;
  const int pseg = blockIdx.x - tile * npseg;
  int g = 0;
  while (g + 1 < segs.nseg && segs.tile_start[g + 1] <= tile) ++g;
  const int64_t row0 = (int64_t)segs.row_lo[g] + (int64_t)(tile - segs.tile_start[g]) * kTileRows;
  const int nrows = (int)min<int64_t>(kTileRows, segs.row_hi[g] - row0);
  const int64_t t0 = row0 - segs.seq_start[g];
  const int npv = (int)((t0 + nrows - 1) / kpool) + 1;  // pools visible to the tile's last row
  const int p_begin = pseg * pseg_pools;
  if (p_begin >= npv) return;  // whole workgroup leaves together
  const int p_end = min(npv, p_begin + pseg_pools);
  const uint16_t *kps = kp + (int64_t)segs.pool_base[g] * D;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform (SGPR)
  const int lg = lane >> 4;  // lane group: K slice of the operands, head quad of the output
  const int lc = lane & 15;  // operand row (head) / output column (pool)
  const int wr0 = wave * kRowsPerWave;

  // ---- per-row operands, resident for the whole kernel --------------------
  bf16x8 a[kRowsPerWave][S::MB][S::KS];
  float sw[kRowsPerWave][S::MB][4];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const bool valid = wr0 + r < nrows;
    const int64_t grow = row0 + wr0 + r;
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) {
      const int head = mb * 16 + lc;
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        const int kk = lg * S::KG + ks * 8;
        bf16x8 v = {};
        if (valid && head < H && kk < D)
          v = *reinterpret_cast<const bf16x8 *>(q + (grow * H + head) * D + kk);
        a[r][mb][ks] = v;
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = mb * 16 + lg * 4 + i;
        sw[r][mb][i] = (valid && h < H) ? scale * w[grow * H + h] : 0.0f;
      }
    }
  }
  // visible pools of the row this lane stores (row wr0 + lg), and of the wave's last row
  const int my_nvis = (wr0 + lg < nrows) ? (int)((t0 + wr0 + lg) / kpool) + 1 : 0;
  const int wave_last = min(nrows, wr0 + kRowsPerWave) - 1;
  const int wave_nvis = __builtin_amdgcn_readfirstlane(
      (wave_last >= wr0) ? (int)((t0 + wave_last) / kpool) + 1 : 0);
  float *orow = out + (row0 + wr0 + lg - chunk_row0) * ld;

  // ---- pooled-key stages through LDS ---------------------------------------
  uint4 pre[S::CPT];
  auto fetch = [&](int stage_base) {
#pragma unroll
    for (int c = 0; c < S::CPT; ++c) {
      const int piece = threadIdx.x + c * kWaves * 64;
      const int pl = piece / (S::DP / 8);
      const int part = piece - pl * (S::DP / 8);
      const int pool = stage_base + pl;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (piece < S::CHUNKS && pool < p_end && part * 8 < D)
        v = *reinterpret_cast<const uint4 *>(kps + (int64_t)pool * D + part * 8);
      pre[c] = v;
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int c = 0; c < S::CPT; ++c) {
      const int piece = threadIdx.x + c * kWaves * 64;
      if (piece < S::CHUNKS) {
        const int pl = piece / (S::DP / 8);
        const int part = piece - pl * (S::DP / 8);
        *reinterpret_cast<uint4 *>(lds + buf * S::STAGE_BYTES + pl * S::PITCH + part * 16) = pre[c];
      }
    }
  };

  const int nstage = (p_end - p_begin + kStagePools - 1) / kStagePools;
  fetch(p_begin);
  stash(0);
  __syncthreads();
  for (int st = 0; st < nstage; ++st) {
    const int stage_base = p_begin + st * kStagePools;
    if (st + 1 < nstage) fetch(stage_base + kStagePools);
    const unsigned char *sb = lds + (st & 1) * S::STAGE_BYTES;
    // 16-pool sub-tiles of this stage that hold pools visible to this wave's rows
    const int lim = min(wave_nvis, p_end) - stage_base;
    const int nsub = __builtin_amdgcn_readfirstlane(
        lim <= 0 ? 0 : min(kStagePools / kSub, (lim + kSub - 1) / kSub));
#pragma unroll 1
    for (int sub = 0; sub < nsub; ++sub) {
      const int pbase = stage_base + sub * kSub;
      bf16x8 b[S::KS];
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks)
        b[ks] = *reinterpret_cast<const bf16x8 *>(sb + (sub * kSub + lc) * S::PITCH +
                                                  (lg * S::KG + ks * 8) * 2);
      // all (row, M block) accumulators advance together: 8 independent MFMAs per K step
      floatx4 acc[kRowsPerWave][S::MB];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
        for (int mb = 0; mb < S::MB; ++mb) acc[r][mb] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks)
#pragma unroll
        for (int r = 0; r < kRowsPerWave; ++r)
#pragma unroll
          for (int mb = 0; mb < S::MB; ++mb)
            acc[r][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r][mb][ks], b[ks], acc[r][mb], 0, 0, 0);
      float x[kRowsPerWave];
#pragma unroll
      for (int r = 0; r < kRowsPerWave; ++r) {
        x[r] = 0.0f;
#pragma unroll
        for (int mb = 0; mb < S::MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) x[r] = fmaf(fmaxf(acc[r][mb][i], 0.0f), sw[r][mb][i], x[r]);
      }
      // lane group g ends up holding row g: ((g0 + g1) + (g2 + g3)) for every row
      const float y01 = swap16_sum(x[0], x[1]);
      const float y23 = swap16_sum(x[2], x[3]);
      // permlane32_swap(y01, y23): [y01.lo, y23.lo] + [y01.hi, y23.hi]
      auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(y01), __float_as_uint(y23), false, false);
      const float val = __uint_as_float(z[0]) + __uint_as_float(z[1]);
      const int p = pbase + lc;
      if (p < my_nvis) orow[p] = val;
    }
    if (st + 1 < nstage) stash((st + 1) & 1);
    __syncthreads();
  }
}

template <int H, int D>
hipError_t launch_t(const uint16_t *q, const uint16_t *kp, const float *w, float scale,
                    int32_t kpool, const SegList &segs, int32_t ntiles, int32_t npseg,
                    int32_t pseg_pools, int64_t chunk_row0, int64_t ld, float *out,
                    hipStream_t stream) {
  using S = Shape<H, D>;
  const size_t lds = 2 * S::STAGE_BYTES;
  const unsigned grid = (unsigned)ntiles * (unsigned)npseg;
  hipLaunchKernelGGL((score_kernel<H, D>), dim3(grid), dim3(kWaves * 64), lds, stream, q, kp, w,
                     scale, kpool, segs, npseg, pseg_pools, chunk_row0, ld, out);
  return hipGetLastError();
}

}  // namespace

bool score_supported(int H, int D) { return (H == 32 && D == 128) || (H == 4 && D == 16); }
int score_tile_rows() { return kTileRows; }

hipError_t launch_score(int H, int D, const uint16_t *q, const uint16_t *kp, const float *w,
                        float scale, int32_t kpool, const SegList &segs, int32_t ntiles,
                        int32_t npseg, int32_t pseg_pools, int64_t chunk_row0, int64_t ld,
                        float *out, hipStream_t stream) {
  if (pseg_pools % kStagePools != 0) return hipErrorInvalidValue;
  if (H == 32 && D == 128)
    return launch_t<32, 128>(q, kp, w, scale, kpool, segs, ntiles, npseg, pseg_pools, chunk_row0,
                             ld, out, stream);
  if (H == 4 && D == 16)
    return launch_t<4, 16>(q, kp, w, scale, kpool, segs, ntiles, npseg, pseg_pools, chunk_row0,
                           ld, out, stream);
  return hipErrorInvalidValue;
}

}  // namespace kpool
