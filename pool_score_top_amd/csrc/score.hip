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
//   * Causal skipping: a tile only visits pools visible to its last row.  Each
//     row's scores are stored in 16-byte pieces up to its own visible count (the
//     last piece may run past it; the selection reads each row only up to its
//     visible count).
//   * The ReLU / weight epilogue of one MFMA chain (row, 16-head block) runs on the
//     VALU while the next chains' MFMAs run, so the two pipes overlap.
//   * The head dim is split across the 4 lane groups as contiguous runs of
//     D/4 (a fixed permutation of K applied to q and kp alike), so every lane
//     reads 16-byte contiguous pieces.
//   * Score bits depend only on (row, pool): each row has its own MFMA chain,
//     every pool column is reduced the same way, and the head sum runs in one
//     fixed order, so tiling, chunking and row-range splits cannot change them.
//   Arithmetic: bf16 x bf16 products accumulated by the MFMA in fp32; the
//   epilogue forms relu(dot) * (scale * w[h]) in fp32 (scale > 0, so this is
//   the same quantity as w * relu(scale * dot)) and sums the heads in fp32.
#include <atomic>
#include <type_traits>

#include "kpool_internal.h"

namespace kpool {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Rows per wave: 4 (8 waves, two per SIMD).  8 rows per wave (4 waves, one per SIMD,
// halving the B-fragment reads per flop) needs the q fragments in AGPRs, which the
// operand loads below force, and the MFMA results in VGPRs (build flag
// -mllvm -amdgpu-mfma-vgpr-form=1); it passes the same tests and measured no faster.
#ifndef KPOOL_SCORE_RPW
#define KPOOL_SCORE_RPW 4
#endif
constexpr int kTileRows = 32;
constexpr int kRowsPerWave = KPOOL_SCORE_RPW;
static_assert(kRowsPerWave % 4 == 0, "the swap reduction sums 4 rows at a time");
constexpr int kQuads = kRowsPerWave / 4;  // row quads per wave
constexpr int kWaves = kTileRows / kRowsPerWave;  // waves per workgroup
constexpr int kStagePools = 64;
constexpr int kSub = 16;

template <int H, int D>
struct Shape {
  static constexpr int MB = (H + 15) / 16;        // 16-head M blocks per row
  static constexpr int DP = (D + 31) / 32 * 32;   // head dim padded to the K step
  static constexpr int KS = DP / 32;              // K steps per dot product
  static constexpr int KG = DP / 4;               // contiguous dims per lane group
  static constexpr int ROWB = DP * 2;             // LDS bytes per pooled key (no padding)
  static constexpr int NSLOT = DP / 8;            // 16-byte slots per key row
  static constexpr int STAGE_BYTES = kStagePools * ROWB;
  static constexpr int NREG = STAGE_BYTES / 1024; // 1 KiB DMA regions per stage (one per wave op)
  static constexpr int RGW = (NREG + kWaves - 1) / kWaves;  // regions per wave
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
    int64_t ld, float *__restrict__ out, int64_t ldg, float *__restrict__ gmax) {
  using S = Shape<H, D>;
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];

  // (This file is built with the IEEE mode off, so the device library's id functions
  // behind blockIdx / threadIdx are called rather than inlined.  Replacing them with
  // the id builtins, or pinning these values to SGPRs, changes the compiler's schedule
  // of the stage loop and measured 2-3% slower, so the plain form stays.)
  const int tile = blockIdx.x / npseg;
  const int pseg = blockIdx.x - tile * npseg;
  int g = 0;
  while (g + 1 < segs.nseg && segs.tile_start[g + 1] <= tile) ++g;
  const int64_t row0 = (int64_t)segs.row_lo[g] + (int64_t)(tile - segs.tile_start[g]) * kTileRows;
  const int nrows = (int)min<int64_t>(kTileRows, segs.row_hi[g] - row0);
  const int64_t t0 = row0 - segs.seq_start[g];
  // pools visible to the tile's last row (at most the sequence's pool count, which only
  // tail mode's full-pool count can undercut); each row's own limit below is capped by it
  const int npv = min((int)((t0 + nrows - 1) / kpool) + 1, segs.pool_count[g]);
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
  // Loads are unconditional from clamped, in-bounds addresses (the tile's last row,
  // the last head / dim slice), and masked lanes are zeroed afterwards, so the
  // compiler issues all of them back to back with no branch or wait in between.
  bf16x8 a[kRowsPerWave][S::MB][S::KS];
  float sw[kRowsPerWave][S::MB][4];
#pragma unroll
  for (int r = 0; r < kRowsPerWave; ++r) {
    const bool valid = wr0 + r < nrows;
    const int64_t grow = row0 + min(wr0 + r, nrows - 1);
#pragma unroll
    for (int mb = 0; mb < S::MB; ++mb) {
      const int head = mb * 16 + lc;
#pragma unroll
      for (int ks = 0; ks < S::KS; ++ks) {
        const int kk = lg * S::KG + ks * 8;
        const bool ok = valid && head < H && kk < D;
        const uint4 v = *reinterpret_cast<const uint4 *>(q + (grow * H + min(head, H - 1)) * D +
                                                         min(kk, D - 8));
        const uint4 z = ok ? v : make_uint4(0, 0, 0, 0);
        a[r][mb][ks] = __builtin_bit_cast(bf16x8, z);
        if (kRowsPerWave > 4) asm volatile("" : "+a"(a[r][mb][ks]));
      }
      const int h0 = mb * 16 + lg * 4;  // this lane's 4 output heads; H % 4 == 0
      const float4 wv = *reinterpret_cast<const float4 *>(w + grow * H + min(h0, H - 4));
      const bool wok = valid && h0 < H;
      sw[r][mb][0] = wok ? scale * wv.x : 0.0f;
      sw[r][mb][1] = wok ? scale * wv.y : 0.0f;
      sw[r][mb][2] = wok ? scale * wv.z : 0.0f;
      sw[r][mb][3] = wok ? scale * wv.w : 0.0f;
    }
  }
  // Global accesses of the loop go through buffer resources built from wave-uniform
  // values (forced into SGPRs) with 32-bit per-lane byte offsets: a chunk's score rows
  // stay within 2 GiB, and no 64-bit address arithmetic occupies VGPRs.  The resource
  // sizes cover exactly this workgroup's tile rows and pools below p_end.
  // Lane group lg stores row wr0 + 4j + lg of every row quad j.
  uint32_t orow_off[kQuads], grow_off[kQuads];
#pragma unroll
  for (int j = 0; j < kQuads; ++j) {
    const uint32_t my_row = (uint32_t)(row0 + min(wr0 + 4 * j + lg, nrows - 1) - chunk_row0);
    orow_off[j] = my_row * (uint32_t)ld * 4u;
    grow_off[j] = my_row * (uint32_t)ldg * 4u;
  }
  const uint32_t tile_end = __builtin_amdgcn_readfirstlane((uint32_t)(row0 + nrows - chunk_row0));
  auto uni_ptr = [](const void *p) {
    const uint64_t a = (uint64_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return (void *)(((uint64_t)hi << 32) | lo);
  };
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kRsrcWord3 = 0x00020000;  // raw buffer, 32-bit data format
  const __amdgpu_buffer_rsrc_t rs_out = __builtin_amdgcn_make_buffer_rsrc(
      uni_ptr(out), 0, (int)__builtin_amdgcn_readfirstlane(tile_end * (uint32_t)ld * 4u), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rs_gmax = __builtin_amdgcn_make_buffer_rsrc(
      uni_ptr(gmax), 0, (int)__builtin_amdgcn_readfirstlane(tile_end * (uint32_t)ldg * 4u), kRsrcWord3);
#endif

  // ---- pooled-key stages through LDS ---------------------------------------
  // Keys go global -> LDS with direct DMA loads (buffer_load_dwordx4 ... lds): one wave
  // instruction fills one contiguous 1 KiB region, lane i writing bytes [16i, 16i+16).
  // Within a key row, 16-byte slot j holds chunk j ^ swz(pool) of the key: an XOR swizzle
  // that makes the B-fragment reads of a sub-tile free of bank conflicts.  A 64-lane
  // ds_read_b128 is served in four phases of 16 lanes, each reading 256 bytes over the 64
  // banks: lanes {0-3, 12-15, 20-23, 24-27} and that set XOR 4, XOR 32 and XOR 36
  // (measured on gfx950 with the LDS bank-conflict counter over 26 lane patterns, which
  // this model predicts to within 0.02 cycles per read).  In a sub-tile's read, lane
  // (lg, lc) reads chunk 4 lg + ks of pool 4 lc + sub, and each phase holds every lc once,
  // with lane groups 2m on lc in {0-3, 12-15} and 2m + 1 on lc in {4-11} (or the reverse).
  // swz = lc ^ 4 [lc in 4..11] therefore puts the 16 lanes of a phase on 16 distinct
  // slots for every ks and sub, since the chunks of the two lane groups differ by 4.  (The
  // plain lc, which assumes phases of 16 consecutive lanes, costs 4 conflict cycles per
  // read.)  Shapes with fewer slots per row (the small test head dim) keep the plain
  // (pool / 4) mod NSLOT.  Chunks past D (padding of the K step) meet zero q fragments.
  auto swz = [](int pool) {
    const int lc = (pool >> 2) & (S::NSLOT - 1);
    return S::NSLOT == 16 ? lc ^ ((((lc >> 2) ^ (lc >> 3)) & 1) << 2) : lc;
  };
  // Per-lane byte offsets of the DMA regions inside a stage (a stage starts at a multiple
  // of 64 pools, so the swizzle of a lane's pool does not depend on the stage), computed
  // once.  Each stage's loads go through a buffer resource based at the stage's first
  // pool whose range ends at p_end: loads of pools at or past p_end fall outside it and
  // are dropped by the hardware range check (their LDS rows then hold zeros or an older
  // stage's keys; their scores are never stored).
  uint32_t dma_off[S::RGW];
#pragma unroll
  for (int i = 0; i < S::RGW; ++i) {
    const int byte = (wave + i * kWaves) * 1024 + lane * 16;
    const int pl = byte / S::ROWB;
    const int off = min((((byte % S::ROWB) / 16) ^ swz(pl)) * 8, D - 8);
    dma_off[i] = (uint32_t)(pl * D + off) * 2u;
  }
  const int p_begin_u = __builtin_amdgcn_readfirstlane(p_begin);
  const int p_end_u = __builtin_amdgcn_readfirstlane(p_end);
  const uint16_t *kps_u = (const uint16_t *)uni_ptr(kps);
  auto dma_stage = [&](int stage_base, int buf) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only emits the launch stub
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(kps_u + (int64_t)stage_base * D), 0, (p_end_u - stage_base) * D * 2, kRsrcWord3);
#endif
#pragma unroll
    for (int i = 0; i < S::RGW; ++i) {
      if (S::NREG % kWaves == 0 || wave + i * kWaves < S::NREG) {  // wave-uniform
#if defined(__HIP_DEVICE_COMPILE__)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs,
            (__attribute__((address_space(3))) void *)(lds + buf * S::STAGE_BYTES +
                                                       (wave + i * kWaves) * 1024),
            16, dma_off[i], 0, 0, 0);
#else
        (void)buf;
#endif
      }
    }
  };
  // B fragment of (pool row `pl` of a stage, chunk `c`) under the swizzle
  auto b_addr = [&](int pl, int c) { return pl * S::ROWB + ((c ^ swz(pl)) * 16); };

  // Sub-tile `sub` of a stage holds the pools 4c + sub (c = 0..15, the MFMA column), so
  // the 4 sub-tiles of a stage give a lane 4 consecutive pools of its row (one 16-byte
  // store), and every 16-pool group of a row sits in one lane quad.
  constexpr int kSubs = kStagePools / kSub;
  static_assert(kSubs == 4, "one 16-byte store per lane per stage");
  // Every stage computes all its sub-tiles (no branches between the LDS prefetches and
  // the MFMAs).  Alongside the scores, the max of every 16-pool group of a row (over
  // its visible pools) goes to `gmax`; the selection reads those first and then only
  // the groups that can hold a winner.  Pools at or past p_end are invisible to every
  // row of the tile, so store_lim (visible and below p_end) bounds both stores.
  int store_lim[kQuads];
#pragma unroll
  for (int j = 0; j < kQuads; ++j) {
    const int rr = wr0 + 4 * j + lg;
    store_lim[j] = rr < nrows ? min((int)((t0 + rr) / kpool) + 1, p_end) : 0;
  }
  // Lane-constant parts, so that a stage (base = its first pool, a multiple of 64, the
  // same for the whole wave) adds one scalar: the lane's pools are base + 4 lc + sub,
  // visible while sub < lim_rel - base; its score bytes start at so_lane + 4 base and its
  // group max at go_lane + base / 4 (pool base + 4 lc is in group base / 16 + lc / 4).
  int lim_rel[kQuads];
  uint32_t so_lane[kQuads], go_lane[kQuads];
#pragma unroll
  for (int j = 0; j < kQuads; ++j) {
    lim_rel[j] = store_lim[j] - 4 * lc;
    so_lane[j] = orow_off[j] + 16u * (uint32_t)lc;
    go_lane[j] = grow_off[j] + 4u * (uint32_t)(lc >> 2);
  }
  // A stage's reduced scores stay in registers (lane (g, c) holds pools 4c .. 4c + 3 of
  // row g) until its last sub-tile is reduced, then go out with one 16-byte store per
  // lane, so every score row is written in whole 256-byte runs.  A lane stores when its
  // first pool is visible to its row; up to 3 pools past the row's visible count then
  // receive finite values that the selection never reads (it reads each row only up to
  // its visible count), inside this workgroup's 64-aligned stage and the row's pitch.
  // The max of each 16-pool group (over the row's visible pools) is formed from the
  // same 4 values plus 2 quad steps.  Both stores are issued by every wave, lanes with
  // nothing to store giving an offset at or past the buffer's range (the hardware range
  // check drops such stores; the ranges are at most 2 GiB), so a wave issues exactly 2
  // stores per row quad and stage; the wait for the key DMA below relies on it.
  constexpr uint32_t kDrop = 0x80000000u;
  float vals[kQuads][kSubs] = {};
  // lane-local part of the group max (the lane's 4 pools, over the row's visible pools)
  auto flush_max = [&](int j, int base) {
    const int d = lim_rel[j] - base;  // this lane's pools base + 4 lc + sub are visible for sub < d
    float m = -__builtin_inff();
#pragma unroll
    for (int sub = 0; sub < kSubs; ++sub) m = fmaxf(m, sub < d ? vals[j][sub] : -__builtin_inff());
    return m;
  };
  auto flush_store = [&](int j, int base, bool live, float m) {
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0xB1, 0xF, 0xF, true)));
    m = fmaxf(m, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m), 0x4E, 0xF, 0xF, true)));
    const bool vis = live && 0 < lim_rel[j] - base;
#if defined(__HIP_DEVICE_COMPILE__)
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 u = {__float_as_uint(vals[j][0]), __float_as_uint(vals[j][1]),
                     __float_as_uint(vals[j][2]), __float_as_uint(vals[j][3])};
    // Scores are stored non-temporally (cache policy NT): they are written once and most of
    // them are never read back, so they should not push the group maxima, which the
    // selection reads next, out of the caches.
    constexpr int kNonTemporal = 2;
    __builtin_amdgcn_raw_buffer_store_b128(u, rs_out, vis ? so_lane[j] + 4u * (uint32_t)base : kDrop, 0,
                                           kNonTemporal);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(m), rs_gmax,
                                          vis && (lc & 3) == 0 ? go_lane[j] + (uint32_t)base / 4u : kDrop,
                                          0, 0);
#endif
  };

  // Each sub-tile's MFMAs run chain by chain: chain c = (row r, head block mb) takes its
  // K steps back to back (the accumulator dependence is forwarded inside the matrix
  // pipe), and while chain c runs, the VALU works on the epilogue (ReLU and head weights
  // of its 4 outputs) of the chain two places before it, whose MFMAs have completed by
  // then (chains 0 and 1 take the previous sub-tile's last two).  The epilogue thus
  // interleaves with the MFMAs at two VALU instructions per MFMA, and only three
  // chains' accumulators are live.  Every row accumulates its heads in the same order
  // (block 0, then block 1; the lane's 4 heads in order), so a score does not depend on
  // which slot of a wave its row occupies.
  constexpr int NCH = kRowsPerWave * S::MB;
  float x[kRowsPerWave] = {};  // head sums in progress (this lane's heads)
  // the two chains whose epilogues are pending (pb is the older)
  floatx4 pa = floatx4{0.0f, 0.0f, 0.0f, 0.0f}, pb = pa;
  auto epi = [&](int c) {
    const int r = c / S::MB, mb = c % S::MB;
#pragma unroll
    for (int i = 0; i < 4; ++i) x[r] = fmaf(fmaxf(pb[i], 0.0f), sw[r][mb][i], x[r]);
  };
  // row quad j: lane group g ends up holding row 4j + g, ((g0 + g1) + (g2 + g3)) for
  // every row
  auto reduce = [&](int j) {
    const float y01 = swap16_sum(x[4 * j], x[4 * j + 1]);
    const float y23 = swap16_sum(x[4 * j + 2], x[4 * j + 3]);
    // permlane32_swap(y01, y23): [y01.lo, y23.lo] + [y01.hi, y23.hi]
    auto z = __builtin_amdgcn_permlane32_swap(__float_as_uint(y01), __float_as_uint(y23), false, false);
#pragma unroll
    for (int r = 0; r < 4; ++r) x[4 * j + r] = 0.0f;
    return __uint_as_float(z[0]) + __uint_as_float(z[1]);
  };
  auto b_read = [&](const unsigned char *sb, int sub, int ks) {
    return *reinterpret_cast<const bf16x8 *>(sb + b_addr(4 * lc + sub, lg * (S::KG / 8) + ks));
  };

  const int nstage = (p_end_u - p_begin_u + kStagePools - 1) / kStagePools;  // wave-uniform
  dma_stage(p_begin_u, 0);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the first stage's keys have landed
  __syncthreads();
  // Explicit schedule.  Each chain is one scheduling region (a full scheduling barrier
  // after it), in which its K-step MFMAs alternate with the VALU work assigned to it:
  // the epilogue of the chain two places before it, and at fixed chain positions the
  // reduction of a row quad or one half of its store, so no VALU work piles up between
  // MFMAs.  Positions count chains from the start of a stage; quad j of sub-tile s is
  // complete once the epilogue of its last chain has run, and is reduced one chain
  // later, at red_pos(j, s), which for the last quad of the last sub-tile falls into
  // the next stage (kStageChains and beyond).  The stores of a stage's quad follow its
  // last reduction (first half: masked group max; second half: quad max and the two
  // stores).
  constexpr int kStageChains = kSubs * NCH;
  auto red_pos = [](int j, int s) { return s * NCH + 4 * (j + 1) * S::MB + 2; };
  auto fa_pos = [&](int j) { return red_pos(j, kSubs - 1) + 1; };
  float mloc[kQuads];
#pragma unroll
  for (int j = 0; j < kQuads; ++j) mloc[j] = -__builtin_inff();
  auto extras = [&](int pos, int stage_base, int st) {
#pragma unroll
    for (int j = 0; j < kQuads; ++j) {
#pragma unroll
      for (int s = 0; s < kSubs; ++s)
        if (red_pos(j, s) == pos) vals[j][s] = reduce(j);
      // wa / wb: the half runs in the stage after the one whose values it stores
      const int wa = fa_pos(j) >= kStageChains, wb = fa_pos(j) + 1 >= kStageChains;
      if (fa_pos(j) == pos) mloc[j] = flush_max(j, stage_base - wa * kStagePools);
      if (fa_pos(j) + 1 == pos) flush_store(j, stage_base - wb * kStagePools, st >= wb, mloc[j]);
    }
  };
  // a scheduling group of n VALU instructions (the builtin takes a constant)
  auto valu_group = [](int n) {
    if (n <= 2) __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
    else if (n == 3) __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    else if (n == 4) __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
    else if (n == 5) __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
    else if (n == 6) __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    else if (n == 7) __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
    else __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
  };
  auto extra_valu = [&](int pos) {
    int n = 0;
#pragma unroll
    for (int j = 0; j < kQuads; ++j) {
#pragma unroll
      for (int s = 0; s < kSubs; ++s) n += red_pos(j, s) == pos ? 8 : 0;
      n += fa_pos(j) == pos ? 14 : 0;
      n += fa_pos(j) + 1 == pos ? 6 : 0;
    }
    return n;
  };
  // The stage loop is unrolled by two so that the LDS buffer of a stage is a constant:
  // the B-fragment reads then carry it in their immediate offset.
  auto stage = [&](int st, auto buf_c) {
    constexpr int BUF = decltype(buf_c)::value;
    const int stage_base = p_begin_u + st * kStagePools;
    const unsigned char *sb = lds + BUF * S::STAGE_BYTES;
    // One set of B fragments: the next sub-tile's are read into the same registers
    // right after the last chain's MFMAs of this one (a second set, read a whole
    // sub-tile ahead, measured 0.5% slower and costs 14 VGPRs).
    bf16x8 b[S::KS];
#pragma unroll
    for (int sub = 0; sub < kSubs; ++sub) {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const int gp = sub * NCH + c;
        if (gp == 0) {
          // the next stage's key DMA goes out before any of this stage's stores
          if (st + 1 < nstage) dma_stage(stage_base + kStagePools, BUF ^ 1);
#pragma unroll
          for (int ks = 0; ks < S::KS; ++ks) b[ks] = b_read(sb, 0, ks);
        }
        // reductions and stores due here (previous stage's when pos wraps); they read
        // the head sums before this chain's epilogue updates them
        extras(gp, stage_base, st);
        extras(gp + kStageChains, stage_base, st);
        const int r = c / S::MB, mb = c % S::MB;
        floatx4 t = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < S::KS; ++ks) t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[r][mb][ks], b[ks], t, 0, 0, 0);
        if (c == NCH - 1 && sub + 1 < kSubs) {
#pragma unroll
          for (int ks = 0; ks < S::KS; ++ks) b[ks] = b_read(sb, sub + 1, ks);
        }
        epi((c + NCH - 2) % NCH);
        pb = pa;
        pa = t;
        if (gp != 0) {  // (the stage's first chain, behind the DMA and LDS reads, is left free)
          // the epilogue's 8 VALU and the extras' estimated count, spread over the K steps
          const int nv = (8 + extra_valu(gp) + extra_valu(gp + kStageChains) + S::KS - 1) / S::KS;
#pragma unroll
          for (int ks = 0; ks < S::KS; ++ks) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            valu_group(nv);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // This wave's key DMA for the next stage must have landed before the barrier
    // releases the other waves to read it: the barrier's fence does not cover LDS DMA,
    // so wait on vmcnt explicitly.  Vector memory operations complete in issue order for
    // this counter, and this stage issued 2 stores per row quad after the DMA, so
    // vmcnt(2 * kQuads) covers the DMA without waiting for them.
    static_assert(2 * kQuads < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | (2 * kQuads));  // vmcnt(2 * kQuads), no other counter
    __syncthreads();
    };
  for (int st = 0; st < nstage; st += 2) {
    stage(st, std::integral_constant<int, 0>{});
    if (st + 1 < nstage) stage(st + 1, std::integral_constant<int, 1>{});
  }
  // drain: the last two chains' epilogues, then the reductions and stores that fall
  // past the last stage
  epi(NCH - 2);
  pb = pa;
  epi(NCH - 1);
  {
    const int last_base = p_begin_u + (nstage - 1) * kStagePools;
#pragma unroll
    for (int pos = kStageChains; pos < 2 * kStageChains; ++pos) extras(pos, last_base + kStagePools, nstage);
  }
}

template <int H, int D>
hipError_t launch_t(const uint16_t *q, const uint16_t *kp, const float *w, float scale,
                    int32_t kpool, const SegList &segs, int32_t ntiles, int32_t npseg,
                    int32_t pseg_pools, int64_t chunk_row0, int64_t ld, float *out,
                    int64_t ldg, float *gmax, hipStream_t stream) {
  using S = Shape<H, D>;
  const size_t lds = 2 * S::STAGE_BYTES;
  const unsigned grid = (unsigned)ntiles * (unsigned)npseg;
  hipLaunchKernelGGL((score_kernel<H, D>), dim3(grid), dim3(kWaves * 64), lds, stream, q, kp, w,
                     scale, kpool, segs, npseg, pseg_pools, chunk_row0, ld, out, ldg, gmax);
  return hipGetLastError();
}

}  // namespace

bool score_supported(int H, int D) { return (H == 32 && D == 128) || (H == 4 && D == 16); }
int score_tile_rows() { return kTileRows; }

int score_slots(int H, int D, int device) {
  // (cached per device and shape; the query runs with the caller's current device, which
  // the library's entry points leave as the stream's device)
  constexpr int kDevs = 64;
  static std::atomic<int> cache[kDevs][2];
  const int shape = (H == 32 && D == 128) ? 0 : 1;
  if (device >= 0 && device < kDevs) {
    const int c = cache[device][shape].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0, per_cu = 0;
  hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
  if (e == hipSuccess) {
    if (shape == 0)
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_kernel<32, 128>, kWaves * 64,
                                                       2 * Shape<32, 128>::STAGE_BYTES);
    else
      e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, score_kernel<4, 16>, kWaves * 64,
                                                       2 * Shape<4, 16>::STAGE_BYTES);
  }
  if (e != hipSuccess || cus <= 0 || per_cu <= 0) return 0;
  const int slots = cus * per_cu;
  if (device >= 0 && device < kDevs) cache[device][shape].store(slots, std::memory_order_relaxed);
  return slots;
}

hipError_t launch_score(int H, int D, const uint16_t *q, const uint16_t *kp, const float *w,
                        float scale, int32_t kpool, const SegList &segs, int32_t ntiles,
                        int32_t npseg, int32_t pseg_pools, int64_t chunk_row0, int64_t ld,
                        float *out, int64_t ldg, float *gmax, hipStream_t stream) {
  if (pseg_pools % kStagePools != 0) return hipErrorInvalidValue;
  if (H == 32 && D == 128)
    return launch_t<32, 128>(q, kp, w, scale, kpool, segs, ntiles, npseg, pseg_pools, chunk_row0,
                             ld, out, ldg, gmax, stream);
  if (H == 4 && D == 16)
    return launch_t<4, 16>(q, kp, w, scale, kpool, segs, ntiles, npseg, pseg_pools, chunk_row0,
                           ld, out, ldg, gmax, stream);
  return hipErrorInvalidValue;
}

}  // namespace kpool
