// Indexer scan (csa2_index): I(t,s) = sum_h w[t][h] * ReLU(q[t][h] . K[b][s]).
//
// Lightning-indexer score of DeepSeek-V4 (gzher.com reading, sec. 4.1), kept by
// CSA2 (DeepSeek-V4.1-Flash report, sec. 2.3) with 32 heads x 128 (sec. 4.2.1).
//
// Per sequence the scan is a [32 heads x 128] x [128 x N] product, far below
// the MFMA ridge (32 flop per key byte), so the kernel is built around the key
// stream: each wave pulls two 16-key tiles (8 KiB) per iteration into the B
// operands of v_mfma_f32_16x16x32_bf16 (idx_tile.h), with the query in LDS.
// Blocks take 128-key chunks round-robin, so at any moment the whole grid
// sweeps one window of each sequence.  Per tile the scan forms the maximum
// score, and per (block, wave, tile slot, iteration mod S) group the maximum
// of those; that is all the selection needs (csa2_topk re-derives the few
// candidate tiles' scores).  The full score matrix is written only when the
// caller asks for it: interleaving 4 bytes of writes per 256 bytes of key
// reads costs about 7 % of the scan's bandwidth.  The same pass accumulates
// partial maxima of ||K_s||^2, from which csa2_topk forms a rigorous per-query
// bound on |fp32 - fp64 score| without a second read of the keys.  The whole
// call is this one kernel.
#include "idx_plan.h"
#include "idx_tile.h"

namespace csa2 {

// One block: sequence b = blockIdx.y, query group blockIdx.z (QG queries of
// that sequence), chunks x, x + gridDim.x, x + 2 gridDim.x, ... of 128 keys;
// wave w takes keys 32w .. 32w+31 of each chunk (kScanWaveKeys per wave).
// Group maxima: group (x * kScanTiles + u) * S + (i % S) holds the maxima of
// tile u of every wave in the block's iterations i, so a group samples the
// whole row and neighbouring tiles never share a group.
//
// With POOL (Reindex: csa2_reindex scores each query's candidate pool),
// "sequence" b is query b's pool: position s holds entry pool.rows[b N + s] of
// key sequence b / pool.qps of k_idx (pool.N_all rows each), or -1 (padding,
// scored -inf), and every position is visible.
struct PoolRows {
  const int32_t* rows;
  int64_t N_all;
  int qps;
};

template <int QG, int S, bool POOL = false>
__global__ __launch_bounds__(kScanThreads, QG == 1 ? 6 : QG == 2 ? 4 : 2) void idx_scan_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int ratio,
    int q_per_seq, int64_t N, float* __restrict__ scores, float* __restrict__ tile_max,
    uint32_t* __restrict__ header, float* __restrict__ group_max, float* __restrict__ norm_partial,
    PoolRows pool = PoolRows{}) {
  __shared__ __attribute__((aligned(16))) uint16_t sq[QG * kIdxHeads * kQRowPad];
  __shared__ float red[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // key within a tile
  const int g = lane >> 4;    // channel group
  const int b = blockIdx.y;
  const int64_t ld = tile_ld(N);
  const int64_t n_groups = group_count(gridDim.x, S);

  int64_t nvis[QG];
  int64_t trow[QG];
  bool valid[QG];
  float wr[QG][8];
  int64_t nvis_max = 0;
#pragma unroll
  for (int qq = 0; qq < QG; ++qq) {
    const int ql = blockIdx.z * QG + qq;
    valid[qq] = ql < q_per_seq;
    const int t = b * q_per_seq + (valid[qq] ? ql : q_per_seq - 1);
    trow[qq] = t;
    stage_query(&sq[qq * kIdxHeads * kQRowPad], q_idx + (size_t)t * kIdxHeads * kIdxDim, threadIdx.x,
                kScanThreads);
    load_head_weights(w_idx + (size_t)t * kIdxHeads, g, wr[qq]);
    nvis[qq] = valid[qq] ? n_visible(q_pos, t, ratio, N) : 0;
    nvis_max = nvis[qq] > nvis_max ? nvis[qq] : nvis_max;
    // the summary header starts at zero (the selection's counters rely on it)
    if (blockIdx.x == 0 && valid[qq] && threadIdx.x < CSA2_STATS_WORDS)
      header[(size_t)t * CSA2_STATS_WORDS + threadIdx.x] = 0u;
  }
  __syncthreads();

  const int64_t nchunks = (N + kChunkKeys - 1) / kChunkKeys;
  const uint16_t* kseq = POOL ? k_idx + (size_t)(b / pool.qps) * pool.N_all * kIdxDim : k_idx + (size_t)b * N * kIdxDim;
  const int64_t last = (nvis_max < N ? (nvis_max > 0 ? nvis_max : 1) : N) - 1;  // last row worth reading
  float maxn2 = 0.f;
  float gm[QG][S];
#pragma unroll
  for (int qq = 0; qq < QG; ++qq)
#pragma unroll
    for (int r = 0; r < S; ++r) gm[qq][r] = -INFINITY;

  int it = 0;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x, ++it) {
    const int64_t base = c * kChunkKeys + kScanWaveKeys * wave;
    // Unconditional loads keep the code branch-free: keys past the end or past
    // every query's visibility re-read row `last`, which is already cached.
    uint4 kv[kScanTiles][4];
    bool live[kScanTiles];
#pragma unroll
    for (int u = 0; u < kScanTiles; ++u) {
      const int64_t s = base + u * kTileKeys + col;
      int64_t row = s < last ? s : last;
      live[u] = true;
      if (POOL) {
        const int32_t e = pool.rows[(size_t)b * N + row];
        live[u] = e >= 0;
        row = e >= 0 ? e : 0;
      }
      load_key_slices(kseq, row, g, kv[u]);
    }
    float sc[QG][kScanTiles];
#pragma unroll
    for (int u = 0; u < kScanTiles; ++u) {
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) sc[qq][u] = -INFINITY;
      const int64_t s = base + u * kTileKeys + col;
      if (base + u * kTileKeys >= nvis_max) continue;  // no query of the group sees this tile
      // this lane's 32 channels of ||K_s||^2 (bf16 dot2); the block sums the four
      // channel groups' maxima over its keys, an upper bound of max_s ||K_s||^2
      float n2 = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w4[4] = {kv[u][j].x, kv[u][j].y, kv[u][j].z, kv[u][j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2 p;
          __builtin_memcpy(&p, &w4[e], 4);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(p, p, n2, false);
        }
      }
      if (s < N) maxn2 = fmaxf(maxn2, n2);
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) {
        if (!valid[qq]) continue;
        const float part = tile_score(&sq[qq * kIdxHeads * kQRowPad], kv[u], wr[qq], col, g);
        sc[qq][u] = (s < nvis[qq] && live[u]) ? part : -INFINITY;
      }
    }
    // Every lane holds the score of key `col` of each tile.  Lane l < 32 stores
    // key l of the wave's 32 (one 128-byte store) and lanes 0..1 the tile maxima.
    const int64_t so = base + lane;
    const int64_t tile = base / kTileKeys + lane;
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      float v = sc[qq][0], m = -INFINITY;
#pragma unroll
      for (int u = 0; u < kScanTiles; ++u) {
        // maximum over the 16 keys of the tile (one 16-lane row) with DPP moves
        const float tm = row_max16(sc[qq][u]);
        if (u > 0) v = g == u ? sc[qq][u] : v;
        m = lane == u ? tm : m;
      }
#pragma unroll
      for (int r = 0; r < S; ++r) gm[qq][r] = (it % S == r) ? fmaxf(gm[qq][r], m) : gm[qq][r];
      if (!valid[qq]) continue;
      if (scores != nullptr && lane < kScanWaveKeys && so < N) scores[trow[qq] * N + so] = v;
      if (lane < kScanTiles && tile * kTileKeys < N) tile_max[trow[qq] * ld + tile] = m;
    }
  }
  // group maxima merged over the block's waves (LDS), and the block's max ||K||^2
  constexpr int kPer = kScanTiles * S;  // groups per block and query
  __shared__ float gml[kScanWaves][QG][kPer];
  if (lane < kScanTiles) {
#pragma unroll
    for (int qq = 0; qq < QG; ++qq)
#pragma unroll
      for (int r = 0; r < S; ++r) gml[wave][qq][lane * S + r] = gm[qq][r];
  }
  // row g of the wave holds channel group g: its maximum over the wave's keys,
  // then the sum over the four groups
  maxn2 = fmaxf(maxn2, dpp_f32<kDppXor1>(maxn2));
  maxn2 = fmaxf(maxn2, dpp_f32<kDppXor2>(maxn2));
  maxn2 = fmaxf(maxn2, dpp_f32<kDppHalfMirror>(maxn2));
  maxn2 = fmaxf(maxn2, dpp_f32<kDppMirror>(maxn2));
  maxn2 = ((lane_f32(maxn2, 0) + lane_f32(maxn2, 16)) + lane_f32(maxn2, 32)) + lane_f32(maxn2, 48);
  if (lane == 0) red[wave] = maxn2;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      if (lane < kPer && valid[qq]) {
        float m = gml[0][qq][lane];
#pragma unroll
        for (int i = 1; i < kScanWaves; ++i) m = fmaxf(m, gml[i][qq][lane]);
        group_max[trow[qq] * n_groups + (int64_t)blockIdx.x * kPer + lane] = m;
      }
      // padding of the row to a multiple of four
      const int64_t used = (int64_t)gridDim.x * kPer;
      if (blockIdx.x == 0 && valid[qq] && lane < n_groups - used) group_max[trow[qq] * n_groups + used + lane] = -INFINITY;
    }
  }
  if (threadIdx.x == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kScanWaves; ++i) m = fmaxf(m, red[i]);
    norm_partial[((size_t)b * gridDim.z + blockIdx.z) * gridDim.x + blockIdx.x] = m;
  }
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_index_stats_bytes(int32_t T, int32_t q_per_seq, int64_t N) {
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return 0;
  return stats_words(T, p) * sizeof(uint32_t);
}

extern "C" int64_t csa2_tile_max_ld(int64_t N) { return N < 1 ? 0 : tile_ld(N); }

// One query per block (decode): the 16 x 16 layout here; several queries per
// sequence: the grouped-query scan (index_group.hip).
template <int S>
static void launch_scan_s(dim3 grid, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                          const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                          uint32_t* header, float* gmax, float* partial) {
  hipLaunchKernelGGL((idx_scan_kernel<1, S>), grid, dim3(kScanThreads), 0, st, q, w, k, q_pos, ratio, q_per_seq, N,
                     scores, tile_max, header, gmax, partial);
}

static void launch_scan(const IndexPlan& p, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                        const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                        uint32_t* header, float* gmax, float* partial) {
  const dim3 grid(p.blocks_x, p.B, p.groups);
  if (p.slots == 1)
    launch_scan_s<1>(grid, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
  else if (p.slots == 2)
    launch_scan_s<2>(grid, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
  else
    launch_scan_s<4>(grid, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
}

namespace csa2 {

// The Reindex scan: query t's pool as its own one-query "sequence" of P
// positions (key rows through the pool, padding scored -inf), with the outputs
// and summary of csa2_index(T, 1, P).
csa2_status index_pool_launch(const void* q_idx, const float* w_idx, const void* k_all, int64_t N_all, int qps,
                              const int32_t* pool, int32_t T, int64_t P, float* scores, float* tile_max,
                              uint32_t* stats, size_t stats_bytes, hipStream_t st) {
  IndexPlan p;
  if (!index_plan(T, 1, P, &p)) return CSA2_ERR_UNSUPPORTED;
  if (stats_bytes < stats_words(T, p) * sizeof(uint32_t)) return CSA2_ERR_INVALID_ARG;
  (void)hipGetLastError();
  float* gmax = (float*)(stats + stats_groups_off(T));
  float* partial = (float*)(stats + stats_parts_off(T, p.n_groups));
  const dim3 grid(p.blocks_x, p.B, p.groups);
  const PoolRows pr{pool, N_all, qps};
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* k = (const uint16_t*)k_all;
  if (p.slots == 1)
    hipLaunchKernelGGL((idx_scan_kernel<1, 1, true>), grid, dim3(kScanThreads), 0, st, q, w_idx, k, nullptr, 1, 1, P,
                       scores, tile_max, stats, gmax, partial, pr);
  else if (p.slots == 2)
    hipLaunchKernelGGL((idx_scan_kernel<1, 2, true>), grid, dim3(kScanThreads), 0, st, q, w_idx, k, nullptr, 1, 1, P,
                       scores, tile_max, stats, gmax, partial, pr);
  else
    hipLaunchKernelGGL((idx_scan_kernel<1, 4, true>), grid, dim3(kScanThreads), 0, st, q, w_idx, k, nullptr, 1, 1, P,
                       scores, tile_max, stats, gmax, partial, pr);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}

}  // namespace csa2

extern "C" csa2_status csa2_index(const void* q_idx, const float* w_idx, const void* k_idx,
                                  const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq,
                                  int64_t N, float* scores, float* tile_max, uint32_t* stats, size_t stats_bytes,
                                  void* hip_stream) {
  if (!q_idx || !w_idx || !k_idx || !tile_max || !stats) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) || (scores && !aligned16(scores)) ||
      !aligned16(tile_max) || !aligned16(stats) || (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || N < 1 || ratio < 1 || T % q_per_seq != 0) return CSA2_ERR_INVALID_ARG;
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  if (stats_bytes < stats_words(T, p) * sizeof(uint32_t)) return CSA2_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  float* gmax = (float*)(stats + stats_groups_off(T));
  float* partial = (float*)(stats + stats_parts_off(T, p.n_groups));
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* k = (const uint16_t*)k_idx;
  if (p.qg == 1)
    launch_scan(p, st, q, w_idx, k, q_pos, ratio, q_per_seq, N, scores, tile_max, stats, gmax, partial);
  else
    launch_scan_grouped(p, st, q, w_idx, k, q_pos, ratio, q_per_seq, N, scores, tile_max, stats, gmax, partial);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
