// Indexer scan over MXFP4 indexer queries and keys (csa2_index_mxfp4):
// I(t,s) = sum_h w[t][h] * ReLU(deq(q[t][h]) . deq(K[b][s])).
//
// The lightning-indexer score (gzher.com reading of DeepSeek-V4, sec. 4.1)
// with the FP4 indexer queries and keys of DeepSeek-V4 that the V4.1-Flash
// report keeps (sec. 2.4.4: MXFP4; 64 + 4 bytes per 128-channel key).  The key
// stream shrinks from 256 to 68 bytes per entry; the product moves to
// v_mfma_scale_f32_16x16x128_f8f6f4, one instruction per 16 keys and 16 heads
// with the E8M0 block scales applied in the instruction (mxfp4.h).  Still far
// below the FP4 MFMA ridge (8192 flop per 68 bytes against ~1260), so the
// kernel is again built around the key stream: each wave requests eight
// 16-key tiles (8.5 KiB) per iteration.  It leaves the bf16 scan's summary
// (tile maxima, group maxima of disjoint groups of whole tiles, partial
// maxima of an upper bound of ||K||^2) for the same selection kernels, plus the
// dequantised queries (bf16, exact) for their fp64 rescoring and norms.
#include "mxfp4.h"

namespace csa2 {

// One block: sequence b = blockIdx.y, query group blockIdx.z (QG queries),
// chunks x, x + gridDim.x, ... of 512 keys; wave w takes keys 128w .. 128w+127
// of each chunk.  Group (x * kMxTiles + u) * S + (i % S) holds the maxima of
// tile u of every wave in the block's iterations i.
static_assert(kMxTiles == 8, "lane l stores keys l and 64 + l of the wave's 128");

template <int QG, int S>
__global__ __launch_bounds__(kMxThreads) void idx_scan_mx_kernel(
    const uint8_t* __restrict__ q_codes, const uint8_t* __restrict__ q_scales, const float* __restrict__ w_idx,
    const uint8_t* __restrict__ k_codes, const uint8_t* __restrict__ k_scales, const int32_t* __restrict__ q_pos,
    int ratio, int q_per_seq, int64_t N, float* __restrict__ scores, float* __restrict__ tile_max,
    uint32_t* __restrict__ header, float* __restrict__ group_max, float* __restrict__ norm_partial,
    uint16_t* __restrict__ q_deq) {
  __shared__ float red[kMxWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int g = lane >> 4;
  const int b = blockIdx.y;
  const int64_t ld = tile_ld(N);
  const int64_t n_groups = mx_group_count(gridDim.x, S);

  int64_t nvis[QG];
  int64_t trow[QG];
  bool valid[QG];
  float wr[QG][8];
  uint4 qa[QG][2];
  uint32_t qsc[QG][2];
  int64_t nvis_max = 0;
#pragma unroll
  for (int qq = 0; qq < QG; ++qq) {
    const int ql = blockIdx.z * QG + qq;
    valid[qq] = ql < q_per_seq;
    const int t = b * q_per_seq + (valid[qq] ? ql : q_per_seq - 1);
    trow[qq] = t;
    const uint8_t* qc = q_codes + (size_t)t * kIdxHeads * kMxRowBytes;
    const uint8_t* qs = q_scales + (size_t)t * kIdxHeads * kMxScales;
    load_query_mx(qc, qs, col, g, qa[qq], qsc[qq]);
    load_head_weights(w_idx + (size_t)t * kIdxHeads, g, wr[qq]);
    nvis[qq] = valid[qq] ? n_visible(q_pos, t, ratio, N) : 0;
    nvis_max = nvis[qq] > nvis_max ? nvis[qq] : nvis_max;
    if (blockIdx.x == 0 && valid[qq]) {
      // the summary header starts at zero; the dequantised query for the selection:
      // thread i takes 8 code bytes (16 channels) of head i / 8
      if (threadIdx.x < CSA2_STATS_WORDS) header[(size_t)t * CSA2_STATS_WORDS + threadIdx.x] = 0u;
      const int h = threadIdx.x >> 3, c16 = threadIdx.x & 7;
      const uint2 cw = *reinterpret_cast<const uint2*>(qc + h * kMxRowBytes + 8 * c16);
      const uint32_t sb = qs[h * kMxScales + (c16 >> 1)];
      uint4* dst = reinterpret_cast<uint4*>(q_deq + ((size_t)t * kIdxHeads + h) * kIdxDim + 16 * c16);
      dst[0] = dequant8(cw.x, sb);
      dst[1] = dequant8(cw.y, sb);
    }
  }

  const int64_t nchunks = (N + kMxChunkKeys - 1) / kMxChunkKeys;
  const uint8_t* kc = k_codes + (size_t)b * N * kMxRowBytes;
  const uint8_t* ks = k_scales + (size_t)b * N * kMxScales;
  const int64_t last = (nvis_max < N ? (nvis_max > 0 ? nvis_max : 1) : N) - 1;  // last row worth reading
  float maxn2 = 0.f;
  float gm[QG][S];
#pragma unroll
  for (int qq = 0; qq < QG; ++qq)
#pragma unroll
    for (int r = 0; r < S; ++r) gm[qq][r] = -INFINITY;

  int it = 0;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x, ++it) {
    const int64_t base = c * kMxChunkKeys + kMxWaveKeys * wave;
    // unconditional loads (rows past the end re-read row `last`, already cached)
    uint4 kv[kMxTiles];
    uint32_t kscale[kMxTiles];
#pragma unroll
    for (int u = 0; u < kMxTiles; ++u) {
      const int64_t s = base + u * kTileKeys + col;
      load_key_mx(kc, ks, s < last ? s : last, g, &kv[u], &kscale[u]);
    }
    float sc[QG][kMxTiles];
#pragma unroll
    for (int u = 0; u < kMxTiles; ++u) {
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) sc[qq][u] = -INFINITY;
      const int64_t s = base + u * kTileKeys + col;
      if (base + u * kTileKeys >= nvis_max) continue;  // no query of the group sees this tile
      if (s < N) maxn2 = fmaxf(maxn2, mx_block_norm2_bound(kscale[u]));
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) {
        if (!valid[qq]) continue;
        const float part = tile_score_mx(qa[qq], qsc[qq], kv[u], kscale[u], wr[qq]);
        sc[qq][u] = (s < nvis[qq]) ? part : -INFINITY;
      }
    }
    // Every lane holds the score of key `col` of each tile.  Lane l stores keys
    // l and 64 + l of the wave's 128 (tiles l / 16 and 4 + l / 16), lanes
    // 0..7 the tile maxima.
    const int64_t tile = base / kTileKeys + lane;
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      float v0 = sc[qq][0], v1 = sc[qq][4], m = -INFINITY;
#pragma unroll
      for (int u = 0; u < kMxTiles; ++u) {
        const float tm = row_max16(sc[qq][u]);
        if (u > 0 && u < 4) v0 = g == u ? sc[qq][u] : v0;
        if (u > 4) v1 = g == u - 4 ? sc[qq][u] : v1;
        m = lane == u ? tm : m;
      }
#pragma unroll
      for (int r = 0; r < S; ++r) gm[qq][r] = (it % S == r) ? fmaxf(gm[qq][r], m) : gm[qq][r];
      if (!valid[qq]) continue;
      if (scores != nullptr) {
        const int64_t s0 = base + lane, s1 = base + 64 + lane;
        if (s0 < N) scores[trow[qq] * N + s0] = v0;
        if (s1 < N) scores[trow[qq] * N + s1] = v1;
      }
      if (lane < kMxTiles && tile * kTileKeys < N) tile_max[trow[qq] * ld + tile] = m;
    }
  }
  // group maxima merged over the block's waves (LDS), and the block's ||K||^2 bound
  constexpr int kPer = kMxTiles * S;
  __shared__ float gml[kMxWaves][QG][kPer];
  if (lane < kMxTiles) {
#pragma unroll
    for (int qq = 0; qq < QG; ++qq)
#pragma unroll
      for (int r = 0; r < S; ++r) gml[wave][qq][lane * S + r] = gm[qq][r];
  }
  // row g of the wave holds scale block g: its maximum over the wave's keys,
  // then the sum over the four blocks
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
        for (int i = 1; i < kMxWaves; ++i) m = fmaxf(m, gml[i][qq][lane]);
        group_max[trow[qq] * n_groups + (int64_t)blockIdx.x * kPer + lane] = m;
      }
      const int64_t used = (int64_t)gridDim.x * kPer;
      if (blockIdx.x == 0 && valid[qq] && lane < n_groups - used) group_max[trow[qq] * n_groups + used + lane] = -INFINITY;
    }
  }
  if (threadIdx.x == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kMxWaves; ++i) m = fmaxf(m, red[i]);
    norm_partial[((size_t)b * gridDim.z + blockIdx.z) * gridDim.x + blockIdx.x] = m;
  }
  // the (at most 3) words between the partials and the 16-byte aligned queries
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    uint32_t* pend = reinterpret_cast<uint32_t*>(norm_partial + (size_t)gridDim.x * gridDim.y * gridDim.z);
    const int64_t pad = reinterpret_cast<uint32_t*>(q_deq) - pend;
    if (threadIdx.x < pad) pend[threadIdx.x] = 0u;
  }
}

template <int QG>
static void launch_scan_mx(const MxPlan& p, hipStream_t st, const uint8_t* qc, const uint8_t* qs, const float* w,
                           const uint8_t* kc, const uint8_t* ks, const int32_t* q_pos, int ratio, int q_per_seq,
                           int64_t N, float* scores, float* tile_max, uint32_t* header, float* gmax, float* partial,
                           uint16_t* q_deq) {
  const dim3 grid(p.blocks_x, p.B, p.groups);
  if (p.slots == 1)
    hipLaunchKernelGGL((idx_scan_mx_kernel<QG, 1>), grid, dim3(kMxThreads), 0, st, qc, qs, w, kc, ks, q_pos, ratio,
                       q_per_seq, N, scores, tile_max, header, gmax, partial, q_deq);
  else if (p.slots == 2)
    hipLaunchKernelGGL((idx_scan_mx_kernel<QG, 2>), grid, dim3(kMxThreads), 0, st, qc, qs, w, kc, ks, q_pos, ratio,
                       q_per_seq, N, scores, tile_max, header, gmax, partial, q_deq);
  else
    hipLaunchKernelGGL((idx_scan_mx_kernel<QG, 4>), grid, dim3(kMxThreads), 0, st, qc, qs, w, kc, ks, q_pos, ratio,
                       q_per_seq, N, scores, tile_max, header, gmax, partial, q_deq);
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_index_mxfp4_stats_bytes(int32_t T, int32_t q_per_seq, int64_t N) {
  MxPlan p;
  if (!mx_plan(T, q_per_seq, N, &p)) return 0;
  return mx_stats_words(T, p) * sizeof(uint32_t);
}

extern "C" csa2_status csa2_index_mxfp4(const uint8_t* q_codes, const uint8_t* q_scales, const float* w_idx,
                                        const uint8_t* k_codes, const uint8_t* k_scales, const int32_t* q_pos,
                                        int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, float* scores,
                                        float* tile_max, uint32_t* stats, size_t stats_bytes, void* hip_stream) {
  if (!q_codes || !q_scales || !w_idx || !k_codes || !k_scales || !tile_max || !stats) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(q_codes) || !aligned16(q_scales) || !aligned16(w_idx) || !aligned16(k_codes) ||
      !aligned16(k_scales) || (scores && !aligned16(scores)) || !aligned16(tile_max) || !aligned16(stats) ||
      (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || N < 1 || ratio < 1 || T % q_per_seq != 0) return CSA2_ERR_INVALID_ARG;
  MxPlan p;
  if (!mx_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  if (stats_bytes < mx_stats_words(T, p) * sizeof(uint32_t)) return CSA2_ERR_INVALID_ARG;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  float* gmax = (float*)(stats + (size_t)T * CSA2_STATS_WORDS);
  float* partial = gmax + (size_t)T * p.n_groups;
  uint16_t* q_deq = (uint16_t*)(stats + mx_qdeq_off(T, p));
  if (p.qg == 1)
    launch_scan_mx<1>(p, st, q_codes, q_scales, w_idx, k_codes, k_scales, q_pos, ratio, q_per_seq, N, scores,
                      tile_max, stats, gmax, partial, q_deq);
  else if (p.qg == 2)
    launch_scan_mx<2>(p, st, q_codes, q_scales, w_idx, k_codes, k_scales, q_pos, ratio, q_per_seq, N, scores,
                      tile_max, stats, gmax, partial, q_deq);
  else
    launch_scan_mx<4>(p, st, q_codes, q_scales, w_idx, k_codes, k_scales, q_pos, ratio, q_per_seq, N, scores,
                      tile_max, stats, gmax, partial, q_deq);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
