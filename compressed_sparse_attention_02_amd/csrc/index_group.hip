// Grouped-query indexer scan (csa2_index with several queries per sequence:
// prefill chunks).  The same score as the one-query scan in index.hip,
// I(t,s) = sum_h w[t][h] * ReLU(q[t][h] . K[b][s]) (lightning indexer of
// DeepSeek-V4, gzher.com reading, sec. 4.1; CSA2 keeps it, DeepSeek-V4.1-Flash
// report, sec. 2.3), the same grid, chunks, outputs and error bound; here
// every key a wave reads serves QG queries, so the products, not the key
// stream, bound the kernel.
#include "idx_plan.h"
#include "idx_tile.h"

namespace csa2 {
// Grouped-query variant (QG >= 2 queries of one sequence per block: prefill
// chunks, several queries per sequence): the same grid, chunks, outputs and
// bound as idx_scan_kernel, with each wave's 32 keys of an iteration as one
// 32 x 32 tile of v_mfma_f32_32x32x16_bf16.  A is the query's 32 heads x 16
// channels of a k-step (lane l: head l % 32, channels 8(l/32) .. +7, from
// LDS), B the 32 keys (lane l: key l % 32, the same channels), and register r
// of the accumulator holds head 8(r/4) + 4(l/32) + r%4 of key l % 32.  One
// instruction covers all heads, and a lane folds 16 heads of one key (two
// chains of eight, then the lane pair), with the tile maxima and the score
// stores once per 32 keys: about half the VALU work per key and query of the
// 16 x 16 layout, whose fold bounds the grouped scan.  The fp32 scores differ
// from that layout's only in summation order (the products are exact; every
// path has at most 128 additions of products and 10 roundings in the head
// fold), so they stay within the selection's error bound.
template <int QG, int S>
__global__ __launch_bounds__(kScanThreads) void idx_scan32_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int ratio,
    int q_per_seq, int64_t N, float* __restrict__ scores, float* __restrict__ tile_max,
    uint32_t* __restrict__ header, float* __restrict__ group_max, float* __restrict__ norm_partial) {
  static_assert(kScanWaveKeys == 32 && kScanTiles == 2, "one 32-key tile (two 16-key tiles) per wave and iteration");
  __shared__ __attribute__((aligned(16))) uint16_t sq[QG * kIdxHeads * kQRowPad];
  __shared__ __attribute__((aligned(16))) float sw[QG][kIdxHeads];
  __shared__ float red[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 31;  // key within the wave's 32
  const int hf = lane >> 5;   // channel half of each k-step
  const int b = blockIdx.y;
  const int64_t ld = tile_ld(N);
  const int64_t n_groups = group_count(gridDim.x, S);

  int64_t nvis[QG];
  int64_t trow[QG];
  bool valid[QG];
  int64_t nvis_max = 0;
#pragma unroll
  for (int qq = 0; qq < QG; ++qq) {
    const int ql = blockIdx.z * QG + qq;
    valid[qq] = ql < q_per_seq;
    const int t = b * q_per_seq + (valid[qq] ? ql : q_per_seq - 1);
    trow[qq] = t;
    stage_query(&sq[qq * kIdxHeads * kQRowPad], q_idx + (size_t)t * kIdxHeads * kIdxDim, threadIdx.x,
                kScanThreads);
    if (threadIdx.x < kIdxHeads) sw[qq][threadIdx.x] = w_idx[(size_t)t * kIdxHeads + threadIdx.x];
    nvis[qq] = valid[qq] ? n_visible(q_pos, t, ratio, N) : 0;
    nvis_max = nvis[qq] > nvis_max ? nvis[qq] : nvis_max;
    // the summary header starts at zero (the selection's counters rely on it)
    if (blockIdx.x == 0 && valid[qq] && threadIdx.x < CSA2_STATS_WORDS)
      header[(size_t)t * CSA2_STATS_WORDS + threadIdx.x] = 0u;
  }
  __syncthreads();

  const int64_t nchunks = (N + kChunkKeys - 1) / kChunkKeys;
  const uint16_t* kseq = k_idx + (size_t)b * N * kIdxDim;
  const int64_t last = (nvis_max < N ? (nvis_max > 0 ? nvis_max : 1) : N) - 1;  // last row worth reading
  // Query group 0 bounds ||K_s||^2 over every key of its chunks, visible or
  // not, and that bound stands for every group of the sequence (the others
  // skip the norms): a bound over all keys bounds each query's visible ones.
  const bool norms = blockIdx.z == 0;
  const int64_t lastk = norms ? N - 1 : last;
  float maxn2 = 0.f;
  float gm[QG][S];
#pragma unroll
  for (int qq = 0; qq < QG; ++qq)
#pragma unroll
    for (int r = 0; r < S; ++r) gm[qq][r] = -INFINITY;

  int it = 0;
  for (int64_t c = blockIdx.x; c < nchunks; c += gridDim.x, ++it) {
    const int64_t base = c * kChunkKeys + kScanWaveKeys * wave;
    const int64_t s = base + col;
    // key s, channels 16j + 8(l/32) .. +7 of k-step j (keys past the end or
    // past every query's visibility re-read row `last`, already cached)
    uint4 kv[8];
    const uint16_t* kp = kseq + (size_t)(s < lastk ? s : lastk) * kIdxDim + 8 * hf;
#pragma unroll
    for (int j = 0; j < 8; ++j) kv[j] = *reinterpret_cast<const uint4*>(kp + 16 * j);
    float sc[QG];
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) sc[qq] = -INFINITY;
    if (norms) {
      // this lane's 64 channels of ||K_s||^2 (bf16 dot2); the block sums the two
      // channel halves' maxima over its keys, an upper bound of max_s ||K_s||^2
      float n2 = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w4[4] = {kv[j].x, kv[j].y, kv[j].z, kv[j].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16x2 pr;
          __builtin_memcpy(&pr, &w4[e], 4);
          n2 = __builtin_amdgcn_fdot2_f32_bf16(pr, pr, n2, false);
        }
      }
      if (s < N) maxn2 = fmaxf(maxn2, n2);
    }
    if (base < nvis_max) {
      // The queries' products in two accumulators, one query ahead of its
      // fold, so that query qq's fold (VALU) overlaps query qq + 1's MFMA
      // chain.  A padding query (past q_per_seq) repeats the last query's
      // row and is computed and discarded.
      floatx16 acc[2];
      const auto chain = [&](int qq, floatx16& a) {
        const uint16_t* qa = &sq[qq * kIdxHeads * kQRowPad] + col * kQRowPad + 8 * hf;
        a = floatx16{};
#pragma unroll
        for (int j = 0; j < 8; ++j)
          a = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8*>(qa + 16 * j),
                                                      as_bf16x8(kv[j]), a, 0, 0, 0);
      };
      chain(0, acc[0]);
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) {
        if (qq + 1 < QG) chain(qq + 1, acc[(qq + 1) & 1]);
        const floatx16& a = acc[qq & 1];
        // heads 8i + 4(l/32) + 0..3 sit in registers 4i .. 4i+3
        float p0 = 0.f, p1 = 0.f;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float4 w0 = *reinterpret_cast<const float4*>(&sw[qq][8 * i + 4 * hf]);
          const float4 w1 = *reinterpret_cast<const float4*>(&sw[qq][8 * (i + 2) + 4 * hf]);
          p0 = fmaf(w0.x, relu_bits(a[4 * i]), p0);
          p0 = fmaf(w0.y, relu_bits(a[4 * i + 1]), p0);
          p0 = fmaf(w0.z, relu_bits(a[4 * i + 2]), p0);
          p0 = fmaf(w0.w, relu_bits(a[4 * i + 3]), p0);
          p1 = fmaf(w1.x, relu_bits(a[4 * i + 8]), p1);
          p1 = fmaf(w1.y, relu_bits(a[4 * i + 9]), p1);
          p1 = fmaf(w1.z, relu_bits(a[4 * i + 10]), p1);
          p1 = fmaf(w1.w, relu_bits(a[4 * i + 11]), p1);
        }
        const float tot = sum_xor32(p0 + p1);
        sc[qq] = (valid[qq] && s < nvis[qq]) ? tot : -INFINITY;
      }
    }
    // Lanes 0..31 store keys base .. base + 31 (one 128-byte store); the tile
    // maxima are the 16-lane row maxima, moved to lanes 0 and 1.
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      const float tm = row_max16(sc[qq]);
      const float m = __shfl(tm, 16 * (lane & 1), 64);
#pragma unroll
      for (int r = 0; r < S; ++r) gm[qq][r] = (it % S == r) ? fmaxf(gm[qq][r], m) : gm[qq][r];
      if (!valid[qq]) continue;
      if (scores != nullptr && lane < kScanWaveKeys && s < N) scores[trow[qq] * N + s] = sc[qq];
      const int64_t tile = base / kTileKeys + lane;
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
  // lanes 0..31 hold channel half 0, lanes 32..63 half 1: each half's maximum
  // over the wave's keys (16-lane rows, then the row pair), then their sum
  maxn2 = fmaxf(maxn2, dpp_f32<kDppXor1>(maxn2));
  maxn2 = fmaxf(maxn2, dpp_f32<kDppXor2>(maxn2));
  maxn2 = fmaxf(maxn2, dpp_f32<kDppHalfMirror>(maxn2));
  maxn2 = fmaxf(maxn2, dpp_f32<kDppMirror>(maxn2));
  maxn2 = fmaxf(lane_f32(maxn2, 0), lane_f32(maxn2, 16)) + fmaxf(lane_f32(maxn2, 32), lane_f32(maxn2, 48));
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
  if (norms && wave == 0) {  // the same bound into every group's slot of this key range
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kScanWaves; ++i) m = fmaxf(m, red[i]);
    for (int z = lane; z < (int)gridDim.z; z += 64)
      norm_partial[((size_t)b * gridDim.z + z) * gridDim.x + blockIdx.x] = m;
  }
}

template <int QG, int S>
static void launch_s(dim3 grid, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                     const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                     uint32_t* header, float* gmax, float* partial) {
  hipLaunchKernelGGL((idx_scan32_kernel<QG, S>), grid, dim3(kScanThreads), 0, st, q, w, k, q_pos, ratio, q_per_seq, N,
                     scores, tile_max, header, gmax, partial);
}

template <int QG>
static void launch_q(const IndexPlan& p, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                     const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                     uint32_t* header, float* gmax, float* partial) {
  const dim3 grid(p.blocks_x, p.B, p.groups);
  if (p.slots == 1)
    launch_s<QG, 1>(grid, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
  else
    launch_s<QG, 2>(grid, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
}

void launch_scan_grouped(const IndexPlan& p, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                         const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                         uint32_t* header, float* gmax, float* partial) {
  if (p.qg == 2)
    launch_q<2>(p, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
  else
    launch_q<4>(p, st, q, w, k, q_pos, ratio, q_per_seq, N, scores, tile_max, header, gmax, partial);
}

}  // namespace csa2
