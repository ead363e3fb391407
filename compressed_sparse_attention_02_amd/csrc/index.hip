// Indexer scan (csa2_index): I(t,s) = sum_h w[t][h] * ReLU(q[t][h] . K[b][s]).
//
// Lightning-indexer score of DeepSeek-V4 (gzher.com reading, sec. 4.1), kept by
// CSA2 (DeepSeek-V4.1-Flash report, sec. 2.3) with 32 heads x 128 (sec. 4.2.1).
//
// Per sequence the scan is a [32 heads x 128] x [128 x N] product, far below
// the MFMA ridge (32 flop per key byte), so the kernel is built around the key
// stream: each wave pulls four 16-key tiles (16 KiB) per iteration into the B
// operands of v_mfma_f32_16x16x32_bf16 (idx_tile.h), with the query in LDS.
// Per tile it also forms the maximum score, which is all the selection needs
// from the scan (csa2_topk re-derives the few candidate tiles' scores); the
// full score matrix is written only when the caller asks for it, because
// interleaving 4 bytes of writes per 256 bytes of key reads costs about 7 %
// of the scan's bandwidth.  The same pass accumulates ||K_s||^2 so that a
// rigorous per-query bound on |fp32 score - fp64 score| can be formed without
// a second read of the keys.
#include "idx_tile.h"

namespace csa2 {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanTiles = 4;      // tiles per wave per iteration: 64 keys, 16 KiB
constexpr int kScanWaveKeys = kTileKeys * kScanTiles;
constexpr int kScanBlocks = 2048;  // blocks per launch the grid aims for (8 per CU)

// One block: sequence b = blockIdx.y, query group blockIdx.z (QG queries of
// that sequence), keys [x*kpb, (x+1)*kpb).  Each wave takes 64 consecutive
// keys per iteration; the block's waves cover 256 consecutive keys.
template <int QG>
__global__ __launch_bounds__(kScanThreads, QG == 1 ? 4 : 2) void idx_scan_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int ratio,
    int q_per_seq, int64_t N, int keys_per_block, float* __restrict__ scores,
    float* __restrict__ tile_max, float* __restrict__ norm_partial) {
  __shared__ __attribute__((aligned(16))) uint16_t sq[QG * kIdxHeads * kQRowPad];
  __shared__ float red[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // key within a tile
  const int g = lane >> 4;    // channel group
  const int b = blockIdx.y;
  const int64_t ld = tile_ld(N);

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
  }
  __syncthreads();

  const int64_t key0 = (int64_t)blockIdx.x * keys_per_block;
  const int64_t key1 = key0 + keys_per_block < N ? key0 + keys_per_block : N;
  const uint16_t* kseq = k_idx + (size_t)b * N * kIdxDim;
  const int64_t last = (nvis_max < N ? (nvis_max > 0 ? nvis_max : 1) : N) - 1;  // last row worth reading
  float maxn2 = 0.f;

  for (int64_t base = key0 + kScanWaveKeys * wave; base < key1; base += kScanWaveKeys * kScanWaves) {
    // Unconditional loads keep the code branch-free: keys past the end or past
    // every query's visibility re-read row `last`, which is already cached.
    uint4 kv[kScanTiles][4];
#pragma unroll
    for (int u = 0; u < kScanTiles; ++u) {
      const int64_t s = base + u * kTileKeys + col;
      load_key_slices(kseq, s < last ? s : last, g, kv[u]);
    }
    float sc[QG][kScanTiles];
#pragma unroll
    for (int u = 0; u < kScanTiles; ++u) {
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) sc[qq][u] = -INFINITY;
      const int64_t s = base + u * kTileKeys + col;
      if (base + u * kTileKeys >= nvis_max) continue;  // no query of the group sees this tile
      // ||K_s||^2: 32 channels per lane with bf16 dot2, then the other three groups
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
      n2 += __shfl_xor(n2, 16, 64);
      n2 += __shfl_xor(n2, 32, 64);
      if (s < key1) maxn2 = fmaxf(maxn2, n2);
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) {
        if (!valid[qq]) continue;
        const float part = tile_score(&sq[qq * kIdxHeads * kQRowPad], kv[u], wr[qq], col, g);
        sc[qq][u] = (s < nvis[qq]) ? part : -INFINITY;
      }
    }
    // Every lane holds the score of key `col` of each tile.  Lane l stores
    // key l of the 64 (one 256-byte store) and lanes 0..3 the tile maxima.
    const int64_t so = base + lane;
    const int64_t tile = base / kTileKeys + lane;
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      float v = sc[qq][0], m = -INFINITY;
#pragma unroll
      for (int u = 0; u < kScanTiles; ++u) {
        float tm = sc[qq][u];
        tm = fmaxf(tm, __shfl_xor(tm, 1, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 2, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 4, 64));
        tm = fmaxf(tm, __shfl_xor(tm, 8, 64));
        if (u > 0) v = g == u ? sc[qq][u] : v;
        m = lane == u ? tm : m;
      }
      if (!valid[qq]) continue;
      if (scores != nullptr && so < key1) scores[trow[qq] * N + so] = v;
      if (lane < kScanTiles && tile * kTileKeys < key1) tile_max[trow[qq] * ld + tile] = m;
    }
  }

  maxn2 = wave_max(maxn2);
  if (lane == 0) red[wave] = maxn2;
  __syncthreads();
  if (threadIdx.x == 0) {
    float m = red[0];
#pragma unroll
    for (int i = 1; i < kScanWaves; ++i) m = fmaxf(m, red[i]);
    norm_partial[((size_t)b * gridDim.z + blockIdx.z) * gridDim.x + blockIdx.x] = m;
  }
}

// eps_t = 2^-14 * sum_h |w_h| ||q_h||_2 * max_s ||K_s||_2 + 2^-100 (1 + sum_h |w_h|), rounded up.
//
// Derivation: the bf16 products are exact in fp32; four chained MFMA steps
// of 32 products each (at most 132 additions on any path), even with every
// addition rounded or truncated, stay within 136 * 2^-23 * sum_c |q_c K_c|
// <= 2^-15.9 ||q_h|| ||K_s|| (Cauchy-Schwarz); ReLU is 1-Lipschitz; the fp32
// head reduction (10 roundings on any path, fewer than 17) adds at most
// 2^-19.9 sum_h |w_h| |dot_h|; the fp64 reference itself is within 2^-44 of
// the exact value.  The sum is below 1.1 * 2^-15; 2^-14 leaves a factor 1.8
// of margin.  The absolute term covers products that flush to zero.
// ||K||^2 is accumulated with bf16 dot2 steps in fp32 over nonnegative terms
// (relative error below 2^-16 even with two roundings per step), so it is
// inflated by (1 + 2^-10) before the square root.  ||q_h||^2 is summed in
// fp64 (relative error below 2^-45 in any order), covered by (1 + 2^-40).
constexpr int kFinThreads = 256;
__global__ __launch_bounds__(kFinThreads) void idx_finalize_kernel(const uint16_t* __restrict__ q_idx,
                                                                  const float* __restrict__ w_idx,
                                                                  const float* __restrict__ norm_partial,
                                                                  int q_per_seq, int parts_per_seq,
                                                                  float* __restrict__ err_bound) {
  __shared__ float smax[kFinThreads / 64];
  __shared__ double sqf[kFinThreads / 64], ssw[kFinThreads / 64];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = t / q_per_seq;
  float m = 0.f;
  for (int i = tid; i < parts_per_seq; i += kFinThreads) m = fmaxf(m, norm_partial[(size_t)b * parts_per_seq + i]);
  // head h = tid / 8 sums channels 16 * (tid % 8) .. +16 of q_h
  const int h = tid >> 3;
  const uint4* qv = reinterpret_cast<const uint4*>(q_idx + ((size_t)t * kIdxHeads + h) * kIdxDim + 16 * (tid & 7));
  const uint4 a = qv[0], c = qv[1];
  const uint32_t wd[8] = {a.x, a.y, a.z, a.w, c.x, c.y, c.z, c.w};
  double ss = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const double lo = (double)bf16lo(wd[i]), hi = (double)bf16hi(wd[i]);
    ss = fma(lo, lo, ss);
    ss = fma(hi, hi, ss);
  }
  ss += __shfl_xor(ss, 1, 64);
  ss += __shfl_xor(ss, 2, 64);
  ss += __shfl_xor(ss, 4, 64);
  const double aw = fabs((double)w_idx[(size_t)t * kIdxHeads + h]);
  double qf = (tid & 7) == 0 ? aw * sqrt(ss) * (1.0 + 0x1p-40) : 0.0;
  double sw = (tid & 7) == 0 ? aw : 0.0;
  m = wave_max(m);
  qf = wave_sum_f64(qf);
  sw = wave_sum_f64(sw);
  if (lane == 0) { smax[wave] = m; sqf[wave] = qf; ssw[wave] = sw; }
  __syncthreads();
  if (tid == 0) {
    m = smax[0]; qf = sqf[0]; sw = ssw[0];
#pragma unroll
    for (int i = 1; i < kFinThreads / 64; ++i) { m = fmaxf(m, smax[i]); qf += sqf[i]; sw += ssw[i]; }
    const double kmax = sqrt((double)m * (1.0 + 0x1p-10) + 0x1p-100) * (1.0 + 0x1p-40);
    const double eps = (0x1p-14 * qf * kmax + 0x1p-100 * (1.0 + sw)) * (1.0 + 0x1p-20);
    float e = (float)eps;
    if ((double)e < eps) e = __int_as_float(__float_as_int(e) + 1);  // round up (positive, finite)
    err_bound[t] = e;
  }
}

struct IndexPlan {
  int qg = 1;             // queries per group (template)
  int groups = 1;         // gridDim.z
  int B = 1;              // gridDim.y
  int blocks_x = 1;       // gridDim.x
  int keys_per_block = kScanWaveKeys * kScanWaves;
};

static bool index_plan(int32_t T, int32_t q_per_seq, int64_t N, IndexPlan* p) {
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || N >= ((int64_t)1 << 31)) return false;
  p->qg = q_per_seq == 1 ? 1 : q_per_seq == 2 ? 2 : 4;
  p->groups = (q_per_seq + p->qg - 1) / p->qg;
  p->B = T / q_per_seq;
  // aim for ~2048 blocks over 256 CUs; each block a multiple of one iteration of its waves
  const int64_t per_iter = (int64_t)kScanWaveKeys * kScanWaves;
  int64_t want = (kScanBlocks + (int64_t)p->B * p->groups - 1) / ((int64_t)p->B * p->groups);
  const int64_t max_blocks = (N + per_iter - 1) / per_iter;
  if (want > max_blocks) want = max_blocks;
  if (want < 1) want = 1;
  int64_t kpb = (N + want - 1) / want;
  kpb = (kpb + per_iter - 1) / per_iter * per_iter;
  p->keys_per_block = (int)kpb;
  p->blocks_x = (int)((N + kpb - 1) / kpb);
  return p->B <= 65535 && p->groups <= 65535;
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_index_workspace_bytes(int32_t T, int32_t q_per_seq, int64_t N) {
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return 0;
  return align_up((size_t)p.B * p.groups * p.blocks_x * sizeof(float), 256);
}

extern "C" int64_t csa2_tile_max_ld(int64_t N) { return N < 1 ? 0 : tile_ld(N); }

extern "C" csa2_status csa2_index(const void* q_idx, const float* w_idx, const void* k_idx,
                                  const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq,
                                  int64_t N, float* scores, float* tile_max, float* err_bound, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  if (!q_idx || !w_idx || !k_idx || !tile_max || !err_bound) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) || (scores && !aligned16(scores)) ||
      !aligned16(tile_max) || !aligned16(err_bound) || (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || N < 1 || ratio < 1 || T % q_per_seq != 0) return CSA2_ERR_INVALID_ARG;
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_index_workspace_bytes(T, q_per_seq, N);
  if (!workspace || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  float* partial = (float*)workspace;
  dim3 grid(p.blocks_x, p.B, p.groups);
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* k = (const uint16_t*)k_idx;
  if (p.qg == 1)
    hipLaunchKernelGGL(idx_scan_kernel<1>, grid, dim3(kScanThreads), 0, st, q, w_idx, k, q_pos, ratio, q_per_seq, N,
                       p.keys_per_block, scores, tile_max, partial);
  else if (p.qg == 2)
    hipLaunchKernelGGL(idx_scan_kernel<2>, grid, dim3(kScanThreads), 0, st, q, w_idx, k, q_pos, ratio, q_per_seq, N,
                       p.keys_per_block, scores, tile_max, partial);
  else
    hipLaunchKernelGGL(idx_scan_kernel<4>, grid, dim3(kScanThreads), 0, st, q, w_idx, k, q_pos, ratio, q_per_seq, N,
                       p.keys_per_block, scores, tile_max, partial);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  hipLaunchKernelGGL(idx_finalize_kernel, dim3(T), dim3(kFinThreads), 0, st, q, w_idx, (const float*)partial,
                     q_per_seq, p.groups * p.blocks_x, err_bound);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
