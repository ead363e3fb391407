// Indexer scan (csa2_index): I(t,s) = sum_h w[t][h] * ReLU(q[t][h] . K[b][s]).
//
// Lightning-indexer score of DeepSeek-V4 (gzher.com reading, sec. 4.1), kept by
// CSA2 (DeepSeek-V4.1-Flash report, sec. 2.3) with 32 heads x 128 (sec. 4.2.1).
//
// Per sequence the scan is a [32 heads x 128] x [128 x N] product, far below
// the MFMA ridge (32 flop per key byte), so the kernel is built around the key
// stream.  Keys are the B operand of v_mfma_f32_16x16x32_bf16: a 16-key tile
// per MFMA, lane l holding key l%16 and channels 32j + 8(l/16) .. +8 at step
// j, i.e. 64 contiguous bytes of one row per lane and load instruction.  The
// query (two 16-head halves, the A operands) sits in LDS.  ReLU(dot) * w is
// reduced over the heads in the accumulator's layout (8 heads per lane plus
// two cross-lane adds), and the scores of a wave's four tiles leave as one
// fully coalesced 256-byte store.  The same pass accumulates ||K_s||^2 so that
// a rigorous per-query bound on |fp32 score - fp64 score| can be formed
// without a second read of the keys.
#include "csa2_common.h"

namespace csa2 {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanTileKeys = 16;  // keys per MFMA tile
constexpr int kScanTiles = 4;      // tiles per wave per iteration: 64 keys, 16 KiB
constexpr int kScanWaveKeys = kScanTileKeys * kScanTiles;
constexpr int kQRowPad = kIdxDim + 8;  // bf16 per q row in LDS (272 B: spreads rows over banks)
constexpr int kScanBlocks = 2048;      // blocks per launch the grid aims for (8 per CU)

// One block: sequence b = blockIdx.y, query group blockIdx.z (QG queries of
// that sequence), keys [x*kpb, (x+1)*kpb).  Each wave takes 64 consecutive
// keys per iteration; the block's waves cover 256 consecutive keys.
// Accumulator register i of half m holds head 16m + 4(l/16) + i of key l%16.
template <int QG>
__global__ __launch_bounds__(kScanThreads, QG == 1 ? 4 : 2) void idx_scan_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int ratio,
    int q_per_seq, int64_t N, int keys_per_block, float* __restrict__ scores,
    float* __restrict__ norm_partial) {
  __shared__ __attribute__((aligned(16))) uint16_t sq[QG * kIdxHeads * kQRowPad];
  __shared__ float red[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // key within a tile
  const int g = lane >> 4;    // channel group: 32j + 8g .. +8
  const int b = blockIdx.y;

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
    trow[qq] = (int64_t)t * N;
    // stage q[t] (32 x 128 bf16) into LDS: 512 chunks of 16 B over 256 threads
    for (int i = threadIdx.x; i < kIdxHeads * kIdxDim / 8; i += kScanThreads) {
      const int h = i >> 4, c8 = i & 15;
      *reinterpret_cast<uint4*>(&sq[(qq * kIdxHeads + h) * kQRowPad + c8 * 8]) =
          *reinterpret_cast<const uint4*>(q_idx + ((size_t)t * kIdxHeads + h) * kIdxDim + c8 * 8);
    }
#pragma unroll
    for (int r = 0; r < 8; ++r) wr[qq][r] = w_idx[(size_t)t * kIdxHeads + 16 * (r >> 2) + 4 * g + (r & 3)];
    nvis[qq] = valid[qq] ? n_visible(q_pos, t, ratio, N) : 0;
    nvis_max = nvis[qq] > nvis_max ? nvis[qq] : nvis_max;
  }
  __syncthreads();

  const int64_t key0 = (int64_t)blockIdx.x * keys_per_block;
  const int64_t key1 = key0 + keys_per_block < N ? key0 + keys_per_block : N;
  const uint16_t* kseq = k_idx + (size_t)b * N * kIdxDim + g * 8;
  const int64_t last = (nvis_max < N ? (nvis_max > 0 ? nvis_max : 1) : N) - 1;  // last row worth reading
  float maxn2 = 0.f;

  for (int64_t base = key0 + kScanWaveKeys * wave; base < key1; base += kScanWaveKeys * kScanWaves) {
    // Unconditional loads keep the code branch-free: keys past the end or past
    // every query's visibility re-read row `last`, which is already cached.
    uint4 kv[kScanTiles][4];
#pragma unroll
    for (int u = 0; u < kScanTiles; ++u) {
      const int64_t s = base + u * kScanTileKeys + col;
      const uint16_t* kp = kseq + (size_t)(s < last ? s : last) * kIdxDim;
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[u][j] = *reinterpret_cast<const uint4*>(kp + 32 * j);
    }
    float sc[QG][kScanTiles];
#pragma unroll
    for (int u = 0; u < kScanTiles; ++u) {
#pragma unroll
      for (int qq = 0; qq < QG; ++qq) sc[qq][u] = -INFINITY;
      const int64_t s = base + u * kScanTileKeys + col;
      if (base + u * kScanTileKeys >= nvis_max) continue;  // no query of the group sees this tile
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
        floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* q0 = &sq[(qq * kIdxHeads + col) * kQRowPad + 8 * g];
        const uint16_t* q1 = q0 + 16 * kQRowPad;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const bf16x8 bk = as_bf16x8(kv[u][j]);
          acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(q0 + 32 * j), bk, acc0, 0, 0, 0);
          acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*reinterpret_cast<const bf16x8*>(q1 + 32 * j), bk, acc1, 0, 0, 0);
        }
        float part = 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          part = fmaf(wr[qq][r], fmaxf(acc0[r], 0.f), part);
          part = fmaf(wr[qq][4 + r], fmaxf(acc1[r], 0.f), part);
        }
        part += __shfl_xor(part, 16, 64);
        part += __shfl_xor(part, 32, 64);
        sc[qq][u] = (s < nvis[qq]) ? part : -INFINITY;
      }
    }
    // every lane holds the score of key `col` of each tile; lane l stores key l of the 64
    const int64_t so = base + lane;
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      float v = sc[qq][0];
#pragma unroll
      for (int u = 1; u < kScanTiles; ++u) v = g == u ? sc[qq][u] : v;
      if (valid[qq] && so < key1) scores[trow[qq] + so] = v;
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
// <= 2^-15.9 ||q_h|| ||K_s|| (Cauchy-Schwarz); ReLU is 1-Lipschitz; the fp32 head reduction (17 roundings) adds at
// most 2^-19.9 sum_h |w_h| |dot_h|; the fp64 reference itself is within
// 2^-44 of the exact value.  The sum is below 1.1 * 2^-15; 2^-14 leaves a
// factor 1.8 of margin.  The absolute term covers products that flush to zero.
// ||K||^2 is accumulated with bf16 dot2 steps in fp32 over nonnegative terms
// (relative error below 2^-16 even with two roundings per step), so it is
// inflated by (1 + 2^-10) before the square root.
__global__ __launch_bounds__(64) void idx_finalize_kernel(const uint16_t* __restrict__ q_idx,
                                                          const float* __restrict__ w_idx,
                                                          const float* __restrict__ norm_partial,
                                                          int q_per_seq, int parts_per_seq,
                                                          float* __restrict__ err_bound) {
  const int t = blockIdx.x;
  const int lane = threadIdx.x;
  const int b = t / q_per_seq;
  float m = 0.f;
  for (int i = lane; i < parts_per_seq; i += 64) m = fmaxf(m, norm_partial[(size_t)b * parts_per_seq + i]);
  m = wave_max(m);
  double qf = 0.0, sw = 0.0;
  if (lane < kIdxHeads) {
    const uint16_t* qh = q_idx + ((size_t)t * kIdxHeads + lane) * kIdxDim;
    double ss = 0.0;
    for (int c = 0; c < kIdxDim; ++c) {
      const double v = bf16_to_f64(qh[c]);
      ss = fma(v, v, ss);
    }
    const double aw = fabs((double)w_idx[(size_t)t * kIdxHeads + lane]);
    qf = aw * sqrt(ss) * (1.0 + 0x1p-40);
    sw = aw;
  }
  qf = wave_sum_f64(qf);
  sw = wave_sum_f64(sw);
  if (lane == 0) {
    const double kmax = sqrt((double)m * (1.0 + 0x1p-10) + 0x1p-100) * (1.0 + 0x1p-40);
    double eps = (0x1p-14 * qf * kmax + 0x1p-100 * (1.0 + sw)) * (1.0 + 0x1p-20);
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

extern "C" csa2_status csa2_index(const void* q_idx, const float* w_idx, const void* k_idx,
                                  const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq,
                                  int64_t N, float* scores, float* err_bound, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  if (!q_idx || !w_idx || !k_idx || !scores || !err_bound) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) || !aligned16(scores) ||
      !aligned16(err_bound) || (q_pos && !aligned16(q_pos)))
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
                       p.keys_per_block, scores, partial);
  else if (p.qg == 2)
    hipLaunchKernelGGL(idx_scan_kernel<2>, grid, dim3(kScanThreads), 0, st, q, w_idx, k, q_pos, ratio, q_per_seq, N,
                       p.keys_per_block, scores, partial);
  else
    hipLaunchKernelGGL(idx_scan_kernel<4>, grid, dim3(kScanThreads), 0, st, q, w_idx, k, q_pos, ratio, q_per_seq, N,
                       p.keys_per_block, scores, partial);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  hipLaunchKernelGGL(idx_finalize_kernel, dim3(T), dim3(64), 0, st, q, w_idx, (const float*)partial, q_per_seq,
                     p.groups * p.blocks_x, err_bound);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
