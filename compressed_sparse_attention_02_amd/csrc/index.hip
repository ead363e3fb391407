// Indexer scan (csa2_index): I(t,s) = sum_h w[t][h] * ReLU(q[t][h] . K[b][s]).
//
// Lightning-indexer score of DeepSeek-V4 (gzher.com reading, sec. 4.1), kept by
// CSA2 (DeepSeek-V4.1-Flash report, sec. 2.3) with 32 heads x 128 (sec. 4.2.1).
//
// Per sequence the scan is a [32 heads x 128] x [128 x N] product, far below
// the MFMA ridge (32 flop per key byte), so the kernel is built around the key
// stream: each wave pulls four 16-key tiles (16 KiB) per iteration into the B
// operands of v_mfma_f32_16x16x32_bf16 (idx_tile.h), with the query in LDS.
// Blocks take 256-key chunks round-robin, so at any moment the whole grid
// sweeps one window of each sequence.  Per tile the scan forms the maximum
// score, and per (block, wave, tile slot, iteration mod S) group the maximum
// of those; that is all the selection needs (csa2_topk re-derives the few
// candidate tiles' scores).  The full score matrix is written only when the
// caller asks for it: interleaving 4 bytes of writes per 256 bytes of key
// reads costs about 7 % of the scan's bandwidth.  The same pass accumulates
// ||K_s||^2 so that a rigorous per-query bound on |fp32 - fp64 score| can be
// formed without a second read of the keys.  A second kernel forms, per
// query, that bound and a floor below the k-th largest score.
#include "idx_tile.h"

namespace csa2 {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanTiles = 4;      // tiles per wave per iteration: 64 keys, 16 KiB
constexpr int kScanWaveKeys = kTileKeys * kScanTiles;
constexpr int kChunkKeys = kScanWaveKeys * kScanWaves;  // 256 keys per block iteration
constexpr int kScanBlocks = 2048;  // blocks per launch the grid aims for (8 per CU)
constexpr int kGroupsWanted = 4096;

// One block: sequence b = blockIdx.y, query group blockIdx.z (QG queries of
// that sequence), chunks x, x + gridDim.x, x + 2 gridDim.x, ... of 256 keys;
// wave w takes keys 64w .. 64w+63 of each chunk.  Group maxima: group
// ((x * 4 + w) * 4 + u) * S + (i % S) holds the maxima of tile u of wave w in
// the block's iterations i, so a group samples the whole row and neighbouring
// tiles never share a group.
template <int QG, int S>
__global__ __launch_bounds__(kScanThreads, QG == 1 ? 4 : 2) void idx_scan_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos, int ratio,
    int q_per_seq, int64_t N, float* __restrict__ scores, float* __restrict__ tile_max,
    float* __restrict__ group_max, float* __restrict__ norm_partial) {
  __shared__ __attribute__((aligned(16))) uint16_t sq[QG * kIdxHeads * kQRowPad];
  __shared__ float red[kScanWaves];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;  // key within a tile
  const int g = lane >> 4;    // channel group
  const int b = blockIdx.y;
  const int64_t ld = tile_ld(N);
  const int64_t n_groups = (int64_t)gridDim.x * 16 * S;

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

  const int64_t nchunks = (N + kChunkKeys - 1) / kChunkKeys;
  const uint16_t* kseq = k_idx + (size_t)b * N * kIdxDim;
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
      if (s < N) maxn2 = fmaxf(maxn2, n2);
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
#pragma unroll
      for (int r = 0; r < S; ++r) gm[qq][r] = (it % S == r) ? fmaxf(gm[qq][r], m) : gm[qq][r];
      if (!valid[qq]) continue;
      if (scores != nullptr && so < N) scores[trow[qq] * N + so] = v;
      if (lane < kScanTiles && tile * kTileKeys < N) tile_max[trow[qq] * ld + tile] = m;
    }
  }
  if (lane < kScanTiles) {
#pragma unroll
    for (int qq = 0; qq < QG; ++qq) {
      if (!valid[qq]) continue;
#pragma unroll
      for (int r = 0; r < S; ++r)
        group_max[trow[qq] * n_groups + (((int64_t)blockIdx.x * kScanWaves + wave) * kScanTiles + lane) * S + r] =
            gm[qq][r];
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
constexpr int kFinThreads = 512;
constexpr int kFloorVals = 16384;            // maxima a finalize block ranks
constexpr int kFloorPer = kFloorVals / kFinThreads;  // 32 per thread, in registers

// LDS of the finalize block.
struct alignas(16) FinalLds {
  uint32_t hist[256];
  uint32_t bmin[256];   // order-preserving keys
  float fred[4][kFinThreads / 64];
  double dred[2][kFinThreads / 64];
  uint32_t ured[2][kFinThreads / 64];
  uint32_t res;
};

// Per query (grid T, 512 threads): the error bound eps and the selection
// floor tau, written to stats[t] = {eps, tau, 0, 0} (the last two words are
// csa2_topk's counters).  tau: at least CSA2_TOPK visible fp32 scores are >=
// tau, because it bounds from below the CSA2_TOPK-th largest of a set of
// maxima of disjoint groups of entries (each maximum is a distinct visible
// entry); -inf when the row has fewer than CSA2_TOPK non-empty tiles.  The
// maxima ranked are the tile maxima when the row has at most 16384 tiles,
// else the scan's group maxima (when there are at least 4096 of them) or the
// tile maxima folded to 16384 groups of tiles j, j + 16384, ...; folding
// unions groups, which keeps them disjoint.
//
// Ranking: each thread holds 32 of the maxima; the smallest per-thread
// maximum L0 is already a valid lower bound when at least CSA2_TOPK threads
// hold one (that many distinct maxima reach it), so only values >= L0 enter a
// histogram of 256 bins over [L0, max] that also keeps each bin's minimum.
// The bins at and above the one holding the CSA2_TOPK-th largest hold at
// least CSA2_TOPK values, and tau is the smallest of them.
__global__ __launch_bounds__(kFinThreads) void idx_finalize_kernel(
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, const float* __restrict__ norm_partial,
    const float* __restrict__ tile_max, const float* __restrict__ group_max, const int32_t* __restrict__ q_pos,
    int ratio, int q_per_seq, int64_t N, int parts_per_seq, int64_t n_groups, uint32_t* __restrict__ stats) {
  __shared__ FinalLds L;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = t / q_per_seq;
  for (int i = tid; i < 256; i += kFinThreads) { L.hist[i] = 0u; L.bmin[i] = 0xFFFFFFFFu; }

  // ---- floor: gather the maxima into registers (folded into at most 16384 values)
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t ntv = (nv + kTileKeys - 1) / kTileKeys;
  const bool use_groups = ntv > kFloorVals && n_groups >= kGroupsWanted;
  const float* src = use_groups ? group_max + (size_t)t * n_groups : tile_max + (size_t)t * tile_ld(N);
  const int64_t nsrc = nv > kTopK ? (use_groups ? n_groups : ntv) : 0;
  // value j = src[j] (rows are 16-byte aligned: four per load); past 16384,
  // fold: value j is the maximum over j, j + 16384, ...
  float v[kFloorPer];
#pragma unroll
  for (int m = 0; m < kFloorPer / 4; ++m) {
    const int64_t j = 4 * ((int64_t)m * kFinThreads + tid);
    const float4 x = j < nsrc ? *reinterpret_cast<const float4*>(src + j)
                              : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    v[4 * m] = x.x;
    v[4 * m + 1] = j + 1 < nsrc ? x.y : -INFINITY;
    v[4 * m + 2] = j + 2 < nsrc ? x.z : -INFINITY;
    v[4 * m + 3] = j + 3 < nsrc ? x.w : -INFINITY;
  }
  if (nsrc > kFloorVals) {
#pragma unroll
    for (int m = 0; m < kFloorPer; ++m) {
      const int64_t j = 4 * ((int64_t)(m / 4) * kFinThreads + tid) + (m % 4);
      for (int64_t i = j + kFloorVals; i < nsrc; i += kFloorVals) v[m] = fmaxf(v[m], src[i]);
    }
  }
  float lmax = -INFINITY, lmin = INFINITY;
  uint32_t finite = 0;
#pragma unroll
  for (int m = 0; m < kFloorPer; ++m) {
    if (v[m] > -INFINITY) { lmax = fmaxf(lmax, v[m]); lmin = fminf(lmin, v[m]); ++finite; }
  }

  // ---- eps: max ||K||^2 over the sequence's scan blocks, sum_h |w_h| ||q_h||
  float m2 = 0.f;
  for (int i = tid; i < parts_per_seq; i += kFinThreads) m2 = fmaxf(m2, norm_partial[(size_t)b * parts_per_seq + i]);
  double qf = 0.0, sw = 0.0;
  if (tid < 256) {
    // head h = tid / 8 sums channels 16 * (tid % 8) .. +16 of q_h
    const int h = tid >> 3;
    const uint4* qv =
        reinterpret_cast<const uint4*>(q_idx + ((size_t)t * kIdxHeads + h) * kIdxDim + 16 * (tid & 7));
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
    qf = (tid & 7) == 0 ? aw * sqrt(ss) * (1.0 + 0x1p-40) : 0.0;
    sw = (tid & 7) == 0 ? aw : 0.0;
  }

  // ---- one block reduction for both: max ||K||^2, sums, value range, L0, counts
  m2 = wave_max(m2);
  qf = wave_sum_f64(qf);
  sw = wave_sum_f64(sw);
  const float wmax = wave_max(lmax);
  const float wmin = -wave_max(-lmin);
  const float wl0 = -wave_max(lmax > -INFINITY ? -lmax : -INFINITY);  // smallest per-thread maximum
  uint32_t nfin = finite, nthr = finite ? 1u : 0u;
  for (int o = 32; o >= 1; o >>= 1) {
    nfin += __shfl_xor((int)nfin, o, 64);
    nthr += __shfl_xor((int)nthr, o, 64);
  }
  if (lane == 0) {
    L.fred[0][wave] = m2; L.fred[1][wave] = wmax; L.fred[2][wave] = wmin; L.fred[3][wave] = wl0;
    L.dred[0][wave] = qf; L.dred[1][wave] = sw;
    L.ured[0][wave] = nfin; L.ured[1][wave] = nthr;
  }
  __syncthreads();
  m2 = L.fred[0][0]; float mx = L.fred[1][0], gmin = L.fred[2][0], l0 = L.fred[3][0];
  qf = L.dred[0][0]; sw = L.dred[1][0]; nfin = L.ured[0][0]; nthr = L.ured[1][0];
  for (int i = 1; i < kFinThreads / 64; ++i) {
    m2 = fmaxf(m2, L.fred[0][i]); mx = fmaxf(mx, L.fred[1][i]); gmin = fminf(gmin, L.fred[2][i]);
    l0 = fminf(l0, L.fred[3][i]);
    qf += L.dred[0][i]; sw += L.dred[1][i]; nfin += L.ured[0][i]; nthr += L.ured[1][i];
  }
  float tau = -INFINITY;
  if (nfin >= (uint32_t)kTopK) {
    const float lo = nthr >= (uint32_t)kTopK ? l0 : gmin;
    const float scale = mx > lo ? 255.99f / (mx - lo) : 0.f;
#pragma unroll
    for (int m = 0; m < kFloorPer; ++m) {
      if (v[m] >= lo) {
        const uint32_t bin = value_bin(v[m], lo, scale);
        atomicAdd(&L.hist[bin], 1u);
        atomicMin(&L.bmin[bin], f32_key(v[m]));
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns bins 255-4*lane .. 252-4*lane (descending); the bins at or
      // above the one holding the rank-th largest are those whose exclusive
      // count from the top is below rank
      const uint32_t rank = (uint32_t)kTopK;
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c[i] = L.hist[255 - 4 * lane - i]; sum += c[i]; }
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
      }
      uint32_t cum = incl - sum, kmin = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum < rank) kmin = min(kmin, L.bmin[255 - 4 * lane - i]);
        cum += c[i];
      }
#pragma unroll
      for (int o = 32; o >= 1; o >>= 1) kmin = min(kmin, (uint32_t)__shfl_xor((int)kmin, o, 64));
      if (lane == 0) L.res = kmin;
    }
    __syncthreads();
    tau = key_f32(L.res);
  }
  if (tid == 0) {
    const double kmax = sqrt((double)m2 * (1.0 + 0x1p-10) + 0x1p-100) * (1.0 + 0x1p-40);
    const double eps = (0x1p-14 * qf * kmax + 0x1p-100 * (1.0 + sw)) * (1.0 + 0x1p-20);
    float e = (float)eps;
    if ((double)e < eps) e = __int_as_float(__float_as_int(e) + 1);  // round up (positive, finite)
    uint32_t* st = stats + (size_t)t * CSA2_STATS_WORDS;
    st[0] = __float_as_uint(e);
    st[1] = __float_as_uint(tau);
    st[2] = 0u;
    st[3] = 0u;
  }
}

struct IndexPlan {
  int qg = 1;             // queries per group (template)
  int groups = 1;         // gridDim.z
  int B = 1;              // gridDim.y
  int blocks_x = 1;       // gridDim.x
  int slots = 1;          // S: group slots per (block, wave, tile)
  int64_t n_groups = 16;  // group maxima per query
};

static bool index_plan(int32_t T, int32_t q_per_seq, int64_t N, IndexPlan* p) {
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || N >= ((int64_t)1 << 31)) return false;
  p->qg = q_per_seq == 1 ? 1 : q_per_seq == 2 ? 2 : 4;
  p->groups = (q_per_seq + p->qg - 1) / p->qg;
  p->B = T / q_per_seq;
  // aim for ~2048 blocks over 256 CUs, each with at least one chunk
  const int64_t nchunks = (N + kChunkKeys - 1) / kChunkKeys;
  int64_t want = (kScanBlocks + (int64_t)p->B * p->groups - 1) / ((int64_t)p->B * p->groups);
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  p->blocks_x = (int)want;
  // enough group slots for ~4096 groups, within the registers of the query count
  const int max_slots = p->qg == 1 ? 4 : p->qg == 2 ? 2 : 1;
  int slots = 1;
  while (slots < max_slots && (int64_t)p->blocks_x * 16 * slots < kGroupsWanted) slots *= 2;
  p->slots = slots;
  p->n_groups = (int64_t)p->blocks_x * 16 * slots;
  return p->B <= 65535 && p->groups <= 65535;
}

}  // namespace csa2

using namespace csa2;

static size_t index_ws_partials(const IndexPlan& p) {
  return align_up((size_t)p.B * p.groups * p.blocks_x * sizeof(float), 256);
}

extern "C" size_t csa2_index_workspace_bytes(int32_t T, int32_t q_per_seq, int64_t N) {
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return 0;
  return index_ws_partials(p) + align_up((size_t)T * p.n_groups * sizeof(float), 256);
}

extern "C" int64_t csa2_tile_max_ld(int64_t N) { return N < 1 ? 0 : tile_ld(N); }

template <int QG>
static void launch_scan(const IndexPlan& p, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                        const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                        float* gmax, float* partial) {
  const dim3 grid(p.blocks_x, p.B, p.groups);
  if (p.slots == 1)
    hipLaunchKernelGGL((idx_scan_kernel<QG, 1>), grid, dim3(kScanThreads), 0, st, q, w, k, q_pos, ratio, q_per_seq, N,
                       scores, tile_max, gmax, partial);
  else if (p.slots == 2)
    hipLaunchKernelGGL((idx_scan_kernel<QG, 2>), grid, dim3(kScanThreads), 0, st, q, w, k, q_pos, ratio, q_per_seq, N,
                       scores, tile_max, gmax, partial);
  else
    hipLaunchKernelGGL((idx_scan_kernel<QG, 4>), grid, dim3(kScanThreads), 0, st, q, w, k, q_pos, ratio, q_per_seq, N,
                       scores, tile_max, gmax, partial);
}

extern "C" csa2_status csa2_index(const void* q_idx, const float* w_idx, const void* k_idx,
                                  const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq,
                                  int64_t N, float* scores, float* tile_max, uint32_t* stats, void* workspace,
                                  size_t workspace_bytes, void* hip_stream) {
  if (!q_idx || !w_idx || !k_idx || !tile_max || !stats) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) || (scores && !aligned16(scores)) ||
      !aligned16(tile_max) || !aligned16(stats) || (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || N < 1 || ratio < 1 || T % q_per_seq != 0) return CSA2_ERR_INVALID_ARG;
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  const size_t need = csa2_index_workspace_bytes(T, q_per_seq, N);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  float* partial = (float*)workspace;
  float* gmax = (float*)((char*)workspace + index_ws_partials(p));
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* k = (const uint16_t*)k_idx;
  if (p.qg == 1)
    launch_scan<1>(p, st, q, w_idx, k, q_pos, ratio, q_per_seq, N, scores, tile_max, gmax, partial);
  else if (p.qg == 2)
    launch_scan<2>(p, st, q, w_idx, k, q_pos, ratio, q_per_seq, N, scores, tile_max, gmax, partial);
  else
    launch_scan<4>(p, st, q, w_idx, k, q_pos, ratio, q_per_seq, N, scores, tile_max, gmax, partial);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  hipLaunchKernelGGL(idx_finalize_kernel, dim3(T), dim3(kFinThreads), 0, st, q, w_idx, (const float*)partial,
                     (const float*)tile_max, (const float*)gmax, q_pos, ratio, q_per_seq, N,
                     p.groups * p.blocks_x, p.n_groups, stats);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
