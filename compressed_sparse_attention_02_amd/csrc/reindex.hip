// Reindex selection (csa2_reindex).
//
// A Reindex layer (report sec. 2.3.2) scores only the candidate pool the
// preceding Full layer left for its query, with its own indexer query over the
// shared indexer keys, and keeps its own top-k within the pool.  Each query's
// pool is scanned as a "sequence" of its own of P = CSA2_HSI_POOL positions:
// with bf16 keys the scan reads the key rows through the pool (index.hip,
// index_pool_launch); with MXFP4 keys the pool rows are first dequantised
// (exactly) into a contiguous bf16 block per query, which the regular scan then
// reads with the pool size as the visible count.  Padding positions score
// -inf either way.  The selection within each pool (reindex_select_kernel,
// topk.hip) writes the selected positions' entry ids.  The pool is ascending,
// so position order is entry order: the tie rule (lower index first) and the
// ascending output carry over unchanged, and the fp64 scores are those of the
// original rows (same bf16 values, same operation order).
#include "mxfp4.h"

namespace csa2 {

// The selection over the scanned pools (topk.hip); keys are the gathered rows
// (pool_qps == 0) or the shared keys read through the pool.
csa2_status reindex_select_launch(const float* scores, const uint32_t* stats, size_t stats_bytes,
                                  const void* q_bf16, const float* w_idx, const uint16_t* keys, int64_t N_all,
                                  int pool_qps, const int32_t* pool, int32_t T, int32_t k, int32_t* indices,
                                  hipStream_t st);
// The scan of each query's pool through the pool (index.hip).
csa2_status index_pool_launch(const void* q_idx, const float* w_idx, const void* k_all, int64_t N_all, int qps,
                              const int32_t* pool, int32_t T, int64_t P, float* scores, float* tile_max,
                              uint32_t* stats, size_t stats_bytes, hipStream_t st);

constexpr int kPool = CSA2_HSI_POOL;
constexpr int kGatherThreads = 256;
constexpr int kGatherRows = 64;                          // pool rows per block
constexpr int kRowVecs = kIdxDim * 2 / 16;               // 16-byte vectors per key row (16)

struct ReindexWs {
  uint16_t* keys;    // [T][kPool][128] gathered keys (bf16)
  uint16_t* q;       // [T][32][128] the Reindex queries in bf16 (MXFP4 variant)
  int32_t* qpos;     // [T]: pool size - 1
  float* scores;     // [T][kPool]
  float* tile_max;   // [T][tile_ld]
  uint32_t* stats;   // csa2_index summary for (T, 1, kPool)
  size_t stats_bytes;
};

static ReindexWs reindex_ws(void* base, int T, int k, size_t* total) {
  ReindexWs w;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const uintptr_t p = (uintptr_t)base + off;
    off += align_up(bytes, 256);
    return (void*)p;
  };
  w.keys = (uint16_t*)take((size_t)T * kPool * kIdxDim * 2);
  w.q = (uint16_t*)take((size_t)T * kIdxHeads * kIdxDim * 2);
  w.qpos = (int32_t*)take((size_t)T * 4);
  w.scores = (float*)take((size_t)T * kPool * 4);
  w.tile_max = (float*)take((size_t)T * (size_t)csa2_tile_max_ld(kPool) * 4);
  w.stats_bytes = csa2_index_stats_bytes(T, 1, kPool);
  w.stats = (uint32_t*)take(w.stats_bytes);
  *total = off;
  return w;
}

// Block (x, t): pool rows [x*64, x*64+64) of query t into keys[t] as bf16
// (MXFP4 rows dequantised, exactly); zeros for pad slots (-1).  Block (0, t)
// also writes qpos[t] = (number of pool entries) - 1, and block (1, t) the
// query dequantised to bf16 when MXFP4 query codes are given.
template <class Keys>
__global__ __launch_bounds__(kGatherThreads) void reindex_gather_kernel(const int32_t* __restrict__ pool, Keys k_all,
                                                                        int q_per_seq, int64_t N,
                                                                        uint16_t* __restrict__ keys,
                                                                        int32_t* __restrict__ qpos,
                                                                        const uint8_t* __restrict__ q_codes,
                                                                        const uint8_t* __restrict__ q_scales,
                                                                        uint16_t* __restrict__ q_out) {
  const int t = blockIdx.y;
  const int tid = threadIdx.x;
  const int32_t* pl = pool + (size_t)t * kPool;
  const Keys kseq = k_all.seq(t / q_per_seq, N);
  uint4* dst = reinterpret_cast<uint4*>(keys + ((size_t)t * kPool + (size_t)blockIdx.x * kGatherRows) * kIdxDim);
  const int r0 = blockIdx.x * kGatherRows;
#pragma unroll
  for (int u = 0; u < kGatherRows * kRowVecs / kGatherThreads; ++u) {
    const int i = u * kGatherThreads + tid;
    const int r = i / kRowVecs, c = i % kRowVecs;
    const int32_t e = pl[r0 + r];
    dst[i] = e >= 0 ? kseq.piece(e, c) : make_uint4(0u, 0u, 0u, 0u);
  }
  if (blockIdx.x == 1 && q_codes != nullptr) {
    // thread i: 8 code bytes (16 channels) of head i / 8
    const int h = tid >> 3, c16 = tid & 7;
    const uint8_t* qc = q_codes + ((size_t)t * kIdxHeads + h) * kMxRowBytes;
    const uint2 cw = *reinterpret_cast<const uint2*>(qc + 8 * c16);
    const uint32_t sb = q_scales[((size_t)t * kIdxHeads + h) * kMxScales + (c16 >> 1)];
    uint4* qd = reinterpret_cast<uint4*>(q_out + ((size_t)t * kIdxHeads + h) * kIdxDim + 16 * c16);
    qd[0] = dequant8(cw.x, sb);
    qd[1] = dequant8(cw.y, sb);
  }
  if (blockIdx.x == 0) {
    __shared__ uint32_t part[kGatherThreads / 64];
    // 64 entries per thread, as 16 loads of four issued together
    const int4* p4 = reinterpret_cast<const int4*>(pl);
    int4 v[kPool / 4 / kGatherThreads];
#pragma unroll
    for (int u = 0; u < kPool / 4 / kGatherThreads; ++u) v[u] = p4[u * kGatherThreads + tid];
    uint32_t n = 0;
#pragma unroll
    for (int u = 0; u < kPool / 4 / kGatherThreads; ++u)
      n += (v[u].x >= 0) + (v[u].y >= 0) + (v[u].z >= 0) + (v[u].w >= 0);
    n = wave_sum_u32_dpp(n);
    if ((tid & 63) == 0) part[tid >> 6] = n;
    __syncthreads();
    if (tid == 0) {
      uint32_t s = 0;
      for (int i = 0; i < kGatherThreads / 64; ++i) s += part[i];
      qpos[t] = (int32_t)s - 1;
    }
  }
}

}  // namespace csa2

using namespace csa2;

extern "C" size_t csa2_reindex_workspace_bytes(int32_t T, int32_t k) {
  if (T < 1 || T > 65535 || k != kTopK) return 0;
  size_t total;
  reindex_ws(nullptr, T, k, &total);
  return total;
}

extern "C" csa2_status csa2_reindex(const int32_t* pool, const void* q_idx, const float* w_idx, const void* k_idx,
                                    int32_t T, int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices,
                                    void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!pool || !q_idx || !w_idx || !k_idx || !indices) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(pool) || !aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) || !aligned16(indices))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1) return CSA2_ERR_INVALID_ARG;
  if (k != kTopK || N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  size_t need;
  ReindexWs w = reindex_ws(workspace, T, k, &need);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
  // the scan reads the key rows through the pool; the selection rescores its
  // band through the pool too
  const hipStream_t st = (hipStream_t)hip_stream;
  csa2_status s = index_pool_launch(q_idx, w_idx, k_idx, N, q_per_seq, pool, T, kPool, w.scores, w.tile_max, w.stats,
                                    w.stats_bytes, st);
  if (s != CSA2_OK) return s;
  return reindex_select_launch(w.scores, w.stats, w.stats_bytes, q_idx, w_idx, (const uint16_t*)k_idx, N, q_per_seq,
                               pool, T, k, indices, st);
}

extern "C" csa2_status csa2_reindex_mxfp4(const int32_t* pool, const uint8_t* q_codes, const uint8_t* q_scales,
                                          const float* w_idx, const uint8_t* k_codes, const uint8_t* k_scales,
                                          int32_t T, int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices,
                                          void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!pool || !q_codes || !q_scales || !w_idx || !k_codes || !k_scales || !indices) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(pool) || !aligned16(q_codes) || !aligned16(q_scales) || !aligned16(w_idx) || !aligned16(k_codes) ||
      !aligned16(k_scales) || !aligned16(indices))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1) return CSA2_ERR_INVALID_ARG;
  if (k != kTopK || N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  size_t need;
  ReindexWs w = reindex_ws(workspace, T, k, &need);
  if (!workspace || !aligned16(workspace) || workspace_bytes < need) return CSA2_ERR_WORKSPACE;
  (void)hipGetLastError();
  hipLaunchKernelGGL(reindex_gather_kernel<Mx4Keys>, dim3(kPool / kGatherRows, T), dim3(kGatherThreads), 0,
                     (hipStream_t)hip_stream, pool, Mx4Keys{k_codes, k_scales}, q_per_seq, N, w.keys, w.qpos, q_codes,
                     q_scales, w.q);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  // the gathered rows as a batch of T one-query "sequences" of kPool keys
  csa2_status s = csa2_index(w.q, w_idx, w.keys, w.qpos, 1, T, 1, kPool, w.scores, w.tile_max, w.stats,
                             w.stats_bytes, hip_stream);
  if (s != CSA2_OK) return s;
  return reindex_select_launch(w.scores, w.stats, w.stats_bytes, w.q, w_idx, w.keys, kPool, 0, pool, T, k, indices,
                               (hipStream_t)hip_stream);
}
