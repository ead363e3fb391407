// Launch plan of the indexer scan and the layout of the per-call summary it
// leaves for the selection (csa2_index -> csa2_topk).
//
// Summary (32-bit words, caller-allocated, csa2_index_stats_bytes):
//   [T][4]            header per query: {eps, floor, counter, counter}; the scan
//                     writes zeros, the selection writes eps and the floor and
//                     leaves the counters zero
//   [T][n_groups]     fp32 maxima of disjoint groups of the query's entries
//   [B * parts]       fp32 partial maxima of ||K_s||^2, `parts` per sequence
#pragma once

#include "csa2_common.h"

namespace csa2 {

constexpr int kScanThreads = 256;  // 4 waves
constexpr int kScanWaves = kScanThreads / 64;
constexpr int kScanTiles = 2;      // 16-key tiles per wave per iteration: 32 keys, 8 KiB
constexpr int kScanWaveKeys = 16 * kScanTiles;
constexpr int kChunkKeys = kScanWaveKeys * kScanWaves;  // 128 keys per block iteration
static_assert(kScanTiles >= 1 && kScanTiles <= 4, "a wave's lane groups take one tile each");
constexpr int kScanBlocks = 16384;  // blocks per launch the grid aims for: short blocks balance the load
constexpr int kGroupsWanted = 4096;

// Group maxima per query: kScanTiles * S per block, rounded up to a multiple of
// four (16-byte rows); the scan writes -inf to the padding.
__host__ __device__ inline int64_t group_count(int64_t blocks_x, int S) {
  return (blocks_x * kScanTiles * S + 3) / 4 * 4;
}

struct IndexPlan {
  int qg = 1;             // queries per group (template)
  int groups = 1;         // gridDim.z
  int B = 1;              // gridDim.y
  int blocks_x = 1;       // gridDim.x
  int slots = 1;          // S: group slots per (block, wave, tile)
  int64_t n_groups = 16;  // group maxima per query
  int64_t parts() const { return (int64_t)groups * blocks_x; }  // norm partials per sequence
};

inline bool index_plan(int32_t T, int32_t q_per_seq, int64_t N, IndexPlan* p) {
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || N >= ((int64_t)1 << 31)) return false;
  p->qg = q_per_seq == 1 ? 1 : q_per_seq == 2 ? 2 : 4;
  p->groups = (q_per_seq + p->qg - 1) / p->qg;
  p->B = T / q_per_seq;
  // aim for ~16384 blocks over 256 CUs (a few chunks each), each with at least one chunk
  const int64_t nchunks = (N + kChunkKeys - 1) / kChunkKeys;
  int64_t want = (kScanBlocks + (int64_t)p->B * p->groups - 1) / ((int64_t)p->B * p->groups);
  if (want > nchunks) want = nchunks;
  if (want < 1) want = 1;
  p->blocks_x = (int)want;
  // enough group slots for at least 4096 groups (kScanTiles per block and slot), within
  // the registers of the query count
  const int max_slots = p->qg == 1 ? 4 : p->qg == 2 ? 2 : 1;
  int slots = 1;
  while (slots < max_slots && (int64_t)p->blocks_x * kScanTiles * slots < kGroupsWanted) slots *= 2;
  p->slots = slots;
  p->n_groups = group_count(p->blocks_x, slots);
  return p->B <= 65535 && p->groups <= 65535;
}

// The grouped-query scan (index_group.hip): plans with p.qg >= 2.
void launch_scan_grouped(const IndexPlan& p, hipStream_t st, const uint16_t* q, const float* w, const uint16_t* k,
                         const int32_t* q_pos, int ratio, int q_per_seq, int64_t N, float* scores, float* tile_max,
                         uint32_t* header, float* gmax, float* partial);

// Word offsets of the summary's parts (all multiples of 4: 16-byte aligned).
__host__ __device__ inline size_t stats_groups_off(int T) { return (size_t)T * CSA2_STATS_WORDS; }
__host__ __device__ inline size_t stats_parts_off(int T, int64_t n_groups) {
  return stats_groups_off(T) + (size_t)T * (size_t)n_groups;
}
// Every word is written by the scan (no padding).
inline size_t stats_words(int T, const IndexPlan& p) {
  return stats_parts_off(T, p.n_groups) + (size_t)p.B * (size_t)p.parts();
}

}  // namespace csa2
