// Exact top-k selection (csa2_topk).
//
// Per query: keep the first min(k, n_vis) entries of the order (fp64 score
// descending, index ascending) and return them ascending by index (report
// sec. 2.3: each query keeps its top-k entries, k = 512 per sec. 4.2.1).
//
// The fp32 scores of csa2_index differ from the fp64 reference by at most
// eps (err_bound).  Let T^ be the k-th largest fp32 score.  Then
//   * every true top-k member has fp32 score >= T^ - 2 eps  (k entries have
//     fp32 >= T^, hence fp64 >= T^ - eps; a member's fp64 is at least the
//     k-th fp64 value);
//   * every entry with fp32 score > T^ + 2 eps is a member (fewer than k
//     entries have fp32 > T^).
// Any tau <= T^ therefore gives a candidate set {fp32 >= tau - 2 eps} that
// contains the whole answer.  Two regimes:
//
//  * Large rows (N > kSmallMax): the row is cut into M = 4096 groups, group j
//    holding the float4 runs j, j+M, j+2M, ... (so every group samples the
//    whole row); tau = a lower bound of the k-th largest group maximum, which
//    is <= T^ because those k maxima are k distinct entries.  One pass
//    computes the maxima (topk_gmax_kernel), one block per query brackets
//    tau (topk_tau_kernel), one pass compacts the candidates
//    (topk_compact_kernel), and one block per query finishes
//    (topk_finish_kernel).  For i.i.d. scores about 1.1 k entries pass.
//  * Small rows (N <= kSmallMax, e.g. a prefill chunk): one block per query
//    loads the visible scores into LDS and does everything there
//    (topk_small_kernel).
//
// The finish, in both regimes: bracket T^ among the candidates (lo <= T^ <= hi,
// two levels of 256 value bins; the arguments above hold with T^ replaced by
// hi for the sure side and by lo for the candidate side), accept entries
// above hi + 2 eps, rescore the band [lo - 2 eps, hi + 2 eps] in fp64 with the
// reference's exact operation sequence (fma per channel in order, then fma per
// head in order; IEEE fma is correctly rounded on both sides) and take the
// rest by (fp64 score desc, index asc).  If the candidates or the band exceed
// capacity, the same block falls back to exact streaming passes over the
// whole row (slow, exact).
#include "csa2_common.h"

namespace csa2 {

constexpr int kFinThreads = 1024;
constexpr int kGroups = 4096;            // large regime: group maxima per query
constexpr int kGroupThreads = 256;       // gmax block: 64 groups x 4 sub-ranges
constexpr int kCompactThreads = 256;
constexpr int kCompactChunk = 8192;      // entries per compact block
constexpr int kBandLds = 2048;           // band entries resolved in LDS
constexpr int kCandLds = 4096;           // candidates handled in LDS by the finish
constexpr int kDefaultCap = 2048;        // default candidate capacity per query
constexpr int kSmallMax = 36864;         // small regime: visible scores kept in LDS
constexpr int kHdrWords = 64;            // per query: [0] candidate count, [1] tau (fp32 bits)

// ---------------------------------------------------------------- helpers

// One ulp towards -inf / +inf (identity on infinities and NaN).
__device__ __forceinline__ double next_down(double x) {
  if (!(x > -INFINITY && x < INFINITY)) return x;
  if (x == 0.0) return -0x1p-1074;
  const long long u = __double_as_longlong(x);
  return __longlong_as_double(x > 0.0 ? u - 1 : u + 1);
}
__device__ __forceinline__ double next_up(double x) { return -next_down(-x); }

// fp64 score with the reference's exact operation sequence (global operands;
// used by the streaming fallback only).
__device__ double exact_score(const uint16_t* __restrict__ q, const float* __restrict__ w,
                              const uint16_t* __restrict__ key) {
  double sc = 0.0;
  for (int h = 0; h < kIdxHeads; ++h) {
    double d = 0.0;
    for (int c = 0; c < kIdxDim; ++c) d = fma(bf16_to_f64(q[h * kIdxDim + c]), bf16_to_f64(key[c]), d);
    sc = fma((double)w[h], d > 0.0 ? d : 0.0, sc);
  }
  return sc;
}

// Digit holding the rank-th largest (rank 1-based) of hist[256] (LDS), found by
// wave 0 with a wave prefix sum.  Writes digit and remaining rank to out[0],
// out[1].  Call with all threads.
__device__ __forceinline__ void pick_digit(const uint32_t* hist, uint32_t rank, uint32_t* out) {
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    // lane owns digits 255-4*lane .. 252-4*lane (descending)
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; sum += c[i]; }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t v = __shfl_up(incl, o, 64);
      if (lane >= o) incl += v;
    }
    uint32_t cum = incl - sum;
    if (cum < rank && rank <= incl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum + c[i] >= rank) {
          out[0] = 255u - 4u * lane - i;
          out[1] = rank - cum;
          break;
        }
        cum += c[i];
      }
    }
  }
  __syncthreads();
}

// Selection scratch shared by the bracketing helpers.
struct alignas(16) SelLds {
  uint32_t hist[256];
  uint32_t pick[2];
  float red[2][kFinThreads / 64];
};

// Block min / max (all threads; returns the same pair everywhere).
__device__ __forceinline__ float2 block_minmax(SelLds& s, float mn, float mx) {
  mn = -wave_max(-mn);
  mx = wave_max(mx);
  const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) { s.red[0][w] = mn; s.red[1][w] = mx; }
  __syncthreads();
  mn = s.red[0][0];
  mx = s.red[1][0];
  for (int i = 1; i < nw; ++i) { mn = fminf(mn, s.red[0][i]); mx = fmaxf(mx, s.red[1][i]); }
  return make_float2(mn, mx);
}

__device__ __forceinline__ uint32_t value_bin(float x, float a, float scale) {
  const float f = (x - a) * scale;
  return f >= 255.f ? 255u : (f > 0.f ? (uint32_t)f : 0u);
}

// Visit get(i) for i < n, four at a time per thread so that four loads are in flight.
template <typename Get, typename F>
__device__ __forceinline__ void for_each4(int64_t n, Get get, F f) {
  const int64_t bd = blockDim.x;
  for (int64_t i = threadIdx.x; i < n; i += 4 * bd) {
    float v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = (i + u * bd < n) ? get(i + u * bd) : 0.f;
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u * bd < n) f(v[u]);
  }
}

// Bracket lo <= T <= hi of T = the rank-th largest (1-based) of the n values
// get(i): two levels of 256 value bins over [min, max]; lo and hi are the
// smallest and largest values sharing T's final bin.  With `loose`, stop after
// the first level and return lo = the smallest value in T's bin or above
// (a lower bound with at least `rank` values >= lo).  All threads participate.
template <typename Get>
__device__ void bracket_kth(SelLds& s, int64_t n, uint32_t rank, Get get, bool loose, float* lo, float* hi) {
  const float inf = INFINITY;
  float mn = inf, mx = -inf;
  for_each4(n, get, [&](float v) { mn = fminf(mn, v); mx = fmaxf(mx, v); });
  float2 r = block_minmax(s, mn, mx);
  const float a1 = r.x, s1 = r.y > r.x ? 255.99f / (r.y - r.x) : 0.f;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) s.hist[i] = 0;
  __syncthreads();
  for_each4(n, get, [&](float v) { atomicAdd(&s.hist[value_bin(v, a1, s1)], 1u); });
  pick_digit(s.hist, rank, s.pick);
  const uint32_t b1 = s.pick[0];
  rank = s.pick[1];
  if (loose) {
    mn = inf;
    for_each4(n, get, [&](float v) { if (value_bin(v, a1, s1) >= b1) mn = fminf(mn, v); });
    r = block_minmax(s, mn, -inf);
    *lo = r.x;
    *hi = inf;
    return;
  }
  mn = inf; mx = -inf;
  for_each4(n, get, [&](float v) { if (value_bin(v, a1, s1) == b1) { mn = fminf(mn, v); mx = fmaxf(mx, v); } });
  r = block_minmax(s, mn, mx);
  const float a2 = r.x, s2 = r.y > r.x ? 255.99f / (r.y - r.x) : 0.f;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) s.hist[i] = 0;
  __syncthreads();
  for_each4(n, get, [&](float v) {
    if (value_bin(v, a1, s1) == b1) atomicAdd(&s.hist[value_bin(v, a2, s2)], 1u);
  });
  pick_digit(s.hist, rank, s.pick);
  const uint32_t b2 = s.pick[0];
  mn = inf; mx = -inf;
  for_each4(n, get, [&](float v) {
    if (value_bin(v, a1, s1) == b1 && value_bin(v, a2, s2) == b2) { mn = fminf(mn, v); mx = fmaxf(mx, v); }
  });
  r = block_minmax(s, mn, mx);
  *lo = r.x;
  *hi = r.y;
}

// --------------------------------------------------------- finish (shared)

// LDS of the finishing block.  FinLds::tail is only touched after the
// candidates have been classified, so the small regime overlays it on its
// copy of the scores.
struct alignas(16) FinTail {
  uint32_t out_sorted[kTopK];
  uint64_t band_key[kBandLds];
  uint16_t krows[64][kIdxDim];
  uint16_t qrows[kIdxHeads][kIdxDim + 8];
  double dots[32][kIdxHeads + 1];
};
struct alignas(16) FinLds {
  SelLds sel;
  uint32_t n_out, n_band;
  uint32_t out[kTopK];
  uint32_t band_idx[kBandLds];
};

// fp64 scores of the band (reference operation order): thread (e = tid/32,
// h = tid%32) forms dot(q[h], K[e]) with 128 sequential fmas from LDS, then 32
// threads fold the heads in order.
__device__ void rescore_band(FinLds& sh, FinTail& tl, uint32_t nb, const uint16_t* __restrict__ qt,
                             const float* __restrict__ wt, const uint16_t* __restrict__ kb) {
  const int tid = threadIdx.x;
  const int e = tid >> 5, h = tid & 31;
  for (int i = tid; i < kIdxHeads * 16; i += kFinThreads) {
    const int r = i >> 4, c = i & 15;
    *reinterpret_cast<uint4*>(&tl.qrows[r][8 * c]) = *reinterpret_cast<const uint4*>(qt + r * kIdxDim + 8 * c);
  }
  for (uint32_t base = 0; base < nb; base += 64) {
    // 64 key rows x 256 B: one 16-byte chunk per thread
    {
      const int r = tid >> 4, c = tid & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (base + r < nb) v = *reinterpret_cast<const uint4*>(kb + (size_t)sh.band_idx[base + r] * kIdxDim + 8 * c);
      *reinterpret_cast<uint4*>(&tl.krows[r][8 * c]) = v;
    }
    __syncthreads();
    for (uint32_t half = 0; half < 64 && base + half < nb; half += 32) {
      if (base + half + e < nb) {
        double d = 0.0;
#pragma unroll 4
        for (int i = 0; i < 16; ++i) {
          const uint4 kq = *reinterpret_cast<const uint4*>(&tl.krows[half + e][8 * i]);
          const uint4 qq = *reinterpret_cast<const uint4*>(&tl.qrows[h][8 * i]);
          const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
          const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            d = fma((double)bf16lo(qw[p]), (double)bf16lo(kw[p]), d);
            d = fma((double)bf16hi(qw[p]), (double)bf16hi(kw[p]), d);
          }
        }
        tl.dots[e][h] = d;
      }
      __syncthreads();
      if (tid < 32 && base + half + tid < nb) {
        double sc = 0.0;
#pragma unroll 8
        for (int hh = 0; hh < kIdxHeads; ++hh) {
          const double d = tl.dots[tid][hh];
          sc = fma((double)wt[hh], d > 0.0 ? d : 0.0, sc);
        }
        tl.band_key[base + half + tid] = f64_key(sc);
      }
      __syncthreads();
    }
  }
}

// Complete the selection once T^ is known and the sure entries and band are
// in sh.out / sh.band_idx (n_band <= kBandLds): rescore and pick the band's share.
__device__ void finish_band(FinLds& sh, FinTail& tl, uint32_t kk, const uint16_t* qt, const float* wt,
                            const uint16_t* kb) {
  const uint32_t nb = sh.n_band;
  rescore_band(sh, tl, nb, qt, wt, kb);
  const uint32_t r = kk - sh.n_out;
  const uint32_t base_out = sh.n_out;
  for (uint32_t i = threadIdx.x; i < nb; i += kFinThreads) {
    const uint64_t ki = tl.band_key[i];
    const uint32_t ii = sh.band_idx[i];
    uint32_t rank = 0;
#pragma unroll 4
    for (uint32_t j = 0; j < nb; ++j) {
      const uint64_t kj = tl.band_key[j];
      rank += (kj > ki) | ((kj == ki) & (sh.band_idx[j] < ii));
    }
    if (rank < r) sh.out[base_out + rank] = ii;
  }
  __syncthreads();
}

// Exact streaming fallback over the whole visible row (capacity overflow).
// Gathers sure entries, then radix-selects the band's share over the 96-bit
// composite (fp64 key, ~index), recomputing each band member's fp64 score.
__device__ void finish_streaming(FinLds& sh, uint32_t kk, const float* row, int64_t nv, double lo, double hi,
                                 const uint16_t* qt, const float* wt, const uint16_t* kb) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.n_out = 0;
  __syncthreads();
  for (int64_t s = tid; s < nv; s += kFinThreads)
    if ((double)row[s] > hi) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)s;
  __syncthreads();
  uint32_t rank = kk - sh.n_out;
  uint64_t phi = 0, mhi = 0;
  uint32_t plo = 0, mlo = 0;
  for (int pass = 0; pass < 12; ++pass) {
    for (int i = tid; i < 256; i += kFinThreads) sh.sel.hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < nv; s += kFinThreads) {
      const double v = (double)row[s];
      if (v < lo || v > hi) continue;
      const uint64_t key = f64_key(exact_score(qt, wt, kb + (size_t)s * kIdxDim));
      const uint32_t low = ~(uint32_t)s;
      if ((key & mhi) != phi || (low & mlo) != plo) continue;
      const uint32_t digit = pass < 8 ? (uint32_t)(key >> (56 - 8 * pass)) & 255u
                                      : (low >> (24 - 8 * (pass - 8))) & 255u;
      atomicAdd(&sh.sel.hist[digit], 1u);
    }
    pick_digit(sh.sel.hist, rank, sh.sel.pick);
    const uint32_t digit = sh.sel.pick[0];
    rank = sh.sel.pick[1];
    if (pass < 8) {
      phi |= (uint64_t)digit << (56 - 8 * pass);
      mhi |= (uint64_t)255 << (56 - 8 * pass);
    } else {
      plo |= digit << (24 - 8 * (pass - 8));
      mlo |= 255u << (24 - 8 * (pass - 8));
    }
  }
  for (int64_t s = tid; s < nv; s += kFinThreads) {
    const double v = (double)row[s];
    if (v < lo || v > hi) continue;
    const uint64_t key = f64_key(exact_score(qt, wt, kb + (size_t)s * kIdxDim));
    const uint32_t low = ~(uint32_t)s;
    if (key > phi || (key == phi && low >= plo)) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)s;
  }
  __syncthreads();
}

// Ascending output (indices are distinct): rank by comparison, 4 per LDS read.
__device__ void write_sorted(FinLds& sh, FinTail& tl, uint32_t kk, int k, int32_t* out) {
  for (uint32_t i = kk + threadIdx.x; i < kTopK; i += kFinThreads) sh.out[i] = 0xFFFFFFFFu;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < kk; i += kFinThreads) {
    const uint32_t v = sh.out[i];
    uint32_t pos = 0;
#pragma unroll 8
    for (uint32_t j = 0; j < kTopK; j += 4) {
      const uint4 u = *reinterpret_cast<const uint4*>(&sh.out[j]);
      pos += (u.x < v) + (u.y < v) + (u.z < v) + (u.w < v);
    }
    tl.out_sorted[pos] = v;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < k; i += kFinThreads) out[i] = i < (int)kk ? (int32_t)tl.out_sorted[i] : -1;
}

// Band bounds around the bracket [t_lo, t_hi] of T^ (rounded outwards in fp64).
__device__ __forceinline__ void band_bounds(float t_lo, float t_hi, float eps, double* lo, double* hi) {
  *lo = next_down((double)t_lo - 2.0 * (double)eps);
  *hi = next_up((double)t_hi + 2.0 * (double)eps);
  if (!(*lo <= (double)t_lo)) *lo = -INFINITY;   // eps not finite: everything is in the band
  if (!(*hi >= (double)t_hi)) *hi = INFINITY;
}

// ----------------------------------------------------------- large regime

struct LargeWs {
  uint32_t* hdr;   // [T][kHdrWords]
  float* gmax;     // [T][kGroups]
  uint32_t* cidx;  // [T][cap]
  float* cval;     // [T][cap]
};

__host__ __device__ __forceinline__ size_t large_ws_fixed(int T) {
  return (size_t)T * (kHdrWords * 4 + kGroups * 4);
}
__device__ __forceinline__ LargeWs large_ws(void* base, int T, int64_t cap) {
  LargeWs w;
  w.hdr = (uint32_t*)base;
  w.gmax = (float*)(w.hdr + (size_t)T * kHdrWords);
  w.cidx = (uint32_t*)(w.gmax + (size_t)T * kGroups);
  w.cval = (float*)(w.cidx + (size_t)T * cap);
  return w;
}

// Group maxima: group j = float4 runs j, j+M, j+2M, ... of the visible row.
// grid (kGroups/64, T), 256 threads = 64 groups x 4 interleaved sub-ranges.
template <bool VEC>
__global__ __launch_bounds__(kGroupThreads) void topk_gmax_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ q_pos, int ratio,
                                                                  int64_t N, int k, void* ws, int T, int64_t cap) {
  const int t = blockIdx.y;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  if (nv <= k) return;
  LargeWs w = large_ws(ws, T, cap);
  if (blockIdx.x == 0 && threadIdx.x == 0) w.hdr[(size_t)t * kHdrWords] = 0u;  // candidate count
  const int j = blockIdx.x * 64 + (threadIdx.x & 63);
  const int r = threadIdx.x >> 6;
  const float* row = scores + (size_t)t * N;
  const int64_t n4 = (nv + 3) / 4;
  float m = -INFINITY;
  for (int64_t tile = j + (int64_t)kGroups * r; tile < n4; tile += (int64_t)kGroups * 4 * 4) {
    float4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t tl = tile + (int64_t)kGroups * 4 * u;
      const int64_t s = 4 * tl;
      if (VEC && s + 3 < nv) {
        x[u] = *reinterpret_cast<const float4*>(row + s);
      } else {
        x[u].x = (tl < n4 && s < nv) ? row[s] : -INFINITY;
        x[u].y = (tl < n4 && s + 1 < nv) ? row[s + 1] : -INFINITY;
        x[u].z = (tl < n4 && s + 2 < nv) ? row[s + 2] : -INFINITY;
        x[u].w = (tl < n4 && s + 3 < nv) ? row[s + 3] : -INFINITY;
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) m = fmaxf(m, fmaxf(fmaxf(x[u].x, x[u].y), fmaxf(x[u].z, x[u].w)));
  }
  __shared__ float part[4][64];
  part[r][threadIdx.x & 63] = m;
  __syncthreads();
  if (r == 0) {
    const int l = threadIdx.x;
    w.gmax[(size_t)t * kGroups + j] = fmaxf(fmaxf(part[0][l], part[1][l]), fmaxf(part[2][l], part[3][l]));
  }
}

// tau <= T^: a lower bound of the k-th largest group maximum, with at least
// k maxima (k distinct entries) >= tau; -inf when fewer than k groups are
// non-empty.  grid T, 1024 threads; the maxima are staged in LDS.
__global__ __launch_bounds__(kFinThreads) void topk_tau_kernel(const int32_t* __restrict__ q_pos, int ratio,
                                                               int64_t N, int k, void* ws, int T, int64_t cap) {
  __shared__ SelLds sel;
  __shared__ float g[kGroups];
  const int t = blockIdx.x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  if (nv <= k) return;
  LargeWs w = large_ws(ws, T, cap);
  const int64_t ng = (nv + 3) / 4 < kGroups ? (nv + 3) / 4 : kGroups;
  float tau = -INFINITY;
  if (ng >= k) {
    for (int i = threadIdx.x; i < ng; i += kFinThreads) g[i] = w.gmax[(size_t)t * kGroups + i];
    __syncthreads();
    float lo, hi;
    bracket_kth(sel, ng, (uint32_t)k, [&](int64_t i) { return g[i]; }, true, &lo, &hi);
    tau = lo;
  }
  if (threadIdx.x == 0) w.hdr[(size_t)t * kHdrWords + 1] = __float_as_uint(tau);
}

// Candidates: every visible entry with score >= tau - 2 eps (block-aggregated
// append).  grid (chunks, T), 256 threads x 32 entries.
template <bool VEC>
__global__ __launch_bounds__(kCompactThreads) void topk_compact_kernel(const float* __restrict__ scores,
                                                                       const float* __restrict__ err_bound,
                                                                       const int32_t* __restrict__ q_pos, int ratio,
                                                                       int64_t N, int k, void* ws, int T,
                                                                       int64_t cap) {
  const int t = blockIdx.y;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t s0 = (int64_t)blockIdx.x * kCompactChunk;
  if (nv <= k || s0 >= nv) return;
  LargeWs w = large_ws(ws, T, cap);
  uint32_t* hdr = w.hdr + (size_t)t * kHdrWords;
  const float* row = scores + (size_t)t * N;
  constexpr int kVec = kCompactChunk / kCompactThreads / 4;  // 8 float4 per thread
  float v[4 * kVec];
  // this block's scores: all loads in flight while tau is being found
#pragma unroll
  for (int i = 0; i < kVec; ++i) {
    const int64_t s = s0 + 4 * ((int64_t)i * kCompactThreads + threadIdx.x);
    if (VEC && s + 3 < nv) {
      const float4 x = *reinterpret_cast<const float4*>(row + s);
      v[4 * i] = x.x; v[4 * i + 1] = x.y; v[4 * i + 2] = x.z; v[4 * i + 3] = x.w;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[4 * i + e] = (s + e < nv) ? row[s + e] : -INFINITY;
    }
  }
  const float tau = __uint_as_float(hdr[1]);
  const double thr = next_down((double)tau - 2.0 * (double)err_bound[t]);
  __shared__ uint32_t s_cnt, s_base;
  __shared__ uint32_t s_idx[1024];
  __shared__ float s_val[1024];
  if (threadIdx.x == 0) s_cnt = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4 * kVec; ++i) {
    const int64_t s = s0 + 4 * ((int64_t)(i >> 2) * kCompactThreads + threadIdx.x) + (i & 3);
    if (s < nv && (double)v[i] >= thr) {
      const uint32_t p = atomicAdd(&s_cnt, 1u);
      if (p < 1024) {
        s_idx[p] = (uint32_t)s;
        s_val[p] = v[i];
      } else {  // rare: a block with more than 1024 candidates appends directly
        const uint32_t pos = atomicAdd(&hdr[0], 1u);
        if (pos < (uint64_t)cap) {
          w.cidx[(size_t)t * cap + pos] = (uint32_t)s;
          w.cval[(size_t)t * cap + pos] = v[i];
        }
      }
    }
  }
  __syncthreads();
  const uint32_t n = s_cnt < 1024 ? s_cnt : 1024;
  if (threadIdx.x == 0 && n) s_base = atomicAdd(&hdr[0], n);
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < n; i += kCompactThreads) {
    const uint32_t pos = s_base + i;
    if (pos < (uint64_t)cap) {
      w.cidx[(size_t)t * cap + pos] = s_idx[i];
      w.cval[(size_t)t * cap + pos] = s_val[i];
    }
  }
}

struct LargeFinLds {
  FinLds f;
  FinTail tail;
  alignas(16) float cval[kCandLds];
  uint32_t cidx[kCandLds];
};

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const float* __restrict__ err_bound, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos,
    int ratio, int q_per_seq, int64_t N, int k, int32_t* __restrict__ indices, void* ws, int T, int64_t cap) {
  __shared__ LargeFinLds L;
  FinLds& sh = L.f;
  FinTail& tl = L.tail;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  int32_t* out = indices + (size_t)t * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kFinThreads) out[i] = i < nv ? i : -1;
    return;
  }
  const uint32_t kk = (uint32_t)k;
  const int b = t / q_per_seq;
  const uint16_t* qt = q_idx + (size_t)t * kIdxHeads * kIdxDim;
  const float* wt = w_idx + (size_t)t * kIdxHeads;
  const uint16_t* kb = k_idx + (size_t)b * N * kIdxDim;
  const float* row = scores + (size_t)t * N;
  LargeWs w = large_ws(ws, T, cap);
  const uint32_t cnt = w.hdr[(size_t)t * kHdrWords];
  const float eps = err_bound[t];
  const bool fits = (int64_t)cnt <= cap && cnt <= kCandLds;
  if (tid == 0) { sh.n_out = 0; sh.n_band = 0; }
  if (fits) {
    for (uint32_t i = tid; i < ((cnt + 3) & ~3u); i += kFinThreads) {
      L.cval[i] = i < cnt ? w.cval[(size_t)t * cap + i] : -INFINITY;
      L.cidx[i] = i < cnt ? w.cidx[(size_t)t * cap + i] : 0u;
    }
  }
  __syncthreads();
  float t_lo, t_hi;
  if (fits) bracket_kth(sh.sel, cnt, kk, [&](int64_t i) { return L.cval[i]; }, false, &t_lo, &t_hi);
  else bracket_kth(sh.sel, nv, kk, [&](int64_t i) { return row[i]; }, false, &t_lo, &t_hi);
  double lo, hi;
  band_bounds(t_lo, t_hi, eps, &lo, &hi);
  bool fast = fits;
  if (fast) {
    for (uint32_t i = tid; i < cnt; i += kFinThreads) {
      const double v = (double)L.cval[i];
      if (v > hi) sh.out[atomicAdd(&sh.n_out, 1u)] = L.cidx[i];
      else if (v >= lo) {
        const uint32_t p = atomicAdd(&sh.n_band, 1u);
        if (p < kBandLds) sh.band_idx[p] = L.cidx[i];
      }
    }
    __syncthreads();
    fast = sh.n_band <= kBandLds;
    __syncthreads();
  }
  if (fast) finish_band(sh, tl, kk, qt, wt, kb);
  else finish_streaming(sh, kk, row, nv, lo, hi, qt, wt, kb);
  write_sorted(sh, tl, kk, k, out);
}

// ----------------------------------------------------------- small regime

// One block per query; the visible scores live in LDS (the finishing tail
// overlays them once they have been classified).
struct SmallLds {
  FinLds f;
  union {
    float v[kSmallMax];
    FinTail tail;
  } u;
};

__global__ __launch_bounds__(kFinThreads) void topk_small_kernel(
    const float* __restrict__ scores, const float* __restrict__ err_bound, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos,
    int ratio, int q_per_seq, int64_t N, int k, int32_t* __restrict__ indices) {
  __shared__ SmallLds L;
  FinLds& sh = L.f;
  FinTail& tl = L.u.tail;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  int32_t* out = indices + (size_t)t * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kFinThreads) out[i] = i < nv ? i : -1;
    return;
  }
  const uint32_t kk = (uint32_t)k;
  const int b = t / q_per_seq;
  const uint16_t* qt = q_idx + (size_t)t * kIdxHeads * kIdxDim;
  const float* wt = w_idx + (size_t)t * kIdxHeads;
  const uint16_t* kb = k_idx + (size_t)b * N * kIdxDim;
  const float* row = scores + (size_t)t * N;
  const float eps = err_bound[t];
  if (tid == 0) { sh.n_out = 0; sh.n_band = 0; }
  for (int64_t i = tid; i < nv; i += kFinThreads) L.u.v[i] = row[i];
  __syncthreads();
  float t_lo, t_hi;
  bracket_kth(sh.sel, nv, kk, [&](int64_t i) { return L.u.v[i]; }, false, &t_lo, &t_hi);
  double lo, hi;
  band_bounds(t_lo, t_hi, eps, &lo, &hi);
  for (int64_t i = tid; i < nv; i += kFinThreads) {
    const double v = (double)L.u.v[i];
    if (v > hi) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)i;
    else if (v >= lo) {
      const uint32_t p = atomicAdd(&sh.n_band, 1u);
      if (p < kBandLds) sh.band_idx[p] = (uint32_t)i;
    }
  }
  __syncthreads();
  const bool fast = sh.n_band <= kBandLds;
  __syncthreads();
  if (fast) finish_band(sh, tl, kk, qt, wt, kb);
  else finish_streaming(sh, kk, row, nv, lo, hi, qt, wt, kb);
  write_sorted(sh, tl, kk, k, out);
}

}  // namespace csa2

using namespace csa2;

static int64_t topk_cap_for(size_t ws_bytes, int32_t T, int64_t N) {
  const size_t fixed = large_ws_fixed(T);
  if (ws_bytes < fixed) return -1;
  int64_t cap = (int64_t)((ws_bytes - fixed) / ((size_t)T * 8));
  cap = cap / 4 * 4;  // keep the float array 16-byte aligned
  if (cap > N) cap = (N + 3) / 4 * 4;
  return cap;
}

static bool topk_small_regime(int64_t N) { return N <= kSmallMax; }

extern "C" size_t csa2_topk_workspace_bytes(int32_t T, int64_t N, int32_t k) {
  if (T < 1 || N < 1 || k != kTopK) return 0;
  if (topk_small_regime(N)) return 0;
  int64_t cap = N < kDefaultCap ? (N + 3) / 4 * 4 : kDefaultCap;
  return large_ws_fixed(T) + (size_t)T * (size_t)cap * 8;
}

extern "C" size_t csa2_topk_min_workspace_bytes(int32_t T, int64_t N, int32_t k) {
  if (T < 1 || N < 1 || k != kTopK) return 0;
  if (topk_small_regime(N)) return 0;
  return large_ws_fixed(T);
}

extern "C" csa2_status csa2_topk(const float* scores, const float* err_bound, const void* q_idx,
                                 const float* w_idx, const void* k_idx, const int32_t* q_pos, int32_t ratio,
                                 int32_t T, int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices,
                                 void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!scores || !err_bound || !q_idx || !w_idx || !k_idx || !indices) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(scores) || !aligned16(err_bound) || !aligned16(q_idx) || !aligned16(w_idx) ||
      !aligned16(k_idx) || !aligned16(indices) || (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || ratio < 1) return CSA2_ERR_INVALID_ARG;
  if (k != kTopK || N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  const uint16_t* q = (const uint16_t*)q_idx;
  const uint16_t* kx = (const uint16_t*)k_idx;
  if (topk_small_regime(N)) {
    hipLaunchKernelGGL(topk_small_kernel, dim3(T), dim3(kFinThreads), 0, st, scores, err_bound, q,
                       w_idx, kx, q_pos, ratio, q_per_seq, N, k, indices);
    if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
    return CSA2_OK;
  }
  if (!workspace || !aligned16(workspace) || workspace_bytes < csa2_topk_min_workspace_bytes(T, N, k))
    return CSA2_ERR_WORKSPACE;
  const int64_t cap = topk_cap_for(workspace_bytes, T, N);
  if (cap < 0) return CSA2_ERR_WORKSPACE;
  const bool vec = (N & 3) == 0;
  const dim3 ggrid(kGroups / 64, T);
  if (vec)
    hipLaunchKernelGGL(topk_gmax_kernel<true>, ggrid, dim3(kGroupThreads), 0, st, scores, q_pos, ratio, N, k,
                       workspace, T, cap);
  else
    hipLaunchKernelGGL(topk_gmax_kernel<false>, ggrid, dim3(kGroupThreads), 0, st, scores, q_pos, ratio, N, k,
                       workspace, T, cap);
  hipLaunchKernelGGL(topk_tau_kernel, dim3(T), dim3(kFinThreads), 0, st, q_pos, ratio, N, k, workspace, T, cap);
  const dim3 cgrid((unsigned)((N + kCompactChunk - 1) / kCompactChunk), T);
  if (vec)
    hipLaunchKernelGGL(topk_compact_kernel<true>, cgrid, dim3(kCompactThreads), 0, st, scores, err_bound, q_pos,
                       ratio, N, k, workspace, T, cap);
  else
    hipLaunchKernelGGL(topk_compact_kernel<false>, cgrid, dim3(kCompactThreads), 0, st, scores, err_bound, q_pos,
                       ratio, N, k, workspace, T, cap);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(T), dim3(kFinThreads), 0, st, scores, err_bound, q, w_idx, kx, q_pos,
                     ratio, q_per_seq, N, k, indices, workspace, T, cap);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
