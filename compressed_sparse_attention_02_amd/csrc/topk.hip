// Exact top-k selection (csa2_topk).
//
// Per query: keep the first min(k, n_vis) entries of the order (fp64 score
// descending, index ascending) and return them ascending by index (report
// sec. 2.3: each query keeps its top-k entries, k = 512 per sec. 4.2.1).
//
// The fp32 scores of csa2_index differ from the fp64 reference by at most
// eps, formed here from the scan's summary (partial maxima of ||K||^2) and
// the query.  If k distinct entries have fp32 score >= tau, then the k-th
// largest fp64 score T^ satisfies T^ >= tau - eps, so every true top-k member
// has fp32 score >= tau - 2 eps: {fp32 >= tau - 2 eps} is a candidate set
// that contains the whole answer.  Two regimes:
//
//  * Tile regime (any N; the only one without a score matrix).  tau is a
//    lower bound of the k-th largest of a set of maxima of disjoint groups of
//    entries (those are k distinct entries): the visible tiles' maxima when
//    there are at most 8192 tiles, else the scan's group maxima.
//    topk_floor_kernel (one block per query) forms eps and tau from the
//    summary and writes them to its header; each block of topk_cand_kernel
//    (4096 entries) re-derives the fp32 scores of its tiles whose maximum
//    reaches tau - 2 eps with the scan's own MFMA code, keeps the entries
//    that reach it, computes their fp64 scores with the reference's exact
//    operation sequence and writes them in index order to its slots;
//    topk_select_kernel (one block per query) selects the k largest fp64 keys
//    among the candidates and writes them in index order.  For i.i.d. scores
//    about 1.1 k entries are candidates.  If they exceed the workspace or LDS
//    capacity, the same block falls back to exact radix passes over the
//    candidate tiles (slow, exact).
//  * Row regime (scores given, N <= kSmallMax, e.g. a prefill chunk): one
//    block per query loads the visible scores into LDS, brackets the k-th
//    largest fp32 value (lo <= T^ <= hi, two levels of 256 value bins), accepts
//    entries above hi + 2 eps, rescores the band [lo - 2 eps, hi + 2 eps] in
//    fp64 and takes the rest by (fp64 score desc, index asc).
#include <type_traits>

#include "idx_plan.h"
#include "mxfp4.h"

namespace csa2 {

constexpr int kFinThreads = 1024;        // row-regime block
constexpr int kBandLds = 2048;           // band entries resolved in LDS (row regime)
constexpr int kSmallMax = CSA2_TOPK_ROW_MAX;  // row regime: visible scores kept in LDS

constexpr int kCandThreads = 256;
constexpr int kCandTiles = 256;          // tiles (4096 entries) per candidate block
constexpr int kCandMax = 1024;           // passing entries a candidate block holds (beyond: exact fallback)
constexpr int kSelThreads = 256;
constexpr int kSelLds = 4096;            // candidates a select block holds in LDS
constexpr int kSelBlocks = 4096;         // candidate blocks per query the select block can index (N <= 2^24)
constexpr int kSlots = 32;               // fixed candidate slots per candidate block
constexpr int kDefaultSpill = 2048;      // shared slots per query for blocks with more
constexpr int kMaxSpill = 16384;
constexpr uint32_t kOverflow = 0x80000000u;  // stats[2]: shared slots used, this bit set on overflow

// ---------------------------------------------------------------- helpers

// One ulp towards -inf / +inf (identity on infinities and NaN).
__device__ __forceinline__ double next_down(double x) {
  if (!(x > -INFINITY && x < INFINITY)) return x;
  if (x == 0.0) return -0x1p-1074;
  const long long u = __double_as_longlong(x);
  return __longlong_as_double(x > 0.0 ? u - 1 : u + 1);
}
__device__ __forceinline__ double next_up(double x) { return -next_down(-x); }

// ---- the BF16 selector (gzher.com reading of DeepSeek-V4, FP4 QAT section:
// index scores are quantised to BF16 before the top-k).  The selection order
// is (bf16 rounding of the exact score desc, index asc).

// Nearest bf16 value of x, ties to the even significand (quantum 2^-133 below
// 2^-126, infinity past 0x1.FEp127), as a double.
__device__ __forceinline__ double bf16_round_f64(double x) {
  if (x == 0.0 || !(fabs(x) < INFINITY)) return x;
  int e;
  const double f = frexp(x, &e);
  if (e - 1 < -126) return ldexp(rint(ldexp(x, 133)), -133);
  const double r = ldexp(rint(ldexp(f, 8)), e - 8);
  return fabs(r) > 0x1.FEp127 ? copysign((double)INFINITY, r) : r;
}

// The bf16 value below (above) a finite bf16 value b, from its bit pattern.
__device__ __forceinline__ double bf16_below(double b) {
  const uint32_t u = __float_as_uint((float)b) >> 16;
  uint32_t p;
  if (b == 0.0) p = 0x8001u;            // -2^-133
  else if (b > 0.0) p = u - 1u;
  else p = u + 1u;                      // -max - 1 step is -infinity (0xFF80)
  return (double)__uint_as_float(p << 16);
}
__device__ __forceinline__ double bf16_above(double b) { return -bf16_below(-b); }

// Rounding boundaries of a bf16 value b: every x >= lower_mid rounds to b or
// above, every x > upper_mid strictly above b (midpoints are exact in fp64).
__device__ __forceinline__ double bf16_lower_mid(double b) {
  return (fabs(b) < INFINITY) ? 0.5 * (bf16_below(b) + b) : b;
}
__device__ __forceinline__ double bf16_upper_mid(double b) {
  return (fabs(b) < INFINITY) ? 0.5 * (b + bf16_above(b)) : b;
}

// The value an entry is ranked by: its exact score, or that score's bf16 rounding.
__device__ __forceinline__ double sel_value(double s, int bsel) { return bsel ? bf16_round_f64(s) : s; }

// Candidate threshold of the tile regime.  At least k entries have an fp32
// score >= tau, so the k-th exact score S is >= tau - eps and every selected
// entry has an exact score >= S (exact order) or >= the lower rounding boundary
// of bf16(S) (bf16 order; rounding is monotone): its fp32 score is at least
// that minus eps.
__device__ __forceinline__ double cand_threshold(float tau, float eps, int bsel) {
  if (!bsel) return next_down((double)tau - 2.0 * (double)eps);
  const double lb = next_down((double)tau - (double)eps);
  return next_down(bf16_lower_mid(bf16_round_f64(lb)) - (double)eps);
}

// The scan's norm partials [B][groups][blocks_x] of query t's group (groups of
// qg queries of one sequence): their maximum bounds ||K||^2 over every key
// that a query of the group sees, t's among them.
__device__ __forceinline__ const float* group_parts(const float* parts, int t, int q_per_seq, int qg,
                                                    int64_t blocks_x) {
  const int b = t / q_per_seq, z = (t % q_per_seq) / qg;
  const int groups = (q_per_seq + qg - 1) / qg;
  return parts + ((size_t)b * groups + z) * blocks_x;
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
// The scan's value for max_s ||K_s||^2 is the sum over the four 32-channel
// groups of each group's maximum over the keys, which is at least the maximum
// of the sums; each group is accumulated with bf16 dot2 steps in fp32 over
// nonnegative terms (relative error below 2^-16 even with two roundings per
// step), so it is inflated by (1 + 2^-10) before the square root.  ||q_h||^2
// is summed in fp64 (relative error below 2^-45 in any order), covered by
// (1 + 2^-40).
//
// This thread's share of the three terms: the maximum of its partials of
// max ||K||^2 (the sequence's n_parts scan partials, the first 8 per thread
// requested at once), and for threads below 256 (whole waves), |w_h| ||q_h||
// and |w_h| of head tid / 8, the same in the 8 lanes of each group of eight
// (the sum of squares is folded with DPP moves); 0 in the other threads.
// Reduce m2 with wave_max_dpp and the two sums with wave_sum_groups8_f64.
__device__ __forceinline__ void bound_terms(const uint16_t* __restrict__ q_t, const float* __restrict__ w_t,
                                            const float* __restrict__ parts_b, int64_t n_parts, int tid,
                                            int nthreads, float* m2, double* qf, double* sw) {
  float pm[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int64_t i = tid + (int64_t)u * nthreads;
    pm[u] = i < n_parts ? parts_b[i] : 0.f;
  }
  uint4 x = make_uint4(0u, 0u, 0u, 0u), y = x;
  float wh = 0.f;
  if (tid < 256) {
    const uint4* qv = reinterpret_cast<const uint4*>(q_t + (tid >> 3) * kIdxDim + 16 * (tid & 7));
    x = qv[0];
    y = qv[1];
    wh = w_t[tid >> 3];
  }
  float m = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) m = fmaxf(m, pm[u]);
  // the rest eight loads at a time (a maximum: the order does not matter)
  for (int64_t i0 = 8 * (int64_t)nthreads; i0 < n_parts; i0 += 8 * (int64_t)nthreads) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t i = i0 + tid + (int64_t)u * nthreads;
      pm[u] = i < n_parts ? parts_b[i] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) m = fmaxf(m, pm[u]);
  }
  double a = 0.0, s = 0.0;
  if (tid < 256) {
    const uint32_t wd[8] = {x.x, x.y, x.z, x.w, y.x, y.y, y.z, y.w};
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double lo = (double)bf16lo(wd[i]), hi = (double)bf16hi(wd[i]);
      ss = fma(lo, lo, ss);
      ss = fma(hi, hi, ss);
    }
    ss += dpp_f64<kDppXor1>(ss);
    ss += dpp_f64<kDppXor2>(ss);
    ss += dpp_f64<kDppHalfMirror>(ss);
    const double aw = fabs((double)wh);
    a = aw * sqrt(ss) * (1.0 + 0x1p-40);
    s = aw;
  }
  *m2 = m;
  *qf = a;
  *sw = s;
}

// eps from the block-reduced terms, rounded up to fp32.
__device__ __forceinline__ float bound_eps(float m2, double qf, double sw) {
  const double kmax = sqrt((double)m2 * (1.0 + 0x1p-10) + 0x1p-100) * (1.0 + 0x1p-40);
  const double eps = (0x1p-14 * qf * kmax + 0x1p-100 * (1.0 + sw)) * (1.0 + 0x1p-20);
  float e = (float)eps;
  if ((double)e < eps) e = __int_as_float(__float_as_int(e) + 1);  // positive and finite
  return e;
}

// fp64 score with the reference's exact operation sequence (global operands;
// used by the streaming fallback only).
template <class Keys>
__device__ double exact_score(const uint16_t* __restrict__ q, const float* __restrict__ w, const Keys& keys,
                              int64_t row) {
  double sc = 0.0;
  for (int h = 0; h < kIdxHeads; ++h) {
    double d = 0.0;
    for (int i = 0; i < 16; ++i) {
      const uint4 kp = keys.piece(row, i);
      const uint32_t kw[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d = fma(bf16_to_f64(q[h * kIdxDim + 8 * i + 2 * c]), (double)bf16lo(kw[c]), d);
        d = fma(bf16_to_f64(q[h * kIdxDim + 8 * i + 2 * c + 1]), (double)bf16hi(kw[c]), d);
      }
    }
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
  uint32_t bmin[256];
  uint32_t pick[3];
  float red[3][kFinThreads / 64];
  uint32_t cnt[kFinThreads / 64];
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
// get(i), of which at least rank are finite (the others are -inf).  Thread j's
// values are get(j), get(j + blockDim), ...; when at least rank threads hold
// a finite value, their maxima are distinct values, so the rank-th largest of
// them, L, has at least rank values >= L and T >= L; otherwise L is the
// smallest finite value.  L comes from a 256-bin histogram of the per-thread
// maxima that keeps each bin's minimum; then two levels of 256 value bins
// over [L, max], counting only values >= L, narrow T to one bin; lo and hi are
// the smallest and largest values in it.  The value histograms thus see a few
// times rank values, not n.  All threads call this.
// visit(f) calls f(v) for each of the calling thread's values.
template <typename Visit>
__device__ void bracket_visit(SelLds& s, uint32_t rank, Visit visit, float* lo, float* hi) {
  const float inf = INFINITY;
  float tmax = -inf, tmin = inf, mx = -inf;
  visit([&](float v) { tmax = fmaxf(tmax, v); tmin = fminf(tmin, v > -inf ? v : inf); });
  // one reduction: smallest finite per-thread maximum, maximum, smallest
  // finite value, threads holding a finite value
  float2 r;
  float gmin;
  uint32_t nthr;
  {
    const float a = -wave_max(-(tmax > -inf ? tmax : inf)), b = wave_max(tmax), c = -wave_max(-tmin);
    const uint32_t nt = (uint32_t)__popcll(__ballot(tmax > -inf));
    const int w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { s.red[0][w] = a; s.red[1][w] = b; s.red[2][w] = c; s.cnt[w] = nt; }
    __syncthreads();
    r = make_float2(s.red[0][0], s.red[1][0]);
    gmin = s.red[2][0];
    nthr = s.cnt[0];
    for (int i = 1; i < nw; ++i) {
      r.x = fminf(r.x, s.red[0][i]); r.y = fmaxf(r.y, s.red[1][i]); gmin = fminf(gmin, s.red[2][i]);
      nthr += s.cnt[i];
    }
  }
  mx = r.y;
  if (nthr < rank) {  // too few per-thread maxima: start from the smallest value
    if (threadIdx.x == 0) s.pick[2] = f32_key(gmin);
    __syncthreads();
  } else {
    // 1. L from the per-thread maxima
    const float a0 = r.x, s0 = r.y > r.x ? 255.99f / (r.y - r.x) : 0.f;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) { s.hist[i] = 0; s.bmin[i] = 0xFFFFFFFFu; }
    __syncthreads();
    if (tmax > -inf) {
      const uint32_t bin = value_bin(tmax, a0, s0);
      atomicAdd(&s.hist[bin], 1u);
      atomicMin(&s.bmin[bin], f32_key(tmax));
    }
    pick_digit(s.hist, rank, s.pick);
    // the smallest per-thread maximum in the chosen bin or above
    if (threadIdx.x < 64) {
      uint32_t m = 0xFFFFFFFFu;
      for (int i = threadIdx.x; i < 256; i += 64)
        if ((uint32_t)i >= s.pick[0]) m = min(m, s.bmin[i]);
      m = wave_min_u32_dpp(m);
      if (threadIdx.x == 0) s.pick[2] = m;
    }
    __syncthreads();
  }
  const float L = key_f32(s.pick[2]);
  // 2. first level over [L, max]
  const float a1 = L, s1 = mx > L ? 255.99f / (mx - L) : 0.f;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) s.hist[i] = 0;
  __syncthreads();
  visit([&](float v) { if (v >= L) atomicAdd(&s.hist[value_bin(v, a1, s1)], 1u); });
  pick_digit(s.hist, rank, s.pick);
  const uint32_t b1 = s.pick[0];
  rank = s.pick[1];
  float mn = inf;
  mx = -inf;
  visit([&](float v) {
    if (v >= L && value_bin(v, a1, s1) == b1) { mn = fminf(mn, v); mx = fmaxf(mx, v); }
  });
  r = block_minmax(s, mn, mx);
  // 3. second level within that bin
  const float a2 = r.x, s2 = r.y > r.x ? 255.99f / (r.y - r.x) : 0.f;
  for (int i = threadIdx.x; i < 256; i += blockDim.x) s.hist[i] = 0;
  __syncthreads();
  visit([&](float v) {
    if (v >= L && value_bin(v, a1, s1) == b1) atomicAdd(&s.hist[value_bin(v, a2, s2)], 1u);
  });
  pick_digit(s.hist, rank, s.pick);
  const uint32_t b2 = s.pick[0];
  mn = inf;
  mx = -inf;
  visit([&](float v) {
    if (v >= L && value_bin(v, a1, s1) == b1 && value_bin(v, a2, s2) == b2) { mn = fminf(mn, v); mx = fmaxf(mx, v); }
  });
  r = block_minmax(s, mn, mx);
  *lo = r.x;
  *hi = r.y;
}

template <typename Get>
__device__ void bracket_kth(SelLds& s, int64_t n, uint32_t rank, Get get, float* lo, float* hi) {
  bracket_visit(s, rank, [&](auto f) { for_each4(n, get, f); }, lo, hi);
}

// Inclusive prefix sum over the 64 lanes of a wave, in lane order (DPP: shifts
// by 1, 2, 4 and 8 within each row of 16 lanes, then each row's total carried
// into the rows above by the row broadcasts of lanes 15 and 31).
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Order-preserving key of the rank-th largest (1-based) of n <= MAXN values
// get(i) (finite or -inf, at least rank finite), by one wave and no block
// barrier.  Lane l holds the keys of values l, l + 64, ... in registers.  Every
// key lies between the smallest and the largest, so the high bits those two
// share are the answer's; the bits below are taken 8 at a time from the top,
// each digit by counting the keys that match the answer's bits so far in a
// 256-bin LDS histogram (`hist`, which no other wave touches meanwhile) and
// picking the digit that holds the rank-th.  All 64 lanes of the calling wave
// call this; every lane gets the key.
template <int MAXN, typename Get>
__device__ uint32_t wave_kth_key(int64_t n, uint32_t rank, Get get, uint32_t* hist) {
  static_assert(MAXN % 64 == 0, "whole registers");
  constexpr int J = MAXN / 64;
  const int lane = threadIdx.x & 63;
  const int jn = (int)((n + 63) >> 6);
  uint32_t key[J];
  uint32_t kmin = 0xFFFFFFFFu, nkmax = 0xFFFFFFFFu;  // smallest key, complement of the largest
#pragma unroll
  for (int j = 0; j < J; ++j) {
    key[j] = 0u;  // below every value's key: a slot past n never reaches the rank-th
    if (j < jn && lane + 64 * j < n) {
      key[j] = f32_key(get(lane + 64 * j));
      kmin = min(kmin, key[j]);
      nkmax = min(nkmax, ~key[j]);
    }
  }
  kmin = wave_min_u32_dpp(kmin);
  const uint32_t kmax = ~wave_min_u32_dpp(nkmax);
  if (kmin == kmax) return kmax;  // all keys equal
  int top = 31 - __clz(kmin ^ kmax);                    // highest bit that differs
  uint32_t mask = ~(uint32_t)((2ull << top) - 1ull);  // the bits above it
  uint32_t prefix = kmax & mask;
#pragma unroll 1
  while (top >= 0) {
    const int shift = top >= 7 ? top - 7 : 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) hist[lane + 64 * i] = 0u;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int j = 0; j < J; ++j)
      if (j < jn && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 255u], 1u);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    // lane owns digits 255-4*lane .. 252-4*lane (descending)
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; sum += c[i]; }
    const uint32_t incl = wave_incl_scan_u32(sum);
    uint32_t cum = incl - sum, digit = 0u, left = 0u;
    bool mine = false;
    if (cum < rank && rank <= incl) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!mine && cum + c[i] >= rank) { digit = 255u - 4u * lane - i; left = rank - cum; mine = true; }
        cum += c[i];
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;
    digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, src);
    rank = (uint32_t)__builtin_amdgcn_readlane((int)left, src);
    prefix |= (digit & 255u) << shift;
    mask |= 255u << shift;
    top = shift - 1;
  }
  return prefix;
}

// --------------------------------------------------------- finish (shared)

// LDS of the finishing block, for a band of up to BAND entries resolved in
// LDS and KROWS key rows staged per rescoring round.  The tail is only
// touched after the candidates have been classified, so the row kernels
// overlay it on their copy of the scores or their candidate list.
template <int BAND, int KROWS>
struct alignas(16) FinTailT {
  static constexpr int kKRows = KROWS;
  uint32_t out_sorted[kTopK];
  uint64_t band_key[BAND];
  uint16_t krows[KROWS][kIdxDim];
  uint16_t qrows[kIdxHeads][kIdxDim + 8];  // directly after krows (the output bitmap spans both)
  double dots[32][kIdxHeads + 1];
  float w[kIdxHeads];
};
template <int BAND>
struct alignas(16) FinLdsT {
  static constexpr int kBand = BAND;
  SelLds sel;
  uint32_t n_out, n_band;
  uint32_t out[kTopK];
  uint32_t band_idx[BAND];
};
using FinTail = FinTailT<kBandLds, 64>;
using FinLds = FinLdsT<kBandLds>;

// fp64 scores of the band (reference operation order), 32 entries per pass:
// thread (e = tid/32, h = tid%32) of an NT-thread block forms dot(q[h], K[x])
// for entries x = e, e + NT/32, ... of the pass (32 / (NT/32) independent
// chains of 128 sequential fmas from LDS), then thread x < 32 folds entry x's
// heads in order.  The query rows, the weights and the first key rows are
// requested together, and each round's key rows are requested while the
// previous round is scored.
template <int NT, class FL, class FT, class Keys>
__device__ void rescore_band(FL& sh, FT& tl, uint32_t nb, const uint16_t* __restrict__ qt,
                             const float* __restrict__ wt, const Keys& kb, int bsel) {
  constexpr int KR = FT::kKRows;                       // key rows per round
  constexpr int EP = NT / 32;                          // entries per chain round
  constexpr int C = 32 / EP;                           // chains per thread
  constexpr int QP = (kIdxHeads * 16 + NT - 1) / NT;   // 16-byte query pieces per thread
  constexpr int KP = (KR * 16 + NT - 1) / NT;          // 16-byte key pieces per thread and round
  static_assert(NT % 32 == 0 && 32 % EP == 0 && C >= 1 && KR % 32 == 0, "32 entries per pass");
  const int tid = threadIdx.x;
  const int e = tid >> 5, h = tid & 31;
  uint4 kv[KP];
  auto load_rows = [&](uint32_t base) {
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int i = tid + u * NT, r = i >> 4, c = i & 15;
      kv[u] = (i < KR * 16 && base + r < nb) ? kb.piece(sh.band_idx[base + r], c) : make_uint4(0, 0, 0, 0);
    }
  };
  load_rows(0);
  {
    uint4 qv[QP];
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int i = tid + u * NT;
      if (i < kIdxHeads * 16) qv[u] = *reinterpret_cast<const uint4*>(qt + (i >> 4) * kIdxDim + 8 * (i & 15));
    }
    const float wv = tid < kIdxHeads ? wt[tid] : 0.f;
#pragma unroll
    for (int u = 0; u < QP; ++u) {
      const int i = tid + u * NT;
      if (i < kIdxHeads * 16) *reinterpret_cast<uint4*>(&tl.qrows[i >> 4][8 * (i & 15)]) = qv[u];
    }
    if (tid < kIdxHeads) tl.w[tid] = wv;
  }
  for (uint32_t base = 0; base < nb; base += KR) {
#pragma unroll
    for (int u = 0; u < KP; ++u) {
      const int i = tid + u * NT;
      if (i < KR * 16) *reinterpret_cast<uint4*>(&tl.krows[i >> 4][8 * (i & 15)]) = kv[u];
    }
    __syncthreads();
    if (base + KR < nb) load_rows(base + KR);
    for (uint32_t half = 0; half < (uint32_t)KR && base + half < nb; half += 32) {
      double d[C];
#pragma unroll
      for (int c = 0; c < C; ++c) d[c] = 0.0;
#pragma unroll 4
      for (int i = 0; i < 16; ++i) {
        const uint4 qq = *reinterpret_cast<const uint4*>(&tl.qrows[h][8 * i]);
        const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
        for (int c = 0; c < C; ++c) {
          const uint4 kq = *reinterpret_cast<const uint4*>(&tl.krows[half + e + c * EP][8 * i]);
          const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            d[c] = fma((double)bf16lo(qw[p]), (double)bf16lo(kw[p]), d[c]);
            d[c] = fma((double)bf16hi(qw[p]), (double)bf16hi(kw[p]), d[c]);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < C; ++c)
        if (base + half + e + c * EP < nb) tl.dots[e + c * EP][h] = d[c];
      __syncthreads();
      if (tid < 32 && base + half + tid < nb) {
        double sc = 0.0;
#pragma unroll 8
        for (int hh = 0; hh < kIdxHeads; ++hh) {
          const double dd = tl.dots[tid][hh];
          sc = fma((double)tl.w[hh], dd > 0.0 ? dd : 0.0, sc);
        }
        tl.band_key[base + half + tid] = f64_key(sel_value(sc, bsel));
      }
      __syncthreads();
    }
  }
}

// Sum over each row of 16 lanes, in every lane of the row (DPP).
__device__ __forceinline__ uint32_t row_sum16_u32(uint32_t v) {
  v += dpp_u32<kDppXor1>(v);
  v += dpp_u32<kDppXor2>(v);
  v += dpp_u32<kDppHalfMirror>(v);
  v += dpp_u32<kDppMirror>(v);
  return v;
}

// Complete the selection once T^ is known and the sure entries and band are
// in sh.out / sh.band_idx (n_band <= FL::kBand): rescore and pick the band's share.
template <int NT, class FL, class FT, class Keys>
__device__ void finish_band(FL& sh, FT& tl, uint32_t kk, const uint16_t* qt, const float* wt,
                            const Keys& kb, int bsel) {
  const uint32_t nb = sh.n_band;
  rescore_band<NT>(sh, tl, nb, qt, wt, kb, bsel);
  const uint32_t r = kk - sh.n_out;
  const uint32_t base_out = sh.n_out;
  // entry i's rank in the band (key descending, then index ascending) by a
  // row of 16 lanes: lane g compares entries g, g + 16, ..., the row sums
  const int g = threadIdx.x & 15;
  for (uint32_t i0 = 0; i0 < nb; i0 += NT / 16) {
    const uint32_t i = i0 + (threadIdx.x >> 4);
    uint64_t ki = 0;
    uint32_t ii = 0, rank = 0;
    if (i < nb) {
      ki = tl.band_key[i];
      ii = sh.band_idx[i];
      for (uint32_t j = g; j < nb; j += 16) {
        const uint64_t kj = tl.band_key[j];
        rank += (kj > ki) | ((kj == ki) & (sh.band_idx[j] < ii));
      }
    }
    rank = row_sum16_u32(rank);
    if (i < nb && g == 0 && rank < r) sh.out[base_out + rank] = ii;
  }
  __syncthreads();
}

// Exact streaming fallback over the whole visible row (capacity overflow).
// Gathers sure entries, then radix-selects the band's share over the 96-bit
// composite (fp64 key, ~index), recomputing each band member's fp64 score.
template <class FL, class Keys>
__device__ void finish_streaming(FL& sh, uint32_t kk, const float* row, int64_t nv, double lo, double hi,
                                 const uint16_t* qt, const float* wt, const Keys& kb, int bsel) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.n_out = 0;
  __syncthreads();
  for (int64_t s = tid; s < nv; s += (int)blockDim.x)
    if ((double)row[s] > hi) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)s;
  __syncthreads();
  uint32_t rank = kk - sh.n_out;
  uint64_t phi = 0, mhi = 0;
  uint32_t plo = 0, mlo = 0;
  for (int pass = 0; pass < 12; ++pass) {
    for (int i = tid; i < 256; i += (int)blockDim.x) sh.sel.hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < nv; s += (int)blockDim.x) {
      const double v = (double)row[s];
      if (v < lo || v > hi) continue;
      const uint64_t key = f64_key(sel_value(exact_score(qt, wt, kb, s), bsel));
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
  for (int64_t s = tid; s < nv; s += (int)blockDim.x) {
    const double v = (double)row[s];
    if (v < lo || v > hi) continue;
    const uint64_t key = f64_key(sel_value(exact_score(qt, wt, kb, s), bsel));
    const uint32_t low = ~(uint32_t)s;
    if (key > phi || (key == phi && low >= plo)) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)s;
  }
  __syncthreads();
}

// Ascending output (indices are distinct): rank by comparison, 4 per LDS read.
template <class FL, class FT>
__device__ void write_sorted(FL& sh, FT& tl, uint32_t kk, int k, int32_t* out) {
  for (uint32_t i = kk + threadIdx.x; i < kTopK; i += (int)blockDim.x) sh.out[i] = 0xFFFFFFFFu;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < kk; i += (int)blockDim.x) {
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
  for (int i = threadIdx.x; i < k; i += (int)blockDim.x) out[i] = i < (int)kk ? (int32_t)tl.out_sorted[i] : -1;
}

// Block-wide exclusive prefix sum (all threads, blockDim.x a multiple of 64).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  __syncthreads();
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const uint32_t c = wsum[i];
    off += i < wave ? c : 0u;
    tot += c;
  }
  *total = tot;
  return off + x - v;
}

// Position of this thread's flag among the block's set flags (ascending
// thread order) and their total: one ballot per wave and one barrier.
// `wsum` (one word per wave) must not be read by a previous call any more.
__device__ __forceinline__ uint32_t block_flag_scan(bool flag, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const uint64_t b = __ballot(flag);
  const uint32_t below = (uint32_t)__popcll(b & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = (uint32_t)__popcll(b);
  __syncthreads();
  uint32_t off = 0, tot = 0;
  for (int i = 0; i < nw; ++i) {
    const uint32_t c = wsum[i];
    off += i < wave ? c : 0u;
    tot += c;
  }
  *total = tot;
  return off + below;
}

// Slot of this lane's item in an LDS array appended to through `counter`: one
// atomic add per wave for the wave's set flags (ascending lane order within
// the wave).  Every lane of the wave calls this; the result is meaningful
// only where flag is set.
__device__ __forceinline__ uint32_t wave_append(bool flag, uint32_t* counter) {
  const int lane = threadIdx.x & 63;
  const uint64_t b = __ballot(flag);
  if (b == 0ull) return 0u;
  const int leader = __ffsll((unsigned long long)b) - 1;
  uint32_t base = 0u;
  if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(b));
  base = __shfl(base, leader, 64);
  return base + (uint32_t)__popcll(b & ((1ull << lane) - 1ull));
}

// Ascending output for rows of at most kSmallMax entries: a bitmap of the
// selected indices in LDS (over the finishing tail's key and query rows, free
// by then), word popcounts prefix-summed over the block, and map(index)
// stored at the index's rank.  `wsum`: one word per wave for the block scan.
constexpr int kBitWords = (kSmallMax + 31) / 32;
template <class FL, class FT, class Map>
__device__ void write_sorted_bits(FL& sh, FT& tl, uint32_t kk, int k, int64_t nv, uint32_t* wsum,
                                  int32_t* out, Map map) {
  static_assert(offsetof(FT, qrows) == offsetof(FT, krows) + sizeof(tl.krows) &&
                    2 * kBitWords * sizeof(uint32_t) <= sizeof(tl.krows) + sizeof(tl.qrows),
                "bitmap and prefix fit the key and query rows");
  uint32_t* bits = reinterpret_cast<uint32_t*>(&tl.krows[0][0]);
  uint32_t* pre = bits + kBitWords;
  const int tid = threadIdx.x, bd = (int)blockDim.x;
  const int nw = (int)((nv + 31) / 32);
  for (int i = tid; i < nw; i += bd) bits[i] = 0u;
  __syncthreads();
  for (uint32_t i = tid; i < kk; i += bd) atomicOr(&bits[sh.out[i] >> 5], 1u << (sh.out[i] & 31u));
  __syncthreads();
  // thread j takes words j*per .. j*per + per - 1
  const int per = (nw + bd - 1) / bd;
  uint32_t c = 0;
  for (int u = 0; u < per; ++u) {
    const int w = tid * per + u;
    if (w < nw) c += (uint32_t)__popc(bits[w]);
  }
  uint32_t tot;
  uint32_t off = block_excl_scan(c, wsum, &tot);
  for (int u = 0; u < per; ++u) {
    const int w = tid * per + u;
    if (w < nw) { pre[w] = off; off += (uint32_t)__popc(bits[w]); }
  }
  __syncthreads();
  for (uint32_t i = tid; i < kk; i += bd) {
    const uint32_t v = sh.out[i];
    out[pre[v >> 5] + (uint32_t)__popc(bits[v >> 5] & ((1u << (v & 31u)) - 1u))] = map(v);
  }
  for (int i = (int)kk + tid; i < k; i += bd) out[i] = -1;
}

// Band bounds around the bracket [t_lo, t_hi] of T^ (rounded outwards in fp64).
// The k-th exact score S lies in [t_lo - eps, t_hi + eps].  Exact order: an
// entry whose fp32 score is above t_hi + 2 eps is in, below t_lo - 2 eps out.
// BF16 order: in only when its exact score rounds strictly above
// bf16(t_hi + eps) >= bf16(S), out when below the lower rounding boundary of
// bf16(t_lo - eps) <= bf16(S); everything between is ranked exactly.
__device__ __forceinline__ void band_bounds(float t_lo, float t_hi, float eps, int bsel, double* lo, double* hi) {
  if (bsel) {
    const double a = next_down((double)t_lo - (double)eps), b = next_up((double)t_hi + (double)eps);
    *lo = next_down(bf16_lower_mid(bf16_round_f64(a)) - (double)eps);
    *hi = next_up(bf16_upper_mid(bf16_round_f64(b)) + (double)eps);
  } else {
    *lo = next_down((double)t_lo - 2.0 * (double)eps);
    *hi = next_up((double)t_hi + 2.0 * (double)eps);
  }
  if (!(*lo <= (double)t_lo)) *lo = -INFINITY;   // eps not finite: everything is in the band
  if (!(*hi >= (double)t_hi)) *hi = INFINITY;
}

// ------------------------------------------------------------- row regime

// One block per query; the visible scores live in LDS (the finishing tail
// overlays them once they have been classified).
struct SmallLds {
  FinLds f;
  union {
    float v[kSmallMax];
    FinTail tail;
  } u;
  float bm[kFinThreads / 64];
  double bq[kFinThreads / 64], bs[kFinThreads / 64];
};

template <class Keys>
__global__ __launch_bounds__(kFinThreads) void topk_small_kernel(
    const float* __restrict__ scores, uint32_t* __restrict__ stats, const float* __restrict__ parts,
    int64_t n_parts, int qg, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, Keys keys,
    const int32_t* __restrict__ q_pos, int ratio, int q_per_seq, int64_t N, int k, int32_t* __restrict__ indices,
    int bsel) {
  __shared__ SmallLds L;
  FinLds& sh = L.f;
  FinTail& tl = L.u.tail;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  int32_t* out = indices + (size_t)t * k;
  const uint32_t kk = (uint32_t)k;
  const int b = t / q_per_seq;
  const uint16_t* qt = q_idx + (size_t)t * kIdxHeads * kIdxDim;
  const float* wt = w_idx + (size_t)t * kIdxHeads;
  const Keys kb = keys.seq(b, N);
  const float* row = scores + (size_t)t * N;
  if (tid == 0) { sh.n_out = 0; sh.n_band = 0; }
  if (nv > k) {
    // eight loads in flight per thread (indices past the row re-read its last score)
    for (int64_t i0 = tid; i0 < nv; i0 += 8 * kFinThreads) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + (int64_t)u * kFinThreads;
        v[u] = row[i < nv ? i : nv - 1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t i = i0 + (int64_t)u * kFinThreads;
        if (i < nv) L.u.v[i] = v[u];
      }
    }
  }
  {
    float m2;
    double qf, sw;
    bound_terms(qt, wt, group_parts(parts, t, q_per_seq, qg, n_parts), n_parts, tid, kFinThreads, &m2, &qf, &sw);
    m2 = wave_max_dpp(m2);
    qf = wave_sum_groups8_f64(qf);
    sw = wave_sum_groups8_f64(sw);
    if ((tid & 63) == 0) { L.bm[tid >> 6] = m2; L.bq[tid >> 6] = qf; L.bs[tid >> 6] = sw; }
  }
  __syncthreads();
  float eps;
  {
    float m2 = L.bm[0];
    double qf = L.bq[0], sw = L.bs[0];
    for (int i = 1; i < kFinThreads / 64; ++i) { m2 = fmaxf(m2, L.bm[i]); qf += L.bq[i]; sw += L.bs[i]; }
    eps = bound_eps(m2, qf, sw);
    if (tid == 0) stats[(size_t)t * CSA2_STATS_WORDS] = __float_as_uint(eps);
  }
  if (nv <= k) {
    for (int i = tid; i < k; i += kFinThreads) out[i] = i < nv ? i : -1;
    return;
  }
  float t_lo, t_hi;
  bracket_kth(sh.sel, nv, kk, [&](int64_t i) { return L.u.v[i]; }, &t_lo, &t_hi);
  double lo, hi;
  band_bounds(t_lo, t_hi, eps, bsel, &lo, &hi);
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
  if (fast) finish_band<kFinThreads>(sh, tl, kk, qt, wt, kb, bsel);
  else finish_streaming(sh, kk, row, nv, lo, hi, qt, wt, kb, bsel);
  write_sorted(sh, tl, kk, k, out);
}

// ------------------------------------------------ row regime, prefiltered
//
// The scan's tile maxima give a floor before any score is read: the k-th
// largest visible tile maximum is at most the k-th largest score (its k tiles
// each hold a distinct entry at or above it), so, as in the tile regime,
// every entry that can be selected has fp32 score >= thr = cand_threshold(tau,
// eps) with tau a lower bracket of that maximum.  Only tiles whose maximum
// reaches thr are read (64 bytes each), their entries that reach it are
// compacted into LDS, and the bracket of the k-th score, the band and its fp64
// rescoring run over that list.  An entry left out has an exact score below the
// k-th exact score, so the list holds every entry the full-row selection
// could pick and the result is the same.  More than kPfMax listed entries
// (planted ties) go to the exact streaming pass over the row.

#ifndef CSA2_PF_THREADS
#define CSA2_PF_THREADS 256
#endif
constexpr int kPfThreads = CSA2_PF_THREADS;                         // four blocks per CU (256)
constexpr int kPfMax = 2048;                                        // listed entries held in LDS
constexpr int kPfBand = 512;                                        // band entries resolved in LDS
constexpr int kPfTiles = (kSmallMax + kTileKeys - 1) / kTileKeys;  // tile maxima of a row
static_assert(kPfTiles <= 65536, "tile ids are listed as 16-bit values");

template <int NT>
struct PfLdsT {
  static constexpr int kPer = (kPfTiles + NT - 1) / NT;  // tile maxima per thread
  FinLdsT<kPfBand> f;
  union {
    struct {
      float v[kPfMax];
      uint32_t i[kPfMax];
      uint16_t tiles[kPfTiles];  // the tiles that reach the floor
    } c;
    FinTailT<kPfBand, 32> tail;
  } u;
  float fr[4][NT / 64];
  double dr[2][NT / 64];
  uint32_t wsum[NT / 64];
  uint32_t res;
};

// Steps 4-6 of the row selection over n listed values getv(i) (entry geti(i);
// at least k of them finite): bracket the k-th, split sure entries from the
// band, rescore the band (or stream the row when the band overflows) and
// write the ordered result.
template <int NT, class Lds, class Keys, class GetV, class GetI, class Map>
__device__ __forceinline__ void pf_finish(Lds& L, int64_t n, GetV getv, GetI geti, uint32_t kk, int k, float eps,
                                          const float* row, int64_t nv, const uint16_t* qt, const float* wt,
                                          const Keys& kb, int bsel, int32_t* out, Map map) {
  auto& sh = L.f;
  auto& tl = L.u.tail;
  float t_lo, t_hi;
  if (n <= kPfMax) {  // a list in LDS: the exact k-th by one wave
    if (threadIdx.x < 64) {
      const uint32_t key = wave_kth_key<kPfMax>(n, kk, getv, sh.sel.hist);
      if (threadIdx.x == 0) sh.sel.pick[2] = key;
    }
    __syncthreads();
    t_lo = t_hi = key_f32(sh.sel.pick[2]);
  } else {
    bracket_kth(sh.sel, n, kk, getv, &t_lo, &t_hi);
  }
  double lo, hi;
  band_bounds(t_lo, t_hi, eps, bsel, &lo, &hi);
  for (int64_t i0 = 0; i0 < n; i0 += NT) {  // every lane takes every round (wave appends)
    const int64_t i = i0 + threadIdx.x;
    const double v = i < n ? (double)getv(i) : -INFINITY;
    const bool sure = v > hi, band = !sure && v >= lo;
    const uint32_t ps = wave_append(sure, &sh.n_out);
    const uint32_t pb = wave_append(band, &sh.n_band);
    if (sure) sh.out[ps] = geti(i);
    if (band && pb < (uint32_t)kPfBand) sh.band_idx[pb] = geti(i);
  }
  __syncthreads();
  const bool fast = sh.n_band <= (uint32_t)kPfBand;
  __syncthreads();
  if (fast) finish_band<NT>(sh, tl, kk, qt, wt, kb, bsel);
  else finish_streaming(sh, kk, row, nv, lo, hi, qt, wt, kb, bsel);
  write_sorted_bits(sh, tl, kk, k, nv, L.wsum, out, map);
}

// The floor tau over PER values per thread (distinct entries' scores, -inf
// where absent; the block's finite count is above k): at least k values are
// >= tau.  When k threads hold a value their k maxima reach the smallest
// per-thread maximum l0, so the k-th largest is >= l0; otherwise it is >= the
// smallest value gmin.  Values at or above that bound enter a 256-bin
// histogram over [bound, mx] that keeps each bin's minimum; the bins at and
// above the one holding the k-th largest hold at least k values, and tau is
// the smallest of them.  hist / bmin start zeroed / all ones; all threads call
// this; `res` is one LDS word.
template <int PER>
__device__ float floor_of_values(SelLds& sel, const float (&tv)[PER], uint32_t kk, uint32_t tthr, float l0,
                                 float gmin, float mx, uint32_t* res) {
  const int tid = threadIdx.x, lane = tid & 63;
  const float lo = tthr >= kk ? l0 : gmin;
  const float scale = mx > lo ? 255.99f / (mx - lo) : 0.f;
#pragma unroll
  for (int r = 0; r < PER; ++r) {
    if (tv[r] >= lo) {
      const uint32_t bin = value_bin(tv[r], lo, scale);
      atomicAdd(&sel.hist[bin], 1u);
      atomicMin(&sel.bmin[bin], f32_key(tv[r]));
    }
  }
  __syncthreads();
  if (tid < 64) {
    // lane owns bins 255-4*lane .. 252-4*lane (descending); the bins at or
    // above the one holding the k-th largest are those whose exclusive
    // count from the top is below k
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = sel.hist[255 - 4 * lane - i]; sum += c[i]; }
    uint32_t incl = sum;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = __shfl_up(incl, o, 64);
      if (lane >= o) incl += x;
    }
    uint32_t cum = incl - sum, kmin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cum < kk) kmin = min(kmin, sel.bmin[255 - 4 * lane - i]);
      cum += c[i];
    }
    kmin = wave_min_u32_dpp(kmin);
    if (lane == 0) *res = kmin;
  }
  __syncthreads();
  return key_f32(*res);
}

template <int NT, class Keys>
__global__ __launch_bounds__(NT) void topk_rows_pf_kernel(
    const float* __restrict__ scores, const float* __restrict__ tile_max, uint32_t* __restrict__ stats,
    const float* __restrict__ parts, int64_t n_parts, int qg, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, Keys keys, const int32_t* __restrict__ q_pos, int ratio, int q_per_seq,
    int64_t N, int k, int32_t* __restrict__ indices, int bsel) {
  using Lds = PfLdsT<NT>;
  constexpr int kPer = Lds::kPer;
  __shared__ Lds L;
  auto& sh = L.f;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  int32_t* out = indices + (size_t)t * k;
  const uint32_t kk = (uint32_t)k;
  const int b = t / q_per_seq;
  const uint16_t* qt = q_idx + (size_t)t * kIdxHeads * kIdxDim;
  const float* wt = w_idx + (size_t)t * kIdxHeads;
  const Keys kb = keys.seq(b, N);
  const float* row = scores + (size_t)t * N;
  const int64_t ntv = (nv + kTileKeys - 1) / kTileKeys;
  // 1. this thread's tile maxima (tiles tid, tid + NT, ...) and the bound
  // terms, every load issued before any is used
  float tv[kPer];
  const float* tmr = tile_max + (size_t)t * tile_ld(N);
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    const int64_t j = tid + (int64_t)r * NT;
    tv[r] = j < ntv ? tmr[j] : -INFINITY;
  }
  float m2;
  double qf, sw;
  bound_terms(qt, wt, group_parts(parts, t, q_per_seq, qg, n_parts), n_parts, tid, NT, &m2, &qf, &sw);
  for (int i = tid; i < 256; i += NT) { sh.sel.hist[i] = 0u; sh.sel.bmin[i] = 0xFFFFFFFFu; }
  if (tid == 0) { sh.n_out = 0; sh.n_band = 0; }
  float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
  for (int r = 0; r < kPer; ++r) {
    lmax = fmaxf(lmax, tv[r]);
    lmin = fminf(lmin, tv[r] > -INFINITY ? tv[r] : INFINITY);
  }
  // one block reduction: bound terms, value range, smallest per-thread maximum,
  // threads holding a tile (every visible tile's maximum is finite)
  m2 = wave_max_dpp(m2);
  qf = wave_sum_groups8_f64(qf);
  sw = wave_sum_groups8_f64(sw);
  const float wmax = wave_max_dpp(lmax);
  const float wmin = wave_min_dpp(lmin);
  const float wl0 = wave_min_dpp(lmax > -INFINITY ? lmax : INFINITY);
  const uint32_t wthr = (uint32_t)__popcll(__ballot(lmax > -INFINITY));
  if (lane == 0) {
    L.fr[0][wave] = m2; L.fr[1][wave] = wmax; L.fr[2][wave] = wmin; L.fr[3][wave] = wl0;
    L.dr[0][wave] = qf; L.dr[1][wave] = sw;
    L.wsum[wave] = wthr;
  }
  __syncthreads();
  m2 = L.fr[0][0];
  float mx = L.fr[1][0], gmin = L.fr[2][0], l0 = L.fr[3][0];
  qf = L.dr[0][0];
  sw = L.dr[1][0];
  uint32_t tthr = L.wsum[0];
  for (int i = 1; i < NT / 64; ++i) {
    m2 = fmaxf(m2, L.fr[0][i]); mx = fmaxf(mx, L.fr[1][i]); gmin = fminf(gmin, L.fr[2][i]);
    l0 = fminf(l0, L.fr[3][i]);
    qf += L.dr[0][i]; sw += L.dr[1][i]; tthr += L.wsum[i];
  }
  const float eps = bound_eps(m2, qf, sw);
  if (tid == 0) stats[(size_t)t * CSA2_STATS_WORDS] = __float_as_uint(eps);
  if (nv <= k) {
    for (int i = tid; i < k; i += NT) out[i] = i < nv ? i : -1;
    return;
  }
  // 2. the floor tau from the tile maxima, which are distinct visible entries'
  // scores (all tiles are kept when there are at most k)
  double thr = -INFINITY;
  if (ntv > k) {
    const float tau = floor_of_values<kPer>(sh.sel, tv, kk, tthr, l0, gmin, mx, &L.res);
    thr = cand_threshold(tau, eps, bsel);
    if (!(thr <= (double)tau)) thr = -INFINITY;  // eps not finite: keep everything
  }
  // 3. the tiles that reach it, listed in tile order; then their entries that
  // reach it, compacted (512 tiles per round, a thread's loads issued
  // together; the list's order is immaterial: every later step ranks by value
  // and index)
  uint32_t n_t;
  {
    uint32_t ct = 0;
#pragma unroll
    for (int r = 0; r < kPer; ++r) ct += ((double)tv[r] >= thr && tid + (int64_t)r * NT < ntv) ? 1u : 0u;
    uint32_t off = block_excl_scan(ct, L.wsum, &n_t);
#pragma unroll
    for (int r = 0; r < kPer; ++r) {
      const int64_t j = tid + (int64_t)r * NT;
      if ((double)tv[r] >= thr && j < ntv) L.u.c.tiles[off++] = (uint16_t)j;
    }
    __syncthreads();
  }
  constexpr int TR = NT >= 512 ? 1 : 512 / NT;  // tiles per thread and round
  uint32_t n = 0;
  for (uint32_t p0 = 0; p0 < n_t; p0 += TR * NT) {
    float vs[TR][16];
    int64_t s0[TR];
#pragma unroll
    for (int h = 0; h < TR; ++h) {
      const uint32_t p = p0 + h * NT + tid;
      s0[h] = p < n_t ? (int64_t)L.u.c.tiles[p] * kTileKeys : -1;
      if (s0[h] >= 0) {
        const float4* q4 = reinterpret_cast<const float4*>(row + s0[h]);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float4 x = q4[u];
          vs[h][4 * u] = x.x; vs[h][4 * u + 1] = x.y; vs[h][4 * u + 2] = x.z; vs[h][4 * u + 3] = x.w;
        }
      }
    }
    uint32_t c = 0;
#pragma unroll
    for (int h = 0; h < TR; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e) c += (s0[h] >= 0 && s0[h] + e < nv && (double)vs[h][e] >= thr) ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = n + block_excl_scan(c, L.wsum, &tot);
#pragma unroll
    for (int h = 0; h < TR; ++h)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (s0[h] >= 0 && s0[h] + e < nv && (double)vs[h][e] >= thr) {
          if (pos < (uint32_t)kPfMax) { L.u.c.v[pos] = vs[h][e]; L.u.c.i[pos] = (uint32_t)(s0[h] + e); }
          ++pos;
        }
    n += tot;
  }
  __syncthreads();
  // 4-6. the full-row selection over the list, or, when it is too long to
  // hold (short rows keep every entry), over the row itself with the entries
  // below the floor counting as -inf
  const bool listed = n <= (uint32_t)kPfMax;
  pf_finish<NT>(
      L, listed ? (int64_t)n : nv,
      [&](int64_t i) {
        if (listed) return L.u.c.v[i];
        const float v = row[i];
        return (double)v >= thr ? v : -INFINITY;
      },
      [&](int64_t i) { return listed ? L.u.c.i[i] : (uint32_t)i; }, kk, k, eps, row, nv, qt, wt, kb, bsel, out,
      [](uint32_t i) { return (int32_t)i; });
}

// ------------------------------------------------------ Reindex selection

// Top-k within one Reindex query's candidate pool (report sec. 2.3.2), one
// block per query over the scan of its pool.  The pool's P fp32 scores sit in
// registers (P / kRxThreads per thread; 512 threads leave every wave 256
// VGPRs, so nothing spills) and its entry ids in LDS.  One histogram of the
// scores at or above the smallest per-thread maximum (kRxBins value bins)
// brackets the k-th largest fp32 score by the float range of its bin; the
// scores above the bracket's band are in, those in it form the band, rescored
// in fp64 from the pool rows' own bf16 values, and the selected pool positions
// are written as the entry ids they hold, ascending (the pool is ascending, so
// position order is entry order and the lower-index tie rule carries over).
// Positions past the pool's entry count are pad and never selected.
constexpr int kRxThreads = 512;
constexpr int kRxPer = CSA2_HSI_POOL / kRxThreads;
constexpr int kRxBins = 2048;  // four per thread
static_assert(CSA2_HSI_POOL % kRxThreads == 0 && CSA2_HSI_POOL <= kSmallMax, "pool positions fit the bitmap");
static_assert(kRxBins == 4 * kRxThreads, "four bins per thread");

// Band key rows read through the pool: position p is entry pool[p] of the
// query's key sequence (the positions rescored are never padding).
struct PoolKeys {
  const uint16_t* k;    // the query's key sequence
  const int32_t* pool;  // the query's pool (entry ids by position)
  __device__ __forceinline__ uint4 piece(int64_t row, int i) const {
    return *reinterpret_cast<const uint4*>(k + (size_t)pool[row] * kIdxDim + 8 * i);
  }
};

struct RxLds {
  FinLdsT<kPfBand> f;
  union {
    uint32_t cnt[kRxBins];       // the histogram
    FinTailT<kPfBand, 32> tail;  // after the band is known
  } u;
  int32_t ent[CSA2_HSI_POOL];  // the pool's entry ids
  float fr[4][kRxThreads / 64];
  double dr[2][kRxThreads / 64];
  uint32_t wsum[kRxThreads / 64], wsum2[kRxThreads / 64];
  uint32_t pick[2];
};

__device__ __forceinline__ uint32_t rx_bin(float x, float a, float scale) {
  const float f = (x - a) * scale;
  return f >= (float)(kRxBins - 1) ? (uint32_t)(kRxBins - 1) : (f > 0.f ? (uint32_t)f : 0u);
}

// The smallest float x in [a, mx] with rx_bin(x) >= b (0 < b < kRxBins), by
// all 64 lanes of a wave: rx_bin is monotone in x, 0 at a and kRxBins - 1 at
// mx, so a search over the float keys that keeps bin(lo) < b <= bin(hi) and
// tries 64 evenly spaced keys per round ends at it.  The first interval is the
// 64 floats around a + b / scale (a few floats from the answer when a >= 0),
// else the whole range.
__device__ float rx_edge(uint32_t b, float a, float scale, float mx) {
  const int lane = threadIdx.x & 63;
  const uint32_t ka = f32_key(a), km = f32_key(mx);
  const uint32_t ke = f32_key(fminf(fmaxf(a + (float)b / scale, a), mx));
  uint32_t lo = ke - ka > 32u ? ke - 32u : ka;
  uint32_t hi = km - ke > 32u ? ke + 32u : km;
  if (!(rx_bin(key_f32(lo), a, scale) < b && rx_bin(key_f32(hi), a, scale) >= b)) { lo = ka; hi = km; }
  while (hi - lo > 1u) {
    const uint32_t step = (hi - lo) / 64u + 1u;
    const uint32_t off = (uint32_t)(lane + 1) * step;
    const uint32_t c = off < hi - lo ? lo + off : hi;
    const uint64_t ge = __ballot(rx_bin(key_f32(c), a, scale) >= b);  // lane 63 (c = hi) always
    const int f = __ffsll((unsigned long long)ge) - 1;
    const uint32_t cf = (uint32_t)__builtin_amdgcn_readlane((int)c, f);
    lo = f > 0 ? (uint32_t)__builtin_amdgcn_readlane((int)c, f - 1) : lo;
    hi = cf;
  }
  return key_f32(hi);
}

// keys: the gathered pool keys ([T][P][128] bf16, row = position) or, with
// pool_qps > 0, the shared keys [B][N_all][128] read through the pool.
template <bool GATHERED>
__global__ __launch_bounds__(kRxThreads) void reindex_select_kernel(
    const float* __restrict__ scores, const float* __restrict__ parts, int64_t n_parts,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, const uint16_t* __restrict__ keys,
    int64_t N_all, int pool_qps, const int32_t* __restrict__ pool, int k, int32_t* __restrict__ indices) {
  __shared__ RxLds L;
  auto& sh = L.f;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t kk = (uint32_t)k;
  const uint16_t* qt = q_idx + (size_t)t * kIdxHeads * kIdxDim;
  const float* wt = w_idx + (size_t)t * kIdxHeads;
  const float* row = scores + (size_t)t * CSA2_HSI_POOL;
  const int32_t* pl = pool + (size_t)t * CSA2_HSI_POOL;
  using Keys = std::conditional_t<GATHERED, Bf16Keys, PoolKeys>;
  Keys kb;
  if constexpr (GATHERED) kb = Bf16Keys{keys}.seq(t, CSA2_HSI_POOL);
  else kb = PoolKeys{keys + (size_t)(t / pool_qps) * N_all * kIdxDim, L.ent};
  int32_t* out = indices + (size_t)t * k;
  // the pool's scores and entries (positions tid, tid + kRxThreads, ...; the
  // scan scored the positions past the pool -inf) and the bound terms, every
  // load issued before any is used
  float v[kRxPer];
  int32_t pe[kRxPer];
#pragma unroll
  for (int r = 0; r < kRxPer; ++r) {
    v[r] = row[tid + r * kRxThreads];
    pe[r] = pl[tid + r * kRxThreads];
  }
  float m2;
  double qf, sw;
  bound_terms(qt, wt, parts + (size_t)t * n_parts, n_parts, tid, kRxThreads, &m2, &qf, &sw);
#pragma unroll
  for (int i = 0; i < 4; ++i) L.u.cnt[tid + i * kRxThreads] = 0u;
  if (tid == 0) { sh.n_out = 0; sh.n_band = 0; }
  // entry ids to LDS (the count of entries is the visible count: the pool is a
  // prefix); the thread's largest and smallest score
  uint32_t nin = 0;
  float lmax = -INFINITY, lmin = INFINITY;
#pragma unroll
  for (int r = 0; r < kRxPer; ++r) {
    L.ent[tid + r * kRxThreads] = pe[r];
    nin += pe[r] >= 0 ? 1u : 0u;
    lmax = fmaxf(lmax, v[r]);
    lmin = fminf(lmin, v[r] > -INFINITY ? v[r] : INFINITY);
  }
  m2 = wave_max_dpp(m2);
  qf = wave_sum_groups8_f64(qf);
  sw = wave_sum_groups8_f64(sw);
  const float wmax = wave_max_dpp(lmax);
  const float wmin = wave_min_dpp(lmin);
  const float wl0 = wave_min_dpp(lmax > -INFINITY ? lmax : INFINITY);
  const uint32_t wthr = (uint32_t)__popcll(__ballot(lmax > -INFINITY));
  const uint32_t win = wave_sum_u32_dpp(nin);
  if (lane == 0) {
    L.fr[0][wave] = m2; L.fr[1][wave] = wmax; L.fr[2][wave] = wmin; L.fr[3][wave] = wl0;
    L.dr[0][wave] = qf; L.dr[1][wave] = sw;
    L.wsum[wave] = wthr | (win << 16);
  }
  __syncthreads();
  m2 = L.fr[0][0];
  float mx = L.fr[1][0], gmin = L.fr[2][0], l0 = L.fr[3][0];
  qf = L.dr[0][0];
  sw = L.dr[1][0];
  uint32_t tthr = L.wsum[0] & 0xFFFFu, cnt_in = L.wsum[0] >> 16;
  for (int i = 1; i < kRxThreads / 64; ++i) {
    m2 = fmaxf(m2, L.fr[0][i]); mx = fmaxf(mx, L.fr[1][i]); gmin = fminf(gmin, L.fr[2][i]);
    l0 = fminf(l0, L.fr[3][i]);
    qf += L.dr[0][i]; sw += L.dr[1][i]; tthr += L.wsum[i] & 0xFFFFu; cnt_in += L.wsum[i] >> 16;
  }
  const int64_t nv = cnt_in;  // pool entries (a prefix of the positions)
  const float eps = bound_eps(m2, qf, sw);
  if (nv <= k) {
    for (int i = tid; i < k; i += kRxThreads) out[i] = i < nv ? L.ent[i] : -1;
    return;
  }
  // The histogram over [lo_h, mx]: when k threads hold a score, their maxima
  // put at least k scores at or above the smallest of them, l0; else every
  // finite score counts.  Bins are monotone in the score, so the k-th largest
  // lies in the bin where the count from the top first reaches k, between the
  // smallest float of that bin and the float below the next bin's smallest.
  const float lo_h = tthr >= kk ? l0 : gmin;
  const float scale = mx > lo_h ? ((float)kRxBins - 0.01f) / (mx - lo_h) : 0.f;
  if (tid == 0) { L.pick[0] = f32_key(lo_h); L.pick[1] = f32_key(mx); }  // the whole range until a bin is picked
#pragma unroll
  for (int r = 0; r < kRxPer; ++r) {
    if (v[r] >= lo_h) atomicAdd(&L.u.cnt[rx_bin(v[r], lo_h, scale)], 1u);
  }
  __syncthreads();
  {
    // thread j owns bins kRxBins-1-4j .. kRxBins-4-4j (descending)
    uint32_t c[4], sum = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = L.u.cnt[kRxBins - 1 - 4 * tid - i]; sum += c[i]; }
    uint32_t tot;
    uint32_t cum = block_excl_scan(sum, L.wsum, &tot);
    const bool mine = cum < kk && kk <= cum + sum;
    uint32_t bin = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (mine && cum < kk && kk <= cum + c[i]) bin = kRxBins - 1 - 4 * tid - i;
      cum += c[i];
    }
    // the wave holding that bin finds its float range: [start(bin), start(bin + 1))
    const uint64_t who = __ballot(mine);
    if (who != 0ull && scale > 0.f) {
      const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)bin, __ffsll((unsigned long long)who) - 1);
      const float t_lo = b > 0u ? rx_edge(b, lo_h, scale, mx) : lo_h;
      const float t_hi = b + 1u < (uint32_t)kRxBins ? key_f32(f32_key(rx_edge(b + 1u, lo_h, scale, mx)) - 1u) : mx;
      if (lane == 0) { L.pick[0] = f32_key(t_lo); L.pick[1] = f32_key(t_hi); }
    }
  }
  __syncthreads();
  double lo, hi;
  band_bounds(key_f32(L.pick[0]), key_f32(L.pick[1]), eps, 0, &lo, &hi);
  // sure entries (above the band) and the band, placed by one block scan of
  // the packed counts (each total is at most P < 2^16).  For a float x,
  // x > hi exactly when x > hi rounded down to float, and x >= lo exactly when
  // x >= lo rounded up.
  {
    const float fhi = __double2float_rd(hi), flo = __double2float_ru(lo);
    const uint32_t nvu = (uint32_t)nv;
    uint32_t sb = 0u, bb = 0u;  // one bit per register: sure, band
#pragma unroll
    for (int r = 0; r < kRxPer; ++r) {
      const bool in = (uint32_t)(tid + r * kRxThreads) < nvu;
      sb |= (in && v[r] > fhi ? 1u : 0u) << r;
      bb |= (in && !(v[r] > fhi) && v[r] >= flo ? 1u : 0u) << r;
    }
    uint32_t tot;
    const uint32_t pos = block_excl_scan((uint32_t)__popc(sb) | ((uint32_t)__popc(bb) << 16), L.wsum2, &tot);
    uint32_t ps = pos & 0xFFFFu, pb = pos >> 16;
    while (sb != 0u) {
      const int r = __builtin_ctz(sb);
      sb &= sb - 1u;
      if (ps < kk) sh.out[ps] = tid + r * kRxThreads;  // fewer than k lie above the k-th's bin
      ++ps;
    }
    while (bb != 0u) {
      const int r = __builtin_ctz(bb);
      bb &= bb - 1u;
      if (pb < (uint32_t)kPfBand) sh.band_idx[pb] = tid + r * kRxThreads;
      ++pb;
    }
    if (tid == 0) { sh.n_out = tot & 0xFFFFu; sh.n_band = tot >> 16; }
  }
  __syncthreads();
  auto& tl = L.u.tail;
  if (sh.n_band <= (uint32_t)kPfBand) finish_band<kRxThreads>(sh, tl, kk, qt, wt, kb, 0);
  else finish_streaming(sh, kk, row, nv, lo, hi, qt, wt, kb, 0);
  write_sorted_bits(sh, tl, kk, k, nv, L.wsum, out, [&](uint32_t i) { return L.ent[i]; });
}

// ------------------------------------------------------------ tile regime

// Workspace of the tile regime, per query: one {offset, count} record per
// candidate block and `cap` candidates (fp64 score, index): `slots` fixed
// ones per block, then shared ones that blocks with more candidates reserve
// with an atomic add on stats word 2.
struct TileWs {
  uint2* table;     // [T][nblk]
  double* cscore;   // [T][cap]
  uint32_t* cidx;   // [T][cap]
};
__host__ __device__ __forceinline__ int64_t cand_blocks(int64_t N) {
  return ((N + kTileKeys - 1) / kTileKeys + kCandTiles - 1) / kCandTiles;
}
__host__ __device__ __forceinline__ size_t tile_ws_fixed(int T, int64_t N) {
  return align_up((size_t)T * (size_t)cand_blocks(N) * 8, 16);
}
__device__ __forceinline__ TileWs tile_ws(void* base, int T, int64_t N, int64_t cap) {
  TileWs w;
  w.table = (uint2*)base;
  w.cscore = (double*)((char*)base + tile_ws_fixed(T, N));
  w.cidx = (uint32_t*)(w.cscore + (size_t)T * cap);
  return w;
}

// ---- eps and the floor tau: one block per query

constexpr int kFloorThreads = 512;
constexpr int kFloorPer = 16;                           // maxima per thread, in registers
constexpr int kFloorVals = kFloorThreads * kFloorPer;  // 8192 maxima ranked per query

struct alignas(16) FloorLds {
  uint32_t hist[256];
  uint32_t bmin[256];  // order-preserving keys
  float fred[4][kFloorThreads / 64];
  double dred[2][kFloorThreads / 64];
  uint32_t ured[kFloorThreads / 64];
  uint32_t res;
};

// Query t (grid T, kFloorThreads threads): stats[t] = {eps, tau} (words 0, 1).
// tau: at least `rank` visible fp32 scores are >= tau, because it bounds from
// below the rank-th largest of a set of maxima of disjoint groups of entries
// (each maximum is a distinct visible entry -- and the maximum of a distinct
// block of 8 entries, since groups are unions of 16-entry tiles); -inf when
// fewer than `rank` of those maxima are finite or when the row has at most
// `all_below` visible entries (everything is selected then).  The top-k uses
// rank = all_below = CSA2_TOPK; the candidate pool rank = 2048 blocks and
// all_below = 16384 entries.  The maxima ranked are the tile maxima
// when the row has at most kFloorVals tiles, else the scan's group maxima (when
// there are at least kGroupsWanted of them) or the tile maxima; past kFloorVals values
// they are folded (value j is the maximum over j, j + kFloorVals, ...), and
// folding unions groups, which keeps them disjoint.
//
// Ranking: each thread holds 16 of the maxima; the smallest per-thread
// maximum L0 is already a valid lower bound when at least `rank` threads
// hold one (that many distinct maxima reach it), so only values >= L0 enter a
// histogram of 256 bins over [L0, max] that also keeps each bin's minimum.
// The bins at and above the one holding the rank-th largest hold at least
// `rank` values, and tau is the smallest of them.
__global__ __launch_bounds__(kFloorThreads) void topk_floor_kernel(
    const float* __restrict__ tile_max, uint32_t* __restrict__ stats, const float* __restrict__ gmax,
    int64_t n_groups, const float* __restrict__ parts, int64_t n_parts, int qg, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const int32_t* __restrict__ q_pos, int ratio, int q_per_seq, int64_t N,
    int rank, int64_t all_below) {
  __shared__ FloorLds F;
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < 256; i += kFloorThreads) { F.hist[i] = 0u; F.bmin[i] = 0xFFFFFFFFu; }
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t ntv = (nv + kTileKeys - 1) / kTileKeys;
  const bool use_groups = ntv > kFloorVals && n_groups >= kGroupsWanted;
  const float* src = use_groups ? gmax + (size_t)t * n_groups : tile_max + (size_t)t * tile_ld(N);
  const int64_t nsrc = nv > all_below ? (use_groups ? n_groups : ntv) : 0;
  // value j = src[j] (rows are 16-byte aligned: four per load)
  float v[kFloorPer];
#pragma unroll
  for (int m = 0; m < kFloorPer / 4; ++m) {
    const int64_t j = 4 * ((int64_t)m * kFloorThreads + tid);
    const float4 x = j < nsrc ? *reinterpret_cast<const float4*>(src + j)
                              : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    v[4 * m] = x.x;
    v[4 * m + 1] = j + 1 < nsrc ? x.y : -INFINITY;
    v[4 * m + 2] = j + 2 < nsrc ? x.z : -INFINITY;
    v[4 * m + 3] = j + 3 < nsrc ? x.w : -INFINITY;
  }
  float m2;
  double qf, sw;
  bound_terms(q_idx + (size_t)t * kIdxHeads * kIdxDim, w_idx + (size_t)t * kIdxHeads,
              group_parts(parts, t, q_per_seq, qg, n_parts), n_parts, tid, kFloorThreads, &m2, &qf, &sw);
  // folding: one level of kFloorVals values at a time, each level's loads issued together
  for (int64_t lvl = kFloorVals; lvl < nsrc; lvl += kFloorVals) {
    float4 x[kFloorPer / 4];
#pragma unroll
    for (int m = 0; m < kFloorPer / 4; ++m) {
      const int64_t j = lvl + 4 * ((int64_t)m * kFloorThreads + tid);
      x[m] = j < nsrc ? *reinterpret_cast<const float4*>(src + j)
                      : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
    }
#pragma unroll
    for (int m = 0; m < kFloorPer / 4; ++m) {
      const int64_t j = lvl + 4 * ((int64_t)m * kFloorThreads + tid);
      v[4 * m] = fmaxf(v[4 * m], x[m].x);
      v[4 * m + 1] = fmaxf(v[4 * m + 1], j + 1 < nsrc ? x[m].y : -INFINITY);
      v[4 * m + 2] = fmaxf(v[4 * m + 2], j + 2 < nsrc ? x[m].z : -INFINITY);
      v[4 * m + 3] = fmaxf(v[4 * m + 3], j + 3 < nsrc ? x[m].w : -INFINITY);
    }
  }
  float lmax = -INFINITY, lmin = INFINITY;
  uint32_t finite = 0;
#pragma unroll
  for (int m = 0; m < kFloorPer; ++m) {
    const bool f = v[m] > -INFINITY;
    lmax = fmaxf(lmax, v[m]);
    lmin = fminf(lmin, f ? v[m] : INFINITY);
    finite += f ? 1u : 0u;
  }

  // one block reduction for all: max ||K||^2, sums, value range, L0, counts
  m2 = wave_max_dpp(m2);
  qf = wave_sum_groups8_f64(qf);
  sw = wave_sum_groups8_f64(sw);
  const float wmax = wave_max_dpp(lmax);
  const float wmin = wave_min_dpp(lmin);
  const float wl0 = wave_min_dpp(lmax > -INFINITY ? lmax : INFINITY);  // smallest per-thread maximum
  const uint32_t nfin = wave_sum_u32_dpp(finite);
  const uint32_t nthr = (uint32_t)__popcll(__ballot(finite > 0));
  if (lane == 0) {
    F.fred[0][wave] = m2; F.fred[1][wave] = wmax; F.fred[2][wave] = wmin; F.fred[3][wave] = wl0;
    F.dred[0][wave] = qf; F.dred[1][wave] = sw;
    F.ured[wave] = nfin | (nthr << 16);
  }
  __syncthreads();
  m2 = F.fred[0][0]; float mx = F.fred[1][0], gmin = F.fred[2][0], l0 = F.fred[3][0];
  qf = F.dred[0][0]; sw = F.dred[1][0];
  uint32_t tfin = F.ured[0] & 0xFFFFu, tthr = F.ured[0] >> 16;
  for (int i = 1; i < kFloorThreads / 64; ++i) {
    m2 = fmaxf(m2, F.fred[0][i]); mx = fmaxf(mx, F.fred[1][i]); gmin = fminf(gmin, F.fred[2][i]);
    l0 = fminf(l0, F.fred[3][i]);
    qf += F.dred[0][i]; sw += F.dred[1][i]; tfin += F.ured[i] & 0xFFFFu; tthr += F.ured[i] >> 16;
  }
  float tau = -INFINITY;
  if (tfin >= (uint32_t)rank) {
    const float lo = tthr >= (uint32_t)rank ? l0 : gmin;
    const float scale = mx > lo ? 255.99f / (mx - lo) : 0.f;
#pragma unroll
    for (int m = 0; m < kFloorPer; ++m) {
      if (v[m] >= lo) {
        const uint32_t bin = value_bin(v[m], lo, scale);
        atomicAdd(&F.hist[bin], 1u);
        atomicMin(&F.bmin[bin], f32_key(v[m]));
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane owns bins 255-4*lane .. 252-4*lane (descending); the bins at or
      // above the one holding the rank-th largest are those whose exclusive
      // count from the top is below rank
      const uint32_t rk = (uint32_t)rank;
      uint32_t c[4], sum = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c[i] = F.hist[255 - 4 * lane - i]; sum += c[i]; }
      uint32_t incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_up(incl, o, 64);
        if (lane >= o) incl += x;
      }
      uint32_t cum = incl - sum, kmin = 0xFFFFFFFFu;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (cum < rk) kmin = min(kmin, F.bmin[255 - 4 * lane - i]);
        cum += c[i];
      }
      kmin = wave_min_u32_dpp(kmin);
      if (lane == 0) F.res = kmin;
    }
    __syncthreads();
    tau = key_f32(F.res);
  }
  if (tid == 0) {
    uint32_t* st = stats + (size_t)t * CSA2_STATS_WORDS;
    st[0] = __float_as_uint(bound_eps(m2, qf, sw));
    st[1] = __float_as_uint(tau);
  }
}

// fp64 scores of entries eidx[0..n) in the reference's operation order,
// 32 entries per round: the block stages their key rows in LDS (all loads in
// flight at once; with erow given and n <= kExactRound the rows are already
// there, row erow[e] for entry e), then entry j of the round goes to wave j % 4, slot j / 4;
// lane (half = lane / 32, h = lane % 32) forms dot(q_h, K) with 128 sequential
// fmas for slots half, half + 2, ... (up to four independent chains), and
// lane s then folds slot s's 32 heads in order.  put(e, score) receives each
// result.  All threads of the block call this.
constexpr int kExactRound = 32;
struct alignas(16) ExactLds {
  uint16_t krows[kExactRound][kIdxDim];
  double dots[kCandThreads / 64][kExactRound / (kCandThreads / 64)][kIdxHeads + 1];
};

// fp32 scores of candidate tiles ctile[0..n_tiles) (offsets from tile0) with
// the scan's arithmetic; cmask[c] gets the entries of tile c that are visible
// and reach thr.  Wave w takes tiles w, w + 4, ...; the rows of up to kMaskTiles of
// its tiles are requested before any is scored.  With kStage the rows of the
// passing entries, already in registers, are also written to X->krows for the
// fp64 rescoring: tile c's passing entries take rows rowbase[c], rowbase[c] + 1,
// ... in entry order (rows reserved with an LDS counter, n_staged, that must be
// zero on entry; rows past kExactRound are not written).
constexpr int kMaskTiles = 3;
template <bool kStage, class Keys>
__device__ __forceinline__ void cand_tile_masks(const uint16_t* __restrict__ sq, const float* __restrict__ w,
                                                const uint16_t* __restrict__ ctile, uint16_t* __restrict__ cmask,
                                                uint32_t n_tiles, int64_t tile0, const Keys& kseq,
                                                int64_t nv, double thr, ExactLds* X, uint16_t* __restrict__ rowbase,
                                                uint32_t* n_staged) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, g = lane >> 4;
  constexpr int kWaves = kCandThreads / 64;
  float wr[8];
  load_head_weights(w, g, wr);
  for (uint32_t c0 = wave; c0 < n_tiles; c0 += kMaskTiles * kWaves) {
    uint4 kv[kMaskTiles][4];
#pragma unroll
    for (int u = 0; u < kMaskTiles; ++u) {
      const uint32_t ci = c0 + u * kWaves;
      if (ci < n_tiles) {
        const int64_t s = (tile0 + ctile[ci]) * kTileKeys + col;
        kseq.slices(s < nv ? s : nv - 1, g, kv[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < kMaskTiles; ++u) {
      const uint32_t ci = c0 + u * kWaves;
      if (ci >= n_tiles) break;
      const int64_t s = (tile0 + ctile[ci]) * kTileKeys + col;
      const float sc = tile_score(sq, kv[u], wr, col, g);
      const uint32_t m16 = (uint32_t)(__ballot(s < nv && (double)sc >= thr) & 0xFFFFull);
      if (lane == 0) cmask[ci] = (uint16_t)m16;
      if (kStage) {
        uint32_t base = 0;
        if (lane == 0 && m16) base = atomicAdd(n_staged, (uint32_t)__popc(m16));
        base = (uint32_t)__shfl((int)base, 0, 64);
        if (lane == 0) rowbase[ci] = (uint16_t)(base < (uint32_t)kExactRound ? base : (uint32_t)kExactRound);
        const uint32_t row = base + (uint32_t)__popc(m16 & ((1u << col) - 1u));
        if (((m16 >> col) & 1u) && row < (uint32_t)kExactRound) {
#pragma unroll
          for (int j = 0; j < 4; ++j) *reinterpret_cast<uint4*>(&X->krows[row][32 * j + 8 * g]) = kv[u][j];
        }
      }
    }
  }
}

template <int C>
__device__ __forceinline__ void exact_dots(const uint16_t* __restrict__ sq, ExactLds& X, const uint8_t* erow,
                                           int wave, int lane) {
  const int h = lane & 31, half = lane >> 5;
  const uint16_t* qr = &sq[h * kQRowPad];
  const uint16_t* kr[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int j = 4 * (half + 2 * i) + wave;
    kr[i] = X.krows[erow ? (erow[j] & (kExactRound - 1)) : j];
  }
  double d[C];
#pragma unroll
  for (int i = 0; i < C; ++i) d[i] = 0.0;
#pragma unroll 2
  for (int c = 0; c < 16; ++c) {
    const uint4 qq = *reinterpret_cast<const uint4*>(qr + 8 * c);
    const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
#pragma unroll
    for (int i = 0; i < C; ++i) {
      const uint4 kq = *reinterpret_cast<const uint4*>(kr[i] + 8 * c);
      const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        d[i] = fma((double)bf16lo(qw[p]), (double)bf16lo(kw[p]), d[i]);
        d[i] = fma((double)bf16hi(qw[p]), (double)bf16hi(kw[p]), d[i]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < C; ++i) X.dots[wave][half + 2 * i][h] = d[i];
}

template <class Keys, class Put>
__device__ __forceinline__ void exact_entry_scores(const uint16_t* __restrict__ sq, const float* __restrict__ w,
                                                   const uint32_t* __restrict__ eidx, const uint8_t* erow,
                                                   uint32_t n, const Keys& kseq, ExactLds& X, Put put) {
  static_assert(kCandThreads == 256, "four waves, two 16-byte pieces of the round's rows per thread");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // all rows already in X.krows (erow[e]: the row of entry e): one round, no loads
  const bool staged = erow != nullptr && n <= (uint32_t)kExactRound;
  for (uint32_t r0 = 0; r0 < n; r0 += kExactRound) {
    const uint32_t m = n - r0 < (uint32_t)kExactRound ? n - r0 : (uint32_t)kExactRound;
    if (!staged) {
      // both pieces requested before either is stored (rows past the round's end re-read row 0)
      const uint32_t row0 = tid >> 4, row1 = (kCandThreads + tid) >> 4, c8 = 8 * (tid & 15);
      const uint4 v0 = kseq.piece(eidx[r0 + (row0 < m ? row0 : 0)], tid & 15);
      const uint4 v1 = kseq.piece(eidx[r0 + (row1 < m ? row1 : 0)], tid & 15);
      if (row0 < m) *reinterpret_cast<uint4*>(&X.krows[row0][c8]) = v0;
      if (row1 < m) *reinterpret_cast<uint4*>(&X.krows[row1][c8]) = v1;
      __syncthreads();
    }
    const uint8_t* rows = staged ? erow : nullptr;
    const int nslot = (int)m > wave ? ((int)m - wave + 3) / 4 : 0;  // this wave's entries this round
    const int chains = (nslot + 1) / 2;
    if (chains == 1) exact_dots<1>(sq, X, rows, wave, lane);
    else if (chains == 2) exact_dots<2>(sq, X, rows, wave, lane);
    else if (chains > 2) exact_dots<4>(sq, X, rows, wave, lane);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < nslot) {
      const double* dr = X.dots[wave][lane];
      double sc = 0.0;
#pragma unroll
      for (int hh = 0; hh < kIdxHeads; ++hh) sc = fma((double)w[hh], dr[hh] > 0.0 ? dr[hh] : 0.0, sc);
      put(r0 + 4 * lane + wave, sc);
    }
    __syncthreads();
  }
}

// fp64 scores of entries eidx[0..n) in the reference's operation order, one
// wave per two entries and no block barrier (the top-k candidates: a few per
// block): lane (e = lane / 32, h = lane % 32) forms dot(q_h, K_e) with 128
// sequential fmas, reading the key row straight from memory (the tile pass has
// just brought it on chip), then lane h == 0 folds the entry's 32 heads in order
// from hrel (this wave's 64 doubles in LDS).  put(e, score) receives each result.
template <class Keys, class Put>
__device__ __forceinline__ void exact_entry_scores_wave(const uint16_t* __restrict__ sq, const float* __restrict__ w,
                                                        const uint32_t* __restrict__ eidx, uint32_t n,
                                                        const Keys& kseq, double* hrel, Put put) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = lane & 31;
  for (uint32_t e0 = 2 * wave; e0 < n; e0 += 2 * (kCandThreads / 64)) {
    const uint32_t e = e0 + (lane >> 5);
    const int64_t kr = eidx[e < n ? e : e0];
    const uint16_t* qr = &sq[h * kQRowPad];
    double d = 0.0;
#pragma unroll 4
    for (int i = 0; i < 16; ++i) {
      const uint4 kq = kseq.piece(kr, i);
      const uint4 qq = *reinterpret_cast<const uint4*>(qr + 8 * i);
      const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
      const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d = fma((double)bf16lo(qw[c]), (double)bf16lo(kw[c]), d);
        d = fma((double)bf16hi(qw[c]), (double)bf16hi(kw[c]), d);
      }
    }
    hrel[lane] = d > 0.0 ? d : 0.0;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (h == 0 && e < n) {
      const double* hr = &hrel[lane & 32];
      double sc = 0.0;
#pragma unroll
      for (int hh = 0; hh < kIdxHeads; ++hh) sc = fma((double)w[hh], hr[hh], sc);
      put(e, sc);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
}

// LDS of a candidate block.
struct alignas(16) CandLds {
  uint16_t sq[kIdxHeads * kQRowPad];
  float w[kIdxHeads];
  uint32_t wsum[2][kCandThreads / 64];
  uint32_t base;
  uint16_t ctile[kCandTiles];   // candidate tiles (offset in the block's range), ascending
  uint16_t cmask[kCandTiles];   // entries of each candidate tile that reach the threshold
  uint32_t eidx[kCandMax];      // passing entries, ascending
  union {
    double hrel[kCandThreads / 64][64];  // per wave: ReLU(dot) of (entry, head) for the in-order head fold
    ExactLds ex;                         // score-matrix path: key rows staged per round of 32 entries
  };
};

// Candidates of tiles [x*kCandTiles, (x+1)*kCandTiles) of query t
// (grid (nblk, T), one thread per tile).  Every block writes its table record.
// With the scan's score matrix (scores non-null) the candidate tiles' fp32
// scores are read from it (the values the scan computed, 64 bytes per tile)
// instead of re-derived from the keys (4 KiB per tile).
template <class Keys>
__global__ __launch_bounds__(kCandThreads, 4) void topk_cand_kernel(
    const float* __restrict__ scores, const float* __restrict__ tile_max, uint32_t* __restrict__ stats,
    const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx, Keys keys,
    const int32_t* __restrict__ q_pos, int ratio, int q_per_seq, int64_t N, int k, void* ws, int T, int64_t cap,
    int slots, int bsel) {
  __shared__ CandLds L;
  const int t = blockIdx.y;
  const int x = blockIdx.x;
  const int tid = threadIdx.x;
  TileWs w = tile_ws(ws, T, N, cap);
  uint32_t* st = stats + (size_t)t * CSA2_STATS_WORDS;
  uint2* rec = w.table + (size_t)t * cand_blocks(N) + x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t ntv = (nv + kTileKeys - 1) / kTileKeys;
  const int64_t tile0 = (int64_t)x * kCandTiles;
  if (nv <= k || tile0 >= ntv) {
    if (tid == 0) *rec = make_uint2(0u, 0u);
    return;
  }
  // all of this block's inputs at once: its tile maxima, tau, eps, the query
  const int64_t my_tile = tile0 + tid;
  const float tm = my_tile < ntv ? tile_max[(size_t)t * tile_ld(N) + my_tile] : -INFINITY;
  const float eps = __uint_as_float(st[0]);
  const float tau = __uint_as_float(st[1]);
  stage_query(L.sq, q_idx + (size_t)t * kIdxHeads * kIdxDim, tid, kCandThreads);
  if (tid < kIdxHeads) L.w[tid] = w_idx[(size_t)t * kIdxHeads + tid];
  const double thr = cand_threshold(tau, eps, bsel);

  // 1. candidate tiles in order
  const bool cand = my_tile < ntv && (double)tm >= thr;
  uint32_t n_tiles;
  const uint32_t p = block_flag_scan(cand, L.wsum[0], &n_tiles);
  if (cand) L.ctile[p] = (uint16_t)tid;
  __syncthreads();

  // 2. fp32 scores of the candidate tiles: the scan's, from its score matrix
  // (16 lanes per tile) or re-derived with its arithmetic
  const Keys kseq = keys.seq(t / q_per_seq, N);
  if (scores) {
    const float* srow = scores + (size_t)t * N;
    const int e = tid & 15;
    for (uint32_t c0 = 0; c0 < n_tiles; c0 += kCandThreads / 16) {
      const uint32_t ci = c0 + (uint32_t)(tid >> 4);
      bool pass = false;
      if (ci < n_tiles) {
        const int64_t s = (tile0 + L.ctile[ci]) * kTileKeys + e;
        pass = s < nv && (double)srow[s] >= thr;
      }
      const uint64_t bal = __ballot(pass);
      if (e == 0 && ci < n_tiles) L.cmask[ci] = (uint16_t)((bal >> (tid & 48)) & 0xFFFFull);
    }
  } else {
    cand_tile_masks<false>(L.sq, L.w, L.ctile, L.cmask, n_tiles, tile0, kseq, nv, thr, nullptr, nullptr, nullptr);
  }
  __syncthreads();

  // 3. output slots in (tile, entry) order: thread ci expands candidate tile ci
  const uint32_t mine = (uint32_t)tid < n_tiles ? (uint32_t)__popc((uint32_t)L.cmask[tid]) : 0u;
  uint32_t n_pass;
  uint32_t q0 = block_excl_scan(mine, L.wsum[1], &n_pass);
  if (n_pass > kCandMax) {  // more than this block can hold: exact fallback for this query
    if (tid == 0) {
      atomicOr(&st[2], kOverflow);
      *rec = make_uint2(0u, 0u);
    }
    return;
  }
  if ((uint32_t)tid < n_tiles) {
    uint32_t m = L.cmask[tid];
    const int64_t e0 = (tile0 + L.ctile[tid]) * kTileKeys;
    while (m) {
      const int c = __ffs(m) - 1;
      m &= m - 1;
      L.eidx[q0++] = (uint32_t)(e0 + c);
    }
  }
  // 4. the block's fixed slots, or a reserved run of shared ones
  if (tid == 0) {
    uint32_t off = (uint32_t)x * (uint32_t)slots;
    if (n_pass > (uint32_t)slots) {
      const uint64_t first = (uint64_t)cand_blocks(N) * slots + (atomicAdd(&st[2], n_pass) & ~kOverflow);
      if (first + n_pass > (uint64_t)cap) atomicOr(&st[2], kOverflow);
      off = (uint32_t)(first < (uint64_t)cap ? first : cap);
    }
    L.base = off;
    *rec = make_uint2(off, n_pass);
  }
  __syncthreads();
  const uint32_t base = L.base;
  for (uint32_t e = tid; e < n_pass; e += kCandThreads) {
    const uint64_t pos = (uint64_t)base + e;
    if (pos < (uint64_t)cap) w.cidx[(size_t)t * cap + pos] = L.eidx[e];
  }

  // 5. fp64 scores of the passing entries, reference operation order, into the
  // slots.  After the tile pass the key rows are on chip and each wave reads its
  // entries' rows directly; with the score matrix they are not, so the rows of
  // each round of 32 entries are requested together and staged in LDS.
  double* cs = w.cscore + (size_t)t * cap;
  auto put = [&](uint32_t e, double sc) {
    if ((uint64_t)base + e < (uint64_t)cap) cs[base + e] = sel_value(sc, bsel);
  };
  if (scores) exact_entry_scores(L.sq, L.w, L.eidx, nullptr, n_pass, kseq, L.ex, put);
  else exact_entry_scores_wave(L.sq, L.w, L.eidx, n_pass, kseq, L.hrel[tid >> 6], put);
}

// LDS of a select block.
struct alignas(16) SelectLds {
  double v[kSelLds];                 // candidates' fp64 scores, index order
  uint32_t idx[kSelLds];
  uint32_t src[kSelLds];             // slot of each candidate, index order
  unsigned long long bmin[256], bmax[256];
  uint32_t hist[256];
  uint32_t wsum[2][kSelThreads / 64];
  uint32_t pick[2];
  uint32_t pick2;
  uint32_t n_bin;
  double red[2][kSelThreads / 64];
  double range[2];
  double bin_vals[64];
  double result;
  uint64_t selm[kSelLds / 64], eqm[kSelLds / 64];
  uint32_t wbase[kSelLds / 64];
  uint16_t sq[kIdxHeads * kQRowPad];   // query rows for the fallback's fp64 scores
  float w[kIdxHeads];
  uint32_t hist_pad;
};

__device__ __forceinline__ double key_f64(unsigned long long k) {
  const unsigned long long u = (k & 0x8000000000000000ull) ? (k & 0x7FFFFFFFFFFFFFFFull) : ~k;
  return __longlong_as_double((long long)u);
}

__device__ __forceinline__ uint32_t bin_f64(double v, double a, double scale) {
  const double f = (v - a) * scale;
  return f >= 255.0 ? 255u : (f > 0.0 ? (uint32_t)f : 0u);
}

// Wave 0: the bin holding the rank-th largest of hist (descending from 255)
// and the rank left inside it.
__device__ __forceinline__ void wave_pick(const uint32_t* hist, uint32_t rank, uint32_t* bin, uint32_t* left) {
  const int lane = threadIdx.x & 63;
  uint32_t c[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; sum += c[i]; }
  uint32_t incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  uint32_t cum = incl - sum, b = 0, l = 0;
  bool found = false;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!found && cum < rank && rank <= cum + c[i]) { b = 255u - 4u * lane - i; l = rank - cum; found = true; }
    cum += c[i];
  }
  const uint64_t who = __ballot(found);
  const int src = who ? __ffsll((long long)who) - 1 : 0;
  *bin = (uint32_t)__shfl((int)b, src, 64);
  *left = (uint32_t)__shfl((int)l, src, 64);
}

// The kk-th largest of L.v[0..n) (1 <= kk <= n), given their range [lo, hi]
// (NT threads; L: the LDS layout of the caller, with the members used here):
// value-binned levels (each keeps the chosen bin's min and max) narrow it to
// at most 64 members, which one wave ranks directly; a bin that stays larger
// is resolved exactly by radix passes over the 64-bit order keys.
// L.hist / L.bmin / L.bmax must be cleared on entry.
template <int NT, class Lds>
__device__ double kth_largest_f64(Lds& L, uint32_t n, uint32_t kk, double lo, double hi, uint32_t* n_gt,
                                 uint32_t* n_eq) {
  const int tid = threadIdx.x;
  uint32_t r = kk;
  uint32_t count = n;
  // Fast path: counts of 256 value bins over [lo, hi]; when the bin holding
  // the kk-th largest has at most 64 values, those are ranked directly (bin
  // membership recomputed with the same arithmetic).  Otherwise the levels
  // below narrow the range with per-bin minima and maxima.
  if (lo < hi && n > 64) {
    const double scale = 256.0 / (hi - lo);
    for (uint32_t i = tid; i < n; i += NT) atomicAdd(&L.hist[bin_f64(L.v[i], lo, scale)], 1u);
    __syncthreads();
    if (tid < 64) {
      uint32_t b, left;
      wave_pick(L.hist, r, &b, &left);
      const uint32_t cb = L.hist[b];
#pragma unroll
      for (int i = 0; i < 4; ++i) L.hist[4 * tid + i] = 0u;
      if (tid == 0) {
        L.pick[0] = cb;
        L.pick[1] = left;
        L.pick2 = b;
        L.n_bin = 0;
      }
    }
    __syncthreads();
    if (L.pick[0] <= 64) {
      const uint32_t bsel = L.pick2, cnt_b = L.pick[0], rr = L.pick[1];
      for (uint32_t i = tid; i < n; i += NT) {
        const double v = L.v[i];
        if (bin_f64(v, lo, scale) == bsel) L.bin_vals[atomicAdd(&L.n_bin, 1u)] = v;
      }
      __syncthreads();
      if (tid < (int)cnt_b) {
        const double va = L.bin_vals[tid];
        uint32_t gt = 0, ge = 0;
        for (uint32_t b = 0; b < cnt_b; ++b) {
          const double vb = L.bin_vals[b];
          gt += vb > va;
          ge += vb >= va;
        }
        if (gt < rr && rr <= ge) {  // every writer writes the same values
          L.result = va;
          L.pick[0] = kk - rr + gt;
          L.pick[1] = ge - gt;
        }
      }
      __syncthreads();
      *n_gt = L.pick[0];
      *n_eq = L.pick[1];
      return L.result;
    }
    // the histogram is clear again; bmin / bmax are untouched
  }
  for (int level = 0; level < 6 && lo < hi && count > 64; ++level) {
    const double scale = 256.0 / (hi - lo);
    for (uint32_t i = tid; i < n; i += NT) {
      const double v = L.v[i];
      if (v >= lo && v <= hi) {
        const uint32_t b = bin_f64(v, lo, scale);
        const unsigned long long key = f64_key(v);
        atomicAdd(&L.hist[b], 1u);
        atomicMin(&L.bmin[b], key);
        atomicMax(&L.bmax[b], key);
      }
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t b, left;
      wave_pick(L.hist, r, &b, &left);
      const uint32_t cb = L.hist[b];
      const unsigned long long kmin = L.bmin[b], kmax = L.bmax[b];
#pragma unroll
      for (int i = 0; i < 4; ++i) { L.hist[4 * tid + i] = 0u; L.bmin[4 * tid + i] = ~0ull; L.bmax[4 * tid + i] = 0ull; }
      if (tid == 0) {
        L.pick[0] = cb;
        L.pick[1] = left;
        L.range[0] = key_f64(kmin);
        L.range[1] = key_f64(kmax);
      }
    }
    __syncthreads();
    count = L.pick[0];
    r = L.pick[1];
    lo = L.range[0];
    hi = L.range[1];
  }
  if (!(lo < hi)) {  // every value in [lo, hi] is the answer; kk - r values lie above
    *n_gt = kk - r;
    *n_eq = count;
    return lo;
  }
  if (count <= 64) {
    if (tid == 0) L.n_bin = 0;
    __syncthreads();
    for (uint32_t i = tid; i < n; i += NT) {
      const double v = L.v[i];
      if (v >= lo && v <= hi) {
        const uint32_t p = atomicAdd(&L.n_bin, 1u);
        if (p < 64) L.bin_vals[p] = v;
      }
    }
    __syncthreads();
    if (tid < (int)count) {
      const double va = L.bin_vals[tid];
      uint32_t gt = 0, ge = 0;
      for (uint32_t b = 0; b < count; ++b) {
        const double vb = L.bin_vals[b];
        gt += vb > va;
        ge += vb >= va;
      }
      if (gt < r && r <= ge) {  // every writer writes the same values
        L.result = va;
        L.pick[0] = kk - r + gt;
        L.pick[1] = ge - gt;
      }
    }
    __syncthreads();
    *n_gt = L.pick[0];
    *n_eq = L.pick[1];
    return L.result;
  }
  unsigned long long pre = 0, mask = 0;
  for (int pass = 0; pass < 8; ++pass) {
    for (uint32_t i = tid; i < n; i += NT) {
      const double v = L.v[i];
      const unsigned long long key = f64_key(v);
      if (v >= lo && v <= hi && (key & mask) == pre)
        atomicAdd(&L.hist[(uint32_t)(key >> (56 - 8 * pass)) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t b, left;
      wave_pick(L.hist, r, &b, &left);
#pragma unroll
      for (int i = 0; i < 4; ++i) L.hist[4 * tid + i] = 0u;
      if (tid == 0) { L.pick[0] = b; L.pick[1] = left; }
    }
    __syncthreads();
    pre |= (unsigned long long)L.pick[0] << (56 - 8 * pass);
    mask |= 255ull << (56 - 8 * pass);
    r = L.pick[1];
  }
  const double V = key_f64(pre);
  uint32_t gt = 0, eq = 0;
  for (uint32_t i = tid; i < n; i += NT) {
    gt += L.v[i] > V;
    eq += L.v[i] == V;
  }
  uint32_t tgt, teq;
  block_excl_scan(gt, L.wsum[0], &tgt);
  block_excl_scan(eq, L.wsum[1], &teq);
  *n_gt = tgt;
  *n_eq = teq;
  return V;
}

// fp64 score of one key row with the reference's operation sequence, query
// and weights in LDS (fallback path).
template <class Keys>
__device__ double exact_score_lds(const uint16_t* __restrict__ sq, const float* __restrict__ w, const Keys& keys,
                                  int64_t row) {
  uint4 kr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) kr[i] = keys.piece(row, i);
  double sc = 0.0;
  for (int h = 0; h < kIdxHeads; ++h) {
    const uint16_t* qr = sq + h * kQRowPad;
    double d = 0.0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 qq = *reinterpret_cast<const uint4*>(qr + 8 * i);
      const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
      const uint32_t kw[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        d = fma((double)bf16lo(qw[c]), (double)bf16lo(kw[c]), d);
        d = fma((double)bf16hi(qw[c]), (double)bf16hi(kw[c]), d);
      }
    }
    sc = fma((double)w[h], d > 0.0 ? d : 0.0, sc);
  }
  return sc;
}

// Exact fallback of the tile regime: radix passes over the 96-bit composite
// (fp64 key, ~index) of every visible entry of the candidate tiles, fp64
// scores recomputed in each pass, then an ordered gather.
template <class Keys>
__device__ void select_streaming(SelectLds& L, uint32_t kk, const float* tm_row, int64_t nv, double thr,
                                 const uint16_t* qt, const float* wt, const Keys& kb, int32_t* out, int bsel) {
  const int tid = threadIdx.x;
  stage_query(L.sq, qt, tid, kSelThreads);
  if (tid < kIdxHeads) L.w[tid] = wt[tid];
  const int64_t ntv = (nv + kTileKeys - 1) / kTileKeys;
  uint32_t rank = kk;
  uint64_t phi = 0, mhi = 0;
  uint32_t plo = 0, mlo = 0;
  for (int pass = 0; pass < 12; ++pass) {
    for (int i = tid; i < 256; i += kSelThreads) L.hist[i] = 0;
    __syncthreads();
    for (int64_t s = tid; s < nv; s += kSelThreads) {
      if (!((double)tm_row[s / kTileKeys] >= thr)) continue;
      const uint64_t key = f64_key(sel_value(exact_score_lds(L.sq, L.w, kb, s), bsel));
      const uint32_t low = ~(uint32_t)s;
      if ((key & mhi) != phi || (low & mlo) != plo) continue;
      const uint32_t digit = pass < 8 ? (uint32_t)(key >> (56 - 8 * pass)) & 255u
                                      : (low >> (24 - 8 * (pass - 8))) & 255u;
      atomicAdd(&L.hist[digit], 1u);
    }
    pick_digit(L.hist, rank, L.pick);
    const uint32_t digit = L.pick[0];
    rank = L.pick[1];
    if (pass < 8) {
      phi |= (uint64_t)digit << (56 - 8 * pass);
      mhi |= (uint64_t)255 << (56 - 8 * pass);
    } else {
      plo |= digit << (24 - 8 * (pass - 8));
      mlo |= 255u << (24 - 8 * (pass - 8));
    }
  }
  // (phi, plo) is the kk-th largest composite: keep everything >= it, in index order
  uint32_t written = 0;
  for (int64_t s0 = 0; s0 < ntv * kTileKeys; s0 += kSelThreads) {
    const int64_t s = s0 + tid;
    bool keep = false;
    if (s < nv && (double)tm_row[s / kTileKeys] >= thr) {
      const uint64_t key = f64_key(sel_value(exact_score_lds(L.sq, L.w, kb, s), bsel));
      const uint32_t low = ~(uint32_t)s;
      keep = key > phi || (key == phi && low >= plo);
    }
    uint32_t tot;
    const uint32_t pos = written + block_excl_scan(keep ? 1u : 0u, L.wsum[0], &tot);
    if (keep && pos < kk) out[pos] = (int32_t)s;
    written += tot;
  }
}

// Final selection of query t (grid T, 256 threads): the k largest fp64 keys
// among the candidates, written ascending by index.
template <class Keys>
__global__ __launch_bounds__(kSelThreads) void topk_select_kernel(
    const float* __restrict__ tile_max, uint32_t* __restrict__ stats, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, Keys keys, const int32_t* __restrict__ q_pos,
    int ratio, int q_per_seq, int64_t N, int k, int32_t* __restrict__ indices, void* ws, int T, int64_t cap,
    int bsel) {
  __shared__ SelectLds L;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  int32_t* out = indices + (size_t)t * k;
  if (nv <= k) {
    for (int i = tid; i < k; i += kSelThreads) out[i] = i < nv ? i : -1;
    return;
  }
  const uint32_t kk = (uint32_t)k;
  TileWs w = tile_ws(ws, T, N, cap);
  uint32_t* st = stats + (size_t)t * CSA2_STATS_WORDS;
  const int64_t nblk = cand_blocks(N);
  const uint2* rec = w.table + (size_t)t * nblk;
  const uint32_t ovf = st[2] & kOverflow;
#pragma unroll
  for (int i = 0; i < 4; ++i) { L.hist[4 * (tid & 63) + i] = 0u; L.bmin[4 * (tid & 63) + i] = ~0ull; L.bmax[4 * (tid & 63) + i] = 0ull; }
  // candidates in index order: block records in block order, each in index
  // order.  Records are taken 256 at a time, one per thread; each thread
  // expands its record into source offsets (LDS), then every candidate is
  // fetched in one round of loads.  (The counter word has been read by every
  // thread once the first scan's barrier has passed; it is reset at the end.)
  uint32_t cnt = 0;
  const bool small_table = nblk <= kSelBlocks;
  for (int64_t x0 = 0; small_table && x0 < nblk; x0 += kSelThreads) {
    const int64_t xb = x0 + tid;
    const uint2 r = xb < nblk ? rec[xb] : make_uint2(0u, 0u);
    uint32_t tot;
    const uint32_t p = cnt + block_excl_scan(r.y, L.wsum[0], &tot);
    if (cnt + tot <= kSelLds)
      for (uint32_t j = 0; j < r.y; ++j) L.src[p + j] = r.x + j;
    cnt += tot;
  }
  const bool fits = ovf == 0u && small_table && cnt <= kSelLds && cnt >= kk;
  if (!fits) {
    const float tau = __uint_as_float(st[1]);
    const double thr = cand_threshold(tau, __uint_as_float(st[0]), bsel);
    select_streaming(L, kk, tile_max + (size_t)t * tile_ld(N), nv, thr, q_idx + (size_t)t * kIdxHeads * kIdxDim,
                     w_idx + (size_t)t * kIdxHeads, keys.seq(t / q_per_seq, N), out, bsel);
    if (tid == 0) st[2] = 0u;
    return;
  }
  __syncthreads();
  double lo = INFINITY, hi = -INFINITY;
  for (uint32_t i0 = 0; i0 < cnt; i0 += 4 * kSelThreads) {
    double v[4];
    uint32_t ix[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + u * kSelThreads + tid;
      v[u] = -INFINITY;
      ix[u] = 0u;
      if (i < cnt) {
        const uint32_t o = L.src[i];
        if (o < (uint64_t)cap) {  // always true for a consistent table
          v[u] = w.cscore[(size_t)t * cap + o];
          ix[u] = w.cidx[(size_t)t * cap + o];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t i = i0 + u * kSelThreads + tid;
      if (i < cnt) {
        L.v[i] = v[u];
        L.idx[i] = ix[u];
        lo = fmin(lo, v[u]);
        hi = fmax(hi, v[u]);
      }
    }
  }
  {
    const int lane = tid & 63, wv = tid >> 6;
    lo = wave_min_f64_dpp(lo);
    hi = wave_max_f64_dpp(hi);
    if (lane == 0) { L.red[0][wv] = lo; L.red[1][wv] = hi; }
    __syncthreads();
    lo = L.red[0][0];
    hi = L.red[1][0];
    for (int i = 1; i < kSelThreads / 64; ++i) { lo = fmin(lo, L.red[0][i]); hi = fmax(hi, L.red[1][i]); }
  }
  uint32_t n_gt, n_eq;
  const double V = kth_largest_f64<kSelThreads>(L, cnt, kk, lo, hi, &n_gt, &n_eq);

  // Entries above V are in; of those equal to V, the lowest indices (first in
  // order).  Selection masks per 64 consecutive candidates (word j covers
  // candidates 64 j .. 64 j + 63), then one wave turns their popcounts into
  // output positions.
  const int lane = tid & 63, wv = tid >> 6;
  const uint32_t need_eq = kk - n_gt;
  const int nwords = (int)((cnt + 63) / 64);
  for (int j0 = 0; j0 < nwords; j0 += kSelThreads / 64) {
    const int j = j0 + wv;
    const uint32_t i = 64u * j + lane;
    const double v = (j < nwords && i < cnt) ? L.v[i] : -INFINITY;
    const uint64_t gt = __ballot(v > V), eq = __ballot(v == V);
    if (lane == 0 && j < nwords) { L.selm[j] = gt; L.eqm[j] = eq; }
  }
  __syncthreads();
  if (tid < 64) {
    const int j = tid;
    uint64_t sel = j < nwords ? L.selm[j] : 0ull, eq = j < nwords ? L.eqm[j] : 0ull;
    if (need_eq >= n_eq) {
      sel |= eq;  // every tie is in
    } else {       // ties straddle the boundary: the first need_eq of them in index order
      const uint32_t c = (uint32_t)__popcll(eq);
      uint32_t incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_up(incl, o, 64);
        if (j >= o) incl += x;
      }
      uint32_t take = incl - c < need_eq ? need_eq - (incl - c) : 0u;
      while (eq && take) {
        const uint64_t low = eq & (~eq + 1ull);
        sel |= low;
        eq ^= low;
        --take;
      }
    }
    const uint32_t c = (uint32_t)__popcll(sel);
    uint32_t incl = c;
    for (int o = 1; o < 64; o <<= 1) {
      const uint32_t x = __shfl_up(incl, o, 64);
      if (j >= o) incl += x;
    }
    if (j < nwords) { L.selm[j] = sel; L.wbase[j] = incl - c; }
  }
  __syncthreads();
  for (int j0 = 0; j0 < nwords; j0 += kSelThreads / 64) {
    const int j = j0 + wv;
    if (j >= nwords) break;
    const uint64_t sel = L.selm[j];
    if ((sel >> lane) & 1ull) {
      const uint32_t pos = L.wbase[j] + (uint32_t)__popcll(sel & ((1ull << lane) - 1ull));
      if (pos < kk) out[pos] = (int32_t)L.idx[64u * j + lane];
    }
  }
  if (tid == 0) st[2] = 0u;
}

// ======================================== hierarchical sparse indexer: pool

// Report sec. 2.3.2 (and sec. 4.2.1 for the sizes): blocks of 8 entries get
// the maximum score of their visible entries; the first 2048 blocks in the
// order (fp64 block score desc, block asc) are kept and their visible entries,
// ascending, are the candidate pool.  The fp32 scores decide only which blocks
// are examined: with tau a floor (at least 2048 blocks have an fp32 maximum
// >= tau), every block that can be kept has an fp64 maximum >= tau - eps,
// reached by an entry whose fp32 score is >= tau - 2 eps.  So the fp64
// maximum over the entries that reach tau - 2 eps equals the true fp64 block
// score of every block that can be kept, and is below the 2048th block score
// for every other block: ranking blocks by it gives the exact selection.
constexpr int kHsiBlock = CSA2_HSI_BLOCK;                        // 8
constexpr int kHsiBlocks = CSA2_HSI_BLOCKS;                      // 2048
constexpr int kHsiPool = kHsiBlock * kHsiBlocks;                 // 16384
constexpr int kHsiPerCand = kCandTiles * kTileKeys / kHsiBlock;  // 512 blocks per candidate block

// Workspace of the pool, per query: {eps, tau, -, -}, one record count per
// candidate block and kHsiPerCand fixed records (block, fp64 maximum) each.
struct HsiWs {
  uint32_t* hdr;     // [T][4]
  uint32_t* count;   // [T][nblk]
  uint32_t* rblk;    // [T][nblk][kHsiPerCand]
  double* rmax;      // [T][nblk][kHsiPerCand]
};
__host__ __device__ __forceinline__ size_t hsi_ws_bytes(int T, int64_t N) {
  const size_t nb = (size_t)cand_blocks(N);
  return align_up((size_t)T * 16, 256) + align_up((size_t)T * nb * 4, 256) +
         align_up((size_t)T * nb * kHsiPerCand * 4, 256) + (size_t)T * nb * kHsiPerCand * 8;
}
__device__ __forceinline__ HsiWs hsi_ws(void* base, int T, int64_t N) {
  const size_t nb = (size_t)cand_blocks(N);
  HsiWs w;
  char* p = (char*)base;
  w.hdr = (uint32_t*)p;
  p += align_up((size_t)T * 16, 256);
  w.count = (uint32_t*)p;
  p += align_up((size_t)T * nb * 4, 256);
  w.rblk = (uint32_t*)p;
  p += align_up((size_t)T * nb * kHsiPerCand * 4, 256);
  w.rmax = (double*)p;
  return w;
}

struct alignas(16) HsiCandLds {
  uint16_t sq[kIdxHeads * kQRowPad];
  float w[kIdxHeads];
  uint32_t wsum[2][kCandThreads / 64];
  uint32_t total;
  uint16_t ctile[kCandTiles];
  uint16_t cmask[kCandTiles];
  uint32_t tpre[kCandTiles];               // passing entries before candidate tile c
  uint32_t eidx[kCandMax];                 // one round of passing entries
  uint16_t rowbase[kCandTiles];            // first staged row of each candidate tile's passing entries
  uint8_t erow[kCandMax];                  // staged row of each passing entry (first round)
  uint32_t n_staged;
  unsigned long long bkey[kHsiPerCand];    // per block: largest fp64 key so far (0: none)
  ExactLds x;
};

// Candidate blocks of tiles [x*kCandTiles, (x+1)*kCandTiles) of query t
// (grid (nblk, T)): per block of 8 entries, the fp64 maximum over the entries
// whose fp32 score reaches tau - 2 eps, written as records in block order.
// Passing entries are scored in rounds of kCandMax, so that any number of
// them (ties included) is handled.
template <class Keys>
__global__ __launch_bounds__(kCandThreads, 4) void hsi_cand_kernel(
    const float* __restrict__ tile_max, const uint16_t* __restrict__ q_idx, const float* __restrict__ w_idx,
    Keys keys, const int32_t* __restrict__ q_pos, int ratio, int q_per_seq, int64_t N, void* ws, int T) {
  __shared__ HsiCandLds L;
  const int t = blockIdx.y;
  const int x = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nblk = cand_blocks(N);
  HsiWs w = hsi_ws(ws, T, N);
  uint32_t* cnt = w.count + (size_t)t * nblk + x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t ntv = (nv + kTileKeys - 1) / kTileKeys;
  const int64_t tile0 = (int64_t)x * kCandTiles;
  if (nv <= kHsiPool || tile0 >= ntv) {
    if (tid == 0) *cnt = 0u;
    return;
  }
  const int64_t my_tile = tile0 + tid;
  const float tm = my_tile < ntv ? tile_max[(size_t)t * tile_ld(N) + my_tile] : -INFINITY;
  const float eps = __uint_as_float(w.hdr[(size_t)t * 4]);
  const float tau = __uint_as_float(w.hdr[(size_t)t * 4 + 1]);
  stage_query(L.sq, q_idx + (size_t)t * kIdxHeads * kIdxDim, tid, kCandThreads);
  if (tid < kIdxHeads) L.w[tid] = w_idx[(size_t)t * kIdxHeads + tid];
  for (int i = tid; i < kHsiPerCand; i += kCandThreads) L.bkey[i] = 0ull;
  if (tid == 0) L.n_staged = 0u;
  const double thr = next_down((double)tau - 2.0 * (double)eps);

  // candidate tiles in order, then their passing entries (fp32, the scan's arithmetic)
  const bool cand = my_tile < ntv && (double)tm >= thr;
  uint32_t n_tiles;
  const uint32_t p = block_flag_scan(cand, L.wsum[0], &n_tiles);
  if (cand) L.ctile[p] = (uint16_t)tid;
  __syncthreads();
  const Keys kseq = keys.seq(t / q_per_seq, N);
  cand_tile_masks<true>(L.sq, L.w, L.ctile, L.cmask, n_tiles, tile0, kseq, nv, thr, &L.x, L.rowbase, &L.n_staged);
  __syncthreads();
  const uint32_t mine = (uint32_t)tid < n_tiles ? (uint32_t)__popc((uint32_t)L.cmask[tid]) : 0u;
  uint32_t n_pass;
  const uint32_t pre = block_excl_scan(mine, L.wsum[1], &n_pass);
  if ((uint32_t)tid < n_tiles) L.tpre[tid] = pre;
  __syncthreads();

  // rounds of passing entries: fp64 scores in the reference order, block maxima
  const int64_t e_base = tile0 * kTileKeys;
  for (uint32_t r0 = 0; r0 < n_pass; r0 += kCandMax) {
    if ((uint32_t)tid < n_tiles) {
      uint32_t m = L.cmask[tid];
      uint32_t r = L.tpre[tid];
      uint32_t row = L.rowbase[tid];
      const int64_t e0 = (tile0 + L.ctile[tid]) * kTileKeys;
      while (m && r < r0 + kCandMax) {
        const int c = __ffs(m) - 1;
        m &= m - 1;
        if (r >= r0) {
          L.eidx[r - r0] = (uint32_t)(e0 + c);
          L.erow[r - r0] = (uint8_t)(row < (uint32_t)kExactRound ? row : 0u);
        }
        ++r;
        ++row;
      }
    }
    __syncthreads();
    const uint32_t n = n_pass - r0 < (uint32_t)kCandMax ? n_pass - r0 : (uint32_t)kCandMax;
    exact_entry_scores(L.sq, L.w, L.eidx, r0 == 0 ? L.erow : nullptr, n, kseq, L.x, [&](uint32_t e, double sc) {
      atomicMax(&L.bkey[(L.eidx[e] - (uint32_t)e_base) / kHsiBlock], (unsigned long long)f64_key(sc));
    });
    __syncthreads();
  }

  // records of the blocks that have a passing entry, in block order
  uint32_t done = 0;
  for (int i0 = 0; i0 < kHsiPerCand; i0 += kCandThreads) {
    const int i = i0 + tid;
    const unsigned long long key = L.bkey[i];
    uint32_t tot;
    const uint32_t q = done + block_flag_scan(key != 0ull, L.wsum[i0 / kCandThreads & 1], &tot);
    if (key != 0ull) {
      const size_t slot = ((size_t)t * nblk + x) * kHsiPerCand + q;
      w.rblk[slot] = (uint32_t)(e_base / kHsiBlock) + (uint32_t)i;
      w.rmax[slot] = key_f64(key);
    }
    done += tot;
  }
  if (tid == 0) *cnt = done;
}

// Order-preserving key of (fp64 block score, block index): larger is earlier
// in the order (score desc, block asc).
__device__ __forceinline__ void hsi_key(double v, uint32_t blk, unsigned long long* hi, uint32_t* lo) {
  *hi = f64_key(v);
  *lo = ~blk;
}

constexpr int kHsiSelThreads = 1024;
constexpr int kHsiSelLds = 4096;  // records ranked in LDS; more go through the global-memory passes

struct alignas(16) HsiSelLds {
  double v[kHsiSelLds];               // record block scores, ascending by block
  uint32_t blk[kHsiSelLds];           // record blocks
  uint32_t off[kHsiSelThreads];       // record offsets of a chunk of candidate blocks
  uint32_t kblk[kHsiBlocks];          // kept blocks, ascending
  unsigned long long bmin[256], bmax[256];
  uint32_t hist[256];
  uint32_t wsum[2][kHsiSelThreads / 64];
  uint32_t pick[3];
  uint32_t pick2;
  uint32_t n_bin;
  double red[2][kHsiSelThreads / 64];
  double range[2];
  double bin_vals[64];
  double result;
  uint64_t selm[kHsiSelLds / 64], eqm[kHsiSelLds / 64];
  uint32_t wbase[kHsiSelLds / 64];
  unsigned long long found_hi;
  uint32_t found_lo;
};

// The 96-bit key of the rank-th record (1-based, from the top) among n records
// read through rec(i, &hi, &lo): radix passes of 8 bits, most significant
// first, until the chosen bin holds a single record (that record is the
// answer) or all 96 bits are fixed.  Keys are distinct (block indices are).
template <class Rec>
__device__ void hsi_kth_key(HsiSelLds& L, int64_t n, uint32_t rank, Rec rec, unsigned long long* key_hi,
                            uint32_t* key_lo) {
  const int tid = threadIdx.x;
  unsigned long long pre_hi = 0, mask_hi = 0;
  uint32_t pre_lo = 0, mask_lo = 0;
  for (int pass = 0; pass < 12; ++pass) {
    for (int i = tid; i < 256; i += blockDim.x) L.hist[i] = 0u;
    __syncthreads();
    const int sh = pass < 8 ? 56 - 8 * pass : 24 - 8 * (pass - 8);
    for (int64_t i = tid; i < n; i += blockDim.x) {
      unsigned long long hi;
      uint32_t lo;
      rec(i, &hi, &lo);
      if ((hi & mask_hi) == pre_hi && (lo & mask_lo) == pre_lo)
        atomicAdd(&L.hist[pass < 8 ? (uint32_t)(hi >> sh) & 255u : (lo >> sh) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t bsel, left;
      wave_pick(L.hist, rank, &bsel, &left);
      if (tid == 0) { L.pick[0] = bsel; L.pick[1] = left; L.pick[2] = L.hist[bsel]; }
    }
    __syncthreads();
    const uint32_t d = L.pick[0];
    rank = L.pick[1];
    const bool single = L.pick[2] == 1u;
    if (pass < 8) {
      pre_hi |= (unsigned long long)d << sh;
      mask_hi |= 255ull << sh;
    } else {
      pre_lo |= d << sh;
      mask_lo |= 255u << sh;
    }
    __syncthreads();
    if (single) {
      for (int64_t i = tid; i < n; i += blockDim.x) {
        unsigned long long hi;
        uint32_t lo;
        rec(i, &hi, &lo);
        if ((hi & mask_hi) == pre_hi && (lo & mask_lo) == pre_lo) { L.found_hi = hi; L.found_lo = lo; }
      }
      __syncthreads();
      pre_hi = L.found_hi;
      pre_lo = L.found_lo;
      __syncthreads();
      break;
    }
  }
  *key_hi = pre_hi;
  *key_lo = pre_lo;
}

// Pool of query t (grid T, kHsiSelThreads threads): over the records of all
// candidate blocks, the 2048th block in the order (score desc, block asc) is
// found by radix passes over the 96-bit keys (score key, ~block); the pool is
// the visible entries of every block at or before it, ascending.  The records
// (ascending by block: candidate blocks in order, each in block order) are
// first copied to LDS when they fit.
__global__ __launch_bounds__(kHsiSelThreads) void hsi_select_kernel(const int32_t* __restrict__ q_pos, int ratio,
                                                                    int64_t N, void* ws, int T,
                                                                    int32_t* __restrict__ pool) {
  __shared__ HsiSelLds L;
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  int32_t* out = pool + (size_t)t * kHsiPool;
  if (nv <= kHsiPool) {  // every visible block is kept
    for (int i = tid; i < kHsiPool; i += kHsiSelThreads) out[i] = i < nv ? i : -1;
    return;
  }
  const int64_t nblk = cand_blocks(N);
  HsiWs w = hsi_ws(ws, T, N);
  const uint32_t* cnt = w.count + (size_t)t * nblk;
  const uint32_t* rb = w.rblk + (size_t)t * nblk * kHsiPerCand;
  const double* rv = w.rmax + (size_t)t * nblk * kHsiPerCand;

  // 1. records into LDS, chunk by chunk of candidate blocks
  uint32_t n_rec = 0;
  bool in_lds = true;
  for (int64_t x0 = 0; x0 < nblk && in_lds; x0 += kHsiSelThreads) {
    const int64_t x = x0 + tid;
    const uint32_t c = x < nblk ? cnt[x] : 0u;
    uint32_t tot;
    const uint32_t o = block_excl_scan(c, L.wsum[0], &tot);
    L.off[tid] = o;
    __syncthreads();
    if (n_rec + tot > (uint32_t)kHsiSelLds) {
      in_lds = false;
      break;
    }
    // record p of the chunk: its candidate block is the last one whose offset is <= p
    for (uint32_t p0 = 0; p0 < tot; p0 += 4 * kHsiSelThreads) {
      double v[4];
      uint32_t bk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t p = p0 + u * kHsiSelThreads + tid;
        const uint32_t pp = p < tot ? p : 0u;
        int lo = 0, hi = kHsiSelThreads - 1;  // largest xi with off[xi] <= pp (counts may be zero)
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (L.off[mid] <= pp) lo = mid; else hi = mid - 1;
        }
        const size_t r = (size_t)(x0 + lo) * kHsiPerCand + (pp - L.off[lo]);
        v[u] = rv[r];
        bk[u] = rb[r];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t p = p0 + u * kHsiSelThreads + tid;
        if (p < tot) {
          L.v[n_rec + p] = v[u];
          L.blk[n_rec + p] = bk[u];
        }
      }
    }
    n_rec += tot;
    __syncthreads();
  }

  if (in_lds) {
    // 2. the 2048th largest block score V (value bins, then a direct rank)
    double lo = INFINITY, hi = -INFINITY;
    for (uint32_t i = tid; i < n_rec; i += kHsiSelThreads) { lo = fmin(lo, L.v[i]); hi = fmax(hi, L.v[i]); }
    for (int i = tid; i < 256; i += kHsiSelThreads) { L.hist[i] = 0u; L.bmin[i] = ~0ull; L.bmax[i] = 0ull; }
    {
      const int lane = tid & 63, wv = tid >> 6;
      lo = wave_min_f64_dpp(lo);
      hi = wave_max_f64_dpp(hi);
      if (lane == 0) { L.red[0][wv] = lo; L.red[1][wv] = hi; }
      __syncthreads();
      lo = L.red[0][0];
      hi = L.red[1][0];
      for (int i = 1; i < kHsiSelThreads / 64; ++i) { lo = fmin(lo, L.red[0][i]); hi = fmax(hi, L.red[1][i]); }
    }
    uint32_t n_gt, n_eq;
    const double V = kth_largest_f64<kHsiSelThreads>(L, n_rec, kHsiBlocks, lo, hi, &n_gt, &n_eq);
    // 3. kept: scores above V, and of those equal to V the lowest blocks (first in
    // record order).  Masks per 64 records, then one wave turns them into ranks.
    const int lane = tid & 63, wv = tid >> 6;
    const uint32_t need_eq = kHsiBlocks - n_gt;
    const int nwords = (int)((n_rec + 63) / 64);
    for (int j = wv; j < nwords; j += kHsiSelThreads / 64) {
      const uint32_t i = 64u * j + lane;
      const double v = i < n_rec ? L.v[i] : -INFINITY;
      const uint64_t gt = __ballot(v > V), eq = __ballot(v == V);
      if (lane == 0) { L.selm[j] = gt; L.eqm[j] = eq; }
    }
    __syncthreads();
    if (tid < 64) {
      const int j = tid;
      uint64_t sel = j < nwords ? L.selm[j] : 0ull, eq = j < nwords ? L.eqm[j] : 0ull;
      if (need_eq >= n_eq) {
        sel |= eq;
      } else {
        const uint32_t c = (uint32_t)__popcll(eq);
        uint32_t incl = c;
        for (int o = 1; o < 64; o <<= 1) {
          const uint32_t x = __shfl_up(incl, o, 64);
          if (j >= o) incl += x;
        }
        uint32_t take = incl - c < need_eq ? need_eq - (incl - c) : 0u;
        while (eq && take) {
          const uint64_t low = eq & (~eq + 1ull);
          sel |= low;
          eq ^= low;
          --take;
        }
      }
      const uint32_t c = (uint32_t)__popcll(sel);
      uint32_t incl = c;
      for (int o = 1; o < 64; o <<= 1) {
        const uint32_t x = __shfl_up(incl, o, 64);
        if (j >= o) incl += x;
      }
      if (j < nwords) { L.selm[j] = sel; L.wbase[j] = incl - c; }
    }
    __syncthreads();
    for (int j = wv; j < nwords; j += kHsiSelThreads / 64) {
      const uint64_t sel = L.selm[j];
      if ((sel >> lane) & 1ull) {
        const uint32_t r = L.wbase[j] + (uint32_t)__popcll(sel & ((1ull << lane) - 1ull));
        if (r < (uint32_t)kHsiBlocks) L.kblk[r] = L.blk[64 * j + lane];
      }
    }
    __syncthreads();
    // 4. every kept block but the last visible one is full, so kept block r fills
    // pool slots 8r .. 8r + 7 (slots past n_vis in the last block get -1)
    for (int i = tid; i < kHsiPool; i += kHsiSelThreads) {
      const int64_t e = (int64_t)L.kblk[i / kHsiBlock] * kHsiBlock + (i % kHsiBlock);
      out[i] = e < nv ? (int32_t)e : -1;
    }
    return;
  }

  // beyond LDS: radix passes over every record slot where the candidate blocks left them
  unsigned long long piv_hi;
  uint32_t piv_lo;
  hsi_kth_key(L, nblk * kHsiPerCand, kHsiBlocks, [&](int64_t i, unsigned long long* hi, uint32_t* lo) {
    const int64_t x = i / kHsiPerCand;
    const uint32_t j = (uint32_t)(i % kHsiPerCand);
    if (j < cnt[x]) hsi_key(rv[i], rb[i], hi, lo);
    else { *hi = 0ull; *lo = 0u; }  // below every record's key: never counted
  }, &piv_hi, &piv_lo);

  // visible entries of the kept blocks (key >= pivot), ascending: per chunk of candidate
  // blocks, an ordered scan of their kept entries gives the offsets
  const auto kept = [&](unsigned long long hi, uint32_t lo) { return hi > piv_hi || (hi == piv_hi && lo >= piv_lo); };
  const auto entries = [&](uint32_t blk) {
    const int64_t e0 = (int64_t)blk * kHsiBlock;
    return (uint32_t)(nv - e0 < kHsiBlock ? nv - e0 : kHsiBlock);
  };
  uint32_t written = 0;
  for (int64_t x0 = 0; x0 < nblk; x0 += kHsiSelThreads) {
    const int64_t x = x0 + tid;
    const uint32_t c = x < nblk ? cnt[x] : 0u;
    uint32_t mine = 0;
    for (uint32_t j = 0; j < c; ++j) {
      unsigned long long hi;
      uint32_t lo;
      hsi_key(rv[x * kHsiPerCand + j], rb[x * kHsiPerCand + j], &hi, &lo);
      if (kept(hi, lo)) mine += entries(rb[x * kHsiPerCand + j]);
    }
    uint32_t tot;
    uint32_t o = written + block_excl_scan(mine, L.wsum[1], &tot);
    for (uint32_t j = 0; j < c; ++j) {
      unsigned long long hi;
      uint32_t lo;
      const uint32_t blk = rb[x * kHsiPerCand + j];
      hsi_key(rv[x * kHsiPerCand + j], blk, &hi, &lo);
      if (!kept(hi, lo)) continue;
      const uint32_t ne = entries(blk);
      for (uint32_t e = 0; e < ne; ++e)
        if (o + e < (uint32_t)kHsiPool) out[o + e] = (int32_t)(blk * kHsiBlock + e);
      o += ne;
    }
    written += tot;
  }
  for (int64_t i = (int64_t)written + tid; i < kHsiPool; i += kHsiSelThreads) out[i] = -1;
}

}  // namespace csa2

using namespace csa2;

// Candidate layout a workspace of ws_bytes provides: per-block fixed slots
// (kSlots, or 0 when it is small) and the per-query capacity; false if too small.
static bool topk_layout(size_t ws_bytes, int32_t T, int64_t N, int* slots, int64_t* cap) {
  const size_t fixed = tile_ws_fixed(T, N);
  if (ws_bytes < fixed) return false;
  const int64_t per = (int64_t)((ws_bytes - fixed) / ((size_t)T * 12));
  const int64_t fixed_slots = cand_blocks(N) * kSlots;
  int64_t c;
  if (per >= fixed_slots + kDefaultSpill) {
    *slots = kSlots;
    c = per < fixed_slots + kMaxSpill ? per : fixed_slots + kMaxSpill;
  } else {
    *slots = 0;
    c = per < kMaxSpill ? per : kMaxSpill;
  }
  *cap = c / 4 * 4;  // keeps the index array 16-byte aligned
  return true;
}

static bool topk_row_regime(const float* scores, int64_t N) { return scores != nullptr && N <= kSmallMax; }

extern "C" size_t csa2_topk_workspace_bytes(int32_t T, int64_t N, int32_t k) {
  if (T < 1 || N < 1 || k != kTopK) return 0;
  const int64_t cap = cand_blocks(N) * kSlots + kDefaultSpill;
  return tile_ws_fixed(T, N) + (size_t)T * (size_t)cap * 12;
}

extern "C" size_t csa2_topk_min_workspace_bytes(int32_t T, int64_t N, int32_t k) {
  if (T < 1 || N < 1 || k != kTopK) return 0;
  return tile_ws_fixed(T, N);
}

// What the selection reads from a scan's summary: group maxima, norm partials
// and the (bf16) indexer queries.
struct Summary {
  const float* gmax;
  int64_t n_groups;
  const float* parts;
  int64_t n_parts;  // norm partials per query group (the scan's blocks_x)
  int qg;           // queries per group
  const uint16_t* q;
};

static bool summary_bf16(const uint32_t* stats, size_t stats_bytes, const void* q_idx, int32_t T, int32_t q_per_seq,
                         int64_t N, Summary* sm) {
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p) || stats_bytes < stats_words(T, p) * sizeof(uint32_t)) return false;
  sm->gmax = (const float*)(stats + stats_groups_off(T));
  sm->n_groups = p.n_groups;
  sm->parts = (const float*)(stats + stats_parts_off(T, p.n_groups));
  sm->n_parts = p.blocks_x;
  sm->qg = p.qg;
  sm->q = (const uint16_t*)q_idx;
  return true;
}

static bool summary_mx(const uint32_t* stats, size_t stats_bytes, int32_t T, int32_t q_per_seq, int64_t N,
                       Summary* sm) {
  MxPlan p;
  if (!mx_plan(T, q_per_seq, N, &p) || stats_bytes < mx_stats_words(T, p) * sizeof(uint32_t)) return false;
  sm->gmax = (const float*)(stats + (size_t)T * CSA2_STATS_WORDS);
  sm->n_groups = p.n_groups;
  sm->parts = sm->gmax + (size_t)T * p.n_groups;
  sm->n_parts = p.blocks_x;
  sm->qg = p.qg;
  sm->q = (const uint16_t*)(stats + mx_qdeq_off(T, p));
  return true;
}

namespace csa2 {

// The Reindex selection over the scan of a batch of gathered pools (one
// one-query "sequence" of CSA2_HSI_POOL keys per query; stats is that scan's
// summary).  Used by csa2_reindex.
// keys: the gathered pool keys (pool_qps == 0) or the shared keys [B][N_all][128]
// read through the pool (pool_qps queries per key sequence).
csa2_status reindex_select_launch(const float* scores, const uint32_t* stats, size_t stats_bytes,
                                  const void* q_bf16, const float* w_idx, const uint16_t* keys, int64_t N_all,
                                  int pool_qps, const int32_t* pool, int32_t T, int32_t k, int32_t* indices,
                                  hipStream_t st) {
  Summary sm;
  if (!summary_bf16(stats, stats_bytes, q_bf16, T, 1, CSA2_HSI_POOL, &sm)) return CSA2_ERR_INVALID_ARG;
  (void)hipGetLastError();
  if (pool_qps == 0)
    hipLaunchKernelGGL(reindex_select_kernel<true>, dim3(T), dim3(kRxThreads), 0, st, scores, sm.parts, sm.n_parts,
                       sm.q, w_idx, keys, N_all, 1, pool, k, indices);
  else
    hipLaunchKernelGGL(reindex_select_kernel<false>, dim3(T), dim3(kRxThreads), 0, st, scores, sm.parts, sm.n_parts,
                       sm.q, w_idx, keys, N_all, pool_qps, pool, k, indices);
  return hipGetLastError() == hipSuccess ? CSA2_OK : CSA2_ERR_LAUNCH;
}

}  // namespace csa2

template <class Keys>
static csa2_status topk_launch(const float* scores, const float* tile_max, uint32_t* stats, const Summary& sm,
                               const float* w_idx, Keys keys, const int32_t* q_pos, int32_t ratio, int32_t T,
                               int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices, void* workspace,
                               size_t workspace_bytes, hipStream_t st, int bsel) {
  (void)hipGetLastError();
  if (topk_row_regime(scores, N)) {
    if (tile_max)
      hipLaunchKernelGGL((topk_rows_pf_kernel<kPfThreads, Keys>), dim3(T), dim3(kPfThreads), 0, st, scores, tile_max, stats,
                         sm.parts, sm.n_parts, sm.qg, sm.q, w_idx, keys, q_pos, ratio, q_per_seq, N, k, indices, bsel);
    else
      hipLaunchKernelGGL(topk_small_kernel<Keys>, dim3(T), dim3(kFinThreads), 0, st, scores, stats, sm.parts,
                         sm.n_parts, sm.qg, sm.q, w_idx, keys, q_pos, ratio, q_per_seq, N, k, indices, bsel);
    if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
    return CSA2_OK;
  }
  if (!tile_max) return CSA2_ERR_INVALID_ARG;
  if (!workspace || !aligned16(workspace) || workspace_bytes < csa2_topk_min_workspace_bytes(T, N, k))
    return CSA2_ERR_WORKSPACE;
  int slots;
  int64_t cap;
  if (!topk_layout(workspace_bytes, T, N, &slots, &cap)) return CSA2_ERR_WORKSPACE;
  const int64_t nblk = cand_blocks(N);
  hipLaunchKernelGGL(topk_floor_kernel, dim3(T), dim3(kFloorThreads), 0, st, tile_max, stats, sm.gmax, sm.n_groups,
                     sm.parts, sm.n_parts, sm.qg, sm.q, w_idx, q_pos, ratio, q_per_seq, N, kTopK, (int64_t)kTopK);
  hipLaunchKernelGGL(topk_cand_kernel<Keys>, dim3((unsigned)nblk, T), dim3(kCandThreads), 0, st, scores, tile_max,
                     stats, sm.q, w_idx, keys, q_pos, ratio, q_per_seq, N, k, workspace, T, cap, slots, bsel);
  hipLaunchKernelGGL(topk_select_kernel<Keys>, dim3(T), dim3(kSelThreads), 0, st, tile_max, stats, sm.q, w_idx, keys,
                     q_pos, ratio, q_per_seq, N, k, indices, workspace, T, cap, bsel);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}

extern "C" csa2_status csa2_topk_ex(const float* scores, const float* tile_max, uint32_t* stats,
                                    size_t stats_bytes, const void* q_idx, const float* w_idx, const void* k_idx,
                                    const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                                    int32_t k, int32_t select, int32_t* indices, void* workspace,
                                    size_t workspace_bytes, void* hip_stream) {
  if (!stats || !q_idx || !w_idx || !k_idx || !indices) return CSA2_ERR_INVALID_ARG;
  if (select != CSA2_SELECT_EXACT && select != CSA2_SELECT_BF16) return CSA2_ERR_UNSUPPORTED;
  if ((scores && !aligned16(scores)) || (tile_max && !aligned16(tile_max)) || !aligned16(stats) ||
      !aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) || !aligned16(indices) ||
      (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || ratio < 1) return CSA2_ERR_INVALID_ARG;
  if (k != kTopK || N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  Summary sm;
  if (!summary_bf16(stats, stats_bytes, q_idx, T, q_per_seq, N, &sm)) return CSA2_ERR_INVALID_ARG;
  return topk_launch(scores, tile_max, stats, sm, w_idx, Bf16Keys{(const uint16_t*)k_idx}, q_pos, ratio, T,
                     q_per_seq, N, k, indices, workspace, workspace_bytes, (hipStream_t)hip_stream,
                     select == CSA2_SELECT_BF16);
}

extern "C" csa2_status csa2_topk(const float* scores, const float* tile_max, uint32_t* stats, size_t stats_bytes,
                                 const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* q_pos,
                                 int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, int32_t k,
                                 int32_t* indices, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return csa2_topk_ex(scores, tile_max, stats, stats_bytes, q_idx, w_idx, k_idx, q_pos, ratio, T, q_per_seq, N, k,
                      CSA2_SELECT_EXACT, indices, workspace, workspace_bytes, hip_stream);
}

extern "C" csa2_status csa2_topk_mxfp4_ex(const float* scores, const float* tile_max, uint32_t* stats,
                                          size_t stats_bytes, const float* w_idx, const uint8_t* k_codes,
                                          const uint8_t* k_scales, const int32_t* q_pos, int32_t ratio, int32_t T,
                                          int32_t q_per_seq, int64_t N, int32_t k, int32_t select,
                                          int32_t* indices, void* workspace, size_t workspace_bytes,
                                          void* hip_stream) {
  if (!stats || !w_idx || !k_codes || !k_scales || !indices) return CSA2_ERR_INVALID_ARG;
  if (select != CSA2_SELECT_EXACT && select != CSA2_SELECT_BF16) return CSA2_ERR_UNSUPPORTED;
  if ((scores && !aligned16(scores)) || (tile_max && !aligned16(tile_max)) || !aligned16(stats) ||
      !aligned16(w_idx) || !aligned16(k_codes) || !aligned16(k_scales) || !aligned16(indices) ||
      (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || ratio < 1) return CSA2_ERR_INVALID_ARG;
  if (k != kTopK || N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  MxPlan p;
  if (!mx_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  Summary sm;
  if (!summary_mx(stats, stats_bytes, T, q_per_seq, N, &sm)) return CSA2_ERR_INVALID_ARG;
  return topk_launch(scores, tile_max, stats, sm, w_idx, Mx4Keys{k_codes, k_scales}, q_pos, ratio, T, q_per_seq, N,
                     k, indices, workspace, workspace_bytes, (hipStream_t)hip_stream, select == CSA2_SELECT_BF16);
}

extern "C" csa2_status csa2_topk_mxfp4(const float* scores, const float* tile_max, uint32_t* stats,
                                       size_t stats_bytes, const float* w_idx, const uint8_t* k_codes,
                                       const uint8_t* k_scales, const int32_t* q_pos, int32_t ratio, int32_t T,
                                       int32_t q_per_seq, int64_t N, int32_t k, int32_t* indices, void* workspace,
                                       size_t workspace_bytes, void* hip_stream) {
  return csa2_topk_mxfp4_ex(scores, tile_max, stats, stats_bytes, w_idx, k_codes, k_scales, q_pos, ratio, T,
                            q_per_seq, N, k, CSA2_SELECT_EXACT, indices, workspace, workspace_bytes, hip_stream);
}

extern "C" size_t csa2_hsi_pool_workspace_bytes(int32_t T, int64_t N) {
  if (T < 1 || N < 1) return 0;
  return hsi_ws_bytes(T, N);
}

template <class Keys>
static csa2_status hsi_launch(const float* tile_max, const Summary& sm, const float* w_idx, Keys keys,
                              const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N,
                              int32_t* pool, void* workspace, size_t workspace_bytes, hipStream_t st) {
  if (!workspace || !aligned16(workspace) || workspace_bytes < hsi_ws_bytes(T, N)) return CSA2_ERR_WORKSPACE;
  (void)hipGetLastError();
  uint32_t* hdr = (uint32_t*)workspace;  // HsiWs::hdr is at the start of the workspace
  hipLaunchKernelGGL(topk_floor_kernel, dim3(T), dim3(kFloorThreads), 0, st, tile_max, hdr, sm.gmax, sm.n_groups,
                     sm.parts, sm.n_parts, sm.qg, sm.q, w_idx, q_pos, ratio, q_per_seq, N, kHsiBlocks, (int64_t)kHsiPool);
  hipLaunchKernelGGL(hsi_cand_kernel<Keys>, dim3((unsigned)cand_blocks(N), T), dim3(kCandThreads), 0, st, tile_max,
                     sm.q, w_idx, keys, q_pos, ratio, q_per_seq, N, workspace, T);
  hipLaunchKernelGGL(hsi_select_kernel, dim3(T), dim3(kHsiSelThreads), 0, st, q_pos, ratio, N, workspace, T, pool);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}

extern "C" csa2_status csa2_hsi_pool(const float* tile_max, const uint32_t* stats, size_t stats_bytes,
                                     const void* q_idx, const float* w_idx, const void* k_idx, const int32_t* q_pos,
                                     int32_t ratio, int32_t T, int32_t q_per_seq, int64_t N, int32_t* pool,
                                     void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!tile_max || !stats || !q_idx || !w_idx || !k_idx || !pool) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(tile_max) || !aligned16(stats) || !aligned16(q_idx) || !aligned16(w_idx) || !aligned16(k_idx) ||
      !aligned16(pool) || (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || ratio < 1) return CSA2_ERR_INVALID_ARG;
  if (N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  IndexPlan p;
  if (!index_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  Summary sm;
  if (!summary_bf16(stats, stats_bytes, q_idx, T, q_per_seq, N, &sm)) return CSA2_ERR_INVALID_ARG;
  return hsi_launch(tile_max, sm, w_idx, Bf16Keys{(const uint16_t*)k_idx}, q_pos, ratio, T, q_per_seq, N, pool,
                    workspace, workspace_bytes, (hipStream_t)hip_stream);
}

extern "C" csa2_status csa2_hsi_pool_mxfp4(const float* tile_max, const uint32_t* stats, size_t stats_bytes,
                                           const float* w_idx, const uint8_t* k_codes, const uint8_t* k_scales,
                                           const int32_t* q_pos, int32_t ratio, int32_t T, int32_t q_per_seq,
                                           int64_t N, int32_t* pool, void* workspace, size_t workspace_bytes,
                                           void* hip_stream) {
  if (!tile_max || !stats || !w_idx || !k_codes || !k_scales || !pool) return CSA2_ERR_INVALID_ARG;
  if (!aligned16(tile_max) || !aligned16(stats) || !aligned16(w_idx) || !aligned16(k_codes) || !aligned16(k_scales) ||
      !aligned16(pool) || (q_pos && !aligned16(q_pos)))
    return CSA2_ERR_INVALID_ARG;
  if (T < 1 || q_per_seq < 1 || T % q_per_seq != 0 || N < 1 || ratio < 1) return CSA2_ERR_INVALID_ARG;
  if (N >= ((int64_t)1 << 31) || T > 65535) return CSA2_ERR_UNSUPPORTED;
  MxPlan p;
  if (!mx_plan(T, q_per_seq, N, &p)) return CSA2_ERR_UNSUPPORTED;
  Summary sm;
  if (!summary_mx(stats, stats_bytes, T, q_per_seq, N, &sm)) return CSA2_ERR_INVALID_ARG;
  return hsi_launch(tile_max, sm, w_idx, Mx4Keys{k_codes, k_scales}, q_pos, ratio, T, q_per_seq, N, pool, workspace,
                    workspace_bytes, (hipStream_t)hip_stream);
}
