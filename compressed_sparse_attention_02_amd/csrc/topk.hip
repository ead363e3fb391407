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
// So: a threshold bin is found with two radix-histogram passes (11 + 11 key
// bits) over the fp32 scores, every entry at or above (bin floor - 2 eps) is
// compacted into a short candidate list, and one workgroup per query finds T^
// exactly among the candidates, accepts the sure entries, rescores the band
// [T^ - 2 eps, T^ + 2 eps] in fp64 with the reference's exact operation
// sequence (fma per channel in order, then fma per head in order), and picks
// the rest of the set by (fp64 score, index).  If the candidates or the band
// do not fit the workspace / LDS, the same workgroup falls back to streaming
// passes over all scores (slow, exact).
#include "csa2_common.h"

namespace csa2 {

constexpr int kBins = 2048;                       // 11-bit radix digits
constexpr int kHdrWords = 2 * kBins + 64;         // hist1, hist2, counters
constexpr size_t kHdrBytes = kHdrWords * sizeof(uint32_t);
constexpr int kHistThreads = 256;
constexpr int kHistChunk = 8192;                  // entries per histogram block
constexpr int kFinThreads = 1024;
constexpr int kBandLds = 2048;                    // band entries handled in LDS
constexpr int kDefaultCap = 2048;                 // default candidate capacity per query

struct TopkWs {
  uint32_t* hdr;   // [T][kHdrWords]
  uint32_t* cidx;  // [T][cap]
  float* cval;     // [T][cap]
  int64_t cap;
};

__device__ __forceinline__ TopkWs topk_ws(void* base, int T, int64_t cap) {
  TopkWs w;
  w.hdr = (uint32_t*)base;
  w.cidx = w.hdr + (size_t)T * kHdrWords;
  w.cval = (float*)(w.cidx + (size_t)T * cap);
  w.cap = cap;
  return w;
}

// Block-wide: find the digit bin holding the rank-th largest element (rank is
// 1-based) of a descending-order histogram hist[kBins] (global memory).
// Returns bin and the count of elements in higher bins through LDS.
// Must be called by all kHistThreads (or a multiple of 256) threads.
__device__ void find_bin(const uint32_t* __restrict__ hist, uint32_t rank, uint32_t* s_sum,
                         uint32_t* s_out) {
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const int per = kBins / nthr;  // bins per thread, descending
  uint32_t local = 0;
  for (int j = 0; j < per; ++j) local += hist[kBins - 1 - (tid * per + j)];
  s_sum[tid] = local;
  __syncthreads();
  // inclusive scan (Hillis-Steele) over threads in descending-bin order
  for (int off = 1; off < nthr; off <<= 1) {
    uint32_t v = tid >= off ? s_sum[tid - off] : 0;
    __syncthreads();
    s_sum[tid] += v;
    __syncthreads();
  }
  const uint32_t incl = s_sum[tid];
  const uint32_t excl = incl - local;
  if (excl < rank && rank <= incl) {
    uint32_t cum = excl;
    for (int j = 0; j < per; ++j) {
      const int bin = kBins - 1 - (tid * per + j);
      const uint32_t c = hist[bin];
      if (cum + c >= rank) {
        s_out[0] = (uint32_t)bin;
        s_out[1] = cum;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void topk_init_kernel(uint32_t* __restrict__ hdr, size_t words) {
  size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const size_t stride = (size_t)gridDim.x * blockDim.x * 4;
  for (; i < words; i += stride) *reinterpret_cast<uint4*>(hdr + i) = make_uint4(0, 0, 0, 0);
}

// Pass 1: histogram of key bits [31:21] over the visible entries.
__global__ __launch_bounds__(kHistThreads) void topk_hist1_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ q_pos, int ratio,
                                                                  int64_t N, int k, void* ws, int T, int64_t cap) {
  const int t = blockIdx.y;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t s0 = (int64_t)blockIdx.x * kHistChunk;
  if (nv <= k || s0 >= nv) return;
  TopkWs w = topk_ws(ws, T, cap);
  __shared__ uint32_t h[kBins];
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) h[i] = 0;
  __syncthreads();
  const int64_t s1 = s0 + kHistChunk < nv ? s0 + kHistChunk : nv;
  const float* row = scores + (size_t)t * N;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += kHistThreads) atomicAdd(&h[f32_key(row[s]) >> 21], 1u);
  __syncthreads();
  uint32_t* g = w.hdr + (size_t)t * kHdrWords;
  for (int i = threadIdx.x; i < kBins; i += kHistThreads)
    if (h[i]) atomicAdd(&g[i], h[i]);
}

// Pass 2: histogram of key bits [20:10] over entries in the pass-1 bin.
__global__ __launch_bounds__(kHistThreads) void topk_hist2_kernel(const float* __restrict__ scores,
                                                                  const int32_t* __restrict__ q_pos, int ratio,
                                                                  int64_t N, int k, void* ws, int T, int64_t cap) {
  const int t = blockIdx.y;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t s0 = (int64_t)blockIdx.x * kHistChunk;
  if (nv <= k || s0 >= nv) return;
  TopkWs w = topk_ws(ws, T, cap);
  uint32_t* g = w.hdr + (size_t)t * kHdrWords;
  __shared__ uint32_t s_sum[kHistThreads];
  __shared__ uint32_t s_out[2];
  __shared__ uint32_t h[kBins];
  find_bin(g, (uint32_t)k, s_sum, s_out);
  const uint32_t b1 = s_out[0];
  for (int i = threadIdx.x; i < kBins; i += kHistThreads) h[i] = 0;
  __syncthreads();
  const int64_t s1 = s0 + kHistChunk < nv ? s0 + kHistChunk : nv;
  const float* row = scores + (size_t)t * N;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += kHistThreads) {
    const uint32_t key = f32_key(row[s]);
    if ((key >> 21) == b1) atomicAdd(&h[(key >> 10) & (kBins - 1)], 1u);
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kBins; i += kHistThreads)
    if (h[i]) atomicAdd(&g[kBins + i], h[i]);
}

// One ulp towards -inf / +inf (identity on infinities and NaN).
__device__ __forceinline__ double next_down(double x) {
  if (!(x > -INFINITY && x < INFINITY)) return x;
  if (x == 0.0) return -0x1p-1074;
  const long long u = __double_as_longlong(x);
  return __longlong_as_double(x > 0.0 ? u - 1 : u + 1);
}
__device__ __forceinline__ double next_up(double x) { return -next_down(-x); }

// Lower threshold: floor of the 22-bit bin holding the k-th key, minus 2 eps,
// rounded down in fp64 so that no entry at the exact boundary is missed.
__device__ __forceinline__ double cand_threshold(uint32_t b1, uint32_t b2, float eps) {
  const float tau = key_f32((b1 << 21) | (b2 << 10));
  return next_down((double)tau - 2.0 * (double)eps);
}

// Pass 3: compact every entry with score >= threshold into the candidate list.
__global__ __launch_bounds__(kHistThreads) void topk_compact_kernel(const float* __restrict__ scores,
                                                                    const float* __restrict__ err_bound,
                                                                    const int32_t* __restrict__ q_pos, int ratio,
                                                                    int64_t N, int k, void* ws, int T, int64_t cap) {
  const int t = blockIdx.y;
  const int64_t nv = n_visible(q_pos, t, ratio, N);
  const int64_t s0 = (int64_t)blockIdx.x * kHistChunk;
  if (nv <= k || s0 >= nv) return;
  TopkWs w = topk_ws(ws, T, cap);
  uint32_t* g = w.hdr + (size_t)t * kHdrWords;
  __shared__ uint32_t s_sum[kHistThreads];
  __shared__ uint32_t s_out[2];
  find_bin(g, (uint32_t)k, s_sum, s_out);
  const uint32_t b1 = s_out[0], above1 = s_out[1];
  __syncthreads();
  find_bin(g + kBins, (uint32_t)k - above1, s_sum, s_out);
  const uint32_t b2 = s_out[0];
  const double thr = cand_threshold(b1, b2, err_bound[t]);
  const int64_t s1 = s0 + kHistChunk < nv ? s0 + kHistChunk : nv;
  const float* row = scores + (size_t)t * N;
  uint32_t* cnt = g + 2 * kBins;
  for (int64_t s = s0 + threadIdx.x; s < s1; s += kHistThreads) {
    const float v = row[s];
    if ((double)v >= thr) {
      const uint32_t pos = atomicAdd(cnt, 1u);
      if (pos < (uint64_t)cap) {
        w.cidx[(size_t)t * cap + pos] = (uint32_t)s;
        w.cval[(size_t)t * cap + pos] = v;
      }
    }
  }
}

// fp64 score with the reference's exact operation sequence.
__device__ double exact_dot(const uint16_t* __restrict__ q, const uint16_t* __restrict__ key) {
  double d = 0.0;
  for (int c = 0; c < kIdxDim; ++c) d = fma(bf16_to_f64(q[c]), bf16_to_f64(key[c]), d);
  return d;
}
__device__ double exact_score(const uint16_t* __restrict__ q, const float* __restrict__ w,
                              const uint16_t* __restrict__ key) {
  double sc = 0.0;
  for (int h = 0; h < kIdxHeads; ++h) {
    const double d = exact_dot(q + h * kIdxDim, key);
    sc = fma((double)w[h], d > 0.0 ? d : 0.0, sc);
  }
  return sc;
}

constexpr int kBinLds = 1024;   // candidates of the threshold's 22-bit bin handled in LDS

struct FinShared {
  uint32_t hist[256];
  uint32_t s_sum[kFinThreads];
  uint32_t s_bin[2];
  uint32_t out[kTopK];
  uint32_t out_sorted[kTopK];
  uint32_t band_idx[kBandLds];
  uint64_t band_key[kBandLds];
  float binv[kBinLds];
  uint16_t krows[32][kIdxDim];
  uint16_t qrows[kIdxHeads][kIdxDim + 8];
  double dots[32][kIdxHeads + 1];
  uint32_t n_out, n_band, n_bin, sel_digit, sel_rank;
  float that;
};

// Radix step over 8-bit digits, descending: given hist[256] of the elements
// matching the current prefix and the 1-based rank among them, pick the digit
// (thread 0) and the rank within that digit.  Used by the streaming path only.
__device__ __forceinline__ void radix_pick(FinShared& sh) {
  if (threadIdx.x == 0) {
    uint32_t rank = sh.sel_rank, cum = 0;
    int d = 255;
    for (; d > 0; --d) {
      if (cum + sh.hist[d] >= rank) break;
      cum += sh.hist[d];
    }
    sh.sel_digit = (uint32_t)d;
    sh.sel_rank = rank - cum;
  }
  __syncthreads();
}

// Find the kk-th largest fp32 key among values produced by `get(i)` for i < n
// (with 4 passes of 8-bit digits).  All threads participate.
template <typename Get>
__device__ uint32_t select_f32_key(FinShared& sh, int64_t n, uint32_t kk, Get get) {
  uint32_t prefix = 0, mask = 0;
  if (threadIdx.x == 0) sh.sel_rank = kk;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = threadIdx.x; i < 256; i += blockDim.x) sh.hist[i] = 0;
    __syncthreads();
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) {
      const uint32_t key = f32_key(get(i));
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    radix_pick(sh);
    prefix |= sh.sel_digit << shift;
    mask |= 255u << shift;
  }
  return prefix;
}

// fp64 scores of 32 band entries per round (reference operation order): thread
// (e = tid/32, h = tid%32) forms dot(q[h], K[e]) with 128 sequential fmas from
// LDS, then 32 threads fold the heads in order.
__device__ void rescore_band(FinShared& sh, uint32_t nb, const uint16_t* __restrict__ qt,
                             const float* __restrict__ wt, const uint16_t* __restrict__ kb) {
  const int tid = threadIdx.x;
  const int e = tid >> 5, h = tid & 31;
  for (int i = tid; i < kIdxHeads * 16; i += kFinThreads) {
    const int r = i >> 4, c = i & 15;
    *reinterpret_cast<uint4*>(&sh.qrows[r][8 * c]) = *reinterpret_cast<const uint4*>(qt + r * kIdxDim + 8 * c);
  }
  for (uint32_t base = 0; base < nb; base += 32) {
    // stage up to 32 key rows (32 x 256 B): 512 chunks of 16 B
    for (int i = tid; i < 32 * 16; i += kFinThreads) {
      const int r = i >> 4, c = i & 15;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (base + r < nb) v = *reinterpret_cast<const uint4*>(kb + (size_t)sh.band_idx[base + r] * kIdxDim + 8 * c);
      *reinterpret_cast<uint4*>(&sh.krows[r][8 * c]) = v;
    }
    __syncthreads();
    if (base + e < nb) {
      double d = 0.0;
#pragma unroll 2
      for (int i = 0; i < 16; ++i) {
        const uint4 kq = *reinterpret_cast<const uint4*>(&sh.krows[e][8 * i]);
        const uint4 qq = *reinterpret_cast<const uint4*>(&sh.qrows[h][8 * i]);
        const uint32_t qw[4] = {qq.x, qq.y, qq.z, qq.w};
        const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w};
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          d = fma((double)bf16lo(qw[p]), (double)bf16lo(kw[p]), d);
          d = fma((double)bf16hi(qw[p]), (double)bf16hi(kw[p]), d);
        }
      }
      sh.dots[e][h] = d;
    }
    __syncthreads();
    if (tid < 32 && base + tid < nb) {
      double sc = 0.0;
      for (int hh = 0; hh < kIdxHeads; ++hh) {
        const double d = sh.dots[tid][hh];
        sc = fma((double)wt[hh], d > 0.0 ? d : 0.0, sc);
      }
      sh.band_key[base + tid] = f64_key(sc);
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kFinThreads) void topk_finish_kernel(
    const float* __restrict__ scores, const float* __restrict__ err_bound, const uint16_t* __restrict__ q_idx,
    const float* __restrict__ w_idx, const uint16_t* __restrict__ k_idx, const int32_t* __restrict__ q_pos,
    int ratio, int q_per_seq, int64_t N, int k, int32_t* __restrict__ indices, void* ws, int T, int64_t cap) {
  __shared__ FinShared sh;
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
  TopkWs w = topk_ws(ws, T, cap);
  const uint32_t* hdr = w.hdr + (size_t)t * kHdrWords;
  const uint32_t cnt = hdr[2 * kBins];
  const uint32_t* cidx = w.cidx + (size_t)t * cap;
  const float* cval = w.cval + (size_t)t * cap;
  const float eps = err_bound[t];
  if (tid == 0) { sh.n_out = 0; sh.n_band = 0; sh.n_bin = 0; }
  __syncthreads();

  bool fast = (int64_t)cnt <= cap;
  if (fast) {
    // T^ lies in the 22-bit bin (b1, b2) found by the histogram passes; its rank
    // inside that bin is what the two passes leave over.
    find_bin(hdr, kk, sh.s_sum, sh.s_bin);
    const uint32_t b1 = sh.s_bin[0], above1 = sh.s_bin[1];
    __syncthreads();
    find_bin(hdr + kBins, kk - above1, sh.s_sum, sh.s_bin);
    const uint32_t b2 = sh.s_bin[0], above2 = sh.s_bin[1];
    const uint32_t r3 = kk - above1 - above2;   // 1-based rank inside the bin
    const uint32_t prefix = (b1 << 11) | b2;
    for (uint32_t i = tid; i < cnt; i += kFinThreads) {
      const float v = cval[i];
      if ((f32_key(v) >> 10) == prefix) {
        const uint32_t p = atomicAdd(&sh.n_bin, 1u);
        if (p < kBinLds) sh.binv[p] = v;
      }
    }
    __syncthreads();
    const uint32_t nbin = sh.n_bin;
    if (nbin <= kBinLds) {
      for (uint32_t i = tid; i < nbin; i += kFinThreads) {
        const float v = sh.binv[i];
        uint32_t above = 0, tie_before = 0;
        for (uint32_t j = 0; j < nbin; ++j) {
          const float u = sh.binv[j];
          above += u > v;
          tie_before += (u == v) & (j < i);
        }
        if (above + tie_before == r3 - 1) sh.that = v;
      }
      __syncthreads();
    } else {
      const uint32_t key = select_f32_key(sh, (int64_t)cnt, kk, [&](int64_t i) { return cval[i]; });
      if (tid == 0) sh.that = key_f32(key);
      __syncthreads();
    }
  } else {
    const uint32_t key = select_f32_key(sh, nv, kk, [&](int64_t i) { return row[i]; });
    if (tid == 0) sh.that = key_f32(key);
    __syncthreads();
  }
  const double that = (double)sh.that;
  double lo = next_down(that - 2.0 * (double)eps), hi = next_up(that + 2.0 * (double)eps);
  if (!(lo <= that)) lo = -INFINITY;   // eps not finite: everything is in the band
  if (!(hi >= that)) hi = INFINITY;

  if (fast) {
    for (uint32_t i = tid; i < cnt; i += kFinThreads) {
      const double v = (double)cval[i];
      if (v > hi) sh.out[atomicAdd(&sh.n_out, 1u)] = cidx[i];
      else if (v >= lo) {
        const uint32_t p = atomicAdd(&sh.n_band, 1u);
        if (p < kBandLds) sh.band_idx[p] = cidx[i];
      }
    }
    __syncthreads();
    fast = sh.n_band <= kBandLds;
    __syncthreads();
    if (!fast) {
      if (tid == 0) { sh.n_out = 0; sh.n_band = 0; }
      __syncthreads();
    }
  }

  if (fast) {
    const uint32_t nb = sh.n_band;
    rescore_band(sh, nb, qt, wt, kb);
    // the r best band entries by (fp64 score desc, index asc): rank-based, all keys distinct
    const uint32_t r = kk - sh.n_out;
    const uint32_t base_out = sh.n_out;
    for (uint32_t i = tid; i < nb; i += kFinThreads) {
      const uint64_t ki = sh.band_key[i];
      const uint32_t ii = sh.band_idx[i];
      uint32_t rank = 0;
      for (uint32_t j = 0; j < nb; ++j) {
        const uint64_t kj = sh.band_key[j];
        rank += (kj > ki) | ((kj == ki) & (sh.band_idx[j] < ii));
      }
      if (rank < r) sh.out[base_out + rank] = ii;
    }
    __syncthreads();
  } else {
    // Streaming path: candidates or band exceed capacity.  Sure entries are
    // gathered by a pass over all scores; the band's share is selected with a
    // radix select over the 96-bit composite (fp64 key, ~index), recomputing
    // the fp64 score of each band member in every pass.
    for (int64_t s = tid; s < nv; s += kFinThreads)
      if ((double)row[s] > hi) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)s;
    __syncthreads();
    const uint32_t r = kk - sh.n_out;
    uint64_t phi = 0, mhi = 0;
    uint32_t plo = 0, mlo = 0;
    if (tid == 0) sh.sel_rank = r;
    for (int pass = 0; pass < 12; ++pass) {
      for (int i = tid; i < 256; i += kFinThreads) sh.hist[i] = 0;
      __syncthreads();
      for (int64_t s = tid; s < nv; s += kFinThreads) {
        const double v = (double)row[s];
        if (v < lo || v > hi) continue;
        const uint64_t key = f64_key(exact_score(qt, wt, kb + (size_t)s * kIdxDim));
        const uint32_t low = ~(uint32_t)s;
        if ((key & mhi) != phi || (low & mlo) != plo) continue;
        const uint32_t digit = pass < 8 ? (uint32_t)(key >> (56 - 8 * pass)) & 255u
                                        : (low >> (24 - 8 * (pass - 8))) & 255u;
        atomicAdd(&sh.hist[digit], 1u);
      }
      __syncthreads();
      radix_pick(sh);
      if (pass < 8) {
        phi |= (uint64_t)sh.sel_digit << (56 - 8 * pass);
        mhi |= (uint64_t)255 << (56 - 8 * pass);
      } else {
        plo |= sh.sel_digit << (24 - 8 * (pass - 8));
        mlo |= 255u << (24 - 8 * (pass - 8));
      }
    }
    // members with composite >= (phi, plo): exactly r of them
    for (int64_t s = tid; s < nv; s += kFinThreads) {
      const double v = (double)row[s];
      if (v < lo || v > hi) continue;
      const uint64_t key = f64_key(exact_score(qt, wt, kb + (size_t)s * kIdxDim));
      const uint32_t low = ~(uint32_t)s;
      if (key > phi || (key == phi && low >= plo)) sh.out[atomicAdd(&sh.n_out, 1u)] = (uint32_t)s;
    }
    __syncthreads();
  }

  // ascending output by rank (indices are distinct)
  for (uint32_t i = tid; i < kk; i += kFinThreads) {
    const uint32_t v = sh.out[i];
    uint32_t pos = 0;
    for (uint32_t j = 0; j < kk; ++j) pos += sh.out[j] < v;
    sh.out_sorted[pos] = v;
  }
  __syncthreads();
  for (int i = tid; i < k; i += kFinThreads) out[i] = i < (int)kk ? (int32_t)sh.out_sorted[i] : -1;
}

}  // namespace csa2

using namespace csa2;

static int64_t topk_cap_for(size_t ws_bytes, int32_t T, int64_t N) {
  const size_t per = ws_bytes / (size_t)T;
  if (per < kHdrBytes) return -1;
  int64_t cap = (int64_t)((per - kHdrBytes) / 8);
  cap = cap / 4 * 4;  // keep the float array 16-byte aligned
  if (cap > N) cap = (N + 3) / 4 * 4;
  return cap;
}

extern "C" size_t csa2_topk_workspace_bytes(int32_t T, int64_t N, int32_t k) {
  if (T < 1 || N < 1 || k != kTopK) return 0;
  int64_t cap = N < kDefaultCap ? (N + 3) / 4 * 4 : kDefaultCap;
  return (size_t)T * (kHdrBytes + (size_t)cap * 8);
}

extern "C" size_t csa2_topk_min_workspace_bytes(int32_t T, int64_t N, int32_t k) {
  if (T < 1 || N < 1 || k != kTopK) return 0;
  return (size_t)T * kHdrBytes;
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
  if (!workspace || !aligned16(workspace) || workspace_bytes < csa2_topk_min_workspace_bytes(T, N, k))
    return CSA2_ERR_WORKSPACE;
  const int64_t cap = topk_cap_for(workspace_bytes, T, N);
  if (cap < 0) return CSA2_ERR_WORKSPACE;
  hipStream_t st = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  const size_t words = (size_t)T * kHdrWords;
  int init_blocks = (int)((words / 4 + 255) / 256);
  if (init_blocks > 4096) init_blocks = 4096;
  hipLaunchKernelGGL(topk_init_kernel, dim3(init_blocks), dim3(256), 0, st, (uint32_t*)workspace, words);
  const int64_t chunks = (N + kHistChunk - 1) / kHistChunk;
  dim3 grid((unsigned)chunks, (unsigned)T);
  hipLaunchKernelGGL(topk_hist1_kernel, grid, dim3(kHistThreads), 0, st, scores, q_pos, ratio, N, k, workspace, T,
                     cap);
  hipLaunchKernelGGL(topk_hist2_kernel, grid, dim3(kHistThreads), 0, st, scores, q_pos, ratio, N, k, workspace, T,
                     cap);
  hipLaunchKernelGGL(topk_compact_kernel, grid, dim3(kHistThreads), 0, st, scores, err_bound, q_pos, ratio, N, k,
                     workspace, T, cap);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(T), dim3(kFinThreads), 0, st, scores, err_bound,
                     (const uint16_t*)q_idx, w_idx, (const uint16_t*)k_idx, q_pos, ratio, q_per_seq, N, k, indices,
                     workspace, T, cap);
  if (hipGetLastError() != hipSuccess) return CSA2_ERR_LAUNCH;
  return CSA2_OK;
}
