// Row selection shared by the standalone top-k, the candidate top-k for few
// long rows and the fused indexer.
#pragma once

#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr uint32_t kZeroKey = 0x80000000u;  // score_key(+0.0f)

struct TopkShared {
  uint32_t hist[1024];
  uint32_t wave_cnt[kTopkWaves];
  uint32_t sel[2];
};

// Block-wide exclusive prefix count of `pred` (all threads must call).
// Returns the prefix; writes the block total to *total.
template <int NWAVES = kTopkWaves>
__device__ __forceinline__ uint32_t block_prefix(bool pred, uint32_t* wave_cnt, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = ballot(pred);
  if (lane == 0) wave_cnt[w] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    const uint32_t c = wave_cnt[i];
    before += (i < w) ? c : 0u;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + lanes_below(m);
}

// Block-wide exact selection of the m-th largest 32-bit key among n keys
// (key_at(i) for i < n) that are >= lo, given every key is <= hi and at
// least m keys are >= lo.  Radix over d = key - lo with 10-bit digits, so
// the first digit spans only the occupied range [lo, hi].  Histogram updates
// peel the wave's most common bin (one atomic for all its lanes) before the
// per-lane atomics, which keeps heavy ties (ReLU zeros) cheap.
// Returns thr (the m-th largest key) and need (how many keys equal to thr
// belong to the top m).  hist must hold 1024 words; scan holds NT/64 words.
// With MAXPASS < 4 the digits below the last pass are left at zero: thr is
// then a lower bound of the m-th largest key within 2^(top - 10 MAXPASS + 1)
// of it (top = the span's highest bit), and need is not meaningful.
template <int NT, class KeyAt, int MAXPASS = 4>
__device__ inline void radix_select(KeyAt key_at, int64_t n, uint32_t m, uint32_t lo, uint32_t hi,
                                    uint32_t* hist, uint32_t* scan, uint32_t* s_out, uint32_t& thr,
                                    uint32_t& need) {
  constexpr int BINS = 1024, PER = BINS / NT > 0 ? BINS / NT : 1;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const uint32_t span = hi - lo;
  int top = span ? 31 - __builtin_clz(span) : 0;      // highest set bit of the span
  uint32_t prefix = 0, pmask = 0, remaining = m;
  for (int shift = top - 9, pass = 1; ; shift -= 10, ++pass) {
    const int sh = shift > 0 ? shift : 0;
    const uint32_t dmask = shift >= 0 ? 1023u : (1023u >> (-shift));
    for (int i = tid; i < BINS; i += NT) hist[i] = 0;
    __syncthreads();
    for (int64_t b = 0; b < n; b += NT) {
      const int64_t i = b + tid;
      bool in = false;
      uint32_t bin = 0;
      if (i < n) {
        const uint32_t key = key_at(i);
        if (key >= lo) {
          const uint32_t d = key - lo;
          in = (d & pmask) == prefix;
          bin = (d >> sh) & dmask;
        }
      }
      // peel the most common bin of this wave: first active lane's bin
      const uint64_t act = ballot(in);
      if (act) {
        const int first = __builtin_ctzll(act);
        const uint32_t b0 = __shfl(bin, first);
        const uint64_t same = ballot(in && bin == b0);
        if (lane == first) atomicAdd(&hist[b0], (uint32_t)__popcll(same));
        if (in && bin != b0) atomicAdd(&hist[bin], 1u);
      }
    }
    __syncthreads();
    // bins in descending order: thread tid owns bins BINS-1-PER*tid .. -PER+1
    uint32_t own = 0, c[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      const int bi = BINS - 1 - PER * tid - e;
      c[e] = bi >= 0 ? hist[bi] : 0u;
      own += c[e];
    }
    uint32_t incl = own;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) scan[w] = incl;
    __syncthreads();
    uint32_t above = incl - own;
    for (int i = 0; i < w; ++i) above += scan[i];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      if (above < remaining && remaining <= above + c[e]) {
        s_out[0] = (uint32_t)(BINS - 1 - PER * tid - e);
        s_out[1] = above;
      }
      above += c[e];
    }
    __syncthreads();
    const uint32_t dig = s_out[0];
    remaining -= s_out[1];
    prefix |= dig << sh;
    pmask |= dmask << sh;
    __syncthreads();
    if (shift <= 0 || pass >= MAXPASS) break;
  }
  thr = lo + prefix;
  need = remaining;
}

// Dynamic budget (DynK) of a row whose fixed selection of m keys has its
// m-th best key at thr, counted over the keys key_at(0 .. nkeys) (all of the
// row's keys above thr must be among them): m when the m best all lie above
// theta, else max(k_min, #{keys > theta}) (<= m).  All threads must call.
template <int NT, class KeyAt>
__device__ inline int64_t dyn_budget(KeyAt key_at, int64_t nkeys, int64_t m, uint32_t thr, const DynK& dyn,
                                     uint32_t* scan) {
  if (!dyn_on(dyn)) return m;
  const uint32_t tk = score_key(dyn.theta);
  if (thr > tk) return m;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t c = 0;
  for (int64_t i = tid; i < nkeys; i += NT) c += key_at(i) > tk ? 1u : 0u;
  c = wave_sum(c);
  __syncthreads();  // the caller's select may still read scan
  if (lane == 0) scan[w] = c;
  __syncthreads();
  uint32_t tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) tot += scan[i];
  __syncthreads();
  const int64_t mm = (int64_t)tot > dyn.k_min ? (int64_t)tot : dyn.k_min;
  return mm < m ? mm : m;
}

// Whole-row exact selection from fp32 scores p[0 .. n): the m best under
// (score desc, index asc), m = min(n, k) or the row's dynamic budget, written
// ascending to o[0 .. m) with o[m .. k) = -1.  Returns m.  All kTopkThreads
// threads of the block call it; `sh` is block-shared scratch.
__device__ inline int64_t select_row(const float* __restrict__ p, int64_t n, int64_t k, int32_t* __restrict__ o,
                                     TopkShared& sh, DynK dyn = kFixedK) {
  const int tid = threadIdx.x;
  int64_t m = n < k ? n : k;
  if (n <= k && !dyn_on(dyn)) {  // every key is kept
    for (int64_t i = tid; i < k; i += kTopkThreads) o[i] = i < n ? (int32_t)i : -1;
    return m;
  }
  // key range of the row
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int64_t i = tid; i < n; i += kTopkThreads) {
    const uint32_t key = score_key(p[i]);
    mn = min(mn, key);
    mx = max(mx, key);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if ((tid & 63) == 0) {
    sh.wave_cnt[tid >> 6] = mn;
    sh.hist[tid >> 6] = mx;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
  for (int i = 0; i < kTopkWaves; ++i) {
    mn = min(mn, sh.wave_cnt[i]);
    mx = max(mx, sh.hist[i]);
  }
  __syncthreads();
  auto key_at = [&](int64_t i) { return score_key(p[i]); };
  uint32_t thr = mn, need = 0;
  if (n > k) radix_select<kTopkThreads>(key_at, n, (uint32_t)m, mn, mx, sh.hist, sh.wave_cnt, sh.sel, thr, need);
  const int64_t mm = dyn_budget<kTopkThreads>(key_at, n, m, thr, dyn, sh.wave_cnt);
  if (n <= k && mm == m) {  // dynamic budget keeps the whole short row
    for (int64_t i = tid; i < k; i += kTopkThreads) o[i] = i < n ? (int32_t)i : -1;
    return m;
  }
  if (mm < m) {
    m = mm;
    if (m == 0) {
      for (int64_t i = tid; i < k; i += kTopkThreads) o[i] = -1;
      return 0;
    }
    radix_select<kTopkThreads>(key_at, n, (uint32_t)m, mn, mx, sh.hist, sh.wave_cnt, sh.sel, thr, need);
  }

  // ordered selection: keys > thr, and the first `need` keys == thr
  uint32_t carry_eq = 0, carry_sel = 0;
  for (int64_t base = 0; base < n && carry_sel < (uint32_t)m; base += kTopkThreads) {
    const int64_t i = base + tid;
    uint32_t key = 0;
    if (i < n) key = score_key(p[i]);
    const bool gt = i < n && key > thr;
    const bool eq = i < n && key == thr;
    uint32_t tot_eq, tot_sel;
    const uint32_t eq_rank = carry_eq + block_prefix(eq, sh.wave_cnt, &tot_eq);
    const bool sel = gt || (eq && eq_rank < need);
    const uint32_t pos = carry_sel + block_prefix(sel, sh.wave_cnt, &tot_sel);
    if (sel && pos < (uint32_t)m) o[pos] = (int32_t)i;
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  for (int64_t i = m + tid; i < k; i += kTopkThreads) o[i] = -1;
  return m;
}

// Ascending output from a candidate list: given thr / need from radix_select
// over the (key, position) pairs cl[0 .. nslots) of a row of n keys, keep
// every position whose key is above thr and the `need` lowest positions
// whose key equals thr, and write the m kept positions in ascending order to
// o[0 .. m), padding o[m .. topk) with -1.  Kept positions are marked in a
// bitmap of nwords words (zeroed by the caller, as is *s_ntie); keys equal
// to thr go through the tie list `tie` (max_ties entries).  When the list
// overflows (typically ReLU's zeros at the boundary of a short row) and the
// row has at most 32 * kTieBitmapWords positions, the ties are marked in a
// second bitmap `tie_bits` (LDS scratch of kTieBitmapWords words, may be
// null) and the `need` lowest are found by prefix popcounts.  Positions
// outside [0, n) are skipped (invalid slots).  Returns false, with nothing
// written to o, when the ties cannot be settled; the caller settles the row
// elsewhere.
constexpr int kTieBitmapWords = 1024;

template <int NT>
__device__ inline bool output_from_candidates(const uint2* cl, int nslots, uint32_t thr, uint32_t need,
                                              int64_t n, int64_t m, int64_t topk, uint32_t* bitmap,
                                              int nwords, int32_t* tie, int max_ties, int* s_ntie,
                                              uint32_t* wave_cnt, int32_t* __restrict__ o,
                                              uint32_t* tie_bits = nullptr) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  for (int e = tid; e < nslots; e += NT) {
    const uint2 cv = cl[e];
    const uint32_t key = cv.x;
    const int32_t p = (int32_t)cv.y;
    if (key < thr || p < 0 || p >= n) continue;
    if (key > thr) {
      atomicOr(&bitmap[p >> 5], 1u << (p & 31));
    } else {
      const int q = atomicAdd(s_ntie, 1);
      if (q < max_ties) tie[q] = p;
    }
  }
  __syncthreads();
  const int ntie = *s_ntie;
  if (ntie > max_ties) {
    if (!tie_bits || nwords > kTieBitmapWords) return false;
    for (int i = tid; i < nwords; i += NT) tie_bits[i] = 0u;
    __syncthreads();
    for (int e = tid; e < nslots; e += NT) {
      const uint2 cv = cl[e];
      const int32_t p = (int32_t)cv.y;
      if (cv.x == thr && p >= 0 && p < n) atomicOr(&tie_bits[p >> 5], 1u << (p & 31));
    }
    __syncthreads();
    // the `need` lowest tie positions: exclusive prefix of the popcounts over
    // runs of `per` words per thread, then each thread walks its run
    const int per = (nwords + NT - 1) / NT;
    const int w0 = tid * per, w1 = min(nwords, w0 + per);
    uint32_t mine = 0;
    for (int i = w0; i < w1; ++i) mine += __popc(tie_bits[i]);
    uint32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_cnt[w] = incl;
    __syncthreads();
    uint32_t rank = incl - mine;
#pragma unroll
    for (int i = 0; i < NW; ++i) rank += (i < w) ? wave_cnt[i] : 0u;
    for (int i = w0; i < w1 && rank < need; ++i) {
      uint32_t wv = tie_bits[i], keep = 0u;
      while (wv && rank < need) {
        const uint32_t b = wv & (0u - wv);
        keep |= b;
        ++rank;
        wv ^= b;
      }
      if (keep) atomicOr(&bitmap[i], keep);
    }
    __syncthreads();  // wave_cnt is reused below
  } else {
    for (int i = tid; i < ntie; i += NT) {
      const int32_t p = tie[i];
      int rank = 0;
      for (int j = 0; j < ntie; ++j) rank += tie[j] < p ? 1 : 0;
      if (rank < (int)need) atomicOr(&bitmap[p >> 5], 1u << (p & 31));
    }
  }
  __syncthreads();
  // prefix popcount over the bitmap: thread tid owns a run of `per` words
  const int per = (nwords + NT - 1) / NT;
  const int w0 = tid * per, w1 = min(nwords, w0 + per);
  uint32_t mine = 0;
  for (int i = w0; i < w1; ++i) mine += __popc(bitmap[i]);
  uint32_t incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  if (lane == 63) wave_cnt[w] = incl;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) before += (i < w) ? wave_cnt[i] : 0u;
  uint32_t pos = before + incl - mine;
  for (int i = w0; i < w1; ++i) {
    uint32_t wv = bitmap[i];
    while (wv) {
      const int b = __builtin_ctz(wv);
      if (pos < (uint32_t)m) o[pos] = i * 32 + b;
      ++pos;
      wv &= wv - 1;
    }
  }
  for (int64_t i = m + tid; i < topk; i += NT) o[i] = -1;
  return true;
}

// The same output without a bitmap, for rows too long for one in LDS.  The
// kept positions (keys above thr, then the `need` lowest-position keys equal
// to thr) are counted per bucket of 2^shift consecutive positions (4096
// buckets span the row), an exclusive scan gives every bucket its output
// range, each kept position is dropped into its bucket's range, and its
// final place is the bucket start plus the number of smaller positions in
// the same bucket (a bucket holds a handful of kept keys).
// work: LDS, 2 * kOutBuckets words; m <= kOutBuckets.  *s_ntie must be
// zeroed by the caller before a barrier.  Returns false, with nothing
// written to o, when the tie list overflows.
constexpr int kOutBuckets = 4096;

template <int NT>
__device__ inline bool output_bucketed_from_candidates(const uint2* cl, int nslots, uint32_t thr, uint32_t need,
                                                       int64_t n, int64_t m, int64_t topk, uint32_t* work,
                                                       int32_t* tie, int max_ties, int* s_ntie, uint32_t* wave_cnt,
                                                       int32_t* __restrict__ o) {
  constexpr int NW = NT / 64, PER = kOutBuckets / NT;
  static_assert(PER * NT == kOutBuckets, "threads must divide the bucket count");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  uint32_t* start = work;                        // [kOutBuckets] counts, then ranges
  int32_t* buf = (int32_t*)(work + kOutBuckets);  // [m] kept positions by bucket
  const int bits = 64 - __builtin_clzll((uint64_t)(n - 1) | 1ull);
  const int shift = bits > 12 ? bits - 12 : 0;
  for (int i = tid; i < kOutBuckets; i += NT) start[i] = 0u;
  __syncthreads();
  for (int e = tid; e < nslots; e += NT) {
    const uint2 cv = cl[e];
    const int32_t p = (int32_t)cv.y;
    if (cv.x < thr || p < 0 || p >= n) continue;
    if (cv.x > thr) {
      atomicAdd(&start[p >> shift], 1u);
    } else {
      const int q = atomicAdd(s_ntie, 1);
      if (q < max_ties) tie[q] = p;
    }
  }
  __syncthreads();
  const int ntie = *s_ntie;
  if (ntie > max_ties) return false;
  auto tie_kept = [&](int i) {
    const int32_t p = tie[i];
    int rank = 0;
    for (int j = 0; j < ntie; ++j) rank += tie[j] < p ? 1 : 0;
    return rank < (int)need;
  };
  for (int i = tid; i < ntie; i += NT)
    if (tie_kept(i)) atomicAdd(&start[tie[i] >> shift], 1u);
  __syncthreads();
  // exclusive scan of the bucket counts; thread tid owns PER buckets
  uint32_t v[PER], mine = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    v[j] = start[tid * PER + j];
    mine += v[j];
  }
  uint32_t incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t u = __shfl_up(incl, off);
    if (lane >= off) incl += u;
  }
  if (lane == 63) wave_cnt[w] = incl;
  __syncthreads();
  uint32_t run = incl - mine;
#pragma unroll
  for (int i = 0; i < NW; ++i) run += (i < w) ? wave_cnt[i] : 0u;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    start[tid * PER + j] = run;
    run += v[j];
  }
  __syncthreads();
  // drop each kept position into its bucket (start[b] ends as bucket b's end)
  for (int e = tid; e < nslots; e += NT) {
    const uint2 cv = cl[e];
    const int32_t p = (int32_t)cv.y;
    if (cv.x <= thr || p < 0 || p >= n) continue;
    const uint32_t slot = atomicAdd(&start[p >> shift], 1u);
    if (slot < (uint32_t)kOutBuckets) buf[slot] = p;
  }
  for (int i = tid; i < ntie; i += NT) {
    if (!tie_kept(i)) continue;
    const uint32_t slot = atomicAdd(&start[tie[i] >> shift], 1u);
    if (slot < (uint32_t)kOutBuckets) buf[slot] = tie[i];
  }
  __syncthreads();
  for (int i = tid; i < (int)m; i += NT) {
    const int32_t p = buf[i];
    const int b = p >> shift;
    const uint32_t lo = b ? start[b - 1] : 0u, hi = start[b];
    uint32_t rank = 0;
    for (uint32_t j = lo; j < hi; ++j) rank += buf[j] < p ? 1u : 0u;
    o[lo + rank] = p;
  }
  for (int64_t i = m + tid; i < topk; i += NT) o[i] = -1;
  return true;
}

}  // namespace dsa
