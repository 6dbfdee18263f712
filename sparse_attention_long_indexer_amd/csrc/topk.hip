// Per-row top-k selection over materialised scores (DeepSeek-V3.2 write-up,
// section 2.3: keep the k best-scoring keys of each query).
//
// Scores map to order-preserving uint32 keys (larger score -> larger key,
// -0.0 folded onto +0.0).  Two strategies give the same exact result:
//
// Many rows: one 1024-thread block per row.  A most-significant-digit-first
// radix select over the row's key range finds the exact key of the m-th
// best element and how many elements equal to it are kept; a last pass
// walks the row in index order with block-wide prefix counts, keeps every
// key above that threshold and the lowest-index keys equal to it, and
// writes the kept indices in ascending order.
//
// Few long rows (batched decode): one block per row would leave most of the
// chip idle, so the row is cut down first.  A sampled estimate picks a
// threshold key tau per row that about 1.75 m keys reach; a wide filter
// pass over every row appends the keys >= tau to a per-row candidate list;
// one block per row then selects exactly among the candidates.  When at
// least m keys reach tau, the top m are all candidates, so the result is
// exact; a row with too few or too many candidates (or a pathological tie)
// is settled by the same block with the full-row select instead.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace dsa {


struct RowView {
  const float* p;
  int64_t n;
};

__device__ __forceinline__ RowView topk_row_view(const TopkRows& R, int64_t row) {
  RowView v;
  if (R.seq_offsets) {
    const int64_t lo = R.seq_offsets[row];
    v.p = R.scores + lo;
    v.n = R.seq_offsets[row + 1] - lo;
  } else {
    const int64_t t = R.row_begin + row;
    const int64_t pos = R.q_pos ? R.q_pos[t] : R.pos_base + t;
    int64_t n = pos + 1 < R.S ? pos + 1 : R.S;
    v.n = n > 0 ? n : 0;
    v.p = R.scores + (R.row_off ? R.row_off[row] : row * R.ld);
  }
  return v;
}

__global__ __launch_bounds__(kTopkThreads) void topk_radix_kernel(TopkRows R, int64_t k,
                                                                  int32_t* __restrict__ idx_out,
                                                                  int32_t* __restrict__ count_out, DynK dyn) {
  __shared__ TopkShared sh;
  const int64_t row = blockIdx.x;
  const RowView rv = topk_row_view(R, row);
  const int64_t m = select_row(rv.p, rv.n, k, idx_out + row * k, sh, dyn);
  if (count_out && threadIdx.x == 0) count_out[row] = (int32_t)m;
}

// ---- candidate path for few long rows --------------------------------------
constexpr int kCandCap = 8192;          // candidates a row may stage in LDS
constexpr int kCandWin = 64;            // sampled keys per window (one wave)
constexpr int kCandWins = 64;           // windows per row (at least), one per stratum
constexpr int kCandWinsMax = 4096;      // ... and at most
constexpr int kCandSampleLds = 8192;    // samples staged in LDS (rows up to 2^18 keys)
constexpr int kCandSpan = 4096;         // keys per filter block
constexpr int kCandThreads = 512;
constexpr int kCandWaves = kCandThreads / 64;
constexpr int kCandMaxTies = 512;
constexpr int64_t kCandMinN = 16384;    // shorter rows: one block per row is enough
constexpr int64_t kCandBitmapN = 524288;  // rows up to this long: ascending output via an LDS bitmap
constexpr int64_t kCandMaxRows = 512;   // more rows fill the chip one block per row

static bool topk_use_candidates(int64_t rows, int64_t max_n, int64_t k) {
  return rows >= 1 && rows < kCandMaxRows && max_n >= kCandMinN && 2 * k <= kCandCap;
}

// integer hash (the "lowbias32" mixer) for window offsets
__device__ __forceinline__ uint32_t mix32(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// tau[row]: the r-th largest of a sample of the row's scores: one 64-key
// window at a hashed offset inside each of nw equal strata, nw = n / 2048
// clamped to [64, 4096] (one key in 32 up to 8M keys), r chosen so that
// about min(1.75 m, (m + cap) / 2) keys of the row reach it.  0 (below every
// key) when the whole row fits the candidate list.  A threshold on the zero
// score is raised past it, so ReLU's zeros do not flood the list.  Also
// clears the row's candidate count.
__global__ __launch_bounds__(kCandThreads) void topk_cand_estimate_kernel(TopkRows R, int64_t k,
                                                                         uint32_t* __restrict__ tau,
                                                                         int32_t* __restrict__ cnt) {
  __shared__ uint32_t wstart[kCandWinsMax];
  __shared__ uint32_t skey[kCandSampleLds];
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t scan[kCandWaves];
  __shared__ uint32_t s_out[2];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row = blockIdx.x;
  if (tid == 0) cnt[row] = 0;
  const RowView rv = topk_row_view(R, row);
  const int64_t n = rv.n, m = n < k ? n : k;
  if (n <= kCandCap) {
    if (tid == 0) tau[row] = 0u;
    return;
  }
  const int64_t nw64 = n / (32 * kCandWin);
  const int nw = (int)(nw64 < kCandWins ? kCandWins : (nw64 > kCandWinsMax ? kCandWinsMax : nw64));
  const int64_t nsamp = (int64_t)nw * kCandWin;
  const double target = fmin(1.75 * (double)m, 0.5 * (double)(m + kCandCap));
  int64_t r = (int64_t)ceil(target * (double)nsamp / (double)n);
  r = r < 1 ? 1 : (r > nsamp ? nsamp : r);
  // strata hold >= 128 keys (n > cap, nw <= max(64, n / 2048)), so every
  // window fits inside its stratum
  for (int wi = tid; wi < nw; wi += kCandThreads) {
    const int64_t s0 = n * wi / nw, s1 = n * (wi + 1) / nw;
    const uint64_t slots = (uint64_t)(s1 - s0 - kCandWin + 1);
    wstart[wi] = (uint32_t)(s0 + (int64_t)(mix32((uint32_t)(row * kCandWinsMax + wi) ^ 0x9e3779b9u) % slots));
  }
  __syncthreads();
  // samples of rows up to 2^18 keys are staged in LDS for the select's
  // passes; longer rows' samples are read again from the score row
  auto key_at = [&](int64_t i) { return score_key(rv.p[wstart[i >> 6] + (i & (kCandWin - 1))]); };
  const bool staged = nsamp <= kCandSampleLds;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  if (staged) {  // every load issued before the first use
    constexpr int PER = kCandSampleLds / kCandThreads;
    float v[PER];
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = tid + r * kCandThreads;
      v[r] = i < nsamp ? rv.p[wstart[i >> 6] + (i & (kCandWin - 1))] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < PER; ++r) {
      const int i = tid + r * kCandThreads;
      if (i < nsamp) {
        const uint32_t key = score_key(v[r]);
        skey[i] = key;
        mn = min(mn, key);
        mx = max(mx, key);
      }
    }
  } else {
    for (int64_t i = tid; i < nsamp; i += kCandThreads) {
      const uint32_t key = key_at(i);
      mn = min(mn, key);
      mx = max(mx, key);
    }
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    hist[w] = mn;
    hist[kCandWaves + w] = mx;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < kCandWaves; ++i) {
    mn = min(mn, hist[i]);
    mx = max(mx, hist[kCandWaves + i]);
  }
  __syncthreads();
  // the threshold only sets how many candidates the filter keeps, so two
  // digit passes (within 2^(top - 19) of the exact r-th sample) suffice
  uint32_t thr, need;
  auto staged_at = [&](int64_t i) { return skey[i]; };
  if (staged)
    radix_select<kCandThreads, decltype(staged_at), 2>(staged_at, nsamp, (uint32_t)r, mn, mx, hist, scan, s_out, thr,
                                                       need);
  else
    radix_select<kCandThreads, decltype(key_at), 2>(key_at, nsamp, (uint32_t)r, mn, mx, hist, scan, s_out, thr, need);
  if (tid == 0) tau[row] = thr == kZeroKey ? kZeroKey + 1 : thr;
}

// Append (key, position) of every key >= tau[row] in this block's span of
// the row to cand[row]; cnt[row] counts them all, slots past the cap are
// not written.  One atomic per block.
__global__ __launch_bounds__(256) void topk_cand_filter_kernel(TopkRows R, const uint32_t* __restrict__ tau,
                                                              uint2* __restrict__ cand, int32_t* __restrict__ cnt) {
  constexpr int PER = kCandSpan / 256;
  const int64_t row = blockIdx.y;
  const RowView rv = topk_row_view(R, row);
  const int64_t base = (int64_t)blockIdx.x * kCandSpan;
  if (base >= rv.n) return;
  const uint32_t tk = tau[row];
  const int tid = threadIdx.x, lane = tid & 63;
  // every load issued before the first compare (clamped, no branches)
  float v[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t i = base + j * 256 + tid;
    v[j] = rv.p[i < rv.n ? i : rv.n - 1];
  }
  uint32_t keys[PER];
  uint32_t mask = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int64_t i = base + j * 256 + tid;
    keys[j] = score_key(v[j]);
    mask |= (i < rv.n && keys[j] >= tk) ? (1u << j) : 0u;
  }
  const uint32_t mine = (uint32_t)__popc(mask);
  uint32_t incl = mine;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t v = __shfl_up(incl, off);
    if (lane >= off) incl += v;
  }
  // one atomic per block: wave totals in LDS, thread 0 reserves the run
  __shared__ uint32_t s_wt[4], s_base;
  const int w = tid >> 6;
  if (lane == 63) s_wt[w] = incl;
  __syncthreads();
  if (tid == 0) {
    const uint32_t tot = s_wt[0] + s_wt[1] + s_wt[2] + s_wt[3];
    s_base = tot ? (uint32_t)atomicAdd(&cnt[row], (int32_t)tot) : 0u;
  }
  __syncthreads();
  uint32_t pos = s_base + incl - mine;
  for (int i = 0; i < w; ++i) pos += s_wt[i];
  uint2* cr = cand + row * kCandCap;
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    if ((mask >> j) & 1u) {
      if (pos < (uint32_t)kCandCap) cr[pos] = make_uint2(keys[j], (uint32_t)(base + j * 256 + tid));
      ++pos;
    }
  }
}

// Exact top m of a row from its candidates (radix select in LDS, ascending
// output through a bitmap of kept positions); a row the candidates cannot
// settle is selected from its full score row by the same block.
__global__ __launch_bounds__(kTopkThreads) void topk_cand_select_kernel(TopkRows R, int64_t k,
                                                                       const uint32_t* __restrict__ tau,
                                                                       const uint2* __restrict__ cand,
                                                                       const int32_t* __restrict__ cnt,
                                                                       int32_t* __restrict__ idx_out,
                                                                       int32_t* __restrict__ count_out,
                                                                       DynK dyn) {
  constexpr int NT = kTopkThreads;
  extern __shared__ __align__(16) uint32_t sm[];
  uint2* cl = (uint2*)sm;                  // [kCandCap] (key, position)
  uint32_t* bitmap = sm + 2 * kCandCap;    // [nwords], or a long row's position buckets
  __shared__ TopkShared sh;
  __shared__ int32_t s_tie[kCandMaxTies];
  __shared__ int s_ntie;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t row = blockIdx.x;
  const RowView rv = topk_row_view(R, row);
  const int64_t n = rv.n;
  int64_t m = n < k ? n : k;
  int32_t* o = idx_out + row * k;
  const uint32_t tk = tau[row];
  const int c = cnt[row];
  if (n <= k || c > kCandCap || (tk != 0u && c < m)) {  // block-uniform
    m = select_row(rv.p, n, k, o, sh, dyn);
    if (count_out && tid == 0) count_out[row] = (int32_t)m;
    return;
  }
  const bool bucketed = n > kCandBitmapN;
  const int nwords = bucketed ? 0 : (int)((n + 31) >> 5);
  for (int i = tid; i < nwords; i += NT) bitmap[i] = 0u;
  if (tid == 0) s_ntie = 0;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  const uint2* cr = cand + row * kCandCap;
  for (int e = tid; e < c; e += NT) {
    const uint2 v = cr[e];
    cl[e] = v;
    mn = min(mn, v.x);
    mx = max(mx, v.x);
  }
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    sh.hist[w] = mn;
    sh.hist[kTopkWaves + w] = mx;
  }
  __syncthreads();
  mn = 0xFFFFFFFFu;
  mx = 0u;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    mn = min(mn, sh.hist[i]);
    mx = max(mx, sh.hist[kTopkWaves + i]);
  }
  __syncthreads();
  uint32_t thr, need;
  const uint32_t lo = tk != 0u ? tk : mn;
  auto key_at = [&](int64_t e) { return cl[e].x; };
  radix_select<NT>(key_at, c, (uint32_t)m, lo, mx, sh.hist, sh.wave_cnt, sh.sel, thr, need);
  // dynamic k: every key above theta is a candidate once the m-th best is
  // at or below theta (the m-th best is >= tau)
  const int64_t mm = dyn_budget<NT>(key_at, c, m, thr, dyn, sh.wave_cnt);
  if (mm < m) {
    m = mm;
    if (m == 0) {
      for (int64_t i = tid; i < k; i += NT) o[i] = -1;
      if (count_out && tid == 0) count_out[row] = 0;
      return;
    }
    radix_select<NT>(key_at, c, (uint32_t)m, lo, mx, sh.hist, sh.wave_cnt, sh.sel, thr, need);
  }
  const bool ok = bucketed ? output_bucketed_from_candidates<NT>(cl, c, thr, need, n, m, k, bitmap, s_tie, kCandMaxTies,
                                                               &s_ntie, sh.wave_cnt, o)
                          : output_from_candidates<NT>(cl, c, thr, need, n, m, k, bitmap, nwords, s_tie,
                                                       kCandMaxTies, &s_ntie, sh.wave_cnt, o, sh.hist);
  if (!ok) {
    __syncthreads();
    m = select_row(rv.p, n, k, o, sh, dyn);  // a boundary tie too long for the list
  }
  if (count_out && tid == 0) count_out[row] = (int32_t)m;
}

struct CandWs {
  uint32_t* tau;
  int32_t* cnt;
  uint2* cand;
};

// byte offsets of the candidate path's buffers; returns the bytes used
static size_t cand_layout(int64_t rows, char* base, CandWs* out) {
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += (bytes + 255) / 256 * 256;
    return at;
  };
  const size_t tau = take((size_t)rows * 4);
  const size_t cnt = take((size_t)rows * 4);
  const size_t cand = take((size_t)rows * kCandCap * 8);
  if (out) *out = CandWs{(uint32_t*)(base + tau), (int32_t*)(base + cnt), (uint2*)(base + cand)};
  return off;
}

size_t topk_workspace_bytes(int64_t rows, int64_t max_n, int64_t k) {
  if (!topk_use_candidates(rows, max_n, k)) return 0;
  return cand_layout(rows, nullptr, nullptr);
}

hipError_t launch_topk(const TopkRows& r, int64_t rows, int64_t max_n, int64_t k, int32_t* idx_out,
                       int32_t* count_out, void* ws, hipStream_t st, DynK dyn) {
  if (rows <= 0) return hipSuccess;
  if (!ws || !topk_use_candidates(rows, max_n, k)) {
    topk_radix_kernel<<<(unsigned)rows, kTopkThreads, 0, st>>>(r, k, idx_out, count_out, dyn);
    return hipGetLastError();
  }
  CandWs c;
  const size_t used = cand_layout(rows, (char*)ws, &c);
  DSA_DEBUG_CHECK(used <= topk_workspace_bytes(rows, max_n, k));
  (void)used;
  topk_cand_estimate_kernel<<<(unsigned)rows, kCandThreads, 0, st>>>(r, k, c.tau, c.cnt);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  dim3 fgrid((unsigned)((max_n + kCandSpan - 1) / kCandSpan), (unsigned)rows);
  topk_cand_filter_kernel<<<fgrid, 256, 0, st>>>(r, c.tau, c.cand, c.cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  constexpr size_t lds_max = (size_t)kCandCap * 8 + (size_t)(kCandBitmapN / 32) * 4;
  static std::atomic<uint64_t> attr_done{0};
  e = set_lds_limit_once((const void*)topk_cand_select_kernel, (int)lds_max, attr_done);
  if (e != hipSuccess) return e;
  const int64_t bm = max_n > kCandBitmapN ? kCandBitmapN : max_n;
  const size_t words = max_n > kCandBitmapN && (size_t)(2 * kOutBuckets) > (size_t)((bm + 31) / 32)
                           ? (size_t)(2 * kOutBuckets)
                           : (size_t)((bm + 31) / 32);
  const size_t lds = (size_t)kCandCap * 8 + words * 4;
  topk_cand_select_kernel<<<(unsigned)rows, kTopkThreads, lds, st>>>(r, k, c.tau, c.cand, c.cnt, idx_out,
                                                                     count_out, dyn);
  return hipGetLastError();
}

}  // namespace dsa
