// Fused lightning indexer + top-k selection for long causal prefill
// (DeepSeek-V3.2 write-up, sections 2.2 and 2.3: score every causal pair
// with ReLU(q . W . k) in FP8, keep the k best keys per query).
//
// The L^2 scores never reach HBM.  Four kernels:
//  1. estimate: per query row, scores against a fixed pseudo-random sample
//     of one key in every P (P = 32 up to 128K keys) give a threshold tau_t,
//     the score of rank r = ceil(1.75 * m * n_s / n) among the row's n_s
//     samples (16-bit truncated, so tau never exceeds that sample's score).
//     Expected survivors ~1.75 m.  Short rows (n <= kTakeAll) keep every key.
//  2. filter: one FP8 MFMA pass over every causal (query, key) pair with
//     keys in the A operand and queries in the B operand, so a lane owns one
//     query and four keys; a score v = acc * ks survives if v >= tau_t / qs_t
//     (rounded down a little, so the survivors contain every key whose final
//     score u = v * qs reaches tau).  Survivors (v, key) are appended to one
//     of four per-row segments, the segment picked by the lane group; a
//     per-tile rotation of the key order spreads periodic key patterns over
//     the segments.
//  3. select: per row, u = v * qs and ReLU for each survivor, an exact radix
//     select of the m best (score desc, index asc), and ascending output via
//     a bitmap over key positions.  The survivors provably contain the exact
//     answer when at least m of them reach tau; a row that fails this (or
//     overflowed a segment) is queued for
//  4. fallback: recompute that row's scores with the same MFMA and select
//     exactly, as the standalone top-k does.
// Every path uses the same fp32 score u = fl(fl(acc * ks) * qs), so the
// output equals the materialised scores + top-k path bit for bit.
#include "common.h"
#include "kernels.h"
#include "select.h"

namespace dsa {

constexpr int kSeg = 4;                    // survivor segments per row
constexpr int kCap = 1536;                 // survivors per segment
constexpr int kTakeAll = 5632;             // rows this short keep every key
constexpr int kSampleMax = 4096;           // samples per row (max)
constexpr float kAlpha = 1.75f;            // survivor target / m

__host__ __device__ inline int sample_stride(int64_t S) {
  int p = 32;
  while ((int64_t)p * kSampleMax < S) p <<= 1;
  return p;
}
// offset of sample j inside its block of P keys
__device__ __forceinline__ int sample_off(int64_t j, int P) {
  return (int)(((uint32_t)j * 2654435761u) >> 16) & (P - 1);
}
// number of samples with key position <= t
__device__ __forceinline__ int64_t samples_upto(int64_t t, int P) {
  const int64_t j = t / P;
  return j + (sample_off(j, P) <= (int)(t - j * P) ? 1 : 0);
}
__device__ __forceinline__ int tile_rot(int64_t key16) {
  return (int)(((uint32_t)key16 * 0x9E3779B1u) >> 28);
}

__global__ void zero_i32_kernel(int32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

// ---- 1. threshold estimate ------------------------------------------------
__global__ __launch_bounds__(256) void idx_estimate_kernel(const uint8_t* __restrict__ qf,
                                                           const float* __restrict__ qs,
                                                           const uint8_t* __restrict__ k8,
                                                           const float* __restrict__ ks, int64_t T,
                                                           int64_t S, int64_t topk,
                                                           float* __restrict__ tau) {
  __shared__ uint16_t sc[16][kSampleMax];
  __shared__ uint32_t hist[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t R0 = (int64_t)blockIdx.x * 16;
  const int64_t rlast = min(R0 + 15, T - 1);
  const int P = sample_stride(S);
  const int64_t nsb = samples_upto(min(rlast, S - 1), P);  // samples any row of the block uses

  const v8i a = *(const v8i*)(qf + min(R0 + c, T - 1) * kIdxDim + 32 * g);
  float qsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qsc[i] = qs[min(R0 + 4 * g + i, T - 1)];
  for (int64_t j16 = w; j16 * 16 < nsb; j16 += 4) {
    const int64_t j = j16 * 16 + c;
    int64_t s = j * P + sample_off(j, P);
    s = s < S ? s : S - 1;
    const v8i b = *(const v8i*)(k8 + s * kIdxDim + 32 * g);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_fp8_16x16x128(a, b, acc);
    const float kss = ks[s];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float u = acc[i] * kss * qsc[i];
      sc[4 * g + i][j] = (uint16_t)(__float_as_uint(u > 0.f ? u : 0.f) >> 16);
    }
  }
  __syncthreads();

  uint32_t* h = hist[w];
  for (int rr = 0; rr < 4; ++rr) {
    const int row = 4 * w + rr;
    const int64_t t = R0 + row;
    if (t >= T) break;
    const int64_t n = min(t + 1, S);
    const int64_t m = min(topk, n);
    if (n <= kTakeAll) {
      if (lane == 0) tau[t] = -INFINITY;
      continue;
    }
    const int64_t ns = samples_upto(n - 1, P);
    int64_t r = (int64_t)ceilf(kAlpha * (float)m * (float)ns / (float)n);
    r = r < 1 ? 1 : (r > ns ? ns : r);
    uint32_t prefix = 0, remaining = (uint32_t)r;
    for (int pass = 0; pass < 2; ++pass) {
      const int shift = 8 - 8 * pass;
      for (int i = lane; i < 256; i += 64) h[i] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int64_t i0 = 0; i0 < ns; i0 += 64) {
        const int64_t i = i0 + lane;
        bool in = false;
        uint32_t key = 0;
        if (i < ns) {
          key = sc[row][i];
          in = pass == 0 || (key >> 8) == (prefix >> 8);
        }
        const bool z = in && key == 0;
        const uint64_t zb = ballot(z);
        if (in && !z) atomicAdd(&h[(key >> shift) & 255u], 1u);
        if (zb && lane == 0) atomicAdd(&h[0], (uint32_t)__popcll(zb));
      }
      __builtin_amdgcn_wave_barrier();
      // digit of the remaining-th largest
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = h[255 - 4 * lane - e];
        sum += c4[e];
      }
      uint32_t incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (lane >= off) incl += v;
      }
      uint32_t above = incl - sum, dig = 0, ab = 0;
      bool found = false;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < remaining && remaining <= above + c4[e]) {
          dig = 255u - 4u * lane - e;
          ab = above;
          found = true;
        }
        above += c4[e];
      }
      const uint64_t fm = ballot(found);
      const int src = fm ? __builtin_ctzll(fm) : 0;
      dig = __shfl(dig, src);
      ab = __shfl(ab, src);
      remaining -= ab;
      prefix |= dig << shift;
      __builtin_amdgcn_wave_barrier();
    }
    const float tv = __uint_as_float(prefix << 16);
    if (lane == 0) tau[t] = tv > 0.f ? tv : -INFINITY;
  }
}

// ---- 2. filter pass ---------------------------------------------------------
constexpr int kFiltKeys = 64;             // keys per LDS tile
constexpr int kFiltRows = 256;            // queries per block (64 per wave)

__global__ __launch_bounds__(256, 2) void idx_filter_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, int64_t T, int64_t S, const float* __restrict__ tau,
    uint2* __restrict__ cand, int32_t* __restrict__ cnt_out) {
  __shared__ __align__(16) uint8_t ktile[2][kFiltKeys * kIdxDim];
  __shared__ __align__(16) float kst[2][kFiltKeys];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  // longest rows first for a better tail
  const int64_t nblk = (T + kFiltRows - 1) / kFiltRows;
  const int64_t R0 = (nblk - 1 - (int64_t)blockIdx.x) * kFiltRows;
  const int64_t Q0 = R0 + 64 * w;

  v8i bq[4];
  int64_t tq[4];
  float tv[4];
  int cnt[4];
  uint2* seg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = Q0 + 16 * q + c;
    const bool ok = t < T;
    const int64_t tt = ok ? t : T - 1;
    bq[q] = *(const v8i*)(qf + tt * kIdxDim + 32 * g);
    tq[q] = ok ? t : -1;  // an invalid query masks every key
    const float ta = tau[tt];
    // survivors need v * qs >= tau; shave a few ulps so rounding of the
    // product can never drop a key whose final score reaches tau
    tv[q] = !ok ? INFINITY : ta == -INFINITY ? -INFINITY : (ta / qs[tt]) * (1.0f - 1.0f / (1 << 20));
    cnt[q] = 0;
    seg[q] = cand + ((tt * kSeg) + g) * (int64_t)kCap;
  }
  const int64_t kend = min(S, min(R0 + kFiltRows, T));  // keys any row of the block can see
  const int ntiles = (int)((kend + kFiltKeys - 1) / kFiltKeys);

  // tile loader: 64 keys x 128 B = 512 chunks (2 per thread) + 64 scales
  auto issue = [&](int it, int buf) {
    const int64_t kb = (int64_t)it * kFiltKeys;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int chunk = (i * 4 + w) * 64 + lane;       // 16-byte chunk of the tile
      const int64_t key = min(kb + (chunk >> 3), S - 1);
      __builtin_amdgcn_global_load_lds(
          (const void*)(k8 + key * kIdxDim + (chunk & 7) * 16),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint8_t*)ktile[buf] +
                                                    (i * 4 + w) * 1024),
          16, 0, 0);
    }
    // scales: lanes 0..15 of wave 0 fetch 4 each; a group running past S is
    // filled by hand in the last tile
    if (w == 0 && lane < 16 && kb + 4 * lane + 3 < S) {
      __builtin_amdgcn_global_load_lds(
          (const void*)(ks + kb + 4 * lane),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) float*)kst[buf]), 16, 0, 0);
    }
  };
  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    const int64_t kb = (int64_t)it * kFiltKeys;
    if (it + 1 < ntiles) issue(it + 1, buf ^ 1);
    if (kb + kFiltKeys > S) {  // partial last tile: fill its scales by hand
      for (int i = threadIdx.x; i < kFiltKeys; i += 256) {
        const int64_t key = kb + i;
        if ((key & ~3LL) + 3 >= S) kst[buf][i] = key < S ? ks[key] : 0.f;
      }
      __syncthreads();
    }
    const bool mask = kb + kFiltKeys - 1 > Q0;  // some key may lie past a query of this wave
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int64_t k16 = kb + 16 * kt;
      const int rot = tile_rot(k16 >> 4);
      const int ar = (c + rot) & 15;                  // A row c holds key k16 + ar
      const uint8_t* ap = ktile[buf] + (16 * kt + ar) * kIdxDim + 32 * g;
      const v8i a = *(const v8i*)ap;
      int64_t key[4];
      float kss[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = (4 * g + i + rot) & 15;        // C row 4g+i holds key k16 + kr
        key[i] = k16 + kr;
        kss[i] = kst[buf][16 * kt + kr];
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
        acc = mfma_fp8_16x16x128(a, bq[q], acc);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float v = acc[i] * kss[i];
          bool pass = v >= tv[q];
          if (mask) pass = pass && key[i] <= tq[q];
          if (pass) {
            if (cnt[q] < kCap) seg[q][cnt[q]] = make_uint2(__float_as_uint(v), (uint32_t)key[i]);
            ++cnt[q];
          }
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (tq[q] >= 0) cnt_out[tq[q] * kSeg + g] = cnt[q];
}

// ---- 3. exact select over survivors ---------------------------------------
constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / 64;

__global__ __launch_bounds__(kSelThreads) void idx_select_kernel(
    const float* __restrict__ qs, const float* __restrict__ tau, const uint2* __restrict__ cand,
    const int32_t* __restrict__ cnt_in, int64_t T, int64_t S, int64_t topk, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ fb, int force_fallback) {
  extern __shared__ __align__(16) uint32_t sm[];
  uint32_t* ckey = sm;                          // [kSeg*kCap] score keys
  int32_t* cidx = (int32_t*)(sm + kSeg * kCap); // [kSeg*kCap] key positions
  uint32_t* bm = sm + 2 * kSeg * kCap;          // [2][nwords] bitmaps: selected, tied
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_cnt[kSelWaves];
  __shared__ uint32_t s_sel[2];
  __shared__ int s_off[kSeg + 1];
  __shared__ int s_bad;
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t t = blockIdx.x;
  const int64_t n = min(t + 1, S);
  const int64_t m = min(topk, n);
  int32_t* o = idx_out + t * topk;
  if (n <= topk) {
    for (int64_t i = tid; i < topk; i += kSelThreads) o[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const int nwords = (int)((n + 31) >> 5);
  if (tid == 0) {
    int off = 0, bad = 0;
    for (int gq = 0; gq < kSeg; ++gq) {
      const int cq = cnt_in[t * kSeg + gq];
      if (cq > kCap) bad = 1;
      s_off[gq] = off;
      off += cq > kCap ? kCap : cq;
    }
    s_off[kSeg] = off;
    s_bad = bad;
  }
  __syncthreads();
  const int total = s_off[kSeg];
  const float tt = tau[t];
  if (s_bad || force_fallback || (tt == -INFINITY && total != n)) {
    if (tid == 0) fb[1 + atomicAdd(&fb[0], 1)] = (int32_t)t;
    return;
  }
  // load survivors, final score u = v * qs with ReLU
  const float qsc = qs[t];
  uint32_t nge = 0;
  for (int e = tid; e < total; e += kSelThreads) {
    int gq = 0;
    while (gq + 1 < kSeg && e >= s_off[gq + 1]) ++gq;
    const uint2 cv = cand[(t * kSeg + gq) * (int64_t)kCap + (e - s_off[gq])];
    const float u0 = __uint_as_float(cv.x) * qsc;
    const float u = u0 > 0.f ? u0 : 0.f;
    ckey[e] = score_key(u);
    cidx[e] = (int32_t)cv.y;
    nge += (u >= tt) ? 1u : 0u;
  }
  for (int i = tid; i < 2 * nwords; i += kSelThreads) bm[i] = 0;
  {
    uint32_t tot;
    // every survivor already holds v >= tau/qs (rounded down), but only the
    // ones whose final score reaches tau count towards the proof
    nge = wave_sum(nge);
    if (lane == 0) wave_cnt[tid >> 6] = nge;
    __syncthreads();
    tot = 0;
    for (int i = 0; i < kSelWaves; ++i) tot += wave_cnt[i];
    __syncthreads();
    if (tt != -INFINITY && tot < (uint32_t)m) {
      if (tid == 0) fb[1 + atomicAdd(&fb[0], 1)] = (int32_t)t;
      return;
    }
  }
  // radix select of the m-th best key among the survivors
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)m;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kSelThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t zdig = (kZeroKey >> shift) & 255u;
    for (int e0 = 0; e0 < total; e0 += kSelThreads) {
      const int e = e0 + tid;
      bool in = false;
      uint32_t key = 0;
      if (e < total) {
        key = ckey[e];
        in = (key & mask) == prefix;
      }
      const bool z = in && key == kZeroKey;
      const uint64_t zb = ballot(z);
      if (in && !z) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      if (zb && lane == 0) atomicAdd(&hist[zdig], (uint32_t)__popcll(zb));
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = hist[255 - 4 * tid - e];
        sum += c4[e];
      }
      uint32_t incl = sum;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (tid >= off) incl += v;
      }
      uint32_t above = incl - sum;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (above < remaining && remaining <= above + c4[e]) {
          s_sel[0] = 255u - 4u * tid - e;
          s_sel[1] = above;
        }
        above += c4[e];
      }
    }
    __syncthreads();
    remaining -= s_sel[1];
    prefix |= s_sel[0] << shift;
    mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t thr = prefix, need = remaining;
  uint32_t* sel = bm;
  uint32_t* tie = bm + nwords;
  for (int e = tid; e < total; e += kSelThreads) {
    const uint32_t key = ckey[e];
    const int32_t p = cidx[e];
    if (p < 0 || p >= n) continue;
    if (key > thr) atomicOr(&sel[p >> 5], 1u << (p & 31));
    else if (key == thr) atomicOr(&tie[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  // keep the `need` lowest-position ties: prefix popcount over tie words
  const int per = (nwords + kSelThreads - 1) / kSelThreads;
  const int w0 = tid * per, w1 = min(nwords, w0 + per);
  uint32_t mine = 0;
  for (int i = w0; i < w1; ++i) mine += __popc(tie[i]);
  uint32_t tot_tie;
  {
    // exclusive block prefix of `mine`
    uint32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_cnt[tid >> 6] = incl;
    __syncthreads();
    uint32_t before = 0;
    tot_tie = 0;
    for (int i = 0; i < kSelWaves; ++i) {
      before += (i < (tid >> 6)) ? wave_cnt[i] : 0u;
      tot_tie += wave_cnt[i];
    }
    __syncthreads();
    uint32_t run = before + incl - mine;
    for (int i = w0; i < w1; ++i) {
      uint32_t wv = tie[i];
      while (wv) {
        const uint32_t b = wv & (0u - wv);
        if (run < need) sel[i] |= b;
        ++run;
        wv ^= b;
      }
    }
  }
  __syncthreads();
  // ascending output: prefix popcount over the selected bitmap
  mine = 0;
  for (int i = w0; i < w1; ++i) mine += __popc(sel[i]);
  {
    uint32_t incl = mine;
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t v = __shfl_up(incl, off);
      if (lane >= off) incl += v;
    }
    if (lane == 63) wave_cnt[tid >> 6] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (int i = 0; i < kSelWaves; ++i) before += (i < (tid >> 6)) ? wave_cnt[i] : 0u;
    uint32_t pos = before + incl - mine;
    for (int i = w0; i < w1; ++i) {
      uint32_t wv = sel[i];
      while (wv) {
        const int b = __builtin_ctz(wv);
        if (pos < (uint32_t)m) o[pos] = i * 32 + b;
        ++pos;
        wv &= wv - 1;
      }
    }
  }
  for (int64_t i = m + tid; i < topk; i += kSelThreads) o[i] = -1;
}

// ---- 4. exact fallback for rows the survivors cannot settle ---------------
constexpr int kFbBlocks = 64;

__global__ __launch_bounds__(kTopkThreads) void idx_fallback_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, int64_t S, int64_t topk, const int32_t* __restrict__ fb,
    float* __restrict__ scratch, int32_t* __restrict__ idx_out) {
  __shared__ TopkShared sh;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int nfb = fb[0];
  float* row = scratch + (int64_t)blockIdx.x * S;
  for (int f = blockIdx.x; f < nfb; f += gridDim.x) {
    const int64_t t = fb[1 + f];
    const int64_t n = min(t + 1, S);
    const v8i a = *(const v8i*)(qf + t * kIdxDim + 32 * g);
    const float qsc = qs[t];
    for (int64_t s0 = (int64_t)w * 16; s0 < n; s0 += kTopkWaves * 16) {
      const int64_t s = s0 + c;
      const int64_t sb = s < n ? s : n - 1;
      const v8i b = *(const v8i*)(k8 + sb * kIdxDim + 32 * g);
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_fp8_16x16x128(a, b, acc);
      if (g == 0 && s < n) {
        const float u = acc[0] * ks[sb] * qsc;
        row[s] = u > 0.f ? u : 0.f;
      }
    }
    __threadfence_block();
    __syncthreads();
    select_row(row, n, topk, idx_out + t * topk, sh);
    __syncthreads();
  }
}

size_t index_select_workspace_bytes(int64_t T, int64_t S) {
  size_t b = 0;
  auto add = [&](size_t x) { b += (x + 255) / 256 * 256; };
  add((size_t)T * 4);                       // tau
  add((size_t)T * kSeg * kCap * 8);         // survivors
  add((size_t)T * kSeg * 4);                // counts
  add((size_t)(T + 1) * 4);                 // fallback queue
  add((size_t)kFbBlocks * S * 4);           // fallback score rows
  return b;
}

bool index_select_supported(int64_t T, int64_t S) { return T == S && T <= 262144 && T >= 1; }

hipError_t launch_index_select(const uint8_t* qf, const float* qs, const uint8_t* k8, const float* ks,
                               int64_t T, int64_t S, int64_t topk, int32_t* idx_out, void* ws,
                               bool force_fallback, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  char* p = (char*)ws;
  auto take = [&](size_t x) {
    char* q = p;
    p += (x + 255) / 256 * 256;
    return q;
  };
  float* tau = (float*)take((size_t)T * 4);
  uint2* cand = (uint2*)take((size_t)T * kSeg * kCap * 8);
  int32_t* cnt = (int32_t*)take((size_t)T * kSeg * 4);
  int32_t* fb = (int32_t*)take((size_t)(T + 1) * 4);
  float* scratch = (float*)take((size_t)kFbBlocks * S * 4);
  zero_i32_kernel<<<1, 64, 0, st>>>(fb, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  idx_estimate_kernel<<<(unsigned)((T + 15) / 16), 256, 0, st>>>(qf, qs, k8, ks, T, S, topk, tau);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  idx_filter_kernel<<<(unsigned)((T + kFiltRows - 1) / kFiltRows), 256, 0, st>>>(qf, qs, k8, ks, T, S, tau, cand,
                                                                                  cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int nwords = (int)((S + 31) / 32);
  const size_t lds = (size_t)2 * kSeg * kCap * 4 + (size_t)2 * nwords * 4;
  static bool attr = false;
  if (!attr) {
    e = hipFuncSetAttribute((const void*)idx_select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)(2 * kSeg * kCap * 4 + 2 * (262144 / 32) * 4));
    if (e != hipSuccess) return e;
    attr = true;
  }
  idx_select_kernel<<<(unsigned)T, kSelThreads, lds, st>>>(qs, tau, cand, cnt, T, S, topk, idx_out, fb,
                                                          force_fallback ? 1 : 0);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  idx_fallback_kernel<<<kFbBlocks, kTopkThreads, 0, st>>>(qf, qs, k8, ks, S, topk, fb, scratch, idx_out);
  return hipGetLastError();
}

}  // namespace dsa
