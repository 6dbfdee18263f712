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
//     Past 128K keys a refinement pass rescores one key in 32 around tau.
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
//     a bitmap over key positions (position buckets for rows past 256K).  The survivors provably contain the exact
//     answer when at least m of them reach tau; a row that fails this (or
//     overflowed a segment) is queued for
//  4. fallback: recompute that row's scores with the same MFMA and select
//     exactly, as the standalone top-k does.
// Every path uses the same fp32 score u = fl(fl(acc * ks) * qs), so the
// output equals the materialised scores + top-k path bit for bit.
#include "common.h"
#include "dsa.h"
#include "kernels.h"
#include "select.h"

namespace dsa {

constexpr int kSeg = 4;                    // survivor segments per row
constexpr int kCap = 1536;                 // survivors per segment
constexpr int kTakeAll = 5632;             // rows this short keep every key
constexpr int kSampleMax = 4096;           // samples per row (max)
constexpr float kAlpha = 1.75f;            // survivor target / m
constexpr int64_t kSelBitmapN = 262144;    // longer rows emit their indices through buckets, not a bitmap

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
constexpr int kEstWaves = 16;
__global__ __launch_bounds__(kEstWaves * 64) void idx_estimate_kernel(const uint8_t* __restrict__ qf,
                                                           const float* __restrict__ qs,
                                                           const uint8_t* __restrict__ k8,
                                                           const float* __restrict__ ks, int64_t T,
                                                           int64_t S, int64_t topk,
                                                           float* __restrict__ tau) {
  __shared__ uint16_t sc[16][kSampleMax];
  __shared__ uint32_t hist[kEstWaves][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t R0 = (int64_t)blockIdx.x * 16;
  const int64_t p0 = S - T;  // position of row 0
  const int64_t rlast = min(R0 + 15, T - 1);
  const int P = sample_stride(S);
  const int64_t nsb = samples_upto(min(p0 + rlast, S - 1), P);  // samples any row of the block uses

  const v8i a = *(const v8i*)(qf + min(R0 + c, T - 1) * kIdxDim + 32 * g);
  float qsc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) qsc[i] = qs[min(R0 + 4 * g + i, T - 1)];
  // each wave takes sample tiles w, w+16, ...; four tiles' keys are loaded
  // before their MFMAs so the loads overlap
  for (int64_t j0 = (int64_t)w * 16; j0 < nsb; j0 += 4 * kEstWaves * 16) {
    v8i b[4];
    float kss[4];
    int64_t jj[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      jj[u] = j0 + (int64_t)u * kEstWaves * 16 + c;
      int64_t sk = jj[u] * P + sample_off(jj[u], P);
      sk = sk < S ? sk : S - 1;
      b[u] = *(const v8i*)(k8 + sk * kIdxDim + 32 * g);
      kss[u] = ks[sk];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (j0 + (int64_t)u * kEstWaves * 16 >= nsb) break;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_fp8_16x16x128(a, b[u], acc);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float uu = acc[i] * kss[u] * qsc[i];
        sc[4 * g + i][jj[u]] = (uint16_t)(__float_as_uint(uu > 0.f ? uu : 0.f) >> 16);
      }
    }
  }
  __syncthreads();

  uint32_t* h = hist[w];
  for (int rr = 0; rr < 16 / kEstWaves; ++rr) {
    const int row = (16 / kEstWaves) * w + rr;
    const int64_t t = R0 + row;
    if (t >= T) break;
    const int64_t n = min(p0 + t + 1, S);
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
        // peel the wave's most common digit (zeros and clustered scores)
        const uint32_t dg = (key >> shift) & 255u;
        const uint64_t act = ballot(in);
        if (act) {
          const int first = __builtin_ctzll(act);
          const uint32_t d0 = __shfl(dg, first);
          const uint64_t same = ballot(in && dg == d0);
          if (lane == first) atomicAdd(&h[d0], (uint32_t)__popcll(same));
          if (in && dg != d0) atomicAdd(&h[dg], 1u);
        }
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
    // a zero rank-r sample means the row has few positive scores: keep the
    // positive ones (tau = the smallest positive float)
    const float tv = __uint_as_float(prefix << 16);
    if (lane == 0) tau[t] = tv > 0.f ? tv : 1.17549435e-38f;
  }
}

// ---- 1b. threshold refinement for rows past 4096 * 32 keys ----------------
// There the estimate's stride P grows while its sample stays at 4096 keys,
// so the rank r shrinks (r ~ 14 at 2^20 keys) and tau scatters: too few
// survivors send the row to the fallback.  This pass rescores one key in
// every 32, counts per row the scores in [tau/2, 2 tau) on 128 bins evenly
// spaced in the float bit pattern (1/64 of an octave each), and moves tau to
// the lower edge of the bin where the count from the top reaches
// r = ceil(1.75 m n_s / n) of the row's n_s samples.  A row whose r-th
// sample lies below tau/2 gets tau/2.
constexpr int kRefRows = 64;    // rows per block, 16 per wave
constexpr int kRefKeys = 64;    // sampled keys per LDS tile
constexpr int kRefBins = 128;
constexpr int kRefStride = 32;
constexpr int kRefBinShift = 17;  // 2 octaves = 2^24 bit steps over 128 bins

__global__ __launch_bounds__(256) void idx_refine_kernel(const uint8_t* __restrict__ qf, const float* __restrict__ qs,
                                                         const uint8_t* __restrict__ k8, const float* __restrict__ ks,
                                                         int64_t T, int64_t S, int64_t topk, float* __restrict__ tau) {
  __shared__ __align__(16) uint8_t ktile[2][kRefKeys * kIdxDim];
  __shared__ __align__(16) float kst[2][kRefKeys];
  __shared__ uint32_t hist[kRefRows][kRefBins];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t R0 = (int64_t)blockIdx.x * kRefRows;
  const int64_t p0 = S - T;
  // the lane's query row (B operand column c of wave w)
  const int64_t t = R0 + 16 * w + c;
  const int64_t tt = t < T ? t : T - 1;
  const v8i bq = *(const v8i*)(qf + tt * kIdxDim + 32 * g);
  const float qsc = qs[tt];
  const int64_t n = min(p0 + tt + 1, S);
  const float t1 = tau[tt];
  const bool act = t < T && n > kTakeAll && t1 > 1.17549435e-38f && t1 < INFINITY;
  const float lo = act ? 0.5f * t1 : INFINITY;
  const uint32_t lob = __float_as_uint(lo);
  const int64_t ns = act ? samples_upto(n - 1, kRefStride) : 0;  // sample j is the row's iff j < ns
  const int64_t nsb = samples_upto(min(p0 + min(R0 + kRefRows - 1, T - 1), S - 1), kRefStride);

  for (int i = threadIdx.x; i < kRefRows * kRefBins; i += 256) (&hist[0][0])[i] = 0u;

  // 64 sampled keys x 128 B = 512 chunks (2 per thread) + 64 scales
  auto issue = [&](int it, int buf) {
    const int64_t j0 = (int64_t)it * kRefKeys;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int chunk = (i * 4 + w) * 64 + lane;
      const int64_t js = j0 + (chunk >> 3);
      const int64_t key = min(js * kRefStride + sample_off(js, kRefStride), S - 1);
      __builtin_amdgcn_global_load_lds(
          (const void*)(k8 + key * kIdxDim + (chunk & 7) * 16),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint8_t*)ktile[buf] +
                                                    (i * 4 + w) * 1024),
          16, 0, 0);
    }
    if (w == 0) {
      const int64_t js = j0 + lane;
      const int64_t key = min(js * kRefStride + sample_off(js, kRefStride), S - 1);
      __builtin_amdgcn_global_load_lds(
          (const void*)(ks + key),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) float*)kst[buf]), 4, 0, 0);
    }
  };
  const int ntiles = (int)((nsb + kRefKeys - 1) / kRefKeys);
  if (ntiles > 0) issue(0, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    if (it + 1 < ntiles) issue(it + 1, buf ^ 1);
    const int64_t j0 = (int64_t)it * kRefKeys;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const v8i a = *(const v8i*)(ktile[buf] + (16 * kt + c) * kIdxDim + 32 * g);
      const v4f acc = mfma_fp8_16x16x128(a, bq, (v4f){0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int jl = 16 * kt + 4 * g + i;   // C row 4g+i holds sample j0 + jl
        const float u = (acc[i] * kst[buf][jl]) * qsc;
        if (j0 + jl < ns && u >= lo) {
          const uint32_t b = min((__float_as_uint(u) - lob) >> kRefBinShift, (uint32_t)(kRefBins - 1));
          atomicAdd(&hist[16 * w + c][b], 1u);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (g == 0 && act) {
    const int64_t m = min(topk, n);
    int64_t r = (int64_t)ceilf(kAlpha * (float)m * (float)ns / (float)n);
    r = r < 1 ? 1 : (r > ns ? ns : r);
    uint32_t cum = 0;
    float tv = lo;
    for (int b = kRefBins - 1; b >= 0; --b) {
      cum += hist[16 * w + c][b];
      if (cum >= (uint32_t)r) {
        tv = __uint_as_float(lob + ((uint32_t)b << kRefBinShift));
        break;
      }
    }
    tau[t] = tv;
  }
}

// ---- 2. filter pass ---------------------------------------------------------
constexpr int kFiltKeys = 64;             // keys per LDS tile
constexpr int kFiltRows = 256;            // queries per block (64 per wave)
constexpr int kSets = 2;                  // key chunks per row (long rows split in two)
constexpr int kSlack = 16;                // sink slots past kCap (one tile's worth per lane)
constexpr int kSegStride = kCap + kSlack;

// Work items: long row blocks (keys past the chunk boundary kmax) are split
// into chunk 0 = keys [0, kmax) and chunk 1 = keys [kmax, end), each with its
// own survivor set, so no item scans more than kmax keys.  Items are ordered
// longest first.  Row block rb holds rows [256 rb, 256 rb + 256) at
// positions p0 + row (p0 = S - T) and sees keys [0, min(S, p0 + 256 (rb+1))).
struct FilterItem {
  int64_t rb;    // row block
  int set;       // key chunk / survivor set
  int64_t k0, k1;
};
__host__ __device__ inline int64_t filter_kmax(int64_t S) {
  const int64_t h = (S + 1) / 2;
  return (h + kFiltRows - 1) / kFiltRows * kFiltRows;
}
// first row block whose key range passes kmax
__host__ __device__ inline int64_t filter_first_long(int64_t T, int64_t S) {
  const int64_t kmax = filter_kmax(S), p0 = S - T;
  return kmax >= p0 ? (kmax - p0) / kFiltRows : 0;
}
__device__ __forceinline__ FilterItem filter_item(int64_t id, int64_t T, int64_t S) {
  const int64_t nb = (T + kFiltRows - 1) / kFiltRows;
  const int64_t kmax = filter_kmax(S), p0 = S - T;
  const int64_t first_long = filter_first_long(T, S);
  const int64_t nl = nb > first_long ? nb - first_long : 0;
  FilterItem it;
  if (id < nl) {
    it.rb = nb - 1 - id;
    it.set = 0;
  } else if (id < 2 * nl) {
    it.rb = nb - 1 - (id - nl);
    it.set = 1;
  } else {
    it.rb = nb - 1 - (id - nl);
    it.set = 0;
  }
  const int64_t end = min(S, p0 + (it.rb + 1) * kFiltRows);
  if (it.rb >= first_long) {
    it.k0 = it.set ? kmax : 0;
    it.k1 = it.set ? end : min(end, kmax);
  } else {
    it.k0 = 0;
    it.k1 = end;
  }
  return it;
}
inline int64_t filter_items(int64_t T, int64_t S) {
  const int64_t nb = (T + kFiltRows - 1) / kFiltRows;
  const int64_t first_long = filter_first_long(T, S);
  return nb + (nb > first_long ? nb - first_long : 0);
}

__global__ __launch_bounds__(256, 2) void idx_filter_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, int64_t T, int64_t S, const float* __restrict__ tau,
    uint2* __restrict__ cand, int32_t* __restrict__ cnt_out) {
  __shared__ __align__(16) uint8_t ktile[2][kFiltKeys * kIdxDim];
  __shared__ __align__(16) float kst[2][kFiltKeys];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const FilterItem item = filter_item(blockIdx.x, T, S);
  const int64_t R0 = item.rb * kFiltRows;
  const int64_t Q0 = R0 + 64 * w;   // the wave's first row
  const int64_t P0 = S - T + Q0;    // ... and its position

  v8i bq[4];
  int tq[4];
  float tv[4];
  uint32_t cnt[4];
  bool ovf[4];
  uint2* seg[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = Q0 + 16 * q + c;
    const bool ok = t < T;
    const int64_t tt = ok ? t : T - 1;
    bq[q] = *(const v8i*)(qf + tt * kIdxDim + 32 * g);
    tq[q] = ok ? (int)(S - T + t) : -1;  // key bound (position); an invalid query masks every key
    const float ta = tau[tt];
    // survivors need v * qs >= tau; shave a few ulps so rounding of the
    // product can never drop a key whose final score reaches tau
    tv[q] = !ok ? INFINITY : ta == -INFINITY ? -INFINITY : (ta / qs[tt]) * (1.0f - 1.0f / (1 << 20));
    cnt[q] = 0;
    ovf[q] = false;
    seg[q] = cand + ((tt * kSets + item.set) * kSeg + g) * (int64_t)kSegStride;
  }
  const int ntiles = (int)((item.k1 - item.k0 + kFiltKeys - 1) / kFiltKeys);

  // tile loader: 64 keys x 128 B = 512 chunks (2 per thread) + 64 scales
  auto issue = [&](int it, int buf) {
    const int64_t kb = item.k0 + (int64_t)it * kFiltKeys;
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
    const int64_t kb = item.k0 + (int64_t)it * kFiltKeys;
    if (it + 1 < ntiles) issue(it + 1, buf ^ 1);
    if (kb + kFiltKeys > S) {  // partial last tile: fill its scales by hand
      for (int i = threadIdx.x; i < kFiltKeys; i += 256) {
        const int64_t key = kb + i;
        if ((key & ~3LL) + 3 >= S) kst[buf][i] = key < S ? ks[key] : 0.f;
      }
      __syncthreads();
    }
    // a segment grows by at most 16 per tile: clamp once per tile into the
    // sink slots past kCap and remember the overflow
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cnt[q] > (uint32_t)kCap) {
        ovf[q] = true;
        cnt[q] = kCap;
      }
    }
    const bool mask = kb + kFiltKeys - 1 > P0;  // some key may lie past a query of this wave
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int k16 = (int)(kb + 16 * kt);
      const int rot = tile_rot(k16 >> 4);
      const int ar = (c + rot) & 15;                  // A row c holds key k16 + ar
      const v8i a = *(const v8i*)(ktile[buf] + (16 * kt + ar) * kIdxDim + 32 * g);
      v4f acc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[q] = mfma_fp8_16x16x128(a, bq[q], (v4f){0.f, 0.f, 0.f, 0.f});
      int key[4];
      float kss[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = (4 * g + i + rot) & 15;        // C row 4g+i holds key k16 + kr
        key[i] = k16 + kr;
        kss[i] = kst[buf][16 * kt + kr];
      }
      if (mask) {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = acc[q][i] * kss[i];
            const bool pass = (v >= tv[q]) & (key[i] <= tq[q]);
            if (pass) seg[q][cnt[q]] = make_uint2(__float_as_uint(v), (uint32_t)key[i]);
            cnt[q] += pass ? 1u : 0u;
          }
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float v = acc[q][i] * kss[i];
            const bool pass = v >= tv[q];
            if (pass) seg[q][cnt[q]] = make_uint2(__float_as_uint(v), (uint32_t)key[i]);
            cnt[q] += pass ? 1u : 0u;
          }
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  const bool two = item.rb >= filter_first_long(T, S);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (tq[q] < 0) continue;
    const int64_t t = Q0 + 16 * q + c;  // the row (tq holds its position)
    const int v = (ovf[q] || cnt[q] > (uint32_t)kCap) ? kCap + 1 : (int)cnt[q];
    cnt_out[(t * kSets + item.set) * kSeg + g] = v;
    if (!two) cnt_out[(t * kSets + 1) * kSeg + g] = 0;  // rows with one key chunk
  }
}

// ---- 3. exact select over survivors ---------------------------------------
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelMax = 6144;             // survivor slots a row may stage in LDS
constexpr int kChunk = 64;                // survivors per 512-byte direct-to-LDS copy
constexpr int kMaxChunks = kSelMax / kChunk;
constexpr int kMaxTies = 512;             // keys equal to the m-th best kept in a list

__global__ __launch_bounds__(kSelThreads) void idx_select_kernel(
    const float* __restrict__ qs, const float* __restrict__ tau, const uint2* __restrict__ cand,
    const int32_t* __restrict__ cnt_in, int64_t T, int64_t S, int64_t topk, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ fb, int force_fallback, DynK dyn) {
  extern __shared__ __align__(16) uint32_t sm[];
  uint2* cl = (uint2*)sm;                       // [kSelMax] (score key, position) pairs
  uint32_t* sel = sm + 2 * kSelMax;             // [nwords] bitmap of kept positions (or a long row's buckets)
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t wave_cnt[kSelWaves];
  __shared__ uint32_t s_sel[2];
  __shared__ int s_cnt[kSets * kSeg], s_cbase[kSets * kSeg + 1];
  __shared__ int32_t s_tie[kMaxTies];
  __shared__ int s_ntie, s_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t n = min(S - T + t + 1, S);
  int64_t m = min(topk, n);
  int32_t* o = idx_out + t * topk;
  if (n <= topk && !dyn_on(dyn)) {  // (a dynamic k scores short rows too: they keep every key as a survivor)
    for (int64_t i = tid; i < topk; i += kSelThreads) o[i] = i < n ? (int32_t)i : -1;
    return;
  }
  const float qsc = qs[t];
  const float tt = tau[t];
  const bool bucketed = n > kSelBitmapN;
  const int nwords = bucketed ? 0 : (int)((n + 31) >> 5);
  if (tid < kSets * kSeg) s_cnt[tid] = cnt_in[t * kSets * kSeg + tid];
  if (tid == 0) s_ntie = 0;
  for (int i = tid; i < nwords; i += kSelThreads) sel[i] = 0;
  __syncthreads();
  // chunk layout: segment gq owns chunks [s_cbase[gq], s_cbase[gq+1])
  if (tid == 0) {
    int nch = 0, bad = 0, total = 0;
    for (int gq = 0; gq < kSets * kSeg; ++gq) {
      const int cq = s_cnt[gq];
      if (cq > kCap) bad = 1;
      const int cv = cq > kCap ? kCap : cq;
      total += cv;
      s_cbase[gq] = nch;
      nch += (cv + kChunk - 1) / kChunk;
    }
    s_cbase[kSets * kSeg] = nch;
    s_bad = bad || nch > kMaxChunks || (tt == -INFINITY && total != n);
  }
  __syncthreads();
  if (s_bad || force_fallback) {
    if (tid == 0) fb[1 + atomicAdd(&fb[0], 1)] = (int32_t)t;
    return;
  }
  const int nch = s_cbase[kSets * kSeg];
  // stage: one 512-byte direct-to-LDS copy (32 lanes x 16 B) per chunk;
  // reads past a segment's count stay inside its kSegStride slots
  for (int ch = 2 * w + (lane >> 5); ch < nch; ch += 2 * kSelWaves) {
    int gq = 0;
    while (gq + 1 < kSets * kSeg && ch >= s_cbase[gq + 1]) ++gq;
    const int ofs = (ch - s_cbase[gq]) * kChunk;
    const uint2* src = cand + (t * kSets * kSeg + gq) * (int64_t)kSegStride + ofs + 2 * (lane & 31);
    __builtin_amdgcn_global_load_lds(
        (const void*)src,
        (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint2*)cl +
                                                  (ch & ~1) * kChunk),
        16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // final score u = v * qs with ReLU; invalid slots get key 0 (below every
  // real score key, all of which are >= key(+0.0))
  const int nslots = nch * kChunk;
  uint32_t nge = 0, mx = 0u, mn = 0xFFFFFFFFu;
  for (int e = tid; e < nslots; e += kSelThreads) {
    const int ch = e / kChunk;
    int gq = 0;
    while (gq + 1 < kSets * kSeg && ch >= s_cbase[gq + 1]) ++gq;
    const int valid = min(kChunk, min(s_cnt[gq], kCap) - (ch - s_cbase[gq]) * kChunk);
    const uint2 cv = cl[e];
    uint32_t key = 0;
    if ((e & (kChunk - 1)) < valid) {
      const float u0 = __uint_as_float(cv.x) * qsc;
      const float u = u0 > 0.f ? u0 : 0.f;
      key = score_key(u);
      nge += (u >= tt) ? 1u : 0u;
      mx = max(mx, key);
      mn = min(mn, key);
    }
    cl[e].x = key;
  }
  {
    nge = wave_sum(nge);
    mx = wave_max(mx);
    mn = wave_min(mn);
    if (lane == 0) {
      wave_cnt[w] = nge;
      hist[w] = mx;
      hist[16 + w] = mn;
    }
    __syncthreads();
    uint32_t tot = 0;
    mx = 0u;
    mn = 0xFFFFFFFFu;
    for (int i = 0; i < kSelWaves; ++i) {
      tot += wave_cnt[i];
      mx = max(mx, hist[i]);
      mn = min(mn, hist[16 + i]);
    }
    __syncthreads();
    // survivors reaching tau prove the answer is among them
    if (tt != -INFINITY && tot < (uint32_t)m) {
      if (tid == 0) fb[1 + atomicAdd(&fb[0], 1)] = (int32_t)t;
      return;
    }
  }
  // the m-th best key lies in [key(tau), max] (or [min, max] when every key
  // was kept)
  const uint32_t lo = tt != -INFINITY ? score_key(tt) : mn;
  auto key_at = [&](int64_t e) { return cl[e].x; };
  uint32_t thr = lo, need = 0;
  if (n > topk) radix_select<kSelThreads>(key_at, nslots, (uint32_t)m, lo, mx, hist, wave_cnt, s_sel, thr, need);
  // dynamic k: once the m-th best is at or below theta, every key above
  // theta is a survivor (the m-th best is >= tau)
  const int64_t mm = dyn_budget<kSelThreads>(key_at, nslots, m, thr, dyn, wave_cnt);
  if (n <= topk && mm == m) {
    for (int64_t i = tid; i < topk; i += kSelThreads) o[i] = i < n ? (int32_t)i : -1;
    return;
  }
  if (mm < m) {
    m = mm;
    if (m == 0) {
      for (int64_t i = tid; i < topk; i += kSelThreads) o[i] = -1;
      return;
    }
    radix_select<kSelThreads>(key_at, nslots, (uint32_t)m, lo, mx, hist, wave_cnt, s_sel, thr, need);
  }
  // keys above the m-th best go to the bitmap, ties to a list; a
  // pathological tie at the boundary is settled exactly elsewhere
  const bool ok = bucketed ? output_bucketed_from_candidates<kSelThreads>(cl, nslots, thr, need, n, m, topk, sel,
                                                                        s_tie, kMaxTies, &s_ntie, wave_cnt, o)
                          : output_from_candidates<kSelThreads>(cl, nslots, thr, need, n, m, topk, sel, nwords,
                                                                s_tie, kMaxTies, &s_ntie, wave_cnt, o, hist);
  if (!ok) {
    if (tid == 0) fb[1 + atomicAdd(&fb[0], 1)] = (int32_t)t;
  }
}

// ---- 4. exact fallback for rows the survivors cannot settle ---------------
constexpr int kFbBlocks = 64;

__global__ __launch_bounds__(kTopkThreads) void idx_fallback_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, int64_t S, int64_t p0, int64_t topk, const int32_t* __restrict__ fb,
    float* __restrict__ scratch, int32_t* __restrict__ idx_out, DynK dyn) {
  __shared__ TopkShared sh;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int nfb = fb[0];
  float* row = scratch + (int64_t)blockIdx.x * S;
  for (int f = blockIdx.x; f < nfb; f += gridDim.x) {
    const int64_t t = fb[1 + f];
    const int64_t n = min(p0 + t + 1, S);
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
    select_row(row, n, topk, idx_out + t * topk, sh, dyn);
    __syncthreads();
  }
}

size_t index_select_workspace_bytes(int64_t T, int64_t S) {
  size_t b = 0;
  auto add = [&](size_t x) { b += (x + 255) / 256 * 256; };
  add((size_t)T * 4);                       // tau
  add((size_t)T * kSets * kSeg * kSegStride * 8 + kChunk * 8);  // survivors (+ copy overrun pad)
  add((size_t)T * kSets * kSeg * 4);                // counts
  add((size_t)(T + 1) * 4);                 // fallback queue
  add((size_t)kFbBlocks * S * 4);           // fallback score rows
  return b;
}

bool index_select_supported(int64_t T, int64_t S) { return T >= 1 && S >= T && S <= (int64_t(1) << 31) - 1; }

hipError_t launch_index_select(const uint8_t* qf, const float* qs, const uint8_t* k8, const float* ks,
                               int64_t T, int64_t S, int64_t topk, int32_t* idx_out, void* ws,
                               bool force_fallback, hipStream_t st, DynK dyn) {
  if (T <= 0) return hipSuccess;
  char* p = (char*)ws;
  auto take = [&](size_t x) {
    char* q = p;
    p += (x + 255) / 256 * 256;
    return q;
  };
  float* tau = (float*)take((size_t)T * 4);
  uint2* cand = (uint2*)take((size_t)T * kSets * kSeg * kSegStride * 8 + kChunk * 8);
  int32_t* cnt = (int32_t*)take((size_t)T * kSets * kSeg * 4);
  int32_t* fb = (int32_t*)take((size_t)(T + 1) * 4);
  float* scratch = (float*)take((size_t)kFbBlocks * S * 4);
  zero_i32_kernel<<<1, 64, 0, st>>>(fb, 1);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  idx_estimate_kernel<<<(unsigned)((T + 15) / 16), kEstWaves * 64, 0, st>>>(qf, qs, k8, ks, T, S, topk, tau);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (sample_stride(S) > kRefStride) {
    idx_refine_kernel<<<(unsigned)((T + kRefRows - 1) / kRefRows), 256, 0, st>>>(qf, qs, k8, ks, T, S, topk, tau);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  idx_filter_kernel<<<(unsigned)filter_items(T, S), 256, 0, st>>>(qf, qs, k8, ks, T, S, tau, cand, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // bitmap words of the longest row with a bitmap, or the bucket pass's words
  const int64_t bn = S < kSelBitmapN ? S : kSelBitmapN;
  const int64_t words = S > kSelBitmapN && 2 * kOutBuckets > (bn + 31) / 32 ? 2 * kOutBuckets : (bn + 31) / 32;
  const size_t lds = (size_t)2 * kSelMax * 4 + (size_t)words * 4;
  static std::atomic<uint64_t> attr_done{0};
  e = set_lds_limit_once((const void*)idx_select_kernel, (int)(2 * kSelMax * 4 + (kSelBitmapN / 32) * 4), attr_done);
  if (e != hipSuccess) return e;
  idx_select_kernel<<<(unsigned)T, kSelThreads, lds, st>>>(qs, tau, cand, cnt, T, S, topk, idx_out, fb,
                                                          force_fallback ? 1 : 0, dyn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  idx_fallback_kernel<<<kFbBlocks, kTopkThreads, 0, st>>>(qf, qs, k8, ks, S, S - T, topk, fb, scratch, idx_out,
                                                          dyn);
  return hipGetLastError();
}

}  // namespace dsa
