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
//     score u = v * qs reaches tau).  Survivors (v, key) are appended to
//     the row's segment for that key chunk (one segment per row and chunk
//     keeps few partly written cache lines open at a time).
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

#include <climits>
#include <type_traits>

namespace dsa {

constexpr int kSeg = 1;                    // survivor segments per row and key chunk
constexpr int kCap = 6144;                 // survivors per segment
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
__global__ void zero_heads_kernel(int32_t* a, int32_t* b) {
  if (threadIdx.x == 0) {
    a[0] = 0;
    b[0] = 0;
  }
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
constexpr int kSetsMax = 8;               // key chunks per row (survivor sets), at most
constexpr int kSlack = 16;                // sink slots past kCap (one tile's worth per lane)
constexpr int kSegStride = kCap + kSlack;

// Work items: the keys are cut into ns chunks of kmax keys (a multiple of
// 256, kmax >= S / ns; ns = 2, 4 or 8, more for fewer row blocks, so that
// short prefills still fill the chip while long ones keep few survivor sets
// open per row); row block rb (rows [256 rb, 256 rb + 256) at
// positions p0 + row, p0 = S - T, seeing keys [0, end_rb) with end_rb =
// min(S, p0 + 256 (rb+1))) has one item per chunk it reaches, each with its
// own survivor set, so no item scans more than kmax keys and short prefills
// Items run in this order: the full chunks (chunk c
// of every row block that reaches chunk c + 1, c ascending, row blocks
// descending), then each row block's last, partial chunk (row blocks
// descending).  The last-chunk item of a row block also clears the counts
// of the sets its rows do not reach.
struct FilterItem {
  int64_t rb;    // row block
  int set;       // key chunk / survivor set
  int nsets;     // chunks row block rb reaches
  int64_t k0, k1;
};
__host__ __device__ inline int filter_nsets(int64_t T, int64_t S) {
  (void)S;
  const int64_t nb = (T + kFiltRows - 1) / kFiltRows;
  return nb >= 384 ? 2 : nb >= 192 ? 4 : kSetsMax;
}
__host__ __device__ inline int64_t filter_kmax(int64_t T, int64_t S) {
  const int ns = filter_nsets(T, S);
  const int64_t h = (S + ns - 1) / ns;
  return (h + kFiltRows - 1) / kFiltRows * kFiltRows;
}
// first row block whose key range passes j kmax (nb when none does)
__host__ __device__ inline int64_t filter_first_rb(int j, int64_t T, int64_t S) {
  const int64_t nb = (T + kFiltRows - 1) / kFiltRows;
  const int64_t kmax = filter_kmax(T, S), p0 = S - T, lim = (int64_t)j * kmax;
  if (S <= lim) return nb;
  const int64_t r = lim >= p0 ? (lim - p0) / kFiltRows : 0;
  return r < nb ? r : nb;
}
__host__ __device__ inline FilterItem filter_item(int64_t id, int64_t T, int64_t S) {
  const int64_t nb = (T + kFiltRows - 1) / kFiltRows;
  const int ns = filter_nsets(T, S);
  const int64_t kmax = filter_kmax(T, S), p0 = S - T;
  FilterItem it;
  int64_t base = 0;
  it.rb = -1;
  it.set = 0;
  for (int c = 0; c + 1 < ns; ++c) {
    const int64_t cnt = nb - filter_first_rb(c + 1, T, S);   // row blocks reaching chunk c + 1
    if (it.rb < 0 && id < base + cnt) {
      it.rb = nb - 1 - (id - base);
      it.set = c;
    }
    base += cnt;
  }
  const bool tail = it.rb < 0;
  if (tail) it.rb = nb - 1 - (id - base);
  const int64_t end = min(S, p0 + (it.rb + 1) * kFiltRows);
  it.nsets = (int)((end + kmax - 1) / kmax);
  if (tail) it.set = it.nsets - 1;
  it.k0 = (int64_t)it.set * kmax;
  it.k1 = min(end, it.k0 + kmax);
  return it;
}
__host__ __device__ inline int64_t filter_items(int64_t T, int64_t S) {
  const int64_t nb = (T + kFiltRows - 1) / kFiltRows;
  const int ns = filter_nsets(T, S);
  int64_t n = nb;
  for (int c = 1; c < ns; ++c) n += nb - filter_first_rb(c, T, S);
  return n;
}

// A block has kFiltWaves compute waves (64 query rows each) and one producer
// wave that alone moves key tiles into LDS (direct-to-LDS copies, three
// buffers, two tiles in flight) and waits for them; tiles are handed over
// with LDS-only barriers, so the compute waves never wait on their own
// global stores.
//
// Survivors leave the MFMA loop in two steps, so that the per-score work is
// a multiply and a third of a compare:
//  1. a lane's four scores of one MFMA result (one query, keys 4g .. 4g+3 of
//     a 16-key group) pass as a group when their maximum reaches the row's
//     threshold; passing groups take consecutive slots of the wave's LDS
//     ring (ballot + mbcnt): the four scores and a tag naming row and keys;
//  2. whenever the ring holds 64 groups, one flush round gives each lane a
//     group: it keeps the scores that pass exactly (threshold and causal
//     position), takes their places in the row's segment with one LDS
//     atomic, and stores them; a round's stores are 64 lanes wide.
// With kSeg > 1 the 16-key groups of every aligned 64-key block would go to
// the row's segments in an order rotated by a hash of the block.  One
// segment per row is the faster choice: the survivor stores of a block then
// keep 256 partly written cache lines open instead of 1024, so fewer lines
// leave the XCD's L2 before they fill (at 131072 tokens, 3.8 GB of
// survivors were written back as 10.6 GB with four segments, 8.6 GB with
// one).
constexpr int kFiltWaves = kFiltRows / 64;
constexpr int kFiltThreads = (kFiltWaves + 1) * 64;
constexpr int kFiltBufs = 3;
constexpr int kRing = 256;      // group slots per compute wave's ring
constexpr int kTileCopies = 9;  // copies per key tile: 8 of key bytes, 1 of scales

__device__ __forceinline__ int seg_of(uint32_t koff) {
  return (int)(((koff >> 4) + (((koff >> 6) * 0x9E3779B1u) >> 30)) & (uint32_t)(kSeg - 1));
}

__global__ __launch_bounds__(kFiltThreads, 4) void idx_filter_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k8,
    const float* __restrict__ ks, int64_t T, int64_t S, const float* __restrict__ tau,
    uint2* __restrict__ cand, int32_t* __restrict__ cnt_out) {
  __shared__ __align__(16) uint8_t ktile[kFiltBufs][kFiltKeys * kIdxDim];
  __shared__ __align__(16) float kst[kFiltBufs][kFiltKeys];
  __shared__ __align__(16) v4f vring[kFiltWaves][kRing];     // a group's four scores
  __shared__ uint32_t tring[kFiltWaves][kRing];              // ... and its tag
  __shared__ uint32_t rcnt[kFiltWaves][64 * kSeg];           // per (row of the wave, segment)
  __shared__ float tvtab[kFiltWaves][64];                    // per row: survivor threshold on v
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const FilterItem item = filter_item(blockIdx.x, T, S);
  const int ntiles = (int)((item.k1 - item.k0 + kFiltKeys - 1) / kFiltKeys);

  if (w == kFiltWaves) {
    // producer: tile j's 64 keys x 128 B = 512 16-byte chunks (8 per lane),
    // stored fragment-major: copy i = 2 kt + h puts, at LDS byte 1024 i +
    // 16 l, the 16 bytes lane l = (g, c) supplies as half h of its A operand
    // for key subtile kt (key kb + 16 kt + c, bytes 32 g + 16 h), so every
    // operand read is lane-linear (bank-conflict free); then one scale per
    // lane.  Keys past S are clamped to key S - 1 (the causal mask drops
    // them), so every tile is exactly kTileCopies copies and the memory
    // counter tells which tiles have landed.
    auto issue = [&](int it) {
      const int buf = it % kFiltBufs;
      const int64_t kb = item.k0 + (int64_t)it * kFiltKeys;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int kt = i >> 1, h = i & 1;
        const int64_t key = min(kb + 16 * kt + c, S - 1);
        __builtin_amdgcn_global_load_lds(
            (const void*)(k8 + key * kIdxDim + 32 * g + 16 * h),
            (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint8_t*)ktile[buf] +
                                                      i * 1024),
            16, 0, 0);
      }
      __builtin_amdgcn_global_load_lds(
          (const void*)(ks + min(kb + lane, S - 1)),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) float*)kst[buf]), 4, 0, 0);
    };
    // s_waitcnt vmcnt(kTileCopies): all but the last tile issued have landed
    constexpr int kWaitOneTile = 0x3F70 | (kTileCopies & 15) | ((kTileCopies >> 4) << 14);
    if (ntiles > 0) issue(0);
    if (ntiles > 1) {
      issue(1);
      __builtin_amdgcn_s_waitcnt(kWaitOneTile);
    } else {
      __builtin_amdgcn_s_waitcnt(0);
    }
    __builtin_amdgcn_s_barrier();
    // barrier it + 1 hands over tile it + 1 (the consumers are done reading
    // tile it - 1, whose buffer tile it + 2 reuses)
    for (int it = 0; it + 1 < ntiles; ++it) {
      if (it + 2 < ntiles) {
        issue(it + 2);
        __builtin_amdgcn_s_waitcnt(kWaitOneTile);
      } else {
        __builtin_amdgcn_s_waitcnt(0);
      }
      __builtin_amdgcn_s_barrier();
    }
    return;
  }

  const int64_t R0 = item.rb * kFiltRows;
  const int64_t Q0 = R0 + 64 * w;   // the wave's first row
  v4f* const vr = vring[w];
  uint32_t* const tr = tring[w];
  uint32_t* const rc = rcnt[w];
#pragma unroll
  for (int i = 0; i < kSeg; ++i) rc[i * 64 + lane] = 0u;

  v8i bq[4];
  int tq[4];
  float tv[4];
  int tvb[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t t = Q0 + 16 * q + c;
    const bool ok = t < T;
    const int64_t tt = ok ? t : T - 1;
    bq[q] = *(const v8i*)(qf + tt * kIdxDim + 32 * g);
    tq[q] = ok ? (int)(S - T + t) : -1;  // key bound (position); an invalid query masks every key
    const float ta = tau[tt];
    // survivors need v * qs >= tau; shave a few ulps so rounding of the
    // product can never drop a key whose final score reaches tau.  A row
    // that keeps every key gets -FLT_MAX: every finite score passes, a
    // masked (-inf) one does not
    tv[q] = !ok ? INFINITY : ta == -INFINITY ? -3.402823466e38f : (ta / qs[tt]) * (1.0f - 1.0f / (1 << 20));
    // the same test on the bit patterns as signed integers, exact for a
    // threshold >= +0 (negative scores and -inf order below every
    // non-negative float); a row that keeps every key lets every group in
    // and the flush's float compare drops its masked scores
    tvb[q] = tv[q] < 0.f ? INT_MIN : __float_as_int(tv[q]);
  }
  if (g == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) tvtab[w][16 * q + c] = tv[q];
  }
  // tag of a group: bits 0-5 its row within the wave (16 q + c), bits 6-7
  // its segment, bits 8-31 the key offset of its first key from the item's
  // first key.  The segment depends only on the 16-key step, so a step's
  // tags share one wave-uniform part.
  const uint32_t lane_tag = (uint32_t)((4 * g) << 8) | (uint32_t)c;
  uint32_t ptr = 0, tail = 0;   // ring write and flush counts (wave-uniform; slots modulo kRing)

  // one flush round: up to 64 ring groups, one per lane.  Keys past a row's
  // position never pass the float compare (the epilogue masks them to
  // -inf), so only the threshold is tested here; a segment's survivors past
  // kCap all land in its slot kCap (never read: the count reports the
  // overflow).
  const int ns = filter_nsets(T, S);   // survivor sets per row
  char* const wave_seg = (char*)(cand + (Q0 * ns + item.set) * kSeg * (int64_t)kSegStride);
  const uint32_t k0 = (uint32_t)item.k0;
  auto flush = [&](uint32_t n) {
    const v4f vv = vr[(tail + lane) & (kRing - 1)];
    const uint32_t tag = tr[(tail + lane) & (kRing - 1)];
    const uint32_t rl = tag & 63u, sg = (tag >> 6) & 3u;
    const float tvr = tvtab[w][rl];
    const bool live = (uint32_t)lane < n;
    bool p[4];
    uint32_t np = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = live & (vv[i] >= tvr);
      np += p[i] ? 1u : 0u;
    }
    uint32_t r = 0;
    if (np) r = atomicAdd(&rc[sg * 64 + rl], np);
    // segment (row Q0 + rl, this item's key chunk, sg) within the wave's rows
    const uint32_t seg = (rl * (uint32_t)(ns * kSeg) + sg) * (uint32_t)kSegStride;
    const uint32_t key0 = k0 + (tag >> 8);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (p[i]) {
        const uint32_t off = (seg + min(r, (uint32_t)kCap)) * 8u;
        *(uint2*)(wave_seg + off) = make_uint2(__float_as_uint(vv[i]), key0 + (uint32_t)i);
      }
      r += p[i] ? 1u : 0u;
    }
    tail += n;
  };

  // groups of one 16-key step of a tile: four MFMA results, one per query
  // group q, four scores per lane, taken in two halves of two q each: both
  // pass tests first, then one wave-uniform branch appends the passing
  // groups to the ring and flushes whole rounds.  On tiles that reach past
  // the wave's first row position (MASKED), scores of keys past a row's
  // position become -inf; key_lane is the key of the lane's first score.
  auto epilogue = [&](bool MASKED, const v4f (&acc)[4], const v4f& kss, uint32_t step_tag, int key_lane) {
#pragma unroll
    for (int q0 = 0; q0 < 4; q0 += 2) {
      v4f v[2];
      bool pass[2];
      uint64_t mk[2];
      uint32_t tot = 0;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = q0 + j;
        v[j] = (v4f){acc[q][0] * kss[0], acc[q][1] * kss[1], acc[q][2] * kss[2], acc[q][3] * kss[3]};
        if (MASKED) {
#pragma unroll
          for (int i = 0; i < 4; ++i) v[j][i] = key_lane + i <= tq[q] ? v[j][i] : -INFINITY;
        }
        const int mx = max(max(__float_as_int(v[j][0]), __float_as_int(v[j][1])),
                           max(__float_as_int(v[j][2]), __float_as_int(v[j][3])));
        pass[j] = mx >= tvb[q];
        mk[j] = ballot(pass[j]);
        tot += (uint32_t)__popcll(mk[j]);
      }
      // the ring is circular (positions modulo kRing): before each half at
      // most 63 groups are live, so the half's at most 128 new ones fit
      if (tot) {
        uint32_t base = ptr;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (pass[j]) {
            const uint32_t rank = (base + lanes_below(mk[j])) & (uint32_t)(kRing - 1);
            vr[rank] = v[j];
            tr[rank] = step_tag + (uint32_t)(16 * (q0 + j));
          }
          base += (uint32_t)__popcll(mk[j]);
        }
        ptr = base;
        while (ptr - tail >= 64u) flush(64u);
      }
    }
  };
  // one step's operands: A row c (key kb + 16 kt + c), bytes 32 g .. 32 g +
  // 31, in two lane-linear reads; the key scales of C rows 4g .. 4g+3
  auto rd = [&](int buf, int kt, v8i& a, v4f& kss) {
    const v4i a0 = *(const v4i*)(ktile[buf] + (2 * kt) * 1024 + 16 * lane);
    const v4i a1 = *(const v4i*)(ktile[buf] + (2 * kt + 1) * 1024 + 16 * lane);
    a = (v8i){a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    kss = *(const v4f*)(&kst[buf][16 * kt + 4 * g]);
  };
  auto mfmas = [&](const v8i& a, v4f (&acc)[4]) {
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] = mfma_fp8_16x16x128(a, bq[q], (v4f){0.f, 0.f, 0.f, 0.f});
  };

  // software pipeline over the four 16-key steps of each tile, two sets of
  // accumulators in turn: the MFMAs of step s + 1 and the operand reads of
  // step s + 2 are issued before the epilogue of step s (reads issued ahead
  // of the epilogue's ring writes do not wait behind them); the barrier
  // that hands over the next tile sits between the last read of one tile
  // and the first of the next (the epilogue only reads registers and the
  // wave's own ring)
  // tiles [0, nsafe) end at or below the wave's first row position
  const int64_t pq = S - T + Q0;
  const int nsafe = pq >= item.k0 ? (int)min((int64_t)ntiles, (pq - item.k0 + 1) / kFiltKeys) : 0;
  // wave-uniform tag part of step kt of tile it: key offset and segment
  auto step_tag = [&](int it, int kt) {
    const uint32_t koff = (uint32_t)(it * kFiltKeys + 16 * kt);
    return (koff << 8) | ((uint32_t)seg_of(koff) << 6);
  };
  lds_barrier();   // the producer's first tile
  v4f acc_a[4], acc_b[4], kss_a, kss_b, kss_n;
  v8i an;
  if (ntiles > 0) {
    rd(0, 0, an, kss_a);
    mfmas(an, acc_a);
    rd(0, 1, an, kss_n);
  }
  auto tile = [&](bool masked_c, int it) {
    const int key_lane = (int)(item.k0 + it * kFiltKeys + 4 * g);
    const bool more = it + 1 < ntiles;
    kss_b = kss_n;
    mfmas(an, acc_b);
    rd(it % kFiltBufs, 2, an, kss_n);
    epilogue(masked_c, acc_a, kss_a, step_tag(it, 0) + lane_tag, key_lane);
    kss_a = kss_n;
    mfmas(an, acc_a);
    rd(it % kFiltBufs, 3, an, kss_n);
    epilogue(masked_c, acc_b, kss_b, step_tag(it, 1) + lane_tag, key_lane + 16);
    kss_b = kss_n;
    mfmas(an, acc_b);
    if (more) {
      lds_barrier();   // done with tile it; tile it + 1 has landed
      rd((it + 1) % kFiltBufs, 0, an, kss_n);
    }
    epilogue(masked_c, acc_a, kss_a, step_tag(it, 2) + lane_tag, key_lane + 32);
    if (more) {
      kss_a = kss_n;
      mfmas(an, acc_a);
      rd((it + 1) % kFiltBufs, 1, an, kss_n);
    }
    epilogue(masked_c, acc_b, kss_b, step_tag(it, 3) + lane_tag, key_lane + 48);
  };
  for (int it = 0; it < ntiles; ++it) {
    tile(it >= nsafe, it);
  }
  if (ptr != tail) flush(ptr - tail);

  const bool last = item.set == item.nsets - 1;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (tq[q] < 0) continue;
    const int rl = 16 * q + c;
    const int64_t t = Q0 + rl;
    // lane group g reports segment g of its rows
    if (g >= kSeg) continue;
    const uint32_t n = rc[g * 64 + rl];
    cnt_out[(t * ns + item.set) * kSeg + g] = n > (uint32_t)kCap ? kCap + 1 : (int)n;
    if (last) {  // sets of chunks this row block does not reach
      for (int sx = item.set + 1; sx < ns; ++sx) cnt_out[(t * ns + sx) * kSeg + g] = 0;
    }
  }
}

// ---- 3. exact select over survivors ---------------------------------------
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / 64;
constexpr int kSelMax = 6144;             // survivor slots a row may hold
constexpr int kChunk = 64;                // survivors per 512-byte direct-to-LDS copy
constexpr int kMaxChunks = kSelMax / kChunk;
constexpr int kMaxTies = 512;             // keys equal to the m-th best kept in a list
constexpr int kGenericBlocks = 512;       // persistent grid of the generic select

// 3a. Fast path, one block per row.  Every thread holds up to kSfPer of the
// row's survivors in registers (final score key, position).  One histogram
// of kSfBins bins spanning [lo, hi] (lo = the key of the row's threshold,
// or its smallest key when the row kept every key; hi = its largest key)
// finds the bin b of the m-th best key.  Every key in a bin above b is kept;
// the keys in b (at most kSfList) are ranked among themselves under (score
// desc, position asc) and the first m - #(keys above b) of them are kept.
// Kept positions are marked in a bitmap over the row's positions, whose
// prefix popcounts give the ascending output.  Rows this path does not
// settle go to a queue for the generic select (3b): a dynamic k, rows past
// the bitmap length, m above kSfBins, a boundary bin fuller than kSfList.
// Rows whose survivors cannot hold the answer (a segment past capacity,
// more than kSelMax survivors, fewer than m survivors at the threshold) go
// to the exact fallback (4).
constexpr int kSfThreads = 512;
constexpr int kSfWaves = kSfThreads / 64;
constexpr int kSfPer = kSelMax / kSfThreads;
constexpr int kSfBins = 2048;
constexpr int kSfList = 512;
static_assert(kSfPer * kSfThreads == kSelMax, "threads must divide the survivor slots");
static_assert(kSfBins == 4 * kSfThreads, "the bin scan gives each thread four bins");

// NSEG: survivor segments per row (filter_nsets(T, S) * kSeg; the launcher
// picks the instantiation)
template <int NSEG>
__global__ __launch_bounds__(kSfThreads) void idx_select_fast_kernel(
    const float* __restrict__ qs, const float* __restrict__ tau, const uint2* __restrict__ cand,
    const int32_t* __restrict__ cnt_in, int64_t T, int64_t S, int64_t topk, int32_t* __restrict__ idx_out,
    int32_t* __restrict__ gq, int32_t* __restrict__ fb, int force_fallback, DynK dyn) {
  extern __shared__ __align__(16) uint32_t bitmap[];  // [(n + 31) / 32] kept positions
  __shared__ uint32_t hist[kSfBins];                   // bin counts, then the staged output
  __shared__ uint32_t lkey[kSfList];
  __shared__ int32_t lpos[kSfList];
  __shared__ uint32_t red[4][kSfWaves];
  __shared__ uint32_t s_bin, s_above, s_nlist;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t t = blockIdx.x;
  const int64_t n = min(S - T + t + 1, S);
  const int64_t m = min(topk, n);
  int32_t* o = idx_out + t * topk;
  if (n <= topk && !dyn_on(dyn)) {  // every key is kept
    for (int64_t i = tid; i < topk; i += kSfThreads) o[i] = i < n ? (int32_t)i : -1;
    return;
  }
  auto defer = [&](int32_t* q) {
    if (tid == 0) q[1 + atomicAdd(&q[0], 1)] = (int32_t)t;
  };
  if (force_fallback) {
    defer(fb);
    return;
  }
  if (dyn_on(dyn) || n > kSelBitmapN || m > kSfBins) {
    defer(gq);
    return;
  }
  // segment starts in the concatenation of the row's segments
  int cb[NSEG + 1];
  bool over = false;
  cb[0] = 0;
#pragma unroll
  for (int g = 0; g < NSEG; ++g) {
    const int c = cnt_in[t * NSEG + g];
    over |= c > kCap;
    cb[g + 1] = cb[g] + (c > kCap ? kCap : c);
  }
  const int total = cb[NSEG];
  const float tt = tau[t];
  if (over || total > kSelMax || (tt == -INFINITY && total != n)) {
    defer(fb);
    return;
  }
  // load: slot e = tid + kSfThreads j of the concatenation; final score
  // u = v * qs with ReLU, as a score key
  const float qsc = qs[t];
  uint32_t key[kSfPer];
  int32_t pos[kSfPer];
#pragma unroll
  for (int j = 0; j < kSfPer; ++j) {
    const int e = tid + kSfThreads * j;
    int g = 0, start = 0;
#pragma unroll
    for (int i = 1; i < NSEG; ++i)
      if (e >= cb[i]) {
        g = i;
        start = cb[i];
      }
    uint2 cv = make_uint2(0u, 0xFFFFFFFFu);
    if (e < total) cv = cand[(t * NSEG + g) * (int64_t)kSegStride + (e - start)];
    const float u0 = __uint_as_float(cv.x) * qsc;
    const bool ok = e < total && (int32_t)cv.y >= 0 && (int64_t)(int32_t)cv.y < n;
    key[j] = ok ? score_key(u0 > 0.f ? u0 : 0.f) : 0u;   // 0 is below every real key
    pos[j] = ok ? (int32_t)cv.y : -1;
  }
  // range of the keys and the count at or above the threshold; a row that
  // kept every key is ranked over its positive scores (lo = its smallest
  // positive key) when at least m of them are positive
  const uint32_t lo_t = tt != -INFINITY ? score_key(tt) : kZeroKey + 1u;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu, nge = 0u;
#pragma unroll
  for (int j = 0; j < kSfPer; ++j) {
    if (pos[j] >= 0) {
      mx = max(mx, key[j]);
      nge += key[j] >= lo_t ? 1u : 0u;
      if (key[j] >= lo_t) mn = min(mn, key[j]);
    }
  }
  mx = wave_max_u32(mx);
  mn = wave_min_u32(mn);
  nge = wave_sum_u32(nge);
  if (lane == 0) {
    red[0][w] = mx;
    red[1][w] = mn;
    red[2][w] = nge;
  }
  const int nwords = (int)((n + 127) >> 7) * 4;   // whole 16-byte groups
  for (int i = tid; i < kSfBins; i += kSfThreads) hist[i] = 0u;
  for (int i = tid; i < nwords; i += kSfThreads) bitmap[i] = 0u;
  if (tid == 0) s_nlist = 0u;
  __syncthreads();
  mx = 0u;
  mn = 0xFFFFFFFFu;
  nge = 0u;
#pragma unroll
  for (int i = 0; i < kSfWaves; ++i) {
    mx = max(mx, red[0][i]);
    mn = min(mn, red[1][i]);
    nge += red[2][i];
  }
  // survivors at the threshold must hold the m best
  if (tt != -INFINITY && nge < (uint32_t)m) {
    defer(fb);
    return;
  }
  const int ngrp = nwords >> 2;
  const int per = (ngrp + kSfThreads - 1) / kSfThreads;
  const int g0 = tid * per, g1 = min(ngrp, g0 + per);
  uint4* const bm4 = (uint4*)bitmap;
  if (nge < (uint32_t)m) {
    // a row that kept every key with fewer than m positive scores: every
    // positive score is kept, and the m - nge lowest positions scoring zero
#pragma unroll
    for (int j = 0; j < kSfPer; ++j)
      if (pos[j] >= 0 && key[j] >= lo_t) atomicOr(&bitmap[pos[j] >> 5], 1u << (pos[j] & 31));
    __syncthreads();
    // zeros (unset positions below n) per run of groups, then their prefix
    uint32_t z = 0u;
    for (int i = g0; i < g1; ++i) {
      const uint4 q = bm4[i];
      const int64_t b0 = (int64_t)i * 128;
      const uint32_t valid = (uint32_t)(n - b0 >= 128 ? 128 : (n > b0 ? n - b0 : 0));
      z += valid - (uint32_t)(__popc(q.x) + __popc(q.y) + __popc(q.z) + __popc(q.w));
    }
    const uint32_t zincl = wave_incl_scan(z);
    if (lane == 63) red[3][w] = zincl;
    __syncthreads();
    uint32_t zr = zincl - z;
#pragma unroll
    for (int i = 0; i < kSfWaves; ++i) zr += i < w ? red[3][i] : 0u;
    const uint32_t need0 = (uint32_t)m - nge;
    for (int i = g0; i < g1 && zr < need0; ++i) {
      for (int e = 0; e < 4 && zr < need0; ++e) {
        const int wi = 4 * i + e;
        const int64_t b0 = (int64_t)wi * 32;
        const uint32_t inrow = n - b0 >= 32 ? 0xFFFFFFFFu : (n > b0 ? (1u << (n - b0)) - 1u : 0u);
        uint32_t zb = ~bitmap[wi] & inrow, keep = 0u;
        while (zb && zr < need0) {
          const uint32_t bit = zb & (0u - zb);
          keep |= bit;
          ++zr;
          zb ^= bit;
        }
        bitmap[wi] |= keep;   // this thread alone owns word wi
      }
    }
    __syncthreads();
  } else {
    const uint32_t lo = tt != -INFINITY ? lo_t : mn;
    const uint32_t span = mx - lo;
    const int top = span ? 31 - __builtin_clz(span) : 0;
    const int sh = top > 10 ? top - 10 : 0;   // (span >> sh) < kSfBins
#pragma unroll
    for (int j = 0; j < kSfPer; ++j)
      if (pos[j] >= 0 && key[j] >= lo) atomicAdd(&hist[(key[j] - lo) >> sh], 1u);
    __syncthreads();
    // bin of the m-th best: descending scan, thread tid owns bins
    // kSfBins - 1 - 4 tid - e
    uint32_t c4[4], own = 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      c4[e] = hist[kSfBins - 1 - 4 * tid - e];
      own += c4[e];
    }
    uint32_t incl = wave_incl_scan(own);
    if (lane == 63) red[3][w] = incl;
    __syncthreads();
    uint32_t above = incl - own;
#pragma unroll
    for (int i = 0; i < kSfWaves; ++i) above += i < w ? red[3][i] : 0u;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (above < (uint32_t)m && (uint32_t)m <= above + c4[e]) {
        s_bin = (uint32_t)(kSfBins - 1 - 4 * tid - e);
        s_above = above;
      }
      above += c4[e];
    }
    __syncthreads();
    const uint32_t bb = s_bin, remaining = (uint32_t)m - s_above, nl = hist[bb];
    if (nl > (uint32_t)kSfList) {
      defer(gq);
      return;
    }
    // keys above the boundary bin are kept; the boundary bin goes to the list
#pragma unroll
    for (int j = 0; j < kSfPer; ++j) {
      if (pos[j] < 0 || key[j] < lo) continue;
      const uint32_t b = (key[j] - lo) >> sh;
      if (b > bb) {
        atomicOr(&bitmap[pos[j] >> 5], 1u << (pos[j] & 31));
      } else if (b == bb) {
        const uint32_t i = atomicAdd(&s_nlist, 1u);
        lkey[i] = key[j];
        lpos[i] = pos[j];
      }
    }
    __syncthreads();
    for (int i = tid; i < (int)nl; i += kSfThreads) {
      const uint32_t ki = lkey[i];
      const int32_t pi = lpos[i];
      uint32_t r = 0u;
      for (int j = 0; j < (int)nl; ++j) {
        const uint32_t kj = lkey[j];
        r += (kj > ki || (kj == ki && lpos[j] < pi)) ? 1u : 0u;
      }
      if (r < remaining) atomicOr(&bitmap[pi >> 5], 1u << (pi & 31));
    }
    __syncthreads();
  }
  // ascending output: prefix popcounts over runs of `per` 16-byte groups per
  // thread, staged in hist (m <= kSfBins) for one coalesced copy
  uint32_t mine = 0u;
  for (int i = g0; i < g1; ++i) {
    const uint4 q = bm4[i];
    mine += __popc(q.x) + __popc(q.y) + __popc(q.z) + __popc(q.w);
  }
  const uint32_t incl = wave_incl_scan(mine);
  if (lane == 63) red[0][w] = incl;
  __syncthreads();
  uint32_t at = incl - mine;
#pragma unroll
  for (int i = 0; i < kSfWaves; ++i) at += i < w ? red[0][i] : 0u;
  for (int i = g0; i < g1; ++i) {
    const uint4 q = bm4[i];
    const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      uint32_t wv = qw[e];
      while (wv) {
        const int b = __builtin_ctz(wv);
        if (at < (uint32_t)m) hist[at] = (uint32_t)((4 * i + e) * 32 + b);
        ++at;
        wv &= wv - 1;
      }
    }
  }
  __syncthreads();
  for (int64_t i = tid; i < topk; i += kSfThreads) o[i] = i < m ? (int32_t)hist[i] : -1;
}

// 3b. Generic select for the rows the fast path queued: the survivors are
// staged in LDS, a radix select over them finds the m-th best (and a
// dynamic k's budget), and the output goes through a bitmap (or buckets for
// rows past the bitmap length).  A persistent grid walks the queue.
__device__ inline void select_generic_row(
    int64_t t, uint32_t* sm, const float* __restrict__ qs, const float* __restrict__ tau,
    const uint2* __restrict__ cand, const int32_t* __restrict__ cnt_in, int64_t T, int64_t S, int64_t topk,
    int32_t* __restrict__ idx_out, int32_t* __restrict__ fb, DynK dyn) {
  uint2* cl = (uint2*)sm;                       // [kSelMax] (score key, position) pairs
  uint32_t* sel = sm + 2 * kSelMax;             // [nwords] bitmap of kept positions (or a long row's buckets)
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t wave_cnt[kSelWaves];
  __shared__ uint32_t s_sel[2];
  __shared__ int s_cnt[kSetsMax * kSeg], s_cbase[kSetsMax * kSeg + 1];
  __shared__ int32_t s_tie[kMaxTies];
  __shared__ int s_ntie, s_bad;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
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
  const int nseg = filter_nsets(T, S) * kSeg;
  if (tid < nseg) s_cnt[tid] = cnt_in[t * nseg + tid];
  if (tid == 0) s_ntie = 0;
  for (int i = tid; i < nwords; i += kSelThreads) sel[i] = 0;
  __syncthreads();
  // chunk layout: segment gq owns chunks [s_cbase[gq], s_cbase[gq+1])
  if (tid == 0) {
    int nch = 0, bad = 0, total = 0;
    for (int gq = 0; gq < nseg; ++gq) {
      const int cq = s_cnt[gq];
      if (cq > kCap) bad = 1;
      const int cv = cq > kCap ? kCap : cq;
      total += cv;
      s_cbase[gq] = nch;
      nch += (cv + kChunk - 1) / kChunk;
    }
    s_cbase[nseg] = nch;
    s_bad = bad || nch > kMaxChunks || (tt == -INFINITY && total != n);
  }
  __syncthreads();
  if (s_bad) {
    if (tid == 0) fb[1 + atomicAdd(&fb[0], 1)] = (int32_t)t;
    return;
  }
  const int nch = s_cbase[nseg];
  // stage: one 512-byte direct-to-LDS copy (32 lanes x 16 B) per chunk;
  // reads past a segment's count stay inside its kSegStride slots
  for (int ch = 2 * w + (lane >> 5); ch < nch; ch += 2 * kSelWaves) {
    int gq = 0;
    while (gq + 1 < nseg && ch >= s_cbase[gq + 1]) ++gq;
    const int ofs = (ch - s_cbase[gq]) * kChunk;
    const uint2* src = cand + (t * nseg + gq) * (int64_t)kSegStride + ofs + 2 * (lane & 31);
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
    while (gq + 1 < nseg && ch >= s_cbase[gq + 1]) ++gq;
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

__global__ __launch_bounds__(kSelThreads) void idx_select_generic_kernel(
    const float* __restrict__ qs, const float* __restrict__ tau, const uint2* __restrict__ cand,
    const int32_t* __restrict__ cnt_in, int64_t T, int64_t S, int64_t topk, int32_t* __restrict__ idx_out,
    const int32_t* __restrict__ gq, int32_t* __restrict__ fb, DynK dyn) {
  extern __shared__ __align__(16) uint32_t sm[];
  const int nq = gq[0];
  for (int f = blockIdx.x; f < nq; f += gridDim.x) {
    select_generic_row(gq[1 + f], sm, qs, tau, cand, cnt_in, T, S, topk, idx_out, fb, dyn);
    __syncthreads();   // LDS is reused by the next row
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
  add((size_t)T * filter_nsets(T, S) * kSeg * kSegStride * 8 + kChunk * 8);  // survivors (+ copy overrun pad)
  add((size_t)T * filter_nsets(T, S) * kSeg * 4);                             // counts
  add((size_t)(T + 1) * 4);                 // fallback queue
  add((size_t)(T + 1) * 4);                 // generic-select queue
  add((size_t)kFbBlocks * S * 4);           // fallback score rows
  return b;
}

// survivor tags hold key offsets below kmax in 24 bits
bool index_select_supported(int64_t T, int64_t S) { return T >= 1 && S >= T && S <= (int64_t(1) << 25); }

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
  uint2* cand = (uint2*)take((size_t)T * filter_nsets(T, S) * kSeg * kSegStride * 8 + kChunk * 8);
  int32_t* cnt = (int32_t*)take((size_t)T * filter_nsets(T, S) * kSeg * 4);
  int32_t* fb = (int32_t*)take((size_t)(T + 1) * 4);
  int32_t* gq = (int32_t*)take((size_t)(T + 1) * 4);
  float* scratch = (float*)take((size_t)kFbBlocks * S * 4);
  DSA_DEBUG_CHECK((size_t)(p - (char*)ws) <= index_select_workspace_bytes(T, S));
  DSA_DEBUG_CHECK(filter_items(T, S) >= 1 && filter_items(T, S) <= INT32_MAX);
  zero_heads_kernel<<<1, 64, 0, st>>>(fb, gq);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  idx_estimate_kernel<<<(unsigned)((T + 15) / 16), kEstWaves * 64, 0, st>>>(qf, qs, k8, ks, T, S, topk, tau);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (sample_stride(S) > kRefStride) {
    idx_refine_kernel<<<(unsigned)((T + kRefRows - 1) / kRefRows), 256, 0, st>>>(qf, qs, k8, ks, T, S, topk, tau);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  idx_filter_kernel<<<(unsigned)filter_items(T, S), kFiltThreads, 0, st>>>(qf, qs, k8, ks, T, S, tau, cand, cnt);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // bitmap words of the longest row with a bitmap, or the bucket pass's words
  const int64_t bn = S < kSelBitmapN ? S : kSelBitmapN;
  const int64_t words = S > kSelBitmapN && 2 * kOutBuckets > (bn + 31) / 32 ? 2 * kOutBuckets : (bn + 31) / 32;
  const size_t lds_fast = (size_t)((bn + 127) / 128) * 16;
  const size_t lds = (size_t)2 * kSelMax * 4 + (size_t)words * 4;
  static std::atomic<uint64_t> attr_done{0};
  e = set_lds_limit_once((const void*)idx_select_generic_kernel, (int)(2 * kSelMax * 4 + (kSelBitmapN / 32) * 4),
                         attr_done);
  if (e != hipSuccess) return e;
  {
    static_assert(kSeg == 1, "the select instantiations cover 2, 4 and 8 segments per row");
    const int nseg = filter_nsets(T, S) * kSeg;
    const int ff = force_fallback ? 1 : 0;
    if (nseg == 2)
      idx_select_fast_kernel<2><<<(unsigned)T, kSfThreads, lds_fast, st>>>(qs, tau, cand, cnt, T, S, topk, idx_out,
                                                                            gq, fb, ff, dyn);
    else if (nseg == 4)
      idx_select_fast_kernel<4><<<(unsigned)T, kSfThreads, lds_fast, st>>>(qs, tau, cand, cnt, T, S, topk, idx_out,
                                                                            gq, fb, ff, dyn);
    else
      idx_select_fast_kernel<kSetsMax * kSeg><<<(unsigned)T, kSfThreads, lds_fast, st>>>(
          qs, tau, cand, cnt, T, S, topk, idx_out, gq, fb, ff, dyn);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned gen_blocks = (unsigned)(T < kGenericBlocks ? T : kGenericBlocks);
  idx_select_generic_kernel<<<gen_blocks, kSelThreads, lds, st>>>(qs, tau, cand, cnt, T, S, topk, idx_out, gq, fb,
                                                                 dyn);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  idx_fallback_kernel<<<kFbBlocks, kTopkThreads, 0, st>>>(qf, qs, k8, ks, S, S - T, topk, fb, scratch, idx_out,
                                                          dyn);
  return hipGetLastError();
}

}  // namespace dsa
