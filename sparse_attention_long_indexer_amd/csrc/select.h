// Row selection shared by the standalone top-k and the fused indexer's
// exact fallback.
#pragma once

#include "common.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr uint32_t kZeroKey = 0x80000000u;  // score_key(+0.0f)

struct TopkShared {
  uint32_t hist[256];
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

// Exact top-k of one row p[0..n) by (score desc, index asc), written in
// ascending index order to o[0..k) with -1 padding.  All kTopkThreads
// threads of the block call it; `sh` is block-shared scratch.
__device__ inline void select_row(const float* __restrict__ p, int64_t n, int64_t k, int32_t* __restrict__ o,
                           TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t m = n < k ? n : k;
  if (n <= k) {  // every key is kept
    for (int64_t i = tid; i < k; i += kTopkThreads) o[i] = i < n ? (int32_t)i : -1;
    return;
  }
  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)m;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) sh.hist[i] = 0;
    __syncthreads();
    const uint32_t zdig = (kZeroKey >> shift) & 255u;
    for (int64_t base = 0; base < n; base += kTopkThreads) {
      const int64_t i = base + tid;
      uint32_t key = 0;
      bool in = false;
      if (i < n) {
        key = score_key(p[i]);
        in = (key & mask) == prefix;
      }
      const bool z = in && key == kZeroKey;
      const uint64_t zb = ballot(z);
      if (in && !z) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
      if (zb && lane == 0) atomicAdd(&sh.hist[zdig], (uint32_t)__popcll(zb));
    }
    __syncthreads();
    // find the digit holding the remaining-th largest element (wave 0)
    if (tid < 64) {
      // lane handles digits 255-4*lane .. 252-4*lane (descending)
      uint32_t c4[4], sum = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = sh.hist[255 - 4 * tid - e];
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
          sh.sel[0] = 255u - 4u * tid - e;
          sh.sel[1] = above;
        }
        above += c4[e];
      }
    }
    __syncthreads();
    const uint32_t dig = sh.sel[0];
    remaining -= sh.sel[1];
    prefix |= dig << shift;
    mask |= 255u << shift;
    __syncthreads();
  }

  // ordered selection: keys > prefix, and the first `remaining` keys == prefix
  const uint32_t thr = prefix, need = remaining;
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
}


}  // namespace dsa
