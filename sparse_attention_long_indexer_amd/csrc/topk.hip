// Per-row top-k selection over materialised scores (DeepSeek-V3.2 write-up,
// section 2.3: keep the k best-scoring keys of each query).
//
// One 1024-thread block per row.  Scores map to order-preserving uint32 keys
// (larger score -> larger key, -0.0 folded onto +0.0).  A most-significant-
// digit-first radix select with four 8-bit digits finds the exact key of the
// m-th best element and how many elements equal to it are kept; LDS
// histograms take one atomic per element, except the key of a zero score,
// which ReLU makes the common tie and which is counted with a wave ballot.
// A last pass walks the row in index order with block-wide prefix counts
// (wave ballots + per-wave totals in LDS), keeps every key above the
// threshold and the lowest-index keys equal to it, and writes the kept
// indices in ascending order.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kTopkThreads = 1024;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr uint32_t kZeroKey = 0x80000000u;  // score_key(+0.0f)

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
    const int64_t pos = R.q_pos ? R.q_pos[t] : t;
    int64_t n = pos + 1 < R.S ? pos + 1 : R.S;
    v.n = n > 0 ? n : 0;
    v.p = R.scores + (R.row_off ? R.row_off[row] : row * R.ld);
  }
  return v;
}

// Block-wide exclusive prefix count of `pred` (all threads must call).
// Returns the prefix; writes the block total to *total.
__device__ __forceinline__ uint32_t block_prefix(bool pred, uint32_t* wave_cnt, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const uint64_t m = ballot(pred);
  if (lane == 0) wave_cnt[w] = (uint32_t)__popcll(m);
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kTopkWaves; ++i) {
    const uint32_t c = wave_cnt[i];
    before += (i < w) ? c : 0u;
    all += c;
  }
  __syncthreads();
  *total = all;
  return before + lanes_below(m);
}

__global__ __launch_bounds__(kTopkThreads) void topk_radix_kernel(TopkRows R, int64_t k,
                                                                  int32_t* __restrict__ idx_out,
                                                                  int32_t* __restrict__ count_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t wave_cnt[kTopkWaves];
  __shared__ uint32_t s_sel[2];
  const int tid = threadIdx.x, lane = tid & 63;
  const int64_t row = blockIdx.x;
  const RowView rv = topk_row_view(R, row);
  const int64_t n = rv.n;
  const int64_t m = n < k ? n : k;
  int32_t* o = idx_out + row * k;
  if (count_out && tid == 0) count_out[row] = (int32_t)m;
  if (n <= k) {  // every key is kept
    for (int64_t i = tid; i < k; i += kTopkThreads) o[i] = i < n ? (int32_t)i : -1;
    return;
  }

  uint32_t prefix = 0, mask = 0, remaining = (uint32_t)m;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += kTopkThreads) hist[i] = 0;
    __syncthreads();
    const uint32_t zdig = (kZeroKey >> shift) & 255u;
    const bool zero_match = (kZeroKey & mask) == prefix;
    for (int64_t base = 0; base < n; base += kTopkThreads) {
      const int64_t i = base + tid;
      uint32_t key = 0;
      bool in = false;
      if (i < n) {
        key = score_key(rv.p[i]);
        in = (key & mask) == prefix;
      }
      const bool z = in && key == kZeroKey;
      const uint64_t zb = ballot(z);
      if (in && !z) atomicAdd(&hist[(key >> shift) & 255u], 1u);
      if (zb && lane == 0 && zero_match) atomicAdd(&hist[zdig], (uint32_t)__popcll(zb));
    }
    __syncthreads();
    // find the digit holding the remaining-th largest element (wave 0)
    if (tid < 64) {
      // lane handles digits 255-4*lane .. 252-4*lane (descending)
      uint32_t c4[4], s = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c4[e] = hist[255 - 4 * tid - e];
        s += c4[e];
      }
      // exclusive prefix over lanes (descending digits) via shuffles
      uint32_t incl = s;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t v = __shfl_up(incl, off);
        if (tid >= off) incl += v;
      }
      uint32_t above = incl - s;
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
    const uint32_t dig = s_sel[0];
    remaining -= s_sel[1];
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
    if (i < n) key = score_key(rv.p[i]);
    const bool gt = i < n && key > thr;
    const bool eq = i < n && key == thr;
    uint32_t tot_eq, tot_sel;
    const uint32_t eq_rank = carry_eq + block_prefix(eq, wave_cnt, &tot_eq);
    const bool sel = gt || (eq && eq_rank < need);
    const uint32_t p = carry_sel + block_prefix(sel, wave_cnt, &tot_sel);
    if (sel && p < (uint32_t)m) o[p] = (int32_t)i;
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  for (int64_t i = m + tid; i < k; i += kTopkThreads) o[i] = -1;
}

size_t topk_workspace_bytes(int64_t rows, int64_t max_n, int64_t k) {
  (void)rows;
  (void)max_n;
  (void)k;
  return 0;
}

hipError_t launch_topk(const TopkRows& r, int64_t rows, int64_t max_n, int64_t k, int32_t* idx_out,
                       int32_t* count_out, void* ws, hipStream_t st) {
  (void)max_n;
  (void)ws;
  if (rows <= 0) return hipSuccess;
  topk_radix_kernel<<<(unsigned)rows, kTopkThreads, 0, st>>>(r, k, idx_out, count_out);
  return hipGetLastError();
}

}  // namespace dsa
