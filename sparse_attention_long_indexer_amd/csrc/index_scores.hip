// Lightning-indexer scores, materialised (DeepSeek-V3.2 write-up, section
// 2.2: I[t,s] = ReLU(q_t . W_index . k_s) on 128-dim FP8 index vectors).
//
// With W folded into the query, one score is a single 128-wide e4m3 dot
// product, which is exactly one gfx950 v_mfma_f32_16x16x128_f8f6f4 per 16x16
// tile of (query, key) pairs.  Each wave keeps its 16 query rows in the A
// operand and streams 16-key B tiles straight from global memory (each lane
// loads 32 contiguous bytes of one key, so 4 lanes cover a 128-byte key row
// and a 16-key tile is one contiguous 2 KB block).  The epilogue applies the
// per-row and per-key fp32 scales, ReLU (+0.0 for u <= 0) and the causal mask
// (-inf for s > pos(t)).
//
// This path writes 4 bytes per score, so it is bound by HBM writes, not by
// the MFMA rate; the forward pass avoids it at long context.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr int kRowsPerBlock = 64;   // 4 waves x 16 rows
constexpr int kKeysPerBlock = 128;  // 8 MFMA tiles per wave

__global__ __launch_bounds__(256) void index_scores_fp8_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, int64_t S, const int64_t* __restrict__ q_pos, int64_t pos_base, int64_t row_begin,
    int64_t row_end, float* __restrict__ out, int64_t ld) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t rw = row_begin + (int64_t)blockIdx.y * kRowsPerBlock + w * 16;  // wave's first row
  if (rw >= row_end) return;
  const int64_t s0 = (int64_t)blockIdx.x * kKeysPerBlock;

  const int64_t ra = min(rw + c, row_end - 1);
  const v8i a = *(const v8i*)(qf + ra * kIdxDim + 32 * g);

  float qsc[4];
  int64_t pos[4];
  bool rok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = rw + 4 * g + i;
    rok[i] = r < row_end;
    const int64_t rr = rok[i] ? r : row_end - 1;
    qsc[i] = qs[rr];
    pos[i] = q_pos ? q_pos[rr] : pos_base + rr;
  }
#pragma unroll 2
  for (int j = 0; j < kKeysPerBlock / 16; ++j) {
    const int64_t s = s0 + 16 * j + c;
    const int64_t sb = s < S ? s : S - 1;
    const v8i b = *(const v8i*)(k + sb * kIdxDim + 32 * g);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_fp8_16x16x128(a, b, acc);
    const float kss = ks[sb];
    if (s < S) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (!rok[i]) continue;
        const int64_t r = rw + 4 * g + i;
        const float u = acc[i] * kss * qsc[i];
        const float v = (s <= pos[i]) ? (u > 0.f ? u : 0.f) : -INFINITY;
        out[(r - row_begin) * ld + s] = v;
      }
    }
  }
}

// fp32 operands (no quantisation): one thread per score, sequential fp32 FMA.
__global__ __launch_bounds__(256) void index_scores_f32_kernel(
    const float* __restrict__ qf, const float* __restrict__ k, int64_t S,
    const int64_t* __restrict__ q_pos, int64_t pos_base, int64_t row_begin, int64_t row_end, float* __restrict__ out,
    int64_t ld) {
  __shared__ float qt[16][kIdxDim + 1];
  __shared__ float kt[16][kIdxDim + 1];
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;
  const int64_t r0 = row_begin + (int64_t)blockIdx.y * 16, s0 = (int64_t)blockIdx.x * 16;
  for (int e = threadIdx.x; e < 16 * kIdxDim; e += 256) {
    const int rr = e / kIdxDim, cc = e % kIdxDim;
    const int64_t r = min<int64_t>(r0 + rr, row_end - 1);
    const int64_t s = min<int64_t>(s0 + rr, S - 1);
    qt[rr][cc] = qf[r * kIdxDim + cc];
    kt[rr][cc] = k[s * kIdxDim + cc];
  }
  __syncthreads();
  const int64_t r = r0 + ty, s = s0 + tx;
  if (r >= row_end || s >= S) return;
  float acc = 0.f;
#pragma unroll 8
  for (int j = 0; j < kIdxDim; ++j) acc = fmaf(qt[ty][j], kt[tx][j], acc);
  const int64_t p = q_pos ? q_pos[r] : pos_base + r;
  out[(r - row_begin) * ld + s] = (s <= p) ? (acc > 0.f ? acc : 0.f) : -INFINITY;
}

hipError_t launch_index_scores(const void* qf, const float* qs, const void* k, const float* ks,
                               bool fp8, int64_t T, int64_t S, const int64_t* q_pos, int64_t pos_base,
                               int64_t row_begin, int64_t row_end, float* out, int64_t ld,
                               hipStream_t st) {
  (void)T;
  const int64_t rows = row_end - row_begin;
  if (rows <= 0 || S <= 0) return hipSuccess;
  if (fp8) {
    dim3 grid((unsigned)((S + kKeysPerBlock - 1) / kKeysPerBlock),
              (unsigned)((rows + kRowsPerBlock - 1) / kRowsPerBlock));
    index_scores_fp8_kernel<<<grid, 256, 0, st>>>((const uint8_t*)qf, qs, (const uint8_t*)k, ks, S,
                                                   q_pos, pos_base, row_begin, row_end, out, ld);
  } else {
    dim3 grid((unsigned)((S + 15) / 16), (unsigned)((rows + 15) / 16));
    index_scores_f32_kernel<<<grid, 256, 0, st>>>((const float*)qf, (const float*)k, S, q_pos,
                                                   pos_base, row_begin, row_end, out, ld);
  }
  return hipGetLastError();
}

// ---- decode: one query per sequence against its own cache ----------------
//
// Bound by the HBM read of the cached index keys (132 bytes per key with its
// scale).  Block (x, b) covers 512 keys of sequence b, 128 per wave; the
// query row is replicated over the 16 A rows so every C row holds the same
// 16 scores.  Every key and scale load of a wave is issued before the first
// MFMA (clamped addresses, no branches), so each wave keeps 16 KB in flight.
constexpr int kDecWaveKeys = 128;
constexpr int kDecKeysPerBlock = 4 * kDecWaveKeys;

__global__ __launch_bounds__(256) void index_scores_decode_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const int64_t* __restrict__ off, float* __restrict__ out) {
  constexpr int J = kDecWaveKeys / 16;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t b = blockIdx.y;
  const int64_t lo = off[b], n = off[b + 1] - lo;
  const int64_t sw = (int64_t)blockIdx.x * kDecKeysPerBlock + w * kDecWaveKeys;
  if (sw >= n) return;
  v8i bb[J];
  float kss[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t s = sw + 16 * j + c;
    const int64_t sb = lo + (s < n ? s : n - 1);
    bb[j] = *(const v8i*)(k + sb * kIdxDim + 32 * g);
    kss[j] = ks[sb];
  }
  const v8i a = *(const v8i*)(qf + b * kIdxDim + 32 * g);
  const float qsc = qs[b];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int64_t s = sw + 16 * j + c;
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_fp8_16x16x128(a, bb[j], acc);
    if (g == 0 && s < n) {
      const float u = acc[0] * kss[j] * qsc;
      out[lo + s] = u > 0.f ? u : 0.f;
    }
  }
}

hipError_t launch_index_scores_decode(const uint8_t* qf, const float* qs, const uint8_t* k,
                                      const float* ks, const int64_t* offsets, int64_t B,
                                      int64_t max_len, float* out, hipStream_t st) {
  if (B <= 0 || max_len <= 0) return hipSuccess;
  dim3 grid((unsigned)((max_len + kDecKeysPerBlock - 1) / kDecKeysPerBlock), (unsigned)B);
  index_scores_decode_kernel<<<grid, 256, 0, st>>>(qf, qs, k, ks, offsets, out);
  return hipGetLastError();
}

}  // namespace dsa
