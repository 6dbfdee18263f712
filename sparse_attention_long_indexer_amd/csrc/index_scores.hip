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
  if (row_end <= row_begin || S <= 0) return hipSuccess;
  // row blocks run along the grid's y extent (at most 65535 per launch)
  const int64_t per_block = fp8 ? kRowsPerBlock : 16;
  const int64_t per_launch = (int64_t)kMaxGridY * per_block;
  for (int64_t r0 = row_begin; r0 < row_end; r0 += per_launch) {
    const int64_t r1 = row_end - r0 < per_launch ? row_end : r0 + per_launch;
    float* o = out + (r0 - row_begin) * ld;
    if (fp8) {
      dim3 grid((unsigned)((S + kKeysPerBlock - 1) / kKeysPerBlock), (unsigned)((r1 - r0 + per_block - 1) / per_block));
      index_scores_fp8_kernel<<<grid, 256, 0, st>>>((const uint8_t*)qf, qs, (const uint8_t*)k, ks, S, q_pos,
                                                     pos_base, r0, r1, o, ld);
    } else {
      dim3 grid((unsigned)((S + 15) / 16), (unsigned)((r1 - r0 + per_block - 1) / per_block));
      index_scores_f32_kernel<<<grid, 256, 0, st>>>((const float*)qf, (const float*)k, S, q_pos, pos_base, r0, r1, o,
                                                     ld);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ---- decode: one query per sequence against its own cache ----------------
//
// Bound by the HBM read of the cached index keys (132 bytes per key with its
// scale).  The grid covers the concatenated caches of all sequences: block
// x covers flat keys 256 x .. +255, 64 per wave, so no block is spent on the
// gap between a short sequence and the longest one.  A wave copies its 64
// keys (8 KB, contiguous) straight into its own LDS region with eight 1 KB
// direct-to-LDS copies, each covering 8 whole key rows (8 lanes per 128-byte
// row), issued non-temporal since every cached key is read once per step;
// then reads them back in the MFMA's operand layout.  Within a row the
// 16-byte chunk j of key r sits in slot j ^ ((r >> 1) & 7), so that the 16
// lanes reading one chunk of 16 consecutive keys hit 16 distinct bank
// groups.  While the copies fly, the wave finds the sequence b0 of its first
// key (a ballot over 64 sequence ends at a time).  A wave inside one
// sequence replicates that query over the 16 A rows; a wave that straddles
// sequence ends gives A row c of each 16-key group the query of sequence
// (the group's first key's) + c, and each key takes the C row of its own
// sequence (every score is the same per-element MFMA dot product either
// way, so the scores match the prefill scores kernel bit for bit).
constexpr int kDecWaveKeys = 64;     // keys per wave (a straddling wave looks up one sequence end per lane)
constexpr int kDecKeysPerBlock = 4 * kDecWaveKeys;
constexpr int kNtAux = 2;            // cache-policy operand of the copies: 2 = non-temporal

__global__ __launch_bounds__(256) void index_scores_decode_kernel(
    const uint8_t* __restrict__ qf, const float* __restrict__ qs, const uint8_t* __restrict__ k,
    const float* __restrict__ ks, const int64_t* __restrict__ off, int64_t B, int64_t total,
    float* __restrict__ out) {
  constexpr int J = kDecWaveKeys / 16;   // 16-key MFMA groups per wave
  constexpr int NI = kDecWaveKeys / 8;   // 1 KB copies per wave
  __shared__ __align__(16) uint8_t kbuf[4][kDecWaveKeys * kIdxDim];
  __shared__ int64_t send[4][kDecWaveKeys + 1];   // a straddling wave's sequence ends
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t k0 = (int64_t)blockIdx.x * kDecKeysPerBlock + w * kDecWaveKeys;   // flat
  if (k0 >= total) return;
  // copy i: lane l brings chunk (l % 8) ^ f(r) of key r = 8 i + l / 8 (keys
  // past the last cached key read it again; their scores are dropped)
  {
    const int rl = lane >> 3;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = 8 * i + rl;
      const int64_t s = k0 + r;
      const int64_t sb = s < total ? s : total - 1;
      const int j = (lane & 7) ^ ((r >> 1) & 7);
      __builtin_amdgcn_global_load_lds(
          (const void*)(k + sb * kIdxDim + 16 * j),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) uint8_t*)kbuf[w] + 1024 * i),
          16, 0, kNtAux);
    }
  }
  float kss[J];
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int64_t s = k0 + 16 * jj + c;
    kss[jj] = __builtin_nontemporal_load(ks + (s < total ? s : total - 1));
  }
  // b0 = the sequence of key k0 = how many sequence ends off[1..B] are <= k0
  // (off[B] = total > k0, so the search ends in the round holding it)
  int64_t b0 = 0, e0 = total;
  for (int64_t base = 1; base <= B; base += 64) {
    const int64_t i = base + lane;
    const int64_t ov = i <= B ? off[i] : (int64_t)0x7FFFFFFFFFFFFFFFLL;
    const uint64_t le = ballot(ov <= k0);
    const int cnt = __popcll(le);
    b0 += cnt;
    if (cnt < 64) {
      const int lo32 = __shfl((int)(uint32_t)ov, cnt), hi32 = __shfl((int)(ov >> 32), cnt);
      e0 = (int64_t)(((uint64_t)(uint32_t)hi32 << 32) | (uint32_t)lo32);   // end of sequence b0
      break;
    }
  }
  __builtin_amdgcn_s_waitcnt(0);   // this wave's copies have landed (its own LDS region)
  auto keys_of = [&](int jj) {
    const int r = 16 * jj + c;
    const uint8_t* row = kbuf[w] + 1024 * (r >> 3) + 128 * (r & 7);
    const int f = (r >> 1) & 7;
    const v4i h0 = *(const v4i*)(row + 16 * ((2 * g) ^ f));
    const v4i h1 = *(const v4i*)(row + 16 * ((2 * g + 1) ^ f));
    return (v8i){h0[0], h0[1], h0[2], h0[3], h1[0], h1[1], h1[2], h1[3]};
  };
  if (e0 >= k0 + kDecWaveKeys) {
    // the whole wave lies in sequence b0
    const v8i a = *(const v8i*)(qf + b0 * kIdxDim + 32 * g);
    const float qsc = qs[b0];
#pragma unroll
    for (int jj = 0; jj < J; ++jj) {
      const int64_t s = k0 + 16 * jj + c;
      v4f acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma_fp8_16x16x128(a, keys_of(jj), acc);
      if (g == 0 && s < total) {
        const float u = acc[0] * kss[jj] * qsc;
        out[s] = u > 0.f ? u : 0.f;
      }
    }
    return;
  }
  // straddling wave: ends of sequences b0 .. b0 + 64 (at most 64 sequences
  // own its 64 keys), then per key its sequence by binary search
  int64_t* se = send[w];
  se[lane] = off[b0 + lane <= B ? b0 + lane : B];
  if (lane == 0) se[64] = off[b0 + 64 <= B ? b0 + 64 : B];
  __builtin_amdgcn_wave_barrier();
  auto seq_of = [&](int64_t p) {   // largest j with se[j] <= p, for se[0] <= p < se[64]
    int lo = 0, hi = 64;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (se[mid] <= p) lo = mid;
      else hi = mid;
    }
    return lo;
  };
#pragma unroll
  for (int jj = 0; jj < J; ++jj) {
    const int64_t s = k0 + 16 * jj + c;
    const int64_t sv = s < total ? s : total - 1;
    const int sq = seq_of(sv);                       // key's sequence - b0
    const int sa = __shfl(sq, 16 * g);               // the group's first key's (lane c = 0)
    const int64_t qa = b0 + sa + c < B ? b0 + sa + c : B - 1;
    const v8i a = *(const v8i*)(qf + qa * kIdxDim + 32 * g);
    v4f acc = {0.f, 0.f, 0.f, 0.f};
    acc = mfma_fp8_16x16x128(a, keys_of(jj), acc);
    const int d = sq - sa;                           // 0 .. 15: the key's C row
    if (s < total && (d >> 2) == g) {
      const int q = d & 3;
      const float v = q == 0 ? acc[0] : q == 1 ? acc[1] : q == 2 ? acc[2] : acc[3];
      const float u = v * kss[jj] * qs[b0 + sq];
      out[s] = u > 0.f ? u : 0.f;
    }
  }
}

hipError_t launch_index_scores_decode(const uint8_t* qf, const float* qs, const uint8_t* k,
                                      const float* ks, const int64_t* offsets, int64_t B,
                                      int64_t total_keys, float* out, hipStream_t st) {
  if (B <= 0 || total_keys <= 0) return hipSuccess;
  const int64_t blocks = (total_keys + kDecKeysPerBlock - 1) / kDecKeysPerBlock;
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  index_scores_decode_kernel<<<(unsigned)blocks, 256, 0, st>>>(qf, qs, k, ks, offsets, B, total_keys, out);
  return hipGetLastError();
}

}  // namespace dsa
