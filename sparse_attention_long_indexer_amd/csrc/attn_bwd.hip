// Backward pass of the sparse MQA attention (DeepSeek-V3.2 write-up,
// section 4.1: the sparse training stage trains the whole model through
// attention over the selected keys).  For query t, head h and its selected
// latent rows s_j (K = row[:Dk], V = row[:Dv]):
//   P[h,j]  = exp(scale q_h . K_j - lse_h)            (the forward's softmax)
//   dS[h,j] = scale P[h,j] (dO_h . V_j - Delta_h),    Delta_h = dO_h . O_h
//   dq_h    = sum_j dS[h,j] K_j
//   dkv[s_j] += sum_h dS[h,j] q_h  (+ sum_h P[h,j] dO_h in the first Dv columns)
// Three kernels per chunk of queries, all bf16 MFMA (16x16x32):
//   1. ds: one block per query, 16 heads per wave, recomputes S^T = K . Q^T
//      and dP^T = V . dO^T over gathered key tiles (V is the first Dv columns
//      of the same LDS tile, so one K fragment feeds both products) and
//      writes P and dS (bf16) for every (key, head) to the workspace;
//   2. dq: one block per query, dq[16 heads x Dk] per wave = dS . K over the
//      same gathered tiles, both operands by transposed LDS reads;
//   3. dkv: one block per query, 48 latent columns per wave, dkv tile =
//      dS^T . q + P^T . dO with q and dO held in registers (heads on the
//      reduction axis) and P / dS tiles staged in LDS; each (key, column) is
//      added to the fp32 dkv accumulator with one hardware float atomic.
// The row sums over heads (dk, dv) are what make per-query blocks need
// atomics: a latent row is selected by many queries.
#include "common.h"
#include "dsa.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kBH = 128;   // heads
constexpr int kBNK = 32;   // keys per tile
constexpr float kBLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) char lds_c;
typedef __attribute__((address_space(3))) v4s lds_v4;

__device__ __forceinline__ void lds_dma16(const void* src, char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (lds_c*)lds_dst, 16, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, result lane i receives
// element i % 4 of the 4-element chunks addressed by source lanes i/4,
// i/4 + 4, i/4 + 8 and i/4 + 12, in that order
__device__ __forceinline__ v4s lds_read_tr16(const char* lds_base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)((lds_c*)lds_base + byte_off));
}

// two transposed reads (ds_read_b64_tr_b16): lane (c, g) receives column
// c0 + c of rows r0 + 8g .. r0 + 8g + 7 of a row-major bf16 matrix at `base`
// with row stride `rs` bytes -- the 8 reduction values an MFMA operand lane
// supplies when the reduction runs along the rows
__device__ __forceinline__ v8s tr_operand(const char* base, int rs, int r0, int c0) {
  const int lane = threadIdx.x & 63, g = lane >> 4, c = lane & 15;
  const int off = (r0 + 8 * g + (c >> 2)) * rs + (c0 + 4 * (c & 3)) * 2;
  const v4s lo = lds_read_tr16(base, off);
  const v4s hi = lds_read_tr16(base, off + 4 * rs);
  return (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Stage the query's index row: sidx[j] = its latent row (invalid entries
// and entries past the first -1 map to row 0); returns n, the leading valid
// entries.  All threads call.
__device__ __forceinline__ int stage_index(const BwdArgs& a, int64_t t, int32_t* sidx, int* s_cnt) {
  const int32_t* ip = a.idx + t * a.k;
  if (threadIdx.x == 0) *s_cnt = (int)a.k;
  __syncthreads();
  int first = (int)a.k;
  for (int j = threadIdx.x; j < (int)a.k; j += blockDim.x) {
    const int32_t s = ip[j];
    if (s < 0 && j < first) first = j;
    sidx[j] = (s >= 0 && s < a.S) ? s : 0;
  }
  if (first < (int)a.k) atomicMin(s_cnt, first);
  __syncthreads();
  return *s_cnt;
}

// Gather rows sidx[j0 .. j0+32) of the latent KV into a row-major LDS tile
// whose rows are DK*2 + 16 bytes apart (one 16-byte pad chunk per row keeps
// the 16 rows an MFMA operand read touches on different banks).  Slot
// s = row * RC + chunk; a wave copies 64 consecutive slots per instruction;
// pad slots copy chunk 0 of their row.
template <int DK>
__device__ __forceinline__ void gather_tile(const BwdArgs& a, const int32_t* sidx, int j0, char* dst) {
  constexpr int RC = DK / 8 + 1, SLOTS = kBNK * RC;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  const char* kv = (const char*)a.kv;
  for (int base = w * 64; base < SLOTS; base += nw * 64) {
    const int s = base + lane;
    if (s < SLOTS) {
      const int r = s / RC, ch = s - r * RC;
      const char* src = kv + (int64_t)sidx[j0 + r] * a.ld_kv * 2 + (ch < RC - 1 ? ch : 0) * 16;
      lds_dma16(src, dst + base * 16);
    }
  }
}

// Stage rows [j0, j0+32) of a [k][128] bf16 matrix (P or dS of one query)
// into LDS rows 272 bytes apart (16 data chunks + 1 pad chunk).
__device__ __forceinline__ void stage_ph(const uint16_t* src_q, int j0, char* dst) {
  constexpr int RC = 17, SLOTS = kBNK * RC;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int base = w * 64; base < SLOTS; base += nw * 64) {
    const int s = base + lane;
    if (s < SLOTS) {
      const int r = s / RC, ch = s - r * RC;
      lds_dma16(src_q + (int64_t)(j0 + r) * kBH + (ch < RC - 1 ? ch : 0) * 8, dst + base * 16);
    }
  }
}
constexpr int kPhRow = 272;               // bytes per staged P / dS row
constexpr int kPhTile = kBNK * kPhRow;    // bytes per staged P / dS tile

// ---- 1. P and dS ----------------------------------------------------------
template <int DK, int DV>
__global__ __launch_bounds__(512) void attn_bwd_ds_kernel(BwdArgs a, int64_t t0, uint16_t* __restrict__ pbuf,
                                                          uint16_t* __restrict__ dsbuf) {
  constexpr int RS = (DK / 8 + 1) * 16, TILE = kBNK * RS;
  constexpr int KK = DK / 32, VK = DV / 32;
  extern __shared__ __align__(16) char smem[];
  int32_t* sidx = (int32_t*)(smem + 2 * TILE);
  __shared__ int s_cnt;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t tl = blockIdx.x, t = t0 + tl;
  const int n = stage_index(a, t, sidx, &s_cnt);
  const int h = 16 * w + c;
  const uint16_t* qp = (const uint16_t*)a.q + (t * kBH + h) * DK + 8 * g;
  const uint16_t* dop = (const uint16_t*)a.dout + (t * kBH + h) * DV + 8 * g;
  const uint16_t* op = (const uint16_t*)a.out + (t * kBH + h) * DV + 8 * g;
  v8s qf[KK], df[VK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const v8s*)(qp + 32 * kk);
  float delta = 0.f;
#pragma unroll
  for (int kk = 0; kk < VK; ++kk) {
    df[kk] = *(const v8s*)(dop + 32 * kk);
    const v8s ov = *(const v8s*)(op + 32 * kk);
#pragma unroll
    for (int e = 0; e < 8; ++e) delta += bf16_to_f32((uint16_t)df[kk][e]) * bf16_to_f32((uint16_t)ov[e]);
  }
  delta = rows_sum(delta);  // over the four lane groups: dO_h . O_h
  const float l2 = a.lse[t * kBH + h] * kBLog2e;
  const float zs = a.scale * kBLog2e;
  uint16_t* pq = pbuf + tl * a.k * kBH;
  uint16_t* dq = dsbuf + tl * a.k * kBH;

  const int ntiles = (n + kBNK - 1) / kBNK;
  if (ntiles > 0) gather_tile<DK>(a, sidx, 0, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const char* tile = smem + (it & 1) * TILE;
    if (it + 1 < ntiles) gather_tile<DK>(a, sidx, (it + 1) * kBNK, smem + ((it + 1) & 1) * TILE);
    v4f sacc[2], pacc[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) sacc[ks] = pacc[ks] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8s av = *(const v8s*)(tile + (16 * ks + c) * RS + (4 * kk + g) * 16);
        sacc[ks] = mfma_bf16_16x16x32(av, qf[kk], sacc[ks]);
        if (kk < VK) pacc[ks] = mfma_bf16_16x16x32(av, df[kk], pacc[ks]);
      }
    }
    // C layout: lane (c, g) holds keys 16ks + 4g + i of head h
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = it * kBNK + 16 * ks + 4 * g + i;
        const float p = j < n ? exp2f(sacc[ks][i] * zs - l2) : 0.f;
        const float ds = a.scale * p * (pacc[ks][i] - delta);
        pq[(int64_t)j * kBH + h] = f32_to_bf16_rne(p);
        dq[(int64_t)j * kBH + h] = f32_to_bf16_rne(ds);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

// ---- 2. dq = dS . K -----------------------------------------------------
template <int DK>
__global__ __launch_bounds__(512) void attn_bwd_dq_kernel(BwdArgs a, int64_t t0, const uint16_t* __restrict__ dsbuf) {
  constexpr int RS = (DK / 8 + 1) * 16, TILE = kBNK * RS;
  constexpr int ND = DK / 16;
  extern __shared__ __align__(16) char smem[];
  char* dst = smem + 2 * TILE;                       // [2][kPhTile]
  int32_t* sidx = (int32_t*)(dst + 2 * kPhTile);
  __shared__ int s_cnt;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t tl = blockIdx.x, t = t0 + tl;
  const int n = stage_index(a, t, sidx, &s_cnt);
  const uint16_t* dsq = dsbuf + tl * a.k * kBH;
  v4f acc[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) acc[d] = (v4f){0.f, 0.f, 0.f, 0.f};
  const int ntiles = (n + kBNK - 1) / kBNK;
  if (ntiles > 0) {
    gather_tile<DK>(a, sidx, 0, smem);
    stage_ph(dsq, 0, dst);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int b = it & 1;
    if (it + 1 < ntiles) {
      gather_tile<DK>(a, sidx, (it + 1) * kBNK, smem + (b ^ 1) * TILE);
      stage_ph(dsq, (it + 1) * kBNK, dst + (b ^ 1) * kPhTile);
    }
    const char* kt = smem + b * TILE;
    // A = dS [16 heads x 32 keys] (rows = the wave's heads), B = K [32 keys x 16 dims]
    const v8s av = tr_operand(dst + b * kPhTile, kPhRow, 0, 16 * w);
#pragma unroll
    for (int d = 0; d < ND; ++d) acc[d] = mfma_bf16_16x16x32(av, tr_operand(kt, RS, 0, 16 * d), acc[d]);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // lane (c, g) holds heads 16w + 4g + i, column 16d + c
  uint16_t* o = (uint16_t*)a.dq + (t * kBH + 16 * w + 4 * g) * DK + c;
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int i = 0; i < 4; ++i) o[(int64_t)i * DK + 16 * d] = f32_to_bf16_rne(acc[d][i]);
}

// ---- 3. dkv += dS^T . q + P^T . dO ----------------------------------------
constexpr int kKvWaves = 12;   // 48 latent columns (3 MFMA column tiles) per wave

template <int DK, int DV>
__global__ __launch_bounds__(kKvWaves * 64) void attn_bwd_dkv_kernel(BwdArgs a, int64_t t0,
                                                                     const uint16_t* __restrict__ pbuf,
                                                                     const uint16_t* __restrict__ dsbuf) {
  constexpr int NDW = DK / 16 / kKvWaves;   // column tiles per wave
  static_assert(NDW * 16 * kKvWaves == DK, "latent columns split evenly over the waves");
  extern __shared__ __align__(16) char smem[];
  // [2][kPhTile] P tiles | [2][kPhTile] dS tiles (first holding 32 rows of q
  // or dO while the B operands are built) | index row
  constexpr int AREA = 4 * kPhTile > 32 * DK * 2 ? 4 * kPhTile : 32 * DK * 2;
  char* pt = smem;
  char* dt = smem + 2 * kPhTile;
  int32_t* sidx = (int32_t*)(smem + AREA);
  __shared__ int s_cnt;
  const int lane = threadIdx.x & 63, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t tl = blockIdx.x, t = t0 + tl;
  const int n = stage_index(a, t, sidx, &s_cnt);
  // B operands, heads on the reduction axis: lane (c, g) of k-step kk holds
  // q / dO of heads 32kk + 8g .. +7 at column 16 D + c.  Built once per
  // query: 32 heads of q (then of dO) at a time are copied to LDS as they
  // lie in memory and read back transposed.
  v8s qb[NDW][4], db[NDW][4];
  auto stage_rows = [&](const uint16_t* src, int bytes) {
    const int lane_ = threadIdx.x & 63, nw = blockDim.x >> 6;
    for (int base = w * 64; base * 16 < bytes; base += nw * 64)
      if ((base + lane_) * 16 < bytes) lds_dma16((const char*)src + (base + lane_) * 16, smem + base * 16);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    stage_rows((const uint16_t*)a.q + (t * kBH + 32 * kk) * DK, 32 * DK * 2);
#pragma unroll
    for (int d = 0; d < NDW; ++d) qb[d][kk] = tr_operand(smem, DK * 2, 0, 16 * (NDW * w + d));
    __syncthreads();
    stage_rows((const uint16_t*)a.dout + (t * kBH + 32 * kk) * DV, 32 * DV * 2);
#pragma unroll
    for (int d = 0; d < NDW; ++d) {
      const int col0 = 16 * (NDW * w + d);
      db[d][kk] = col0 + 16 <= DV ? tr_operand(smem, DV * 2, 0, col0) : (v8s){0, 0, 0, 0, 0, 0, 0, 0};
    }
    __syncthreads();
  }
  const uint16_t* pq = pbuf + tl * a.k * kBH;
  const uint16_t* dq = dsbuf + tl * a.k * kBH;
  float* dkv = a.dkv;
  const int ntiles = (n + kBNK - 1) / kBNK;
  if (ntiles > 0) {
    stage_ph(pq, 0, pt);
    stage_ph(dq, 0, dt);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const int b = it & 1;
    if (it + 1 < ntiles) {
      stage_ph(pq, (it + 1) * kBNK, pt + (b ^ 1) * kPhTile);
      stage_ph(dq, (it + 1) * kBNK, dt + (b ^ 1) * kPhTile);
    }
    v4f acc[2][NDW];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int d = 0; d < NDW; ++d) acc[ks][d] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        // A = dS^T / P^T [16 keys x 32 heads]: lane (c, g) key 16ks + c, heads 32kk + 8g .. +7
        const int off = (16 * ks + c) * kPhRow + (32 * kk + 8 * g) * 2;
        const v8s ad = *(const v8s*)(dt + b * kPhTile + off);
        const v8s ap = *(const v8s*)(pt + b * kPhTile + off);
#pragma unroll
        for (int d = 0; d < NDW; ++d) {
          acc[ks][d] = mfma_bf16_16x16x32(ad, qb[d][kk], acc[ks][d]);
          if (16 * (NDW * w + d) + 16 <= DV) acc[ks][d] = mfma_bf16_16x16x32(ap, db[d][kk], acc[ks][d]);
        }
      }
    }
    // lane (c, g) holds keys 16ks + 4g + i at column 16 D + c
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = it * kBNK + 16 * ks + 4 * g + i;
        if (j < n) {
          float* row = dkv + (int64_t)sidx[j] * a.ld_dkv + 16 * NDW * w + c;
#pragma unroll
          for (int d = 0; d < NDW; ++d) unsafeAtomicAdd(row + 16 * d, acc[ks][d][i]);
        }
      }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
}

}  // namespace

bool attn_bwd_supported(int64_t H, int64_t Dk, int64_t Dv, int64_t k) {
  return H == kBH && Dk == 576 && Dv == 512 && k >= kBNK && k % kBNK == 0 && k <= DSA_MAX_TOPK;
}

int64_t attn_bwd_chunk(int64_t T, int64_t k) {
  const int64_t per = k * kBH * 2 * 2;   // P + dS, bf16
  int64_t c = ((int64_t)1 << 31) / per;
  c = c < 1 ? 1 : c;
  return T < c ? T : c;
}

size_t attn_bwd_workspace_bytes(int64_t T, int64_t k) {
  const int64_t c = attn_bwd_chunk(T, k);
  return (size_t)(c * k * kBH * 2) * 2 + 256;
}

hipError_t launch_attn_bwd(const BwdArgs& a, void* ws, hipStream_t st) {
  constexpr int DK = 576, DV = 512;
  const int64_t C = attn_bwd_chunk(a.T, a.k);
  uint16_t* pbuf = (uint16_t*)ws;
  uint16_t* dsbuf = (uint16_t*)((char*)ws + (size_t)(C * a.k * kBH * 2 + 255) / 256 * 256);
  DSA_DEBUG_CHECK((char*)(dsbuf + (size_t)C * a.k * kBH) <= (char*)ws + attn_bwd_workspace_bytes(a.T, a.k));
  constexpr int TILE = kBNK * (DK / 8 + 1) * 16;
  const size_t lds_ds = 2 * TILE + a.k * 4;
  const size_t lds_dq = 2 * TILE + 2 * kPhTile + a.k * 4;
  const size_t lds_kv = (size_t)(4 * kPhTile > 32 * DK * 2 ? 4 * kPhTile : 32 * DK * 2) + a.k * 4;
  static std::atomic<uint64_t> ds_done{0}, dq_done{0};
  hipError_t ea = set_lds_limit_once((const void*)attn_bwd_ds_kernel<DK, DV>, (int)(2 * TILE + 16384), ds_done);
  if (ea != hipSuccess) return ea;
  ea = set_lds_limit_once((const void*)attn_bwd_dq_kernel<DK>, (int)(2 * TILE + 2 * kPhTile + 16384), dq_done);
  if (ea != hipSuccess) return ea;
  for (int64_t t0 = 0; t0 < a.T; t0 += C) {
    const unsigned nb = (unsigned)(a.T - t0 < C ? a.T - t0 : C);
    attn_bwd_ds_kernel<DK, DV><<<nb, 512, lds_ds, st>>>(a, t0, pbuf, dsbuf);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    attn_bwd_dq_kernel<DK><<<nb, 512, lds_dq, st>>>(a, t0, dsbuf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    attn_bwd_dkv_kernel<DK, DV><<<nb, kKvWaves * 64, lds_kv, st>>>(a, t0, pbuf, dsbuf);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace dsa
