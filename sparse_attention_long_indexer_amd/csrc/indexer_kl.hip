// KL alignment of the lightning indexer to the dense attention (DeepSeek-V3.2
// write-up, section 4.1, dense warm-up: the frozen model's attention
// distribution is distilled into the indexer with a KL loss).
//
// For a causal prefill of L tokens, query t over keys s <= t:
//   target  p_t[s] = (1/H) sum_h softmax_s(scale q_{t,h} . k_s)  (MLA latent k)
//   indexer I[t,s] = ReLU((q^I_t W) . k^I_s),  log q_t[s] = I[t,s] - LSE_s I[t,.]
//   loss_t = sum_s p (log p - log q),  G[t,s] = (q_t[s] - p_t[s]) [I[t,s] > 0]
//   dqf = G k^I,  dk^I = G^T qf,  dq^I = dqf W^T,  dW = q^I^T dqf   (qf = q^I W)
// Kernels: the fp32 fold and fp32 scores of the inference path fill the score
// matrix I; kl_target_kernel (one block per query, 16 heads per wave, bf16
// MFMA) makes two passes over the causal keys -- the per-head log-sum-exp,
// then the head-averaged probabilities -- and turns row t of I into row t of
// G in place, with the query's loss; four fp32 kernels form the gradients.
#include "common.h"
#include "dsa.h"
#include "kernels.h"

namespace dsa {

namespace {

constexpr int kKH = 128;   // heads
constexpr int kKNK = 32;   // keys per tile
constexpr float kKLog2e = 1.4426950408889634f;

typedef __attribute__((address_space(3))) char lds_k;

// Copy latent rows min(j0 + r, last), r < 32, into a row-major LDS tile with
// rows DK*2 + 16 bytes apart (a pad chunk per row; pad slots copy chunk 0).
template <int DK>
__device__ __forceinline__ void kl_tile(const char* kv, int64_t ldb, int64_t j0, int64_t last, char* dst) {
  constexpr int RC = DK / 8 + 1, SLOTS = kKNK * RC;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
  for (int base = w * 64; base < SLOTS; base += nw * 64) {
    const int s = base + lane;
    if (s < SLOTS) {
      const int r = s / RC, ch = s - r * RC;
      const int64_t row = j0 + r < last ? j0 + r : last;
      __builtin_amdgcn_global_load_lds((const void*)(kv + row * ldb + (ch < RC - 1 ? ch : 0) * 16),
                                       (lds_k*)(dst + base * 16), 16, 0, 0);
    }
  }
}

template <int DK>
__global__ __launch_bounds__(512) void kl_target_kernel(const uint16_t* __restrict__ q, const char* __restrict__ kv,
                                                        int64_t ld_kv, int64_t L, float scale,
                                                        float* __restrict__ gmat, float* __restrict__ loss_out) {
  constexpr int RS = (DK / 8 + 1) * 16, TILE = kKNK * RS, KK = DK / 32, NW = 8;
  extern __shared__ __align__(16) char smem[];   // [2][TILE]
  __shared__ float s_red[NW][kKNK];
  __shared__ float s_m[NW], s_l[NW];
  __shared__ float s_lse;
  const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = blockIdx.x;
  const int n = (int)t + 1;
  float* grow = gmat + t * L;
  const int64_t ldb = ld_kv * 2;

  // log-sum-exp of the indexer row I[t, 0..t]
  {
    float m = -INFINITY;
    for (int s = tid; s < n; s += 512) m = fmaxf(m, grow[s]);
    m = wave_max(m);
    if (lane == 0) s_m[w] = m;
    __syncthreads();
    m = s_m[0];
    for (int i = 1; i < NW; ++i) m = fmaxf(m, s_m[i]);
    float l = 0.f;
    for (int s = tid; s < n; s += 512) l += exp2f((grow[s] - m) * kKLog2e);
    l = wave_sum(l);
    if (lane == 0) s_l[w] = l;
    __syncthreads();
    if (tid == 0) {
      float tot = 0.f;
      for (int i = 0; i < NW; ++i) tot += s_l[i];
      s_lse = m + logf(tot);
    }
    __syncthreads();
  }
  const float lse_i = s_lse;

  const int h = 16 * w + c;
  const uint16_t* qp = q + (t * kKH + h) * DK + 8 * g;
  v8s qf[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const v8s*)(qp + 32 * kk);
  const float zs = scale * kKLog2e;
  const int ntiles = (n + kKNK - 1) / kKNK;

  auto scores = [&](const char* tile, v4f* sacc) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) sacc[ks] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8s av = *(const v8s*)(tile + (16 * ks + c) * RS + (4 * kk + g) * 16);
        sacc[ks] = mfma_bf16_16x16x32(av, qf[kk], sacc[ks]);
      }
  };

  // pass A: per-head running max and sum in the log2 domain (lane: head h,
  // keys 16ks + 4g + i of the tile)
  float m_run = -INFINITY, l_run = 0.f;
  kl_tile<DK>((const char*)kv, ldb, 0, t, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const char* tile = smem + (it & 1) * TILE;
    if (it + 1 < ntiles) kl_tile<DK>((const char*)kv, ldb, (int64_t)(it + 1) * kKNK, t, smem + ((it + 1) & 1) * TILE);
    v4f sacc[2];
    scores(tile, sacc);
    float tm = -INFINITY;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (it * kKNK + 16 * ks + 4 * g + i < n) tm = fmaxf(tm, sacc[ks][i] * zs);
    const float mn = fmaxf(m_run, tm);
    float add = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (it * kKNK + 16 * ks + 4 * g + i < n) add += exp2f(sacc[ks][i] * zs - mn);
    l_run = (m_run == -INFINITY ? 0.f : l_run * exp2f(m_run - mn)) + add;
    m_run = mn;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  // combine the four lane groups of the head
  {
    const float M = rows_max(m_run);
    const float part = m_run == -INFINITY ? 0.f : l_run * exp2f(m_run - M);
    l_run = rows_sum(part);
    m_run = M;
  }
  const float lse2 = m_run + log2f(l_run);   // head h's log2-sum-exp of the scaled scores

  // pass B: head-averaged probabilities, then G and the loss per key
  float loss = 0.f;
  kl_tile<DK>((const char*)kv, ldb, 0, t, smem);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int it = 0; it < ntiles; ++it) {
    const char* tile = smem + (it & 1) * TILE;
    if (it + 1 < ntiles) kl_tile<DK>((const char*)kv, ldb, (int64_t)(it + 1) * kKNK, t, smem + ((it + 1) & 1) * TILE);
    v4f sacc[2];
    scores(tile, sacc);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float p = exp2f(sacc[ks][i] * zs - lse2);
        // sum over the wave's 16 heads (the 16 lanes of the group)
        p += __shfl_xor(p, 1);
        p += __shfl_xor(p, 2);
        p += __shfl_xor(p, 4);
        p += __shfl_xor(p, 8);
        if (c == 0) s_red[w][16 * ks + 4 * g + i] = p;
      }
    __syncthreads();
    if (tid < kKNK) {
      const int s = it * kKNK + tid;
      if (s < n) {
        float p = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) p += s_red[i][tid];
        p *= 1.f / kKH;
        const float iv = grow[s];
        const float logq = iv - lse_i;
        if (p > 0.f) loss += p * (logf(p) - logq);
        grow[s] = iv > 0.f ? expf(logq) - p : 0.f;
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (w == 0) {
    loss = wave_sum(loss);
    if (lane == 0) loss_out[t] = loss;
  }
}

// dqf[t][:] = sum_{s <= t} G[t][s] kI[s][:]: a block owns 32 rows t and the
// 128 columns; key tiles of 32 staged in LDS; thread (r, c4) computes rows
// r, r + 16 and columns 4 c4 .. 4 c4 + 3 (256 threads).
__global__ __launch_bounds__(256) void kl_dqf_kernel(const float* __restrict__ gmat, const float* __restrict__ ki,
                                                     int64_t L, float* __restrict__ dqf) {
  __shared__ float sg[32][33];
  __shared__ __align__(16) float sk[32][128];
  const int tid = threadIdx.x, r = tid >> 4, c4 = tid & 15;
  const int64_t t0 = (int64_t)blockIdx.x * 32;
  float acc[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
  const int64_t tmax = t0 + 31 < L - 1 ? t0 + 31 : L - 1;
  for (int64_t s0 = 0; s0 <= tmax; s0 += 32) {
    for (int e = tid; e < 32 * 32; e += 256) {
      const int rr = e >> 5, cc = e & 31;
      const int64_t t = t0 + rr, s = s0 + cc;
      sg[rr][cc] = (t < L && s <= t) ? gmat[t * L + s] : 0.f;
    }
    for (int e = tid; e < 32 * 32; e += 256) {
      const int rr = e >> 5, cc = e & 31;
      const int64_t s = s0 + rr;
      *(float4*)&sk[rr][4 * cc] = s < L ? *(const float4*)(ki + s * 128 + 4 * cc) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < 32; ++j) {
      const float4 k0 = *(const float4*)&sk[j][4 * c4];
      const float4 k1 = *(const float4*)&sk[j][64 + 4 * c4];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float gv = sg[r + 16 * a][j];
        acc[a][0] += gv * k0.x;
        acc[a][1] += gv * k0.y;
        acc[a][2] += gv * k0.z;
        acc[a][3] += gv * k0.w;
        acc[a][4] += gv * k1.x;
        acc[a][5] += gv * k1.y;
        acc[a][6] += gv * k1.z;
        acc[a][7] += gv * k1.w;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t t = t0 + r + 16 * a;
    if (t < L) {
      *(float4*)(dqf + t * 128 + 4 * c4) = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
      *(float4*)(dqf + t * 128 + 64 + 4 * c4) = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
    }
  }
}

// dk[s][:] = sum_{t >= s} G[t][s] qf[t][:]: a block owns 32 keys s; query
// tiles of 32 from the block's first key on.
__global__ __launch_bounds__(256) void kl_dk_kernel(const float* __restrict__ gmat, const float* __restrict__ qf,
                                                    int64_t L, float* __restrict__ dk) {
  __shared__ float sg[32][33];   // [t][s]
  __shared__ __align__(16) float sq[32][128];
  const int tid = threadIdx.x, r = tid >> 4, c4 = tid & 15;
  const int64_t s0 = (int64_t)blockIdx.x * 32;
  float acc[2][8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 8; ++b) acc[a][b] = 0.f;
  for (int64_t t0 = s0; t0 < L; t0 += 32) {
    for (int e = tid; e < 32 * 32; e += 256) {
      const int rr = e >> 5, cc = e & 31;
      const int64_t t = t0 + rr, s = s0 + cc;
      sg[rr][cc] = (t < L && s < L && s <= t) ? gmat[t * L + s] : 0.f;
    }
    for (int e = tid; e < 32 * 32; e += 256) {
      const int rr = e >> 5, cc = e & 31;
      const int64_t t = t0 + rr;
      *(float4*)&sq[rr][4 * cc] = t < L ? *(const float4*)(qf + t * 128 + 4 * cc) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    __syncthreads();
#pragma unroll 4
    for (int j = 0; j < 32; ++j) {
      const float4 q0 = *(const float4*)&sq[j][4 * c4];
      const float4 q1 = *(const float4*)&sq[j][64 + 4 * c4];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const float gv = sg[j][r + 16 * a];
        acc[a][0] += gv * q0.x;
        acc[a][1] += gv * q0.y;
        acc[a][2] += gv * q0.z;
        acc[a][3] += gv * q0.w;
        acc[a][4] += gv * q1.x;
        acc[a][5] += gv * q1.y;
        acc[a][6] += gv * q1.z;
        acc[a][7] += gv * q1.w;
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int64_t s = s0 + r + 16 * a;
    if (s < L) {
      *(float4*)(dk + s * 128 + 4 * c4) = make_float4(acc[a][0], acc[a][1], acc[a][2], acc[a][3]);
      *(float4*)(dk + s * 128 + 64 + 4 * c4) = make_float4(acc[a][4], acc[a][5], acc[a][6], acc[a][7]);
    }
  }
}

// dq[t][i] = sum_j dqf[t][j] W[i][j]: a block owns 8 rows t, thread (row, i)
__global__ __launch_bounds__(256) void kl_dq_kernel(const float* __restrict__ dqf, const float* __restrict__ w,
                                                    int64_t L, float* __restrict__ dq) {
  __shared__ float sw[128][129];
  __shared__ float sd[2][128];
  const int tid = threadIdx.x;
  for (int e = tid; e < 128 * 128; e += 256) sw[e >> 7][e & 127] = w[e];
  for (int64_t t0 = (int64_t)blockIdx.x * 8; t0 < (int64_t)blockIdx.x * 8 + 8 && t0 < L; t0 += 2) {
    __syncthreads();
    sd[tid >> 7][tid & 127] = t0 + (tid >> 7) < L ? dqf[(t0 + (tid >> 7)) * 128 + (tid & 127)] : 0.f;
    __syncthreads();
    const int rr = tid >> 7, i = tid & 127;
    float acc = 0.f;
#pragma unroll 8
    for (int j = 0; j < 128; ++j) acc += sd[rr][j] * sw[i][j];
    if (t0 + rr < L) dq[(t0 + rr) * 128 + i] = acc;
  }
}

// dW[i][j] = sum_t qI[t][i] dqf[t][j]: one block per row i, thread j; the
// rows t are split over gridDim.y slices whose partial sums go to dw_part
__global__ __launch_bounds__(128) void kl_dw_kernel(const float* __restrict__ qi, const float* __restrict__ dqf,
                                                    int64_t L, float* __restrict__ dw_part) {
  const int i = blockIdx.x, j = threadIdx.x;
  const int64_t per = (L + gridDim.y - 1) / gridDim.y;
  const int64_t t0 = (int64_t)blockIdx.y * per, t1 = t0 + per < L ? t0 + per : L;
  float acc = 0.f;
  for (int64_t t = t0; t < t1; ++t) acc += qi[t * 128 + i] * dqf[t * 128 + j];
  dw_part[((int64_t)blockIdx.y * 128 + i) * 128 + j] = acc;
}

__global__ __launch_bounds__(256) void kl_dw_sum_kernel(const float* __restrict__ dw_part, int nparts,
                                                        float* __restrict__ dw) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= 128 * 128) return;
  float acc = 0.f;
  for (int p = 0; p < nparts; ++p) acc += dw_part[(int64_t)p * 128 * 128 + e];
  dw[e] = acc;
}

constexpr int kDwParts = 64;

}  // namespace

bool indexer_kl_supported(int64_t H, int64_t Dk, int64_t L) {
  return H == kKH && Dk == 576 && L >= 1 && L <= 65536;
}

size_t indexer_kl_workspace_bytes(int64_t L) {
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  return up((size_t)L * 128 * 4) * 2 + up((size_t)L * L * 4) + up((size_t)kDwParts * 128 * 128 * 4);
}

hipError_t launch_indexer_kl(const KlArgs& a, void* ws, hipStream_t st) {
  constexpr int DK = 576;
  auto up = [](size_t b) { return (b + 255) / 256 * 256; };
  char* p = (char*)ws;
  float* qf = (float*)p;
  p += up((size_t)a.L * 128 * 4);
  float* dqf = (float*)p;
  p += up((size_t)a.L * 128 * 4);
  float* gmat = (float*)p;
  p += up((size_t)a.L * a.L * 4);
  float* dw_part = (float*)p;
  DSA_DEBUG_CHECK((char*)(dw_part + (size_t)kDwParts * 128 * 128) <= (char*)ws + indexer_kl_workspace_bytes(a.L));
  hipError_t e = launch_fold(a.q_idx, nullptr, false, a.w, false, a.L, qf, nullptr, st);
  if (e != hipSuccess) return e;
  e = launch_index_scores(qf, nullptr, a.k_idx, nullptr, false, a.L, a.L, nullptr, 0, 0, a.L, gmat, a.L, st);
  if (e != hipSuccess) return e;
  constexpr int TILE = kKNK * (DK / 8 + 1) * 16;
  static std::atomic<uint64_t> attr_done{0};
  e = set_lds_limit_once((const void*)kl_target_kernel<DK>, 2 * TILE, attr_done);
  if (e != hipSuccess) return e;
  kl_target_kernel<DK><<<(unsigned)a.L, 512, 2 * TILE, st>>>((const uint16_t*)a.q, (const char*)a.kv, a.ld_kv, a.L,
                                                              a.scale, gmat, a.loss);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const unsigned nb = (unsigned)((a.L + 31) / 32);
  kl_dqf_kernel<<<nb, 256, 0, st>>>(gmat, a.k_idx, a.L, dqf);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  kl_dk_kernel<<<nb, 256, 0, st>>>(gmat, qf, a.L, a.dk_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  kl_dq_kernel<<<(unsigned)((a.L + 7) / 8), 256, 0, st>>>(dqf, a.w, a.L, a.dq_idx);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  kl_dw_kernel<<<dim3(128, kDwParts), 128, 0, st>>>(a.q_idx, dqf, a.L, dw_part);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  kl_dw_sum_kernel<<<64, 256, 0, st>>>(dw_part, kDwParts, a.dw);
  return hipGetLastError();
}

}  // namespace dsa
