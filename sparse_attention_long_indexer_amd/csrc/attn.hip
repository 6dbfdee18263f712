// Sparse MQA attention over the selected key rows (DeepSeek-V3.2 write-up,
// sections 2.3 and 3.1: ordinary softmax attention restricted to the k
// selected keys, all query heads sharing one key/value head as in MLA's MQA
// mode).
//
// bf16 path: one block per query, 16 heads per wave.  Per tile of 32
// selected keys the block gathers the K rows (row-major) and the V rows
// (transposed, V^T[dv][key]) into LDS, then each wave computes
//   S^T = K . Q^T   with v_mfma_f32_16x16x32_bf16 (A = K tile from LDS,
//                   B = the wave's Q^T held in registers for the whole loop),
//   an online softmax per head in the log2 domain, and
//   O^T += V^T . P^T (A = V^T from LDS, B = P^T straight from the S^T
//                   accumulators: the C layout of S^T gives lane (head c,
//                   group g) the keys {4g..4g+3, 16+4g..16+4g+3}, and the
//                   V^T operand is read with the same key order).
// Keeping heads in the N dimension puts one head per lane column, so the
// softmax rescale of O is a per-lane scalar.
//
// fp32 path: a plain VALU kernel for the small fp32 configuration.
#include "common.h"
#include "kernels.h"

namespace dsa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct AttnRow {
  const int32_t* ip;
  int64_t base;   // row offset of this query's cache
  int64_t len;    // rows available to this query
};

__device__ __forceinline__ AttnRow attn_row(const AttnArgs& a, const int64_t* seq_off, int64_t t) {
  AttnRow r;
  r.ip = a.idx + t * a.k;
  if (seq_off) {
    r.base = seq_off[t];
    r.len = seq_off[t + 1] - r.base;
  } else {
    r.base = 0;
    r.len = a.S;
  }
  return r;
}

// number of leading valid entries of an index row (block-wide)
__device__ __forceinline__ int valid_count(const int32_t* ip, int64_t k, int* s_cnt) {
  if (threadIdx.x == 0) *s_cnt = (int)k;
  __syncthreads();
  int first = (int)k;
  for (int64_t j = threadIdx.x; j < k; j += blockDim.x)
    if (ip[j] < 0 && (int)j < first) first = (int)j;
  if (first < (int)k) atomicMin(s_cnt, first);
  __syncthreads();
  return *s_cnt;
}

template <int DK, int DV, int NW>
__global__ __launch_bounds__(NW * 64) void attn_bf16_kernel(AttnArgs a, const int64_t* seq_off) {
  constexpr int NK = 32;          // keys per tile
  constexpr int KP = DK + 8;      // K tile pitch (bf16), 16-byte pad
  constexpr int VP = NK + 4;      // V^T pitch (bf16), 8-byte pad
  constexpr int NT = NW * 64;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* ks = smem;                 // [NK][KP]
  uint16_t* vt = smem + NK * KP;       // [DV][VP]
  __shared__ int s_cnt;
  __shared__ int32_t s_idx[NK];

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = blockIdx.x;
  const AttnRow row = attn_row(a, seq_off, t);
  const int n = valid_count(row.ip, a.k, &s_cnt);
  const int H = 16 * NW;
  const uint16_t* kv = (const uint16_t*)a.kv;
  const uint16_t* vv = a.v ? (const uint16_t*)a.v : kv;
  const int64_t ldv = a.v ? a.ld_v : a.ld_kv;

  // this wave's Q^T fragments: head 16w + c, dims 32kk + 8g .. +8
  v8s qf[DK / 32];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((t * H) + 16 * w + c) * (int64_t)DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) qf[kk] = *(const v8s*)(qp + 32 * kk);
  }
  v4f o[DV / 16];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) o[d] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float zs = a.scale * kLog2e;

  for (int j0 = 0; j0 < n; j0 += NK) {
    __syncthreads();
    if (tid < NK) {
      const int j = j0 + tid;
      int32_t s = j < n ? row.ip[j] : -1;
      if (s >= row.len) s = (int32_t)(row.len - 1);
      s_idx[tid] = s;
    }
    __syncthreads();
    // gather K rows: NK x DK bf16 in 16-byte chunks
    for (int e = tid; e < NK * (DK / 8); e += NT) {
      const int j = e / (DK / 8), cc = e % (DK / 8);
      const int32_t s = s_idx[j];
      v8s val = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
      if (s >= 0) val = *(const v8s*)(kv + (row.base + s) * a.ld_kv + 8 * cc);
      *(v8s*)(ks + j * KP + 8 * cc) = val;
    }
    // gather V rows, stored transposed
    for (int e = tid; e < NK * (DV / 8); e += NT) {
      const int j = e / (DV / 8), cc = e % (DV / 8);
      const int32_t s = s_idx[j];
      v8s val = (v8s){0, 0, 0, 0, 0, 0, 0, 0};
      if (s >= 0) val = *(const v8s*)(vv + (row.base + s) * ldv + 8 * cc);
#pragma unroll
      for (int q = 0; q < 8; ++q) vt[(8 * cc + q) * VP + j] = (uint16_t)val[q];
    }
    __syncthreads();

    // S^T tiles: keys 0..15 and 16..31 of this tile, head column c
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
      const v8s a0 = *(const v8s*)(ks + c * KP + 32 * kk + 8 * g);
      const v8s a1 = *(const v8s*)(ks + (16 + c) * KP + 32 * kk + 8 * g);
      s0 = mfma_bf16_16x16x32(a0, qf[kk], s0);
      s1 = mfma_bf16_16x16x32(a1, qf[kk], s1);
    }
    float z[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      z[i] = (j0 + 4 * g + i < n) ? s0[i] * zs : -INFINITY;
      z[4 + i] = (j0 + 16 + 4 * g + i < n) ? s1[i] * zs : -INFINITY;
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float corr = exp2f(m_run - m_new);
    float p[8], rs = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = exp2f(z[i] - m_new);
      rs += p[i];
    }
    rs += __shfl_xor(rs, 16);
    rs += __shfl_xor(rs, 32);
    l_run = l_run * corr + rs;
    m_run = m_new;
    v8s pb;
    {
      v4i pk;
      pk[0] = (int)pack_bf16x2(p[0], p[1]);
      pk[1] = (int)pack_bf16x2(p[2], p[3]);
      pk[2] = (int)pack_bf16x2(p[4], p[5]);
      pk[3] = (int)pack_bf16x2(p[6], p[7]);
      pb = (v8s)pk;
    }
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const v4s lo = *(const v4s*)(vt + (16 * d + c) * VP + 4 * g);
      const v4s hi = *(const v4s*)(vt + (16 * d + c) * VP + 16 + 4 * g);
      const v8s av = (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      o[d] = o[d] * corr;
      o[d] = mfma_bf16_16x16x32(av, pb, o[d]);
    }
  }

  // epilogue: lane (c, g) holds O^T[dv = 16d + 4g + i][head c]
  const int h = 16 * w + c;
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  uint16_t* op = (uint16_t*)a.out + (t * H + h) * (int64_t)DV;
#pragma unroll
  for (int d = 0; d < DV / 16; ++d) {
    v2i pk;
    pk[0] = (int)pack_bf16x2(o[d][0] * inv, o[d][1] * inv);
    pk[1] = (int)pack_bf16x2(o[d][2] * inv, o[d][3] * inv);
    *(v2i*)(op + 16 * d + 4 * g) = pk;
  }
  if (a.lse && g == 0) a.lse[t * H + h] = n > 0 ? (m_run + log2f(l_run)) * kLn2 : -INFINITY;
}

// ---- fp32 path -----------------------------------------------------------
constexpr int kF32Keys = 32;

__global__ __launch_bounds__(256) void attn_f32_kernel(AttnArgs a, const int64_t* seq_off) {
  __shared__ float kt[kF32Keys][128 + 1];
  __shared__ float vt[kF32Keys][128 + 1];
  __shared__ float zt[64][kF32Keys];
  __shared__ int s_cnt;
  __shared__ int32_t s_idx[kF32Keys];
  const int tid = threadIdx.x;
  const int64_t t = blockIdx.x;
  const AttnRow row = attn_row(a, seq_off, t);
  const int n = valid_count(row.ip, a.k, &s_cnt);
  const int H = (int)a.H, Dk = (int)a.Dk, Dv = (int)a.Dv;
  const float* q = (const float*)a.q + t * H * (int64_t)Dk;
  const float* kv = (const float*)a.kv;
  const float* vv = a.v ? (const float*)a.v : kv;
  const int64_t ldv = a.v ? a.ld_v : a.ld_kv;
  // each thread owns outputs e = tid + 256 r, (h, d) = (e / Dv, e % Dv)
  constexpr int kMaxOwn = 32;
  float acc[kMaxOwn], mrun[kMaxOwn], lrun[kMaxOwn];
  const int nown = (H * Dv + 255) / 256;
  for (int r = 0; r < kMaxOwn; ++r) {
    acc[r] = 0.f;
    mrun[r] = -INFINITY;
    lrun[r] = 0.f;
  }
  for (int j0 = 0; j0 < n; j0 += kF32Keys) {
    __syncthreads();
    if (tid < kF32Keys) {
      const int j = j0 + tid;
      int32_t s = j < n ? row.ip[j] : -1;
      if (s >= row.len) s = (int32_t)(row.len - 1);
      s_idx[tid] = s;
    }
    __syncthreads();
    for (int e = tid; e < kF32Keys * 128; e += 256) {
      const int j = e / 128, d = e % 128;
      const int32_t s = s_idx[j];
      kt[j][d] = (s >= 0 && d < Dk) ? kv[(row.base + s) * a.ld_kv + d] : 0.f;
      vt[j][d] = (s >= 0 && d < Dv) ? vv[(row.base + s) * ldv + d] : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < H * kF32Keys; e += 256) {
      const int h = e / kF32Keys, j = e % kF32Keys;
      float dot = 0.f;
      for (int d = 0; d < Dk; ++d) dot = fmaf(q[h * Dk + d], kt[j][d], dot);
      zt[h][j] = (j0 + j < n) ? dot * a.scale : -INFINITY;
    }
    __syncthreads();
    for (int r = 0; r < nown; ++r) {
      const int e = tid + 256 * r;
      if (e >= H * Dv) break;
      const int h = e / Dv, d = e % Dv;
      float mx = -INFINITY;
      for (int j = 0; j < kF32Keys; ++j) mx = fmaxf(mx, zt[h][j]);
      const float mn = fmaxf(mrun[r], mx);
      const float corr = expf(mrun[r] - mn);
      float ls = 0.f, os = 0.f;
      for (int j = 0; j < kF32Keys; ++j) {
        const float pj = expf(zt[h][j] - mn);
        ls += pj;
        os = fmaf(pj, vt[j][d], os);
      }
      lrun[r] = lrun[r] * corr + ls;
      acc[r] = acc[r] * corr + os;
      mrun[r] = mn;
    }
  }
  for (int r = 0; r < nown; ++r) {
    const int e = tid + 256 * r;
    if (e >= H * Dv) break;
    const int h = e / Dv, d = e % Dv;
    ((float*)a.out)[(t * H + h) * (int64_t)Dv + d] = lrun[r] > 0.f ? acc[r] / lrun[r] : 0.f;
    if (a.lse && d == 0) a.lse[t * H + h] = n > 0 ? mrun[r] + logf(lrun[r]) : -INFINITY;
  }
}

bool attn_supported(bool f32, int64_t H, int64_t Dk, int64_t Dv) {
  if (f32) return H >= 1 && H <= 64 && Dk >= 4 && Dk <= 128 && Dv >= 4 && Dv <= 128 && Dk % 4 == 0 && Dv % 4 == 0;
  return (H == 16 && Dk == 128 && Dv == 128) || (H == 128 && Dk == 576 && Dv == 512);
}

size_t attn_workspace_bytes(bool f32, int64_t T, int64_t H, int64_t Dv, int64_t k) {
  (void)f32;
  (void)T;
  (void)H;
  (void)Dv;
  (void)k;
  return 0;
}

template <int DK, int DV, int NW>
static hipError_t launch_bf16(const AttnArgs& a, const int64_t* seq_off, hipStream_t st) {
  constexpr size_t lds = (size_t)(32 * (DK + 8) + DV * 36) * sizeof(uint16_t);
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_bf16_kernel<DK, DV, NW>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  attn_bf16_kernel<DK, DV, NW><<<(unsigned)a.T, NW * 64, lds, st>>>(a, seq_off);
  return hipGetLastError();
}

hipError_t launch_attn(const AttnArgs& a, bool f32, void* ws, size_t ws_bytes, hipStream_t st) {
  (void)ws;
  (void)ws_bytes;
  if (a.T <= 0) return hipSuccess;
  if (f32) {
    attn_f32_kernel<<<(unsigned)a.T, 256, 0, st>>>(a, a.seq_offsets);
    return hipGetLastError();
  }
  if (a.H == 16 && a.Dk == 128 && a.Dv == 128) return launch_bf16<128, 128, 1>(a, a.seq_offsets, st);
  if (a.H == 128 && a.Dk == 576 && a.Dv == 512) return launch_bf16<576, 512, 8>(a, a.seq_offsets, st);
  return hipErrorInvalidValue;
}

}  // namespace dsa
