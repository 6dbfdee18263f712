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

#ifndef DSA_MLA_HW
#define DSA_MLA_HW 16   // heads per wave for the 128-head MLA shape
#define DSA_MLA_NW 8    // waves per block
#endif
#ifndef DSA_QK_GROUP
#define DSA_QK_GROUP 4  // QK k-steps the scheduler may interleave
#define DSA_PV_GROUP 4  // PV dv-subtiles the scheduler may interleave
#endif

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

// LDS tile of NK gathered rows, each row C chunks of 16 bytes.  Chunk X of
// row r lives at slot r*C + (X ^ ((r >> 1) & 7)): 16 consecutive rows read at
// the same logical chunk hit 16 distinct 4-bank groups.
template <int C>
__device__ __forceinline__ int tile_slot(int r, int X) {
  return r * C + (X ^ ((r >> 1) & 7));
}

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Transposed LDS read (ds_read_b64_tr_b16).  Within each 16-lane group,
// result lane i receives element (i % 4) of the 4-element chunks addressed
// by source lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  With source lane s of
// group G pointing at row kb + 4G + s/4, columns n0 + 4(s%4) .. +3, lane
// (i, G) receives column n0 + i of rows kb + 4G .. kb + 4G + 3.
__device__ __forceinline__ v4s lds_read_tr16(const char* lds_base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)((lds_char*)lds_base + byte_off));
}

template <int DK, int DV, int HW, int NW, bool SEPV>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(AttnArgs a, const int64_t* seq_off) {
  constexpr int NK = 32;                        // keys per tile
  constexpr int KC = DK / 8;                    // 16-byte chunks per K row
  constexpr int VC = SEPV ? DV / 8 : 0;         // chunks per separate V row
  constexpr int TILE_CHUNKS = NK * (KC + VC);
  constexpr int NT = NW * 64;
  constexpr int LOADS = (TILE_CHUNKS + NT - 1) / NT;  // 16-byte gathers per lane per tile
  constexpr int HS = HW / 16;                   // 16-head subtiles per wave
  constexpr int H = HW * NW;
  constexpr int TILE_BYTES = TILE_CHUNKS * 16;
  static_assert((NK * KC) % 64 == 0, "K region must be whole wave loads");
  static_assert(KC % 8 == 0 && VC % 8 == 0, "swizzle works on groups of 8 chunks");
  extern __shared__ __align__(16) char smem[];  // [2][TILE_BYTES]

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = blockIdx.x;
  __shared__ int s_cnt;
  const AttnRow row = attn_row(a, seq_off, t);
  const int n = valid_count(row.ip, a.k, &s_cnt);
  const char* kvb = (const char*)a.kv;
  const char* vvb = SEPV ? (const char*)a.v : kvb;
  const int64_t ldk = a.ld_kv * 2, ldv = (SEPV ? a.ld_v : a.ld_kv) * 2;  // bytes

  // gather plan: load i of wave w fills slots (i*NW + w)*64 + lane; a wave
  // whose slot range lies past the tile skips that load (wave-uniform)
  auto slot_row = [&](int i, int& r, int& off, bool& isv) {
    const int slot = (i * NW + w) * 64 + lane;
    isv = VC > 0 && slot >= NK * KC;
    const int rs = isv ? slot - NK * KC : slot;
    const int CC = isv ? (VC > 0 ? VC : 8) : KC;
    r = rs / CC;
    const int pc = rs - r * CC;
    off = (pc ^ ((r >> 1) & 7)) * 16;   // logical chunk stored at this slot, in bytes
  };
  auto fetch_idx = [&](int j0, int32_t* keys) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if ((i * NW + w) * 64 >= TILE_CHUNKS) break;
      int r, off;
      bool isv;
      slot_row(i, r, off, isv);
      const int j = j0 + r;
      int32_t s = row.ip[j < n ? j : j0];
      keys[i] = s < row.len ? s : (int32_t)(row.len - 1);
    }
  };
  auto issue_tile = [&](int buf, const int32_t* keys) {
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      if ((i * NW + w) * 64 >= TILE_CHUNKS) break;
      int r, off;
      bool isv;
      slot_row(i, r, off, isv);
      const int64_t kr = row.base + keys[i];
      const char* src = isv ? vvb + kr * ldv + off : kvb + kr * ldk + off;
      __builtin_amdgcn_global_load_lds(
          (const void*)src,
          (__attribute__((address_space(3))) void*)((lds_char*)smem + buf * TILE_BYTES + (i * NW + w) * 1024),
          16, 0, 0);
    }
  };

  // Q^T fragments: head 32w.. (HW per wave), subtile hs: head HW*w + 16hs + c
  v8s qf[HS][DK / 32];
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    const uint16_t* qp = (const uint16_t*)a.q + ((t * H) + HW * w + 16 * hs + c) * (int64_t)DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) qf[hs][kk] = *(const v8s*)(qp + 32 * kk);
  }
  v4f o[DV / 16][HS];
#pragma unroll
  for (int d = 0; d < DV / 16; ++d)
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) o[d][hs] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run[HS], l_part[HS];
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    m_run[hs] = -INFINITY;
    l_part[hs] = 0.f;
  }
  const float zs = a.scale * kLog2e;
  const int ntiles = (n + NK - 1) / NK;
  constexpr int VCH = SEPV ? VC : KC;  // chunks per row of the V rows
  int kbase[2], vbase[4];
  {
    const int sw = (c >> 1) & 7;
    kbase[0] = (c * KC + (g ^ sw)) * 16;
    kbase[1] = (c * KC + ((4 + g) ^ sw)) * 16;
    const int sl = lane & 15, G = lane >> 4;
    const int r0 = 4 * G + (sl >> 2), swv = (r0 >> 1) & 7;
#pragma unroll
    for (int q = 0; q < 4; ++q) vbase[q] = (r0 * VCH + ((2 * q + ((sl & 3) >> 1)) ^ swv)) * 16 + (sl & 1) * 8;
  }

  int32_t keys[LOADS];
  if (ntiles > 0) {
    fetch_idx(0, keys);
    issue_tile(0, keys);
    if (ntiles > 1) fetch_idx(NK, keys);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int it = 0; it < ntiles; ++it) {
    const int j0 = it * NK;
    if (it + 1 < ntiles) {
      issue_tile((it + 1) & 1, keys);
      if (it + 2 < ntiles) fetch_idx(j0 + 2 * NK, keys);
    }
    const char* tb = smem + (it & 1) * TILE_BYTES;

    // S^T = K . Q^T : key subtiles ks (rows 16ks + c), head subtiles hs.
    // Chunk 4kk + g of row r sits at 8*(kk/2) + ((4*(kk%2) + g) ^ sw(r)), and
    // rows c and 16 + c share sw, so two base offsets plus immediates cover
    // every read.
    v4f sacc[2][HS];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) sacc[ks][hs] = (v4f){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < DK / 32; ++kk) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8s kf = *(const v8s*)(tb + kbase[kk & 1] + ks * (16 * KC * 16) + (kk >> 1) * 128);
#pragma unroll
        for (int hs = 0; hs < HS; ++hs) sacc[ks][hs] = mfma_bf16_16x16x32(kf, qf[hs][kk], sacc[ks][hs]);
      }
      if (kk % DSA_QK_GROUP == DSA_QK_GROUP - 1) __builtin_amdgcn_sched_barrier(0);
    }

    // online softmax (log2 domain); the running max only moves when a tile
    // raises it by more than 2^8, so O is rescaled rarely
    v8s pb[HS];
    bool need_any = false;
    float zt[HS][8], mnew[HS];
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zt[hs][i] = (j0 + 4 * g + i < n) ? sacc[0][hs][i] * zs : -INFINITY;
        zt[hs][4 + i] = (j0 + 16 + 4 * g + i < n) ? sacc[1][hs][i] * zs : -INFINITY;
      }
      float mx = zt[hs][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, zt[hs][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool need = mx > m_run[hs] + 8.f;
      mnew[hs] = need ? mx : m_run[hs];
      need_any |= need;
    }
    if (__any(need_any)) {
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) {
        const float corr = exp2f(m_run[hs] - mnew[hs]);
        l_part[hs] *= corr;
#pragma unroll
        for (int d = 0; d < DV / 16; ++d) o[d][hs] *= corr;
        m_run[hs] = mnew[hs];
      }
    }
#pragma unroll
    for (int hs = 0; hs < HS; ++hs) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        p[i] = exp2f(zt[hs][i] - m_run[hs]);
        l_part[hs] += p[i];
      }
      v4i pk;
      pk[0] = (int)pack_bf16x2(p[0], p[1]);
      pk[1] = (int)pack_bf16x2(p[2], p[3]);
      pk[2] = (int)pack_bf16x2(p[4], p[5]);
      pk[3] = (int)pack_bf16x2(p[6], p[7]);
      pb[hs] = (v8s)pk;
    }

    // O^T += V^T . P^T ; V^T fragment via two transposed reads (rows
    // r0 = 4G + sl/4 and r0 + 16, which share a swizzle), dv chunk
    // 2d + (sl%4)/2 at 8*(d/4) + ((2*(d%4) + (sl%4)/2) ^ sw(r0))
    const char* vb = SEPV ? tb + NK * KC * 16 : tb;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      const int off = vbase[d & 3] + (d >> 2) * 128;
      const v4s lo = lds_read_tr16(vb, off);
      const v4s hi = lds_read_tr16(vb, off + 16 * VCH * 16);
      const v8s av = (v8s){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
      for (int hs = 0; hs < HS; ++hs) o[d][hs] = mfma_bf16_16x16x32(av, pb[hs], o[d][hs]);
      if (d % DSA_PV_GROUP == DSA_PV_GROUP - 1) __builtin_amdgcn_sched_barrier(0);
    }

    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }

  // epilogue: lane (c, g) holds O^T[dv = 16d + 4g + i][head HW*w + 16hs + c]
#pragma unroll
  for (int hs = 0; hs < HS; ++hs) {
    float l = l_part[hs];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int h = HW * w + 16 * hs + c;
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = (uint16_t*)a.out + (t * H + h) * (int64_t)DV;
#pragma unroll
    for (int d = 0; d < DV / 16; ++d) {
      v2i pk;
      pk[0] = (int)pack_bf16x2(o[d][hs][0] * inv, o[d][hs][1] * inv);
      pk[1] = (int)pack_bf16x2(o[d][hs][2] * inv, o[d][hs][3] * inv);
      *(v2i*)(op + 16 * d + 4 * g) = pk;
    }
    if (a.lse && g == 0) a.lse[t * H + h] = n > 0 ? (m_run[hs] + log2f(l)) * kLn2 : -INFINITY;
  }
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

template <int DK, int DV, int HW, int NW, bool SEPV>
static hipError_t launch_bf16(const AttnArgs& a, const int64_t* seq_off, hipStream_t st) {
  constexpr size_t lds = 2 * (size_t)32 * (DK / 8 + (SEPV ? DV / 8 : 0)) * 16;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)attn_bf16_kernel<DK, DV, HW, NW, SEPV>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  attn_bf16_kernel<DK, DV, HW, NW, SEPV><<<(unsigned)a.T, NW * 64, lds, st>>>(a, seq_off);
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
  if (a.H == 16 && a.Dk == 128 && a.Dv == 128) {
    if (a.v) return launch_bf16<128, 128, 16, 1, true>(a, a.seq_offsets, st);
    return launch_bf16<128, 128, 16, 1, false>(a, a.seq_offsets, st);
  }
  if (a.H == 128 && a.Dk == 576 && a.Dv == 512) {
    if (a.v) return launch_bf16<576, 512, DSA_MLA_HW, DSA_MLA_NW, true>(a, a.seq_offsets, st);
    return launch_bf16<576, 512, DSA_MLA_HW, DSA_MLA_NW, false>(a, a.seq_offsets, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
