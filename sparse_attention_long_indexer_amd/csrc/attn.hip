// Sparse MQA attention over the selected key rows (DeepSeek-V3.2 write-up,
// sections 2.3 and 3.1: ordinary softmax attention restricted to the k
// selected keys, all query heads sharing one key/value head as in MLA's MQA
// mode).
//
// Three bf16 kernels.  The MLA shape with the shared latent row (128 heads,
// key = 576-wide latent row, value = its first 512 columns) runs
// attn_mla_kernel, where two groups of four waves alternate between S^T +
// softmax and PV so that each SIMD always has one wave feeding its matrix
// core.  16 heads of 128 run attn_h16_kernel: one wave per query over
// 16-key tiles, P^T kept in registers, nine blocks per CU.  MLA with a
// separate value tensor runs attn_bf16_kernel: one block per query (or per
// key split of one), 16 heads per wave.  Each kernel gathers the selected
// rows into LDS with direct-to-LDS copies (the gather of the next tile runs
// during the current one), then
//   S^T = K . Q^T   with v_mfma_f32_16x16x32_bf16 (A = K fragments from LDS,
//                   B = Q^T held in registers for the whole loop),
//   an online softmax per head in the log2 domain, and
//   O^T += V^T . P^T for all heads over the wave's slice of the value
//                   columns (A = V^T via transposed LDS reads, B = P^T).
// Heads sit in the N dimension, one head per lane column, so the softmax
// rescale of O is a per-lane scalar.  Barriers inside the loops order LDS
// only; the gathers are awaited explicitly.  With few queries (batched
// decode) the selected keys are split over blocks and an LSE combine kernel
// merges the parts.  (Each kernel is described where it is defined.)
//
// fp32 path: a plain VALU kernel for the small fp32 configuration.
#include "common.h"
#include "kernels.h"
#include "dsa.h"

namespace dsa {

constexpr int kQkGroup = 4;  // QK k-steps the scheduler may interleave
constexpr int kPvGroup = 4;  // PV head subtiles the scheduler may interleave

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

// LDS tile of NK = 32 gathered rows, stored fragment-major: the rows form
// two 16-row key subtiles, each row C chunks of 16 bytes; fragment
// (ks, q) holds chunks 4q .. 4q+3 of rows 16ks .. 16ks+15 as 64 slots
// (chunk-column major, slot = 16 * (X % 4) + (row % 16 ^ 8 * (X % 2))).  One
// 16x16x32 MFMA operand is then one 1 KB read whose 16-lane quarters each
// cover 256 contiguous bytes, and a transposed V read (4 rows x 2 adjacent
// chunks per 16 lanes) touches two 64-byte runs that the row swizzle puts on
// different LDS banks.  Each gathered fragment is one 64-lane direct-to-LDS
// copy.
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

// Eight transposed reads: value subtiles d = 0..3 (byte offsets 512 d from
// `lds_ptr`) of key subtile 0 and of key subtile 1 (HI bytes further), into
// av[d] = (key rows 0-15 | key rows 16-31).  One asm block that ends with
// its own lgkmcnt wait: through the builtin, each read would also wait for
// the direct-to-LDS gather of the next tile still in flight into the other
// buffer, because the compiler cannot tell the two LDS regions apart.  The
// outputs are early-clobber: a load may land before a later one reads the
// address register.
template <int HI>
__device__ __forceinline__ void lds_read_vt4(const char* lds_ptr, v8s* av) {
  const uint32_t addr = (uint32_t)(uintptr_t)(const lds_char*)lds_ptr;
  v2i r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:512\n\t"
      "ds_read_b64_tr_b16 %2, %8 offset:1024\n\t"
      "ds_read_b64_tr_b16 %3, %8 offset:1536\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%9\n\t"
      "ds_read_b64_tr_b16 %5, %8 offset:%10\n\t"
      "ds_read_b64_tr_b16 %6, %8 offset:%11\n\t"
      "ds_read_b64_tr_b16 %7, %8 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(addr), "i"(HI), "i"(HI + 512), "i"(HI + 1024), "i"(HI + 1536)
      : "memory");
  const v2i lo[4] = {r0, r1, r2, r3}, hi[4] = {r4, r5, r6, r7};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const v4s l = __builtin_bit_cast(v4s, lo[d]), h = __builtin_bit_cast(v4s, hi[d]);
    av[d] = (v8s){l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  }
}

// MLA with a separate value tensor: one block of NW waves per query (or key
// split), wave w owning heads 16w .. 16w+15 for S^T and the softmax and
// value columns w DV/NW .. for PV, 32-key tiles double buffered.
template <int DK, int DV, int NW, bool SEPV>
__global__ __launch_bounds__(NW * 64, 1) void attn_bf16_kernel(AttnArgs a, const int64_t* seq_off) {
  constexpr int NK = 32;                        // keys per tile
  constexpr int KC = DK / 8;                    // 16-byte chunks per K row
  constexpr int VC = SEPV ? DV / 8 : 0;         // chunks per separate V row
  constexpr int VCH = SEPV ? VC : KC;           // chunks per row of the V rows
  constexpr int TILE_CHUNKS = NK * (KC + VC);
  constexpr int NT = NW * 64;
  constexpr int H = 16 * NW;                    // wave w owns heads 16w .. 16w+15 for QK/softmax
  constexpr int DVW = DV / NW;                  // ... and value columns w*DVW .. +DVW for PV
  constexpr int ND = DVW / 16;
  constexpr int TILE_BYTES = TILE_CHUNKS * 16;
  static_assert(KC % 4 == 0 && VC % 4 == 0, "fragments are 4 chunks wide");
  static_assert(DV % (16 * NW) == 0, "value columns split evenly over the waves");
  static_assert(DV / NW == 64, "each wave reads its four value subtiles in one asm block");
  constexpr int KF = 2 * (KC / 4);              // K fragments per tile
  constexpr int NFRAG = KF + 2 * (VC / 4);      // fragments per tile
  constexpr int LOADS = (NFRAG + NW - 1) / NW;  // fragment copies per wave per tile
  constexpr int VF = VCH / 4;
  constexpr int KKW = DK / 32;  // k-steps of 32 dims
  // dynamic LDS: [2][TILE_BYTES] tiles | [NW] P^T fragments (1 KB) | [3][32]
  // index entries of the upcoming tiles (copied from the index row two
  // tiles ahead), which keeps a one-wave block at 33 KB
  extern __shared__ __align__(16) char smem[];
  char* pbuf = smem + 2 * TILE_BYTES;
  int32_t* sring = (int32_t*)(pbuf + NW * 1024);
  __shared__ float s_corr[H], s_l[H];
  __shared__ int s_need[NW];
  __shared__ int s_cnt;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = blockIdx.x / a.splits;
  const int sp = (int)(blockIdx.x % a.splits);
  const AttnRow row = attn_row(a, seq_off, t);
  // n = leading valid entries of the query's index row
  if (tid == 0) s_cnt = (int)a.k;
  __syncthreads();
  {
    int first = (int)a.k;
    for (int j = tid; j < (int)a.k; j += NT)
      if (row.ip[j] < 0 && j < first) first = j;
    if (first < (int)a.k) atomicMin(&s_cnt, first);
  }
  __syncthreads();
  // this block's keys: [kbeg, n) of the valid entries (split in whole tiles)
  const int nvalid = s_cnt;
  const int per = ((nvalid + a.splits - 1) / a.splits + NK - 1) / NK * NK;
  const int kbeg = min(nvalid, sp * per);
  const int n = min(nvalid, kbeg + per);
  // this query's cache rows start at a wave-uniform base; a row's bytes sit
  // at a 32-bit offset from it (the launcher checks rows * ld * 2 < 4 GiB)
  const uint32_t ldk = (uint32_t)(a.ld_kv * 2), ldv = (uint32_t)((SEPV ? a.ld_v : a.ld_kv) * 2);  // bytes
  const char* kvq = (const char*)a.kv + row.base * (int64_t)ldk;
  const char* vvq = SEPV ? (const char*)a.v + row.base * (int64_t)ldv : kvq;

  // gather: copy i of wave w fills fragment f = i*NW + w of the tile; lane
  // l brings chunk 4q + l/16 of row 16ks + (l%16 ^ 8((l/16)%2)), so per tile
  // a lane needs the offsets of two rows (ks = 0, 1); the chunk offset 64q
  // is wave-uniform (a wave past the last fragment skips the copy)
  const int rl = (lane & 15) ^ ((lane & 16) >> 1);
  const uint32_t lofs = 16u * (uint32_t)(lane >> 4);
  // wave 0 copies a tile's 32 index entries into ring slot tile % 3
  auto fetch_idx = [&](int tile) {
    if (w == 0 && lane < NK) {
      const int j = min(tile * NK + lane, (int)a.k - 1);
      __builtin_amdgcn_global_load_lds((const void*)(row.ip + j),
                                       (__attribute__((address_space(3))) void*)(lds_char*)(sring + (tile % 3) * NK),
                                       4, 0, 0);
    }
  };
  const int32_t lenm1 = (int32_t)(row.len - 1);
  auto issue_tile = [&](int tile) {
    const int j0 = tile * NK;
    char* dst = smem + (tile & 1) * TILE_BYTES;
    // past the valid entries: the tile's first one (valid); an index past
    // the query's rows reads its last row
    const int32_t* si = sring + (tile % 3) * NK;
    const int32_t ra = si[j0 + rl < n ? rl : 0], rb = si[j0 + 16 + rl < n ? 16 + rl : 0];
    const uint32_t sa = (uint32_t)(ra < lenm1 ? ra : lenm1), sb = (uint32_t)(rb < lenm1 ? rb : lenm1);
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int f = i * NW + w;
      if (f >= NFRAG) break;
      const bool isv = VC > 0 && f >= KF;
      const int fr = isv ? f - KF : f;
      const int FQ = isv ? (VC > 0 ? VC / 4 : 1) : KC / 4;
      const int ks = fr / FQ, q = fr - ks * FQ;
      const char* src = isv ? vvq + 64 * q + ((ks ? sb : sa) * ldv + lofs)
                            : kvq + 64 * q + ((ks ? sb : sa) * ldk + lofs);
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)((lds_char*)dst + f * 1024), 16, 0,
                                       0);
    }
  };

  // Q^T fragments, dims 32kk + 8g .. +8, of head 16w + c
  v8s qf[KKW];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((t * H) + 16 * w + c) * (int64_t)DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KKW; ++kk) qf[kk] = *(const v8s*)(qp + 32 * kk);
  }
  // O^T accumulators: value subtile d of this wave's columns x head subtile hs
  v4f o[ND][NW];
#pragma unroll
  for (int d = 0; d < ND; ++d)
#pragma unroll
    for (int hs = 0; hs < NW; ++hs) o[d][hs] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  const float zs = a.scale * kLog2e;
  const int ntiles = (n - kbeg + NK - 1) / NK;
  // V^T reads: lane (sl, G) reads row 4G + sl/4 (+16h), dv 16D + 4(sl%4):
  // chunk X = 2D + (sl%4)/2, half sl%2, i.e. slot
  // ((h*VF + D/2)*4 + 2(D%2) + (sl%4)/2)*16 + ((4G + sl/4) ^ 8((sl%4)/2)).
  const int vbase =
      ((((lane & 3) >> 1) * 16) + ((4 * (lane >> 4) + ((lane & 15) >> 2)) ^ (((lane >> 1) & 1) << 3))) * 16 +
      (lane & 1) * 8;
  const int kslot = lane ^ ((lane & 16) >> 1);  // lane's MFMA operand slot in a fragment

  // Per tile: S^T and softmax for the wave's 16 heads, P^T published to
  // LDS, then O^T for all heads over the wave's value columns.  The gather
  // of tile it+1 is issued first, into the buffer every wave finished
  // reading before the barrier that closed the previous tile.
  const int t0 = kbeg / NK;  // first tile of this split
  if (ntiles > 0) {
    fetch_idx(t0);
    if (ntiles > 1) fetch_idx(t0 + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue_tile(t0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int it = t0; it < t0 + ntiles; ++it) {
    if (it + 1 < t0 + ntiles) issue_tile(it + 1);
    // into the slot of tile it - 1, whose gather every wave issued two
    // barriers ago; it lands with the gather, before the tile's end
    if (it + 2 < t0 + ntiles) fetch_idx(it + 2);
    const char* tb = smem + (it & 1) * TILE_BYTES;
    const int j0 = it * NK;
    // S^T = K . Q^T (key subtiles ks = rows 16ks + c)
    v4f sc[2] = {(v4f){0.f, 0.f, 0.f, 0.f}, (v4f){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < KKW; ++kk) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const v8s kf = *(const v8s*)(tb + ((ks * (KC / 4) + kk) * 64 + kslot) * 16);
        sc[ks] = mfma_bf16_16x16x32(kf, qf[kk], sc[ks]);
      }
      if (kk % kQkGroup == kQkGroup - 1) __builtin_amdgcn_sched_barrier(0);
    }
    // online softmax (log2 domain); the running max only moves when a tile
    // raises it by more than 2^8, so O is rescaled rarely
    {
      float zt[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        zt[i] = (j0 + 4 * g + i < n) ? sc[0][i] * zs : -INFINITY;
        zt[4 + i] = (j0 + 16 + 4 * g + i < n) ? sc[1][i] * zs : -INFINITY;
      }
      float mx = zt[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) mx = fmaxf(mx, zt[i]);
      mx = rows_max(mx);
      const bool need = mx > m_run + 8.f;
      const float mnew = need ? mx : m_run;
      const float corr = exp2f(m_run - mnew);
      m_run = mnew;
      float ps = 0.f;
      v4i pk;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = exp2f(zt[2 * i] - mnew), p1 = exp2f(zt[2 * i + 1] - mnew);
        ps += p0 + p1;
        pk[i] = (int)pack_bf16x2(p0, p1);
      }
      l_part = l_part * corr + ps;
      *(v4i*)(pbuf + (w * 64 + lane) * 16) = pk;
      if (g == 0) s_corr[16 * w + c] = corr;
      const bool any = __any(need);
      if (lane == 0) s_need[w] = any ? 1 : 0;
    }
    lds_barrier();  // the gather of tile it+1 may still be in flight
    // a head whose max moved: rescale its O columns (all waves hold them)
    bool resc = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) resc |= s_need[i] != 0;
    if (resc) {
#pragma unroll
      for (int hs = 0; hs < NW; ++hs) {
        const float cr = s_corr[16 * hs + c];
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d][hs] *= cr;
      }
    }
    // O^T += V^T . P^T over this wave's value columns
    {
      const char* vb = SEPV ? tb + KF * 1024 : tb;
      // subtiles D = 4w .. 4w+3 sit in fragments 2w, 2w+1 of each key subtile
      v8s av[ND];
      lds_read_vt4<VF * 1024>(vb + vbase + 2048 * w, av);
#pragma unroll
      for (int hs = 0; hs < NW; ++hs) {
        const v8s pf = *(const v8s*)(pbuf + (hs * 64 + lane) * 16);
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d][hs] = mfma_bf16_16x16x32(av[d], pf, o[d][hs]);
        if (hs % kPvGroup == kPvGroup - 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  }

  // epilogue: row sums of every head, then lane (c, g) of wave w writes
  // O^T[dv = DVW*w + 16d + 4g + i][head 16hs + c]: normalised bf16 output,
  // or with several splits the unnormalised partial as fp16 over its
  // 64-column slice scale, plus (max, sum)
  const bool partial = a.splits > 1;
  {
    const float l = rows_sum(l_part);
    if (g == 0) s_l[16 * w + c] = l;
    if (g == 0) {
      const int h = 16 * w + c;
      if (partial) {
        float* ml = a.part_ml + ((t * a.splits + sp) * H + h) * 2;
        ml[0] = m_run;
        ml[1] = l;
      } else if (a.lse) {
        a.lse[t * H + h] = n > 0 ? (m_run + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
  __syncthreads();
#pragma unroll
  for (int hs = 0; hs < NW; ++hs) {
    const int h = 16 * hs + c;
    if (partial) {
      // slice w of head h: the lane's 16 values, then the four lanes of the head
      float mx = 0.f;
#pragma unroll
      for (int d = 0; d < ND; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(o[d][hs][i]));
      mx = rows_max(mx);
      const float sc = mx > 0.f ? mx : 1.f, isc = 1.f / sc;
      if (g == 0) a.part_sc[((t * a.splits + sp) * H + h) * (DV / 64) + w] = sc;
      uint16_t* op = a.part_o + ((t * a.splits + sp) * H + h) * (int64_t)DV + DVW * w;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        const v2i pk = {(int)pack_f16x2(o[d][hs][0] * isc, o[d][hs][1] * isc),
                        (int)pack_f16x2(o[d][hs][2] * isc, o[d][hs][3] * isc)};
        *(v2i*)(op + 16 * d + 4 * g) = pk;
      }
    } else {
      const float l = s_l[h];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      uint16_t* op = (uint16_t*)a.out + (t * H + h) * (int64_t)DV + DVW * w;
#pragma unroll
      for (int d = 0; d < ND; ++d) {
        v2i pk;
        pk[0] = (int)pack_bf16x2(o[d][hs][0] * inv, o[d][hs][1] * inv);
        pk[1] = (int)pack_bf16x2(o[d][hs][2] * inv, o[d][hs][3] * inv);
        *(v2i*)(op + 16 * d + 4 * g) = pk;
      }
    }
  }
}

// Eight transposed reads for the whole-line tile layout of the MLA kernel:
// value subtile d of key subtile 0 at LDS address a[d], of key subtile 1 at
// a[d] + HI (the per-lane row swizzle permutes the subtiles' positions, so
// each takes its own address).  Same asm discipline as lds_read_vt4.
template <int HI>
__device__ __forceinline__ void lds_read_vt4_at(const uint32_t (&a)[4], v8s* av) {
  v2i r0, r1, r2, r3, r4, r5, r6, r7;
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %9\n\t"
      "ds_read_b64_tr_b16 %2, %10\n\t"
      "ds_read_b64_tr_b16 %3, %11\n\t"
      "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
      "ds_read_b64_tr_b16 %5, %9 offset:%12\n\t"
      "ds_read_b64_tr_b16 %6, %10 offset:%12\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:%12\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3), "=&v"(r4), "=&v"(r5), "=&v"(r6), "=&v"(r7)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(HI)
      : "memory");
  const v2i lo[4] = {r0, r1, r2, r3}, hi[4] = {r4, r5, r6, r7};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const v4s l = __builtin_bit_cast(v4s, lo[d]), h = __builtin_bit_cast(v4s, hi[d]);
    av[d] = (v8s){l[0], l[1], l[2], l[3], h[0], h[1], h[2], h[3]};
  }
}

// ---- 16 heads of 128: one wave per query, 16-key tiles ----------------------
// S^T (16 keys x 16 heads) with 16x16x32 MFMAs over the 128 key dims; the
// result lane (c, g) holds keys 4g .. 4g+3 of head c, which is exactly the
// B operand of a 16x16x16 MFMA, so P^T stays in registers and O^T (128
// value columns x 16 heads, 8 subtiles) accumulates with 16x16x16 MFMAs.
// Every O^T entry of a lane belongs to its head c, so the rescale is
// lane-local too.  A block holds two tiles (4 KB of key rows, plus 4 KB of
// value rows with a separate V) and a 3-slot ring of index entries: about
// 16 KB, so nine one-wave blocks share a CU.
//
// Tile layout: row r (256 bytes) at 256 r, its 16-byte chunk x in slot
// x ^ sw(r), sw(r) = 2 (r % 8) + r / 8.  The 16 lanes of an S^T operand read
// (chunk 4kk + g of rows 0..15) and the 32 lanes of a half-wave transposed
// V read (rows 4G + s/4 of G = 0, 1 or 2, 3; chunks 2D, 2D + 1) each hit
// distinct bank groups.  A 1 KB copy brings four rows, 16 lanes per row, so
// every copy reads whole 128-byte lines.
__device__ __forceinline__ int h16_sw(int r) { return ((r << 1) & 14) | (r >> 3); }

template <bool SEPV>
__global__ __launch_bounds__(64) void attn_h16_kernel(AttnArgs a, const int64_t* seq_off) {
  constexpr int NK = 16, D = 128, H = 16;
  constexpr int KB = NK * D * 2;             // 4 KB of key rows per tile
  constexpr int TILE = SEPV ? 2 * KB : KB;
  constexpr int KK = D / 32;                 // S^T k-steps
  constexpr int ND = D / 16;                 // O^T value subtiles
  extern __shared__ __align__(16) char smem[];
  int32_t* sring = (int32_t*)(smem + 2 * TILE);   // [3][NK] index entries
  __shared__ int s_cnt;

  const int lane = threadIdx.x;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = blockIdx.x / a.splits;
  const int sp = (int)(blockIdx.x % a.splits);
  const AttnRow row = attn_row(a, seq_off, t);
  // n = leading valid entries of the query's index row
  if (lane == 0) s_cnt = (int)a.k;
  __syncthreads();
  {
    int first = (int)a.k;
    for (int j = lane; j < (int)a.k; j += 64)
      if (row.ip[j] < 0 && j < first) first = j;
    if (first < (int)a.k) atomicMin(&s_cnt, first);
  }
  __syncthreads();
  const int nvalid = s_cnt;
  const int per = ((nvalid + a.splits - 1) / a.splits + NK - 1) / NK * NK;
  const int kbeg = min(nvalid, sp * per);
  const int n = min(nvalid, kbeg + per);
  const uint32_t ldk = (uint32_t)(a.ld_kv * 2), ldv = (uint32_t)((SEPV ? a.ld_v : a.ld_kv) * 2);  // bytes
  const char* kvq = (const char*)a.kv + row.base * (int64_t)ldk;
  const char* vvq = SEPV ? (const char*)a.v + row.base * (int64_t)ldv : kvq;
  const int32_t lenm1 = (int32_t)(row.len - 1);

  // lanes 0..15 copy a tile's index entries into ring slot tile % 3
  auto fetch_idx = [&](int tile) {
    if (lane < NK) {
      const int j = min(tile * NK + lane, (int)a.k - 1);
      __builtin_amdgcn_global_load_lds((const void*)(row.ip + j),
                                       (__attribute__((address_space(3))) void*)(lds_char*)(sring + (tile % 3) * NK),
                                       4, 0, 0);
    }
  };
  // copy i brings rows 4 (i % 4) .. +3 (key rows, then value rows); lane l
  // fills slot l % 16 of row 4 (i % 4) + l / 16 with chunk (l % 16) ^ sw(row)
  auto issue_tile = [&](int tile) {
    const int j0 = tile * NK;
    char* dst = smem + (tile & 1) * TILE;
    const int32_t* si = sring + (tile % 3) * NK;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int r = 4 * q + g;
      // past the valid entries: the tile's first one (valid); an index past
      // the query's rows reads its last row
      const int32_t e = si[j0 + r < n ? r : 0];
      const uint32_t rr = (uint32_t)(e < lenm1 ? e : lenm1);
      const uint32_t col = 16u * (uint32_t)(c ^ h16_sw(r));
      __builtin_amdgcn_global_load_lds((const void*)(kvq + (rr * ldk + col)),
                                       (__attribute__((address_space(3))) void*)((lds_char*)dst + q * 1024), 16, 0,
                                       0);
      if (SEPV)
        __builtin_amdgcn_global_load_lds((const void*)(vvq + (rr * ldv + col)),
                                         (__attribute__((address_space(3))) void*)((lds_char*)dst + KB + q * 1024),
                                         16, 0, 0);
    }
  };

  // Q^T fragments, dims 32kk + 8g .. +7, of head c
  v8s qf[KK];
  {
    const uint16_t* qp = (const uint16_t*)a.q + (t * H + c) * (int64_t)D + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const v8s*)(qp + 32 * kk);
  }
  v4f o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = (v4f){0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_part = 0.f;
  const float zs = a.scale * kLog2e;
  const int ntiles = (n - kbeg + NK - 1) / NK;
  // S^T operand of k-step kk: row c, chunk 4kk + g
  const int sw_c = h16_sw(c);
  // V^T operand of subtile d: source lane (s = l % 16, G = l / 16) reads row
  // 4G + s/4, value columns 16d + 4 (s%4) .. +3: chunk 2d + (s%4)/2, half s%2
  const int vr = 4 * g + (c >> 2);
  const int vsw = h16_sw(vr), vh = ((c & 3) >> 1);
  const int voff = 256 * vr + 8 * (c & 1);

  const int t0 = kbeg / NK;
  const int tend = t0 + ntiles;
  if (ntiles > 0) {
    fetch_idx(t0);
    if (ntiles > 1) fetch_idx(t0 + 1);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    issue_tile(t0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  for (int it = t0; it < tend; ++it) {
    if (it + 1 < tend) issue_tile(it + 1);
    // into the slot of tile it - 1, gathered two iterations ago
    if (it + 2 < tend) fetch_idx(it + 2);
    const char* tb = smem + (it & 1) * TILE;
    const int j0 = it * NK;
    // S^T = K . Q^T, even and odd k-steps in separate accumulators
    v4f s0 = {0.f, 0.f, 0.f, 0.f}, s1 = s0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const v8s kf = *(const v8s*)(tb + 256 * c + 16 * ((4 * kk + g) ^ sw_c));
      if (kk & 1)
        s1 = mfma_bf16_16x16x32(kf, qf[kk], s1);
      else
        s0 = mfma_bf16_16x16x32(kf, qf[kk], s0);
    }
    // online softmax (log2 domain); the running max only moves when a tile
    // raises it by more than 2^8, so O is rescaled rarely
    float zt[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) zt[i] = (j0 + 4 * g + i < n) ? (s0[i] + s1[i]) * zs : -INFINITY;
    float mx = fmaxf(fmaxf(zt[0], zt[1]), fmaxf(zt[2], zt[3]));
    mx = rows_max(mx);
    const bool need = mx > m_run + 8.f;
    const float mnew = need ? mx : m_run;
    const float corr = exp2f(m_run - mnew);
    m_run = mnew;
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = exp2f(zt[i] - mnew);
    l_part = l_part * corr + ((p[0] + p[1]) + (p[2] + p[3]));
    if (__any(need)) {
#pragma unroll
      for (int d = 0; d < ND; ++d) o[d] *= corr;
    }
    const v2i pk = {(int)pack_bf16x2(p[0], p[1]), (int)pack_bf16x2(p[2], p[3])};
    const v4s pf = __builtin_bit_cast(v4s, pk);
    // O^T += V^T . P^T
    const char* vb = SEPV ? tb + KB : tb;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      const v4s av = lds_read_tr16(vb, voff + 16 * ((2 * d + vh) ^ vsw));
      o[d] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, pf, o[d], 0, 0, 0);
    }
    if (it + 1 < tend) __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
  }

  // epilogue: row sums per head, then lane (c, g) writes O^T[dv = 16d + 4g
  // + i][head c]: normalised bf16 output, or with several splits the
  // unnormalised partial as fp16 over its 64-column slice scales, plus
  // (max, sum)
  const bool partial = a.splits > 1;
  const float l = rows_sum(l_part);
  if (g == 0) {
    if (partial) {
      float* ml = a.part_ml + ((t * a.splits + sp) * H + c) * 2;
      ml[0] = m_run;
      ml[1] = l;
    } else if (a.lse) {
      a.lse[t * H + c] = n > 0 ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    }
  }
  if (partial) {
    uint16_t* op = a.part_o + ((t * a.splits + sp) * H + c) * (int64_t)D + 4 * g;
#pragma unroll
    for (int q = 0; q < D / 64; ++q) {
      // slice q = subtiles 4q .. 4q+3: the lane's 16 values, then the head's four lanes
      float mx = 0.f;
#pragma unroll
      for (int d = 4 * q; d < 4 * q + 4; ++d)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, fabsf(o[d][i]));
      mx = rows_max(mx);
      const float sc = mx > 0.f ? mx : 1.f, isc = 1.f / sc;
      if (g == 0) a.part_sc[((t * a.splits + sp) * H + c) * (D / 64) + q] = sc;
#pragma unroll
      for (int d = 4 * q; d < 4 * q + 4; ++d) {
        const v2i pk = {(int)pack_f16x2(o[d][0] * isc, o[d][1] * isc), (int)pack_f16x2(o[d][2] * isc, o[d][3] * isc)};
        *(v2i*)(op + 16 * d) = pk;
      }
    }
  } else {
    const float inv = l > 0.f ? 1.f / l : 0.f;
    uint16_t* op = (uint16_t*)a.out + (t * H + c) * (int64_t)D + 4 * g;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      v2i pk;
      pk[0] = (int)pack_bf16x2(o[d][0] * inv, o[d][1] * inv);
      pk[1] = (int)pack_bf16x2(o[d][2] * inv, o[d][3] * inv);
      *(v2i*)(op + 16 * d) = pk;
    }
  }
}

// ---- MLA shape, shared latent row: two wave groups in ping-pong -----------
// 128 heads, key = the 576-wide latent row, value = its first 512 columns.
// Eight waves, two per SIMD (wave w runs on SIMD w % 4), in two groups
// G = w / 4.  Wave w computes S^T and the softmax for heads 16w .. 16w+15
// over all 576 key dims (16x16x32 MFMAs), and accumulates O^T for all 128
// heads over value columns 64w .. 64w+63 (32x32x16 MFMAs, which one wave
// alone issues faster than 16x16x32).  The loop runs in slots closed by block barriers:
// in slot 2j group 0 does S^T + softmax of tile j while group 1 does PV of
// tile j-1, in slot 2j+1 group 1 does S^T + softmax of tile j while group 0
// does PV of tile j-1.  Each SIMD then always holds one wave feeding its
// matrix core while the other is in its softmax or waiting on LDS, and the
// S^T wave runs at raised priority so its softmax starts early.  Tile j is
// read in slots 2j .. 2j+3; group 1 gathers tile j+1 at the start of slot
// 2j into the third buffer and awaits it at the end of slot 2j+1.  P^T and
// the rescale factors are double buffered by tile parity.
//
// Tile layout (whole lines): the 32 rows x 9 lines of 128 bytes arrive as 36
// copies of 1 KB; copy 9 rb + L holds line L (chunks 8L .. 8L+7) of rows
// 8 rb .. 8 rb + 7, row r % 8 in slots 8 (r % 8) .. +7 with chunk x in slot
// position (x % 8) ^ ((r >> 1) & 7).  Every copy reads whole cache lines
// (a gather of random 1152-byte rows into LDS moves 7.2 TB/s this way
// against 5.3 TB/s for copies of half lines), the 16 lanes of an S^T
// operand read hit 16 distinct bank groups, and the transposed V^T reads
// are 2-way conflicted (an eighth of the LDS read traffic).
constexpr int kMlaTile = 32 * (576 / 8) * 16;         // 32 latent rows, 36 KB
constexpr size_t kMlaFixedLds = 3 * kMlaTile + 2 * 8 * 1024;

constexpr int kMlaQkg = 2;  // k-steps of S^T reads in flight ahead of the MFMAs (2 fragments each)

// 2^x with the hardware instruction alone: results below 2^-126 flush to
// zero, which for softmax weights relative to a running max (sum >= 1) is
// far below the bf16 rounding of P
__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

__global__ __launch_bounds__(512, 1) void attn_mla_kernel(AttnArgs a, const int64_t* seq_off) {
  constexpr int NK = 32, DK = 576, DV = 512, H = 128, NW = 8;
  constexpr int KK = DK / 32;       // k-steps of S^T
  extern __shared__ __align__(16) char smem[];
  char* pbuf = smem + 3 * kMlaTile;                 // [parity][wave][lane] 16-byte P^T fragments
  int32_t* sidx = (int32_t*)(pbuf + 2 * 8 * 1024);  // the block's index row
  __shared__ float s_corr[2][H], s_l[H];
  __shared__ int s_need[2][NW];
  __shared__ int s_cnt;

  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int G = w >> 2, gw = w & 3;
  const int g = lane >> 4, c = lane & 15;
  const int64_t t = blockIdx.x / a.splits;
  const int sp = (int)(blockIdx.x % a.splits);
  const AttnRow row = attn_row(a, seq_off, t);
  if (tid == 0) s_cnt = (int)a.k;
  __syncthreads();
  {
    int first = (int)a.k;
    for (int j = tid; j < (int)a.k; j += NW * 64) {
      int32_t s = row.ip[j];
      if (s < 0 && j < first) first = j;
      sidx[j] = s < row.len ? s : (int32_t)(row.len - 1);
    }
    if (first < (int)a.k) atomicMin(&s_cnt, first);
  }
  __syncthreads();
  const int nvalid = s_cnt;
  const int per = ((nvalid + a.splits - 1) / a.splits + NK - 1) / NK * NK;
  const int kbeg = min(nvalid, sp * per);
  const int n = min(nvalid, kbeg + per);
  const int ntiles = (n - kbeg + NK - 1) / NK;
  const uint32_t ldk = (uint32_t)(a.ld_kv * 2);  // bytes; rows * ld * 2 < 4 GiB (checked by the launcher)
  const char* kvq = (const char*)a.kv + row.base * (int64_t)ldk;

  // gather (group 1): wave 4 + gw copies rows 8 gw .. 8 gw + 7 of the tile,
  // line by line; lane l brings chunk 8L + ((l % 8) ^ swz) of row
  // 8 gw + l / 8 to slot l of copy 9 gw + L
  const uint32_t gsw = 16u * (uint32_t)((lane & 7) ^ ((4 * gw + (lane >> 4)) & 7));
  auto issue_tile = [&](int jl) {
    const int j0 = kbeg + jl * NK;
    char* dst = smem + (jl % 3) * kMlaTile + 9 * 1024 * gw;
    const int jr = j0 + 8 * gw + (lane >> 3);
    const uint32_t rr = (uint32_t)sidx[jr < n ? jr : j0];
    const char* src0 = kvq + (rr * ldk + gsw);
#pragma unroll
    for (int L = 0; L < 9; ++L) {
      __builtin_amdgcn_global_load_lds((const void*)(src0 + 128 * L),
                                       (__attribute__((address_space(3))) void*)((lds_char*)dst + L * 1024), 16, 0,
                                       0);
    }
  };

  // Q^T fragments of head 16w + c, dims 32kk + 8g .. +7
  v8s qf[KK];
  {
    const uint16_t* qp = (const uint16_t*)a.q + ((t * H) + 16 * w + c) * (int64_t)DK + 8 * g;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qf[kk] = *(const v8s*)(qp + 32 * kk);
  }
  // O^T blocks of 32 value columns (64w + 32 vb ..) x 32 heads (32 hb ..)
  v16f o[2][4];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[vb][hb][r] = 0.f;
  float m_run = -INFINITY, l_part = 0.f;
  const float zs = a.scale * kLog2e;
  // 32x32x16 PV: A operand (value block vb, k-step m) of lane (G = l/16,
  // s = l%16) is column 64w + 32 vb + 16 (G%2) + s of keys 4 gk .. +3 and
  // 16 + 4 gk .. +3, gk = 2m + G/2 (the keys S^T lane (c, gk) holds); the
  // source lane s reads row 8m + 4 (G/2) + s/4, columns .. + 4 (s%4): chunk
  // 8w + 4 vb + 2 (G%2) + (s%4)/2, half s%2, at vqn ^ 64 (vb ^ m), + 9216 m
  const int G16 = lane >> 4, s16 = lane & 15;
  const int vqn = 1024 * w + 128 * (4 * (G16 >> 1) + (s16 >> 2)) +
                  16 * (2 * ((G16 & 1) ^ (G16 >> 1)) + (((s16 & 3) >> 1) ^ (s16 >> 3))) + 8 * (s16 & 1);
  // B operand (heads 32 hb + j, j = l%32, k-step m): the P^T fragment of
  // S^T wave 2 hb + j/16, lane (j%16) + 16 (2m + l/32)
  const int pq = 1024 * ((lane & 31) >> 4) + 16 * ((lane & 15) + 16 * (lane >> 5));
  // S^T reads: lane (g, c) takes chunk 4 kk + g of row 16 ks + c, at offset
  // sb0 + 1024 (kk / 2) + 18432 ks for even kk and sb0 ^ 64 for odd kk
  const int sswz = (c >> 1) & 7;
  const int sb0 = 9216 * (c >> 3) + 128 * (c & 7) + 16 * (g ^ (sswz & 3)) + 64 * (sswz >> 2);

  // S^T = K . Q^T for the wave's 16 heads (key subtiles 0 and 1, even and
  // odd k-steps in separate accumulators), then the online softmax in the
  // log2 domain; the running max only moves when a tile raises it by more
  // than 2^8.  P^T, the rescale factors and the moved flag go to LDS.
  auto qk_softmax = [&](int jl) {
    const char* tb = smem + (jl % 3) * kMlaTile;
    const int j0 = kbeg + jl * NK;
    __builtin_amdgcn_s_setprio(1);
    v4f sc0 = {0.f, 0.f, 0.f, 0.f}, sc1 = sc0;
    // K fragments in a rolling pipeline: the reads of k-step kk + D are
    // issued before the MFMAs of k-step kk, so D steps of reads are in
    // flight behind the matrix core (the same registers as D reads per
    // round trip)
    constexpr int D = kMlaQkg;
    v8s k0[KK], k1[KK];
#pragma unroll
    for (int kk = 0; kk < D; ++kk) {
      const char* kp = tb + ((kk & 1) ? (sb0 ^ 64) : sb0) + 1024 * (kk >> 1);
      k0[kk] = *(const v8s*)kp;
      k1[kk] = *(const v8s*)(kp + 18432);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      if (kk + D < KK) {
        const char* kp = tb + (((kk + D) & 1) ? (sb0 ^ 64) : sb0) + 1024 * ((kk + D) >> 1);
        k0[kk + D] = *(const v8s*)kp;
        k1[kk + D] = *(const v8s*)(kp + 18432);
      }
      sc0 = mfma_bf16_16x16x32(k0[kk], qf[kk], sc0);
      sc1 = mfma_bf16_16x16x32(k1[kk], qf[kk], sc1);
      if (kk + D < KK) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads of k-step kk + D
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);                  // MFMAs of k-step kk
      __builtin_amdgcn_sched_barrier(0);
    }
    // keys past the block's last valid entry (last tile only) drop out
    if (j0 + NK > n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (j0 + 4 * g + i >= n) sc0[i] = -INFINITY;
        if (j0 + 16 + 4 * g + i >= n) sc1[i] = -INFINITY;
      }
    }
    // zs > 0, so the max of the scaled scores is the scaled max
    float mx = fmaxf(fmaxf(fmaxf(sc0[0], sc0[1]), fmaxf(sc0[2], sc0[3])),
                     fmaxf(fmaxf(sc1[0], sc1[1]), fmaxf(sc1[2], sc1[3])));
    mx = rows_max(mx) * zs;
    const bool need = mx > m_run + 8.f;
    const float mnew = need ? mx : m_run;
    const float corr = exp2_raw(m_run - mnew);
    m_run = mnew;
    float p[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2_raw(fmaf(sc0[i], zs, -mnew));
      p[4 + i] = exp2_raw(fmaf(sc1[i], zs, -mnew));
    }
    v4i pk;
#pragma unroll
    for (int i = 0; i < 4; ++i) pk[i] = (int)pack_bf16x2(p[2 * i], p[2 * i + 1]);
    l_part = fmaf(l_part, corr, ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7])));
    const int par = jl & 1;
    *(v4i*)(pbuf + ((par * 8 + w) * 64 + lane) * 16) = pk;
    if (g == 0) s_corr[par][16 * w + c] = corr;
    const bool any = __any(need);
    if (lane == 0) s_need[par][w] = any ? 1 : 0;
    __builtin_amdgcn_s_setprio(0);
  };
  // O^T += V^T . P^T of tile jl for all heads over the wave's value
  // columns, after the rescale of the heads whose max moved in that tile
  auto pv = [&](int jl) {
    const int par = jl & 1;
    const char* tb = smem + (jl % 3) * kMlaTile;
    bool resc = false;
#pragma unroll
    for (int i = 0; i < NW; ++i) resc |= s_need[par][i] != 0;
    if (resc) {
#pragma unroll
      for (int hb = 0; hb < 4; ++hb) {
        const float cr = s_corr[par][32 * hb + (lane & 31)];
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) o[vb][hb] *= cr;
      }
    }
    v8s av[4];  // [2 m + vb]
    {
      const uint32_t tba = (uint32_t)(uintptr_t)(const lds_char*)tb;
      const uint32_t va[4] = {tba + (uint32_t)vqn, tba + (uint32_t)(vqn ^ 64), tba + (uint32_t)((vqn ^ 64) + 9216),
                              tba + (uint32_t)(vqn + 9216)};
      lds_read_vt4_at<18432>(va, av);
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const char* pb = pbuf + (par * 8 + 2 * hb) * 1024 + pq;
      const v8s pf0 = *(const v8s*)pb;
      const v8s pf1 = *(const v8s*)(pb + 512);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) o[vb][hb] = mfma_bf16_32x32x16(av[vb], pf0, o[vb][hb]);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb) o[vb][hb] = mfma_bf16_32x32x16(av[2 + vb], pf1, o[vb][hb]);
      if (hb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
    }
  };

  // slot 2j: group 0 S^T + softmax of tile j, group 1 PV of tile j-1 (and
  // the gather of tile j+1); slot 2j+1: group 1 S^T + softmax of tile j,
  // group 0 PV of tile j-1.  Both groups pass the same 2 ntiles + 2 barriers.
  // The block that most likely runs next on this CU, query t + a.ahead
  // (a.ahead = the chip's CU count: blocks are dealt round-robin, so it is on
  // the same XCD), finds its index row in the cache: one 4-byte
  // direct-to-LDS copy per 128-byte line of the row into a dummy slot.  One
  // wave of group 0 issues them; its loop has no other global loads, so
  // nothing waits for them.  Its index row is the head of that block's
  // dependent chain (index row, first gather, first S^T).
  auto prefetch_next_index_row = [&]() {
    const int64_t tn = t + a.ahead;
    if (a.ahead <= 0 || tn >= a.T || w != 0) return;
    lds_char* dummy = (lds_char*)(smem + kMlaFixedLds) + a.k * 4;
    const int lines = (int)((a.k + 31) / 32);   // 32 entries per line; each copy reads the line's first entry
    for (int l0 = 0; l0 < lines; l0 += 64) {
      const int ln = min(l0 + lane, lines - 1);
      __builtin_amdgcn_global_load_lds((const void*)(a.idx + tn * a.k + 32 * ln),
                                       (__attribute__((address_space(3))) void*)dummy, 4, 0, 0);
    }
  };
  if (G == 0) {
    __syncthreads();
    for (int jj = 0; jj <= ntiles; ++jj) {
      if (jj == 2) prefetch_next_index_row();
      if (jj < ntiles) qk_softmax(jj);
      lds_barrier();
      if (jj >= 1) pv(jj - 1);
      lds_barrier();
    }
  } else {
    if (ntiles > 0) issue_tile(0);
    __syncthreads();  // waits for the first tile
    for (int jj = 0; jj <= ntiles; ++jj) {
      if (jj + 1 < ntiles) issue_tile(jj + 1);
      if (jj >= 1) pv(jj - 1);
      lds_barrier();
      if (jj < ntiles) qk_softmax(jj);
      if (jj + 1 < ntiles) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile jj+1 has landed
      lds_barrier();
    }
  }

  // epilogue: row sums of every head, then lane (c, g) of wave w writes
  // O^T[dv = 64w + 16d + 4g + i][head 16hs + c]
  const bool partial = a.splits > 1;
  {
    const float l = rows_sum(l_part);
    if (g == 0) {
      const int h = 16 * w + c;
      s_l[h] = l;
      if (partial) {
        float* ml = a.part_ml + ((t * a.splits + sp) * H + h) * 2;
        ml[0] = m_run;
        ml[1] = l;
      } else if (a.lse) {
        a.lse[t * H + h] = n > kbeg ? (m_run + log2f(l)) * kLn2 : -INFINITY;
      }
    }
  }
  __syncthreads();
  if (partial) {
    // the unnormalised partial as fp16 over a scale per (head, 64-column
    // slice w): lanes l and l ^ 32 hold the slice's 64 values of head h
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const int h = 32 * hb + (lane & 31);
      float mx = 0.f;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, fabsf(o[vb][hb][r]));
      {
        const uint32_t u = __float_as_uint(mx);
        auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float sc = mx > 0.f ? mx : 1.f, isc = 1.f / sc;
      if (lane < 32) a.part_sc[((t * a.splits + sp) * H + h) * (DV / 64) + w] = sc;
      uint16_t* op = a.part_o + ((t * a.splits + sp) * H + h) * (int64_t)DV + 64 * w + 4 * (lane >> 5);
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          const v2i pk = {(int)pack_f16x2(o[vb][hb][4 * rq] * isc, o[vb][hb][4 * rq + 1] * isc),
                          (int)pack_f16x2(o[vb][hb][4 * rq + 2] * isc, o[vb][hb][4 * rq + 3] * isc)};
          *(v2i*)(op + 32 * vb + 8 * rq) = pk;
        }
    }
    return;
  }
  // normalised bf16 rows staged in the (now idle) tile buffers, 64 heads at
  // a time with a padded row stride, then written as whole 1 KB head rows
  constexpr int kRow = DV * 2 + 16;
  uint16_t* ob = (uint16_t*)a.out + t * H * (int64_t)DV;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const int hb = 2 * half + hh;
      const float l = s_l[32 * hb + (lane & 31)];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      char* sp_row = smem + (32 * hh + (lane & 31)) * kRow + (64 * w + 4 * (lane >> 5)) * 2;
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int rq = 0; rq < 4; ++rq) {
          v2i pk;
          pk[0] = (int)pack_bf16x2(o[vb][hb][4 * rq] * inv, o[vb][hb][4 * rq + 1] * inv);
          pk[1] = (int)pack_bf16x2(o[vb][hb][4 * rq + 2] * inv, o[vb][hb][4 * rq + 3] * inv);
          *(v2i*)(sp_row + 2 * (32 * vb + 8 * rq)) = pk;
        }
    }
    lds_barrier();
    // 64 rows x 64 lanes of 16 bytes: wave w writes rows w, w + 8, ...
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int r = 8 * rr + w;
      const v4i v = *(const v4i*)(smem + r * kRow + 16 * lane);
      *(v4i*)(ob + (64 * half + r) * (int64_t)DV + 8 * lane) = v;
    }
    lds_barrier();
  }
}

// merge the key splits of each (query, head): weights 2^(m_s - M) with M the
// largest split max; out = sum_s w_s O_s / sum_s w_s l_s (bf16), lse in ln,
// where O_s is the fp16 partial times its 64-column slice scale.  Dv/4
// threads per (query, head), four value columns each.
// NS >= splits slots (2, 4 or 8: the launcher rounds up).
constexpr int kMaxSplits = 8;
template <int NS>
__global__ __launch_bounds__(256) void attn_combine_kernel(AttnArgs a) {
  const int tph = (int)(a.Dv / 4);
  const int per_blk = 256 / tph;
  const int64_t th = (int64_t)blockIdx.x * per_blk + threadIdx.x / tph;
  if ((int)threadIdx.x >= per_blk * tph || th >= a.T * a.H) return;
  const int d = 4 * (threadIdx.x % tph);
  const int64_t t = th / a.H, h = th % a.H;
  const int S = a.splits;
  // every split block writes its (max, sum) and its partial (zeros and
  // (-inf, 0) when it had no keys), so all loads go out at once, with no
  // branch around them (slots past S re-read split S - 1 and are not used)
  const int nsl = (int)(a.Dv / 64);
  float2 ml[NS];
  float sc[NS];
  v2i po[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const int ss = s < S ? s : S - 1;
    const int64_t th_s = (t * S + ss) * a.H + h;
    ml[s] = *(const float2*)(a.part_ml + th_s * 2);
    sc[s] = a.part_sc[th_s * nsl + (d >> 6)];
    po[s] = *(const v2i*)(a.part_o + th_s * a.Dv + d);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s)
    if (s < S) M = fmaxf(M, ml[s].x);
  float L = 0.f;
  v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    // weight 0 for unused slots and empty splits (their partials are finite)
    const bool use = s < S && ml[s].y > 0.f;
    const float wgt = use ? exp2f(ml[s].x - M) : 0.f;
    L += use ? ml[s].y * wgt : 0.f;
    acc += (wgt * sc[s]) * unpack_f16x4(po[s]);
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  v2i pk;
  pk[0] = (int)pack_bf16x2(acc[0] * inv, acc[1] * inv);
  pk[1] = (int)pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *(v2i*)((uint16_t*)a.out + (t * a.H + h) * a.Dv + d) = pk;
  if (a.lse && d == 0) a.lse[t * a.H + h] = L > 0.f ? (M + log2f(L)) * kLn2 : -INFINITY;
}

static void launch_combine_kernel(const AttnArgs& a, int64_t per_blk, hipStream_t st) {
  const unsigned grid = (unsigned)((a.T * a.H + per_blk - 1) / per_blk);
  if (a.splits <= 2)
    attn_combine_kernel<2><<<grid, 256, 0, st>>>(a);
  else if (a.splits <= 4)
    attn_combine_kernel<4><<<grid, 256, 0, st>>>(a);
  else
    attn_combine_kernel<kMaxSplits><<<grid, 256, 0, st>>>(a);
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

// dynamic LDS a block may take (160 KB per CU, less the kernel's static LDS)
constexpr size_t kAttnLdsLimit = 160 * 1024 - 2048;

bool attn_supported(bool f32, int64_t H, int64_t Dk, int64_t Dv, bool sep_v, int64_t k) {
  if (f32) return H >= 1 && H <= 64 && Dk >= 4 && Dk <= 128 && Dv >= 4 && Dv <= 128 && Dk % 4 == 0 && Dv % 4 == 0;
  if (H == 16 && Dk == 128 && Dv == 128) return true;
  if (H == 128 && Dk == 576 && Dv == 512) {
    // shared latent row: three gathered tiles + two P^T sets + the index
    // row; separate V: two tiles of key and value rows + P^T + index ring
    if (!sep_v) return kMlaFixedLds + (size_t)k * 4 <= kAttnLdsLimit;
    const size_t tile = (size_t)32 * (Dk / 8 + Dv / 8) * 16;
    return 2 * tile + 8 * 1024 + 3 * 32 * 4 <= kAttnLdsLimit;
  }
  return false;
}

// key splits per query: about one block per CU when there are few queries
// (batched decode; a block fills a CU's LDS); each split keeps at least 8
// tiles of keys
static int attn_splits(bool f32, int64_t T, int64_t k) {
  if (f32 || T <= 0 || T >= 256) return 1;
  int s = (int)((256 + T - 1) / T);
  const int maxs = (int)(k / 256);
  if (s > maxs) s = maxs;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 1 ? 1 : s;
}

size_t attn_workspace_bytes(bool f32, int64_t T, int64_t H, int64_t Dv, int64_t k) {
  const int s = attn_splits(f32, T, k);
  if (s <= 1) return 0;
  const size_t o = (size_t)T * s * H * Dv * 2, ml = (size_t)T * s * H * 2 * 4, sc = (size_t)T * s * H * (Dv / 64) * 4;
  return (o + 255) / 256 * 256 + (ml + 255) / 256 * 256 + sc;
}

template <int DK, int DV, int NW, bool SEPV>
static hipError_t launch_bf16(const AttnArgs& a, const int64_t* seq_off, hipStream_t st) {
  constexpr size_t tile = (size_t)32 * (DK / 8 + (SEPV ? DV / 8 : 0)) * 16;
  constexpr size_t lds = 2 * tile + (size_t)NW * 1024 + 3 * 32 * 4;
  static_assert(lds <= kAttnLdsLimit, "two tiles, the P^T fragments and the index ring fit in LDS");
  static std::atomic<uint64_t> attr_done{0};
  hipError_t ea = set_lds_limit_once((const void*)attn_bf16_kernel<DK, DV, NW, SEPV>, (int)lds, attr_done);
  if (ea != hipSuccess) return ea;
  attn_bf16_kernel<DK, DV, NW, SEPV><<<(unsigned)(a.T * a.splits), NW * 64, lds, st>>>(a, seq_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  const int64_t per_blk = 256 / (a.Dv / 4);
  launch_combine_kernel(a, per_blk, st);
  return hipGetLastError();
}

template <bool SEPV>
static hipError_t launch_h16(const AttnArgs& a, const int64_t* seq_off, hipStream_t st) {
  constexpr size_t lds = 2 * (size_t)(SEPV ? 8192 : 4096) + 3 * 16 * 4;
  attn_h16_kernel<SEPV><<<(unsigned)(a.T * a.splits), 64, lds, st>>>(a, seq_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  const int64_t per_blk = 256 / (a.Dv / 4);
  launch_combine_kernel(a, per_blk, st);
  return hipGetLastError();
}

static hipError_t launch_combine(const AttnArgs& a, hipStream_t st) {
  const int64_t per_blk = 256 / (a.Dv / 4);
  launch_combine_kernel(a, per_blk, st);
  return hipGetLastError();
}

static hipError_t launch_mla(const AttnArgs& a, const int64_t* seq_off, hipStream_t st) {
  // + 256 bytes: the dummy slot of the index-row prefetch
  constexpr size_t lds_max = kMlaFixedLds + (size_t)DSA_MAX_TOPK * 4 + 256;
  static_assert(lds_max <= kAttnLdsLimit, "three tiles, P^T, the index row and the dummy slot fit in LDS");
  const size_t lds = kMlaFixedLds + (size_t)a.k * 4 + 256;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t ea = set_lds_limit_once((const void*)attn_mla_kernel, (int)lds_max, attr_done);
  if (ea != hipSuccess) return ea;
  attn_mla_kernel<<<(unsigned)(a.T * a.splits), 512, lds, st>>>(a, seq_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits <= 1) return e;
  return launch_combine(a, st);
}

hipError_t launch_attn(const AttnArgs& a_in, bool f32, void* ws, size_t ws_bytes, hipStream_t st) {
  if (a_in.T <= 0) return hipSuccess;
  AttnArgs a = a_in;
  a.splits = attn_splits(f32, a.T, a.k);
  // queries ahead whose index row a block prefetches (one block per query
  // and CU): the device's CU count
  a.ahead = 0;
  if (a.splits == 1) {
    int dev = 0, ncu = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && ncu > 0)
      a.ahead = ncu;
  }
  if (a.splits > 1) {
    if (!ws || ws_bytes < attn_workspace_bytes(f32, a.T, a.H, a.Dv, a.k)) return hipErrorInvalidValue;
    const size_t rows = (size_t)a.T * a.splits * a.H;
    a.part_o = (uint16_t*)ws;
    a.part_ml = (float*)((char*)ws + (rows * a.Dv * 2 + 255) / 256 * 256);
    a.part_sc = (float*)((char*)a.part_ml + (rows * 2 * 4 + 255) / 256 * 256);
    DSA_DEBUG_CHECK((char*)(a.part_sc + rows * (a.Dv / 64)) <= (char*)ws + ws_bytes);
  }
  if (f32) {
    a.splits = 1;
    attn_f32_kernel<<<(unsigned)a.T, 256, 0, st>>>(a, a.seq_offsets);
    return hipGetLastError();
  }
  if (a.H == 16 && a.Dk == 128 && a.Dv == 128) {
    if (a.v) return launch_h16<true>(a, a.seq_offsets, st);
    return launch_h16<false>(a, a.seq_offsets, st);
  }
  if (a.H == 128 && a.Dk == 576 && a.Dv == 512) {
    if (a.v) return launch_bf16<576, 512, 8, true>(a, a.seq_offsets, st);
    return launch_mla(a, a.seq_offsets, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
