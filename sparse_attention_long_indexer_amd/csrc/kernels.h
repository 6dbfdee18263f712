// Launchers of the DSA kernels (internal to the library; the public
// interface is include/dsa.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// Debug builds (-DDSA_DEBUG) check the launch plans on the host: each
// workspace carve-up ends inside the size its *_workspace_bytes() query
// reports, and the plan's derived sizes are in range.  A failed check prints
// the condition and aborts before anything is launched.
#ifdef DSA_DEBUG
#include <cstdio>
#include <cstdlib>
#define DSA_DEBUG_CHECK(cond)                                                                   \
  do {                                                                                          \
    if (!(cond)) {                                                                              \
      std::fprintf(stderr, "DSA_DEBUG check failed: %s (%s:%d)\n", #cond, __FILE__, __LINE__); \
      std::abort();                                                                             \
    }                                                                                           \
  } while (0)
#else
#define DSA_DEBUG_CHECK(cond) ((void)0)
#endif

namespace dsa {

// fold.hip
hipError_t launch_fold(const void* q_in, const float* q_scale, bool fp8_in, const void* w,
                       bool w_bf16, int64_t T, void* q_out, float* s_out, hipStream_t st);

// index_scores.hip: materialised scores for rows [row_begin, row_end); row
// t sits at position q_pos[t], or pos_base + t without q_pos
hipError_t launch_index_scores(const void* qf, const float* qs, const void* k, const float* ks,
                               bool fp8, int64_t T, int64_t S, const int64_t* q_pos, int64_t pos_base,
                               int64_t row_begin, int64_t row_end, float* out, int64_t ld,
                               hipStream_t st);
// decode: scores of query b over its own cache rows, written at key offsets
// (total_keys = offsets[B], the concatenated caches' length)
hipError_t launch_index_scores_decode(const uint8_t* qf, const float* qs, const uint8_t* k,
                                      const float* ks, const int64_t* offsets, int64_t B,
                                      int64_t total_keys, float* out, hipStream_t st);

// Dynamic k (every selection path): a row keeps
// min(n, k, max(k_min, #{scores > theta})) keys; theta = -inf keeps the
// fixed min(n, k).
struct DynK {
  float theta;
  int64_t k_min;
};
__host__ __device__ inline bool dyn_on(const DynK& d) { return d.theta > -__builtin_huge_valf(); }
constexpr DynK kFixedK = {-__builtin_huge_valf(), 0};

// topk.hip: rows are described by (row_off, n) pairs computed on device
struct TopkRows {
  const float* scores;
  int64_t ld;                 // row stride when row_off == nullptr
  const int64_t* row_off;     // optional per-row start offset into scores
  const int64_t* q_pos;       // optional per-row position (n = min(S, pos+1))
  int64_t S;                  // keys available (prefill) when seq_len == nullptr
  const int64_t* seq_offsets; // decode: n_b = off[b+1]-off[b], start = off[b]
  int64_t row_begin;          // first row (for q_pos lookup / output row)
  int64_t pos_base;           // without q_pos, row t sits at position pos_base + t
};
size_t topk_workspace_bytes(int64_t rows, int64_t max_n, int64_t k);
hipError_t launch_topk(const TopkRows& r, int64_t rows, int64_t max_n, int64_t k, int32_t* idx_out,
                       int32_t* count_out, void* ws, hipStream_t st, DynK dyn = kFixedK);

// index_select.hip: fused scores + top-k for a causal prefill chunk: query t
// sits at position p0 + t and sees keys [0, p0 + t]; S = p0 + T keys
bool index_select_supported(int64_t T, int64_t S);
size_t index_select_workspace_bytes(int64_t T, int64_t S);
hipError_t launch_index_select(const uint8_t* qf, const float* qs, const uint8_t* k8, const float* ks,
                               int64_t T, int64_t S, int64_t topk, int32_t* idx_out, void* ws,
                               bool force_fallback, hipStream_t st, DynK dyn = kFixedK);

// attn_bwd.hip: backward of the bf16 sparse attention with a shared latent
// KV row per key (H = 128, Dk = 576, Dv = 512)
struct BwdArgs {
  const void* q;        // [T][H][Dk] bf16
  const void* kv;       // [S][ld_kv] bf16
  int64_t ld_kv;
  const int32_t* idx;   // [T][k]
  int64_t S, T, k;
  float scale;
  const void* out;      // [T][H][Dv] bf16, the forward's output
  const float* lse;     // [T][H], the forward's log-sum-exp (natural log)
  const void* dout;     // [T][H][Dv] bf16
  void* dq;             // [T][H][Dk] bf16 (written)
  float* dkv;           // [S][ld_dkv] fp32 (accumulated)
  int64_t ld_dkv;
};
bool attn_bwd_supported(int64_t H, int64_t Dk, int64_t Dv, int64_t k);
int64_t attn_bwd_chunk(int64_t T, int64_t k);
size_t attn_bwd_workspace_bytes(int64_t T, int64_t k);
hipError_t launch_attn_bwd(const BwdArgs& a, void* ws, hipStream_t st);

// indexer_kl.hip: KL alignment of the indexer to the dense attention
struct KlArgs {
  const float* q_idx;   // [L][128] fp32
  const float* k_idx;   // [L][128] fp32
  const float* w;       // [128][128] fp32
  const void* q;        // [L][128][576] bf16
  const void* kv;       // [L][ld_kv] bf16
  int64_t ld_kv, L;
  float scale;
  float* loss;          // [L]
  float* dq_idx;        // [L][128]
  float* dk_idx;        // [L][128]
  float* dw;            // [128][128]
};
bool indexer_kl_supported(int64_t H, int64_t Dk, int64_t L);
size_t indexer_kl_workspace_bytes(int64_t L);
hipError_t launch_indexer_kl(const KlArgs& a, void* ws, hipStream_t st);

// attn.hip
struct AttnArgs {
  const void* q;        // [T][H][Dk]
  const void* kv;       // [*][ld_kv]
  const void* v;        // [*][ld_v] or nullptr
  int64_t ld_kv, ld_v;
  const int32_t* idx;   // [T][k]
  const int64_t* seq_offsets;  // decode: query t reads cache rows [off[t], off[t+1])
  int64_t S;            // rows of kv/v (prefill)
  int64_t T, H, Dk, Dv, k;
  float scale;
  void* out;            // [T][H][Dv]
  float* lse;           // [T][H] or nullptr
  int splits;           // key splits per query (set by launch_attn)
  uint16_t* part_o;     // [T][splits][H][Dv] fp16: unnormalised partial output / its slice scale
  float* part_ml;       // [T][splits][H][2] running max (log2) and sum
  float* part_sc;       // [T][splits][H][Dv/64] slice scales: max |partial| over 64 value columns
  int64_t ahead;        // MLA kernel: a block prefetches the index row of query t + ahead (0: none)
};
bool attn_supported(bool f32, int64_t H, int64_t Dk, int64_t Dv, bool sep_v, int64_t k);
size_t attn_workspace_bytes(bool f32, int64_t T, int64_t H, int64_t Dv, int64_t k);
hipError_t launch_attn(const AttnArgs& a, bool f32, void* ws, size_t ws_bytes, hipStream_t st);

}  // namespace dsa
