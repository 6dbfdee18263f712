/*
 * dsa.h - C ABI of the DeepSeek Sparse Attention (DSA) forward hot path on
 * AMD MI355X (gfx950).
 *
 * The method (DeepSeek-V3.2 write-up on intelliparadigm.com, "DeepSeek
 * Sparse Attention"): a lightning indexer scores each query token against
 * every earlier token as I[t,s] = ReLU(q_t . W_index . k_s) on 128-dim index
 * vectors kept in FP8 (section 2.2); a fine-grained selection keeps the
 * k = 2048 best-scoring keys per query (section 2.3); softmax attention then
 * runs over the selected keys only, all query heads sharing one key/value
 * head as in MLA's MQA mode (sections 2.3 and 3.1).
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are device memory owned by the caller; the
 *     library keeps no pointer after a call returns and never allocates.
 *     Scratch memory is passed in as a workspace (device pointer + byte
 *     count, 256-byte aligned); each op documents the size it needs.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  The caller keeps buffers alive until the stream has
 *     run the work.  The library never synchronises.
 *   - Arguments are validated on the host before any launch; on an error
 *     status nothing is launched and nothing is written.  A launch failure
 *     maps to DSA_ERR_DEVICE.  Kernel faults surface at the caller's next
 *     synchronisation.  No C++ exception crosses this interface.
 *   - Layouts are row-major with a contiguous last dimension.  Counts and
 *     offsets are int64; key indices are int32.
 *   - FP8 means OCP E4M3 ("e4m3fn": bias 7, max 448, NaN = S.1111.111) with
 *     one fp32 scale per row: value = e4m3(code) * scale[row].
 *   - Devices and threads: a call runs on the caller's current HIP device.
 *     The library's global state is per device and set once: whether the
 *     device is gfx950 (checked on the first call), which kernels already
 *     have their LDS limit raised, and the address of the device's copy of
 *     the static scratch of dsa_forward_static.  Each record is updated
 *     atomically, so calls from several threads, on several streams or
 *     devices, may run concurrently (dsa_forward_static excepted: see there).
 */
#ifndef DSA_H_
#define DSA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DSA_ABI_VERSION 6
#define DSA_INDEX_DIM 128   /* index-key width, write-up section 2.2 */
#define DSA_MAX_TOPK 4096

typedef enum {
  DSA_OK = 0,
  DSA_ERR_NULL = 1,        /* a required pointer is NULL */
  DSA_ERR_SHAPE = 2,       /* a size or leading dimension is out of range */
  DSA_ERR_DTYPE = 3,       /* a dtype code is not valid for that argument */
  DSA_ERR_UNSUPPORTED = 4, /* valid but not implemented (e.g. head shape) */
  DSA_ERR_WORKSPACE = 5,   /* workspace missing, misaligned or too small */
  DSA_ERR_DEVICE = 6       /* HIP error: no gfx950 device, launch failure */
} dsa_status_t;

typedef enum {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2
} dsa_dtype_t;

typedef enum {
  DSA_MODE_PREFILL = 0,
  DSA_MODE_DECODE = 1
} dsa_mode_t;

/* dsa_forward flags (the result is the same on every path) */
#define DSA_FLAG_MATERIALIZE 1u   /* materialise the scores and run dsa_topk's
                                     select even where the fused path runs */
#define DSA_FLAG_FUSED 2u         /* fused scores + select even for short
                                     prefills (FP8 index only) */
#define DSA_FLAG_FORCE_FALLBACK 4u /* fused path: settle every long row with
                                     the exact recompute fallback (testing) */
#define DSA_FLAG_DYNAMIC_K 8u     /* per-query budget from dyn_theta and
                                     dyn_k_min, as dsa_topk_dynamic */

int dsa_abi_version(void);
const char* dsa_status_str(dsa_status_t s);

/*
 * Fold W_index into the index query and re-quantise it (write-up section
 * 2.2: the score is q_t . W_index . k_s, computed in FP8).
 *
 *   qf[t, j] = sum_i dq(q)[t, i] * W[i, j]          (fp64 accumulation)
 *   FP8:  scale[t] = fp32_rne(max_j |qf[t, j]| / 448), or 1 if that max is 0;
 *         qf8[t, j] = e4m3_rne_saturate(qf[t, j] / scale[t])  (fp64 quotient,
 *         a zero encodes as +0)
 *   F32:  qf_out[t, j] = fp32_rne(qf[t, j]); no scale is written.
 *
 * q_idx     device [T][128]: e4m3 codes (q_dtype = DSA_FP8_E4M3) or fp32
 *           (DSA_F32)
 * q_scale   device fp32 [T] for FP8, ignored (may be NULL) for F32
 * w         device [128][128]: bf16 (w_dtype = DSA_BF16) or fp32 (DSA_F32);
 *           FP8 queries require bf16 or fp32 W, F32 queries require fp32 W
 * qf_out    device [T][128]: e4m3 codes (FP8) or fp32 (F32)
 * qf_scale_out  device fp32 [T] (FP8 only)
 * T >= 0 (T = 0 is a no-op).
 */
dsa_status_t dsa_fold_index_query(const void* q_idx, const float* q_scale, dsa_dtype_t q_dtype,
                                  const void* w, dsa_dtype_t w_dtype, int64_t T, void* qf_out,
                                  float* qf_scale_out, void* stream);

/*
 * Lightning-indexer scores, materialised (write-up section 2.2).
 *
 *   u[t, s] = qs[t] * ks[s] * sum_j e4m3(qf8[t, j]) * e4m3(k8[s, j])   (FP8)
 *   u[t, s] = sum_j qf[t, j] * k[s, j]                                  (F32)
 *   scores[t - row_begin][s] = u > 0 ? u : +0.0   for s <= pos(t)
 *                            = -inf              for s >  pos(t)
 * with fp32 accumulation; pos(t) = q_pos[t] if q_pos != NULL, else t.
 *
 * qf, qf_scale  device: the folded index query from dsa_fold_index_query
 * k_idx, k_scale device [S][128] codes + fp32 [S] (FP8) or fp32 [S][128]
 *               with k_scale ignored (F32)
 * q_pos     device int64 [T] or NULL
 * rows      [row_begin, row_end) within [0, T]; the output holds
 *           row_end - row_begin rows of `ld` floats (ld >= S)
 */
dsa_status_t dsa_index_scores(const void* qf, const float* qf_scale, const void* k_idx,
                              const float* k_scale, dsa_dtype_t idx_dtype, int64_t T, int64_t S,
                              const int64_t* q_pos, int64_t row_begin, int64_t row_end,
                              float* scores_out, int64_t ld, void* stream);

/*
 * Top-k selection per row (write-up section 2.3).
 *
 * Row t considers keys s in [0, n_t) with n_t = min(S, pos(t) + 1) and keeps
 * m_t = min(k, n_t) of them: the largest scores, ties to the lower index
 * (-0.0 counts as +0.0; NaN is not allowed).  The kept indices are written
 * in ascending order to idx_out[t][0 .. m_t) and idx_out[t][m_t .. k) = -1.
 *
 * scores    device fp32 [T][ld]
 * q_pos     device int64 [T] or NULL (pos(t) = t)
 * idx_out   device int32 [T][k]
 * count_out device int32 [T] (m_t) or NULL
 * 1 <= k <= DSA_MAX_TOPK.  Workspace: dsa_topk_workspace_size() bytes.
 */
size_t dsa_topk_workspace_size(int64_t T, int64_t S, int64_t k);
dsa_status_t dsa_topk(const float* scores, int64_t ld, int64_t T, int64_t S, const int64_t* q_pos,
                      int64_t k, int32_t* idx_out, int32_t* count_out, void* ws, size_t ws_bytes,
                      void* stream);

/*
 * Top-k with a per-row budget (the write-up's outlook, section 6: a k that
 * adapts per query instead of a fixed top-k).  Row t keeps
 *   m_t = min(n_t, k_max, max(k_min, #{s < n_t : scores[t][s] > theta}))
 * keys, the m_t best under dsa_topk's order, written as dsa_topk writes them
 * (ascending, idx_out[t][m_t .. k_max) = -1); count_out[t] = m_t.
 * theta = -inf is dsa_topk with k = k_max.  0 <= k_min <= k_max <=
 * DSA_MAX_TOPK and theta not NaN, else DSA_ERR_SHAPE.  m_t may be 0 (k_min
 * = 0 and no score above theta): the row is all -1.
 * Workspace: dsa_topk_workspace_size(T, S, k_max) bytes.
 */
dsa_status_t dsa_topk_dynamic(const float* scores, int64_t ld, int64_t T, int64_t S, const int64_t* q_pos,
                              int64_t k_max, int64_t k_min, float theta, int32_t* idx_out,
                              int32_t* count_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Sparse MQA attention over the selected rows (write-up sections 2.3, 3.1).
 * For each query t and head h, over the valid entries s of idx[t] (entries
 * after the first -1 are ignored):
 *   z_s = scale * <Q[t, h, :], K[s, :Dk]>;   p = softmax(z);
 *   out[t, h, :] = sum_s p_s V[s, :Dv]
 * K[s] = kv[s * ld_kv + 0 .. Dk);  V[s] = v[s * ld_v + 0 .. Dv) when v != NULL,
 * else the first Dv entries of the same latent row, kv[s * ld_kv + 0 .. Dv).
 * A query with no valid entry gets out = 0 and lse = -inf.
 *
 * q         device [T][H][Dk] (dtype)
 * kv, v     device [S][ld] (dtype)
 * idx       device int32 [T][k], each valid entry in [0, S)
 * out       device [T][H][Dv] (dtype)
 * lse_out   device fp32 [T][H] (natural log of sum_s exp(z_s)) or NULL
 * Supported (dtype, H, Dk, Dv): (F32, any H <= 64, Dk, Dv <= 128 and
 * multiples of 4), (BF16, 16, 128, 128), (BF16, 128, 576, 512), with or
 * without a separate V pointer.  BF16 also needs S * max(ld_kv, ld_v) * 2 <= 4 GiB (rows are addressed by
 * 32-bit byte offsets); otherwise DSA_ERR_UNSUPPORTED.
 */
size_t dsa_sparse_attn_workspace_size(int64_t T, int64_t H, int64_t Dv, int64_t k, dsa_dtype_t dtype);
dsa_status_t dsa_sparse_attn(const void* q, int64_t T, int64_t H, int64_t Dk, dsa_dtype_t dtype,
                             const void* kv, int64_t ld_kv, const void* v, int64_t ld_v, int64_t Dv,
                             int64_t S, const int32_t* idx, int64_t k, float scale, void* out,
                             float* lse_out, void* ws, size_t ws_bytes, void* stream);

/*
 * Backward of dsa_sparse_attn for the sparse training stage (write-up
 * section 4.1: after the dense warm-up the whole model trains through
 * attention over the selected keys).  Shared latent KV only (v = NULL in the
 * forward: K = kv[s, :Dk], V = kv[s, :Dv]).  With P the forward's softmax
 * weights (from lse_in) and dO = d_out:
 *   dS[t,h,j] = scale P[t,h,j] (dO[t,h] . V_j - dO[t,h] . out[t,h])
 *   dq[t,h]  = sum_j dS[t,h,j] K_j                       (written)
 *   dkv[s]  += sum over (t, h, j) with idx[t][j] = s of
 *              dS[t,h,j] q[t,h]  (all Dk columns)
 *            + P[t,h,j] dO[t,h]  (the first Dv columns)  (accumulated)
 * The caller zeroes dkv before the first call; dkv may then collect the
 * gradients of several calls.  Accumulation order across queries is not
 * fixed (hardware float atomics), so dkv is reproducible to rounding only.
 *
 * q, out, d_out, dq  device bf16 [T][H][Dk], [T][H][Dv], [T][H][Dv], [T][H][Dk]
 * kv        device bf16 [S][ld_kv]; idx device int32 [T][k] as for the forward
 * lse_in    device fp32 [T][H]: the forward's lse_out
 * dkv       device fp32 [S][ld_dkv], ld_dkv >= Dk
 * Supported: dtype = DSA_BF16, H = 128, Dk = 576, Dv = 512, k a multiple of
 * 32 up to DSA_MAX_TOPK; otherwise DSA_ERR_UNSUPPORTED.
 * Workspace: dsa_sparse_attn_bwd_workspace_size(T, H, k) bytes (P and dS of
 * a chunk of queries in bf16; the call walks the queries in chunks).
 */
size_t dsa_sparse_attn_bwd_workspace_size(int64_t T, int64_t H, int64_t k);
dsa_status_t dsa_sparse_attn_bwd(const void* q, int64_t T, int64_t H, int64_t Dk, dsa_dtype_t dtype,
                                 const void* kv, int64_t ld_kv, int64_t Dv, int64_t S, const int32_t* idx,
                                 int64_t k, float scale, const void* out, const float* lse_in,
                                 const void* d_out, void* dq, float* dkv, int64_t ld_dkv, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * KL alignment of the lightning indexer to the dense attention (write-up
 * section 4.1, dense warm-up: the indexer alone learns to imitate the
 * frozen model's attention distribution through a KL loss).  Causal prefill
 * of L tokens; for query t over keys s <= t:
 *   p_t[s]  = (1/H) sum_h softmax_s(scale q[t,h] . kv[s, :Dk])  (target)
 *   I[t,s]  = ReLU((q_idx[t] W) . k_idx[s]),  log q_t = I - logsumexp_s I
 *   loss[t] = sum_s p_t[s] (log p_t[s] - log q_t[s])            (0 log 0 = 0)
 * and with G[t,s] = (q_t[s] - p_t[s]) [I[t,s] > 0], qf = q_idx W:
 *   dq_idx = (G k_idx) W^T,  dk_idx = G^T qf,  dw = q_idx^T (G k_idx).
 * Index vectors and W are real-valued fp32 here (training, no FP8); the
 * attention operands are the model's bf16 tensors.  All outputs are written.
 *
 * q_idx, k_idx  device fp32 [L][128];  w device fp32 [128][128]
 * q             device bf16 [L][H][Dk];  kv device bf16 [L][ld_kv]
 * loss_out      device fp32 [L];  dq_idx, dk_idx device fp32 [L][128];
 * dw            device fp32 [128][128]
 * Supported: dtype = DSA_BF16, H = 128, Dk = 576, 1 <= L <= 65536
 * (otherwise DSA_ERR_UNSUPPORTED).  Workspace:
 * dsa_indexer_kl_workspace_size(L) bytes (it holds the L x L score matrix).
 */
size_t dsa_indexer_kl_workspace_size(int64_t L);
dsa_status_t dsa_indexer_kl(const float* q_idx, const float* k_idx, const float* w, const void* q, int64_t H,
                            int64_t Dk, dsa_dtype_t dtype, const void* kv, int64_t ld_kv, int64_t L, float scale,
                            float* loss_out, float* dq_idx, float* dk_idx, float* dw, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * Whole forward: fold, scores, top-k and sparse attention -- the path of the
 * write-up's sections 2.1-2.3 and 3.1: the lightning indexer scores every
 * causal pair (2.2), the fine-grained selection keeps each query's k best
 * keys (2.3), and attention in MLA's MQA mode runs over those keys (3.1).
 *
 * PREFILL: T query tokens at positions q_offset .. q_offset + T - 1 of one
 *   causal sequence whose first S = q_offset + T tokens are the keys
 *   (q_offset = 0: the whole sequence, queries = keys).  Query t attends
 *   over keys [0, q_offset + t].  q_offset > 0 runs a long prefill in
 *   chunks: each chunk reuses the keys cached by the earlier ones, and the
 *   result equals the rows of the whole-sequence call.
 *   q_idx/q_scale [T][128], k_idx/k_scale [S][128], q [T][H][Dk],
 *   kv [S][ld_kv], v [S][ld_v] or NULL; out [T][H][Dv]; idx_out [T][k].
 *   S <= 2^31 - 1.
 * DECODE: B sequences, one new query each.  Sequence b owns cache rows
 *   [seq_offsets[b], seq_offsets[b+1]) of k_idx/k_scale/kv/v (device int64
 *   [B+1], non-decreasing, seq_offsets[0] = 0, every length >= 1); its
 *   query sits at position n_b - 1 and attends over keys [0, n_b) of its
 *   own cache.  q_offset must be 0.
 *   q_idx/q_scale [B][128], q [B][H][Dk]; out [B][H][Dv];
 *   idx_out [B][k] holds indices local to each sequence's cache.
 *   max_len is an upper bound on every n_b (host value, used to size work;
 *   BF16 attention needs max_len * ld * 2 <= 4 GiB, as for dsa_sparse_attn).
 * With DSA_FLAG_DYNAMIC_K each query keeps m_t keys as dsa_topk_dynamic
 * (k_max = topk) and attends over those; a query with m_t = 0 gets out = 0.
 * idx_out may be NULL (the indices then live only in the workspace).
 * Workspace: dsa_forward_workspace_size(args) bytes.
 */
typedef struct dsa_forward_args {
  int32_t mode;               /* dsa_mode_t */
  uint32_t flags;             /* DSA_FLAG_* */
  int64_t T;                  /* PREFILL: tokens; DECODE: B */
  const int64_t* seq_offsets; /* DECODE: device int64 [B+1] */
  int64_t total_keys;         /* DECODE: seq_offsets[B] (host copy) */
  int64_t max_len;            /* DECODE: max n_b (host) */
  dsa_dtype_t idx_dtype;      /* DSA_FP8_E4M3 or DSA_F32 */
  const void* q_idx;
  const float* q_scale;
  const void* w_index;
  dsa_dtype_t w_dtype;
  const void* k_idx;
  const float* k_scale;
  dsa_dtype_t attn_dtype;     /* DSA_BF16 or DSA_F32 */
  const void* q;
  int64_t H, Dk, Dv;
  const void* kv;
  int64_t ld_kv;
  const void* v;
  int64_t ld_v;
  int64_t topk;
  float scale;
  int64_t q_offset;           /* PREFILL: position of the first query */
  float dyn_theta;            /* DSA_FLAG_DYNAMIC_K: score threshold theta */
  int64_t dyn_k_min;          /* DSA_FLAG_DYNAMIC_K: k_min (k_max = topk) */
} dsa_forward_args;

size_t dsa_forward_workspace_size(const dsa_forward_args* a);
dsa_status_t dsa_forward(const dsa_forward_args* a, int32_t* idx_out, void* out, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * dsa_forward without a workspace argument, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops (a decode
 * step per token), harnesses that forbid allocation.  The call allocates
 * nothing; its scratch memory is a static device array of
 * DSA_STATIC_SCRATCH_BYTES (128 MiB) per device, part of the library's code
 * object, held from the library's first use on that device until the process
 * ends.  Results are those of dsa_forward with the same arguments (the same
 * kernels run).
 *
 * Limit: the call needs what dsa_forward would take as its workspace (the
 * indices count only when idx_out is NULL); above DSA_STATIC_SCRATCH_BYTES
 * it returns DSA_ERR_WORKSPACE and launches nothing.  That covers a decode
 * step of 64 sequences over caches of up to 131072 keys each (about 101 MiB)
 * and short prefills; long prefills need dsa_forward.
 *
 * Every call on a device uses that device's one scratch array: calls whose
 * work overlaps on one device (different streams, or host threads sharing a
 * device) race and corrupt each other's results.  Calls on one stream, one
 * after another, are safe.  Nothing in the scratch carries over between calls.
 */
#define DSA_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
dsa_status_t dsa_forward_static(const dsa_forward_args* a, int32_t* idx_out, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H_ */
