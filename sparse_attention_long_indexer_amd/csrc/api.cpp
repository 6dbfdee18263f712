// C ABI of the DSA forward path: host-side validation, workspace planning and
// kernel launches on the caller's stream.  See include/dsa.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>

#include "dsa.h"
#include "kernels.h"

using namespace dsa;

namespace {

constexpr int kMaxDevices = 64;
// once-initialised per-device check: 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_dev_state[kMaxDevices];

dsa_status_t check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_DEVICE;
  int st = g_dev_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) return DSA_ERR_DEVICE;
    st = (std::strncmp(p.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_dev_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? DSA_OK : DSA_ERR_DEVICE;
}

inline dsa_status_t from_hip(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_DEVICE; }

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

inline hipStream_t as_stream(void* s) { return (hipStream_t)s; }

#define DSA_TRY(expr)                      \
  do {                                     \
    dsa_status_t _s = (expr);              \
    if (_s != DSA_OK) return _s;           \
  } while (0)

// ---- argument checks shared by several entry points ----------------------

dsa_status_t check_fold(const void* q_idx, const float* q_scale, dsa_dtype_t q_dtype, const void* w,
                        dsa_dtype_t w_dtype, int64_t T, const void* qf_out, const float* qf_scale_out) {
  if (T < 0) return DSA_ERR_SHAPE;
  if (q_dtype != DSA_FP8_E4M3 && q_dtype != DSA_F32) return DSA_ERR_DTYPE;
  if (q_dtype == DSA_FP8_E4M3 && w_dtype != DSA_BF16 && w_dtype != DSA_F32) return DSA_ERR_DTYPE;
  if (q_dtype == DSA_F32 && w_dtype != DSA_F32) return DSA_ERR_DTYPE;
  if (T == 0) return DSA_OK;
  if (!q_idx || !w || !qf_out) return DSA_ERR_NULL;
  if (q_dtype == DSA_FP8_E4M3 && (!q_scale || !qf_scale_out)) return DSA_ERR_NULL;
  return DSA_OK;
}

dsa_status_t check_scores(const void* qf, const float* qs, const void* k, const float* ks,
                          dsa_dtype_t dt, int64_t T, int64_t S, int64_t rb, int64_t re,
                          const float* out, int64_t ld) {
  if (dt != DSA_FP8_E4M3 && dt != DSA_F32) return DSA_ERR_DTYPE;
  if (T < 0 || S < 0 || rb < 0 || rb > re || re > T || ld < S) return DSA_ERR_SHAPE;
  if (re == rb || S == 0) return DSA_OK;
  if (!qf || !k || !out) return DSA_ERR_NULL;
  if (dt == DSA_FP8_E4M3) {
    if (!qs || !ks) return DSA_ERR_NULL;
    if (!aligned(qf, 32) || !aligned(k, 32)) return DSA_ERR_SHAPE;
  }
  return DSA_OK;
}

// rows: the most cache rows one query may address (the bf16 kernels gather
// through 32-bit byte offsets from the query's first row)
dsa_status_t check_attn(const void* q, int64_t T, int64_t H, int64_t Dk, dsa_dtype_t dt,
                        const void* kv, int64_t ld_kv, const void* v, int64_t ld_v, int64_t Dv,
                        const int32_t* idx, int64_t k, const void* out, int64_t rows) {
  if (dt != DSA_BF16 && dt != DSA_F32) return DSA_ERR_DTYPE;
  if (T < 0 || H <= 0 || Dk <= 0 || Dv <= 0 || k < 1 || k > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  if (ld_kv < Dk || (v ? ld_v < Dv : ld_kv < Dv)) return DSA_ERR_SHAPE;
  if (!attn_supported(dt == DSA_F32, H, Dk, Dv, v != nullptr, k)) return DSA_ERR_UNSUPPORTED;
  if (T == 0) return DSA_OK;
  if (!q || !kv || !idx || !out) return DSA_ERR_NULL;
  if (dt == DSA_BF16) {
    if (!aligned(q, 16) || !aligned(kv, 16) || (v && !aligned(v, 16)) || !aligned(out, 8))
      return DSA_ERR_SHAPE;
    if (ld_kv % 8 != 0 || (v && ld_v % 8 != 0)) return DSA_ERR_SHAPE;
    const int64_t ld = v && ld_v > ld_kv ? ld_v : ld_kv;
    if (rows > (int64_t(1) << 32) / (ld * 2)) return DSA_ERR_UNSUPPORTED;
  }
  return DSA_OK;
}

// ---- dsa_forward workspace plan -----------------------------------------

struct FwdPlan {
  size_t qf_off, qs_off, idx_off, sc_off, topk_off, topk_bytes, total;
  int64_t chunk_rows;  // prefill: rows of scores materialised at once
  bool fused;          // prefill: fused scores + select
};

constexpr int64_t kFusedMinT = 4096;  // shorter prefills materialise their scores

// keys a prefill chunk sees: the chunk's T queries are the last T of them
int64_t prefill_keys(const dsa_forward_args* a) { return a->q_offset + a->T; }

bool use_fused(const dsa_forward_args* a) {
  return a->mode == DSA_MODE_PREFILL && a->idx_dtype == DSA_FP8_E4M3 &&
         !(a->flags & DSA_FLAG_MATERIALIZE) && index_select_supported(a->T, prefill_keys(a)) &&
         (prefill_keys(a) >= kFusedMinT || (a->flags & DSA_FLAG_FUSED));
}

constexpr size_t kAlign = 256;
constexpr size_t kScoreChunkBytes = size_t(1) << 31;  // cap on one score slab

FwdPlan plan_forward(const dsa_forward_args* a, bool need_idx) {
  FwdPlan p{};
  const int64_t R = a->T;  // rows of queries (prefill T, decode B)
  const size_t qf_elem = a->idx_dtype == DSA_F32 ? 4 : 1;
  size_t off = 0;
  p.qf_off = off;
  off = round_up(off + (size_t)R * 128 * qf_elem, kAlign);
  p.qs_off = off;
  off = round_up(off + (size_t)R * 4, kAlign);
  p.idx_off = off;
  if (need_idx) off = round_up(off + (size_t)R * (size_t)a->topk * 4, kAlign);
  p.sc_off = off;
  p.fused = use_fused(a);
  if (p.fused) {
    p.chunk_rows = R;
    off = round_up(off + index_select_workspace_bytes(a->T, prefill_keys(a)), kAlign);
  } else if (a->mode == DSA_MODE_PREFILL) {
    const int64_t S = prefill_keys(a);
    int64_t rows = S > 0 ? (int64_t)(kScoreChunkBytes / ((size_t)S * 4)) : 1;
    rows = rows / 64 * 64;
    if (rows < 64) rows = 64;
    if (rows > R) rows = R;
    if (rows < 1) rows = 1;
    p.chunk_rows = rows;
    off = round_up(off + (size_t)rows * (size_t)S * 4, kAlign);
  } else {
    p.chunk_rows = R;
    off = round_up(off + (size_t)a->total_keys * 4, kAlign);
    p.topk_off = off;
    p.topk_bytes = topk_workspace_bytes(R, a->max_len, a->topk);
    off = round_up(off + p.topk_bytes, kAlign);
  }
  p.total = off;
  return p;
}

dsa_status_t check_forward(const dsa_forward_args* a) {
  if (!a) return DSA_ERR_NULL;
  if (a->mode != DSA_MODE_PREFILL && a->mode != DSA_MODE_DECODE) return DSA_ERR_UNSUPPORTED;
  if (a->T < 0 || a->topk < 1 || a->topk > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
  if (a->q_offset < 0 || (a->mode == DSA_MODE_DECODE && a->q_offset != 0)) return DSA_ERR_SHAPE;
  if ((a->flags & DSA_FLAG_DYNAMIC_K) &&
      (a->dyn_k_min < 0 || a->dyn_k_min > a->topk || a->dyn_theta != a->dyn_theta))
    return DSA_ERR_SHAPE;
  if (a->mode == DSA_MODE_PREFILL && a->q_offset > (int64_t(1) << 31) - 1 - a->T) return DSA_ERR_SHAPE;
  if (a->mode == DSA_MODE_DECODE) {
    if (a->idx_dtype != DSA_FP8_E4M3) return DSA_ERR_UNSUPPORTED;
    if (a->total_keys < a->T || a->max_len < 1) return DSA_ERR_SHAPE;
    if (a->T > 0 && !a->seq_offsets) return DSA_ERR_NULL;
  }
  const int64_t S = a->mode == DSA_MODE_PREFILL ? prefill_keys(a) : a->total_keys;
  DSA_TRY(check_fold(a->q_idx, a->q_scale, a->idx_dtype, a->w_index, a->w_dtype, a->T, a->q_idx,
                     a->q_scale));
  if (a->T > 0) {
    if (!a->k_idx) return DSA_ERR_NULL;
    if (a->idx_dtype == DSA_FP8_E4M3 && (!a->k_scale || !aligned(a->k_idx, 32))) {
      return a->k_scale ? DSA_ERR_SHAPE : DSA_ERR_NULL;
    }
  }
  DSA_TRY(check_attn(a->q, a->T, a->H, a->Dk, a->attn_dtype, a->kv, a->ld_kv, a->v, a->ld_v, a->Dv,
                     (const int32_t*)a->q /*non-null placeholder*/, a->topk, a->q,
                     a->mode == DSA_MODE_PREFILL ? S : a->max_len));
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_abi_version(void) { return DSA_ABI_VERSION; }

const char* dsa_status_str(dsa_status_t s) {
  switch (s) {
    case DSA_OK: return "ok";
    case DSA_ERR_NULL: return "a required pointer is NULL";
    case DSA_ERR_SHAPE: return "size, leading dimension or alignment out of range";
    case DSA_ERR_DTYPE: return "dtype not valid for this argument";
    case DSA_ERR_UNSUPPORTED: return "configuration not supported";
    case DSA_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case DSA_ERR_DEVICE: return "HIP device error (no gfx950 device or launch failure)";
  }
  return "unknown status";
}

dsa_status_t dsa_fold_index_query(const void* q_idx, const float* q_scale, dsa_dtype_t q_dtype,
                                  const void* w, dsa_dtype_t w_dtype, int64_t T, void* qf_out,
                                  float* qf_scale_out, void* stream) {
  try {
    DSA_TRY(check_fold(q_idx, q_scale, q_dtype, w, w_dtype, T, qf_out, qf_scale_out));
    if (T == 0) return DSA_OK;
    DSA_TRY(check_device());
    return from_hip(launch_fold(q_idx, q_scale, q_dtype == DSA_FP8_E4M3, w, w_dtype == DSA_BF16, T,
                                qf_out, qf_scale_out, as_stream(stream)));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

dsa_status_t dsa_index_scores(const void* qf, const float* qf_scale, const void* k_idx,
                              const float* k_scale, dsa_dtype_t idx_dtype, int64_t T, int64_t S,
                              const int64_t* q_pos, int64_t row_begin, int64_t row_end,
                              float* scores_out, int64_t ld, void* stream) {
  try {
    DSA_TRY(check_scores(qf, qf_scale, k_idx, k_scale, idx_dtype, T, S, row_begin, row_end,
                         scores_out, ld));
    if (row_end == row_begin || S == 0) return DSA_OK;
    DSA_TRY(check_device());
    return from_hip(launch_index_scores(qf, qf_scale, k_idx, k_scale, idx_dtype == DSA_FP8_E4M3, T,
                                        S, q_pos, 0, row_begin, row_end, scores_out, ld,
                                        as_stream(stream)));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

size_t dsa_topk_workspace_size(int64_t T, int64_t S, int64_t k) {
  return topk_workspace_bytes(T, S, k);
}

dsa_status_t dsa_topk_dynamic(const float* scores, int64_t ld, int64_t T, int64_t S, const int64_t* q_pos,
                              int64_t k_max, int64_t k_min, float theta, int32_t* idx_out, int32_t* count_out,
                              void* ws, size_t ws_bytes, void* stream) {
  try {
    if (T < 0 || S < 0 || ld < S || k_max < 1 || k_max > DSA_MAX_TOPK) return DSA_ERR_SHAPE;
    if (k_min < 0 || k_min > k_max || theta != theta) return DSA_ERR_SHAPE;
    if (T == 0) return DSA_OK;
    if (!idx_out || (!scores && S > 0)) return DSA_ERR_NULL;
    const size_t need = topk_workspace_bytes(T, S, k_max);
    if (ws_bytes < need || (need && (!ws || !aligned(ws, kAlign)))) return DSA_ERR_WORKSPACE;
    DSA_TRY(check_device());
    TopkRows r{scores, ld, nullptr, q_pos, S, nullptr, 0, 0};
    return from_hip(launch_topk(r, T, S, k_max, idx_out, count_out, ws, as_stream(stream), DynK{theta, k_min}));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

dsa_status_t dsa_topk(const float* scores, int64_t ld, int64_t T, int64_t S, const int64_t* q_pos,
                      int64_t k, int32_t* idx_out, int32_t* count_out, void* ws, size_t ws_bytes,
                      void* stream) {
  return dsa_topk_dynamic(scores, ld, T, S, q_pos, k, 0, -__builtin_huge_valf(), idx_out, count_out, ws, ws_bytes,
                          stream);
}

size_t dsa_sparse_attn_workspace_size(int64_t T, int64_t H, int64_t Dv, int64_t k,
                                      dsa_dtype_t dtype) {
  return attn_workspace_bytes(dtype == DSA_F32, T, H, Dv, k);
}

dsa_status_t dsa_sparse_attn(const void* q, int64_t T, int64_t H, int64_t Dk, dsa_dtype_t dtype,
                             const void* kv, int64_t ld_kv, const void* v, int64_t ld_v, int64_t Dv,
                             int64_t S, const int32_t* idx, int64_t k, float scale, void* out,
                             float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  try {
    if (S < 1) return DSA_ERR_SHAPE;
    DSA_TRY(check_attn(q, T, H, Dk, dtype, kv, ld_kv, v, ld_v, Dv, idx, k, out, S));
    if (T == 0) return DSA_OK;
    const size_t need = attn_workspace_bytes(dtype == DSA_F32, T, H, Dv, k);
    if (ws_bytes < need || (need && (!ws || !aligned(ws, kAlign)))) return DSA_ERR_WORKSPACE;
    DSA_TRY(check_device());
    AttnArgs a{};
    a.q = q;
    a.kv = kv;
    a.v = v;
    a.ld_kv = ld_kv;
    a.ld_v = ld_v;
    a.idx = idx;
    a.seq_offsets = nullptr;
    a.S = S;
    a.T = T;
    a.H = H;
    a.Dk = Dk;
    a.Dv = Dv;
    a.k = k;
    a.scale = scale;
    a.out = out;
    a.lse = lse_out;
    return from_hip(launch_attn(a, dtype == DSA_F32, ws, ws_bytes, as_stream(stream)));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

size_t dsa_sparse_attn_bwd_workspace_size(int64_t T, int64_t H, int64_t k) {
  if (T < 1 || H != 128 || k < 1) return 0;
  return attn_bwd_workspace_bytes(T, k);
}

dsa_status_t dsa_sparse_attn_bwd(const void* q, int64_t T, int64_t H, int64_t Dk, dsa_dtype_t dtype,
                                 const void* kv, int64_t ld_kv, int64_t Dv, int64_t S, const int32_t* idx,
                                 int64_t k, float scale, const void* out, const float* lse_in,
                                 const void* d_out, void* dq, float* dkv, int64_t ld_dkv, void* ws,
                                 size_t ws_bytes, void* stream) {
  try {
    if (T < 0 || S < 1 || k < 1 || ld_kv < Dk || ld_dkv < Dk || Dv > Dk) return DSA_ERR_SHAPE;
    if (dtype != DSA_BF16) return dtype == DSA_F32 ? DSA_ERR_UNSUPPORTED : DSA_ERR_DTYPE;
    if (!attn_bwd_supported(H, Dk, Dv, k)) return DSA_ERR_UNSUPPORTED;
    if (T == 0) return DSA_OK;
    if (!q || !kv || !idx || !out || !lse_in || !d_out || !dq || !dkv) return DSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv, 16) || !aligned(out, 16) || !aligned(d_out, 16) || (ld_kv * 2) % 16)
      return DSA_ERR_SHAPE;
    const size_t need = attn_bwd_workspace_bytes(T, k);
    if (ws_bytes < need || !ws || !aligned(ws, kAlign)) return DSA_ERR_WORKSPACE;
    DSA_TRY(check_device());
    BwdArgs a{};
    a.q = q;
    a.kv = kv;
    a.ld_kv = ld_kv;
    a.idx = idx;
    a.S = S;
    a.T = T;
    a.k = k;
    a.scale = scale;
    a.out = out;
    a.lse = lse_in;
    a.dout = d_out;
    a.dq = dq;
    a.dkv = dkv;
    a.ld_dkv = ld_dkv;
    return from_hip(launch_attn_bwd(a, ws, as_stream(stream)));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

size_t dsa_indexer_kl_workspace_size(int64_t L) {
  if (L < 1 || L > 65536) return 0;
  return indexer_kl_workspace_bytes(L);
}

dsa_status_t dsa_indexer_kl(const float* q_idx, const float* k_idx, const float* w, const void* q, int64_t H,
                            int64_t Dk, dsa_dtype_t dtype, const void* kv, int64_t ld_kv, int64_t L, float scale,
                            float* loss_out, float* dq_idx, float* dk_idx, float* dw, void* ws, size_t ws_bytes,
                            void* stream) {
  try {
    if (L < 0 || ld_kv < Dk) return DSA_ERR_SHAPE;
    if (dtype != DSA_BF16) return dtype == DSA_F32 ? DSA_ERR_UNSUPPORTED : DSA_ERR_DTYPE;
    if (L == 0) return DSA_OK;
    if (!indexer_kl_supported(H, Dk, L)) return DSA_ERR_UNSUPPORTED;
    if (!q_idx || !k_idx || !w || !q || !kv || !loss_out || !dq_idx || !dk_idx || !dw) return DSA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(kv, 16) || (ld_kv * 2) % 16 || !aligned(k_idx, 16) || !aligned(dq_idx, 16) ||
        !aligned(dk_idx, 16))
      return DSA_ERR_SHAPE;
    const size_t need = indexer_kl_workspace_bytes(L);
    if (ws_bytes < need || !ws || !aligned(ws, kAlign)) return DSA_ERR_WORKSPACE;
    DSA_TRY(check_device());
    KlArgs a{};
    a.q_idx = q_idx;
    a.k_idx = k_idx;
    a.w = w;
    a.q = q;
    a.kv = kv;
    a.ld_kv = ld_kv;
    a.L = L;
    a.scale = scale;
    a.loss = loss_out;
    a.dq_idx = dq_idx;
    a.dk_idx = dk_idx;
    a.dw = dw;
    return from_hip(launch_indexer_kl(a, ws, as_stream(stream)));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

size_t dsa_forward_workspace_size(const dsa_forward_args* a) {
  if (!a || check_forward(a) != DSA_OK) return 0;
  const FwdPlan p = plan_forward(a, true);
  return p.total + attn_workspace_bytes(a->attn_dtype == DSA_F32, a->T, a->H, a->Dv, a->topk);
}

}  // extern "C"

namespace {

// The forward's launches once its arguments are validated, the device is
// checked and `ws` holds at least forward_bytes(a, idx_out) bytes.
dsa_status_t forward_run(const dsa_forward_args* a, int32_t* idx_out, void* out, void* ws, size_t ws_bytes,
                         hipStream_t st) {
  const FwdPlan p = plan_forward(a, idx_out == nullptr);
  const size_t attn_ws = attn_workspace_bytes(a->attn_dtype == DSA_F32, a->T, a->H, a->Dv, a->topk);
  char* base = (char*)ws;
  void* qf = base + p.qf_off;
  float* qs = (float*)(base + p.qs_off);
  int32_t* idx = idx_out ? idx_out : (int32_t*)(base + p.idx_off);
  float* sc = (float*)(base + p.sc_off);
  const bool fp8 = a->idx_dtype == DSA_FP8_E4M3;
  const int64_t R = a->T;
  // the plan's regions follow one another inside the workspace
  DSA_DEBUG_CHECK(p.qf_off + (size_t)R * 128 * (fp8 ? 1 : 4) <= p.qs_off);
  DSA_DEBUG_CHECK(p.qs_off + (size_t)R * 4 <= p.idx_off);
  DSA_DEBUG_CHECK(idx_out || p.idx_off + (size_t)R * (size_t)a->topk * 4 <= p.sc_off);
  DSA_DEBUG_CHECK(!p.fused || p.sc_off + index_select_workspace_bytes(R, prefill_keys(a)) <= p.total);
  DSA_DEBUG_CHECK(p.fused || a->mode != DSA_MODE_PREFILL ||
                  (p.chunk_rows >= 1 && p.sc_off + (size_t)p.chunk_rows * (size_t)prefill_keys(a) * 4 <= p.total));
  DSA_DEBUG_CHECK(a->mode != DSA_MODE_DECODE ||
                  (p.sc_off + (size_t)a->total_keys * 4 <= p.topk_off && p.topk_off + p.topk_bytes <= p.total));
  DSA_DEBUG_CHECK(p.total + attn_ws <= ws_bytes);
  const DynK dyn = (a->flags & DSA_FLAG_DYNAMIC_K) ? DynK{a->dyn_theta, a->dyn_k_min} : kFixedK;

  hipError_t e = launch_fold(a->q_idx, a->q_scale, fp8, a->w_index, a->w_dtype == DSA_BF16, R, qf,
                             qs, st);
  if (e != hipSuccess) return DSA_ERR_DEVICE;

  AttnArgs at{};
  at.q = a->q;
  at.kv = a->kv;
  at.v = a->v;
  at.ld_kv = a->ld_kv;
  at.ld_v = a->ld_v;
  at.idx = idx;
  at.T = R;
  at.H = a->H;
  at.Dk = a->Dk;
  at.Dv = a->Dv;
  at.k = a->topk;
  at.scale = a->scale;
  at.out = out;
  at.lse = nullptr;

  if (p.fused) {
    const int64_t S = prefill_keys(a);
    e = launch_index_select((const uint8_t*)qf, qs, (const uint8_t*)a->k_idx, a->k_scale, R, S, a->topk, idx,
                            sc, (a->flags & DSA_FLAG_FORCE_FALLBACK) != 0, st, dyn);
    if (e != hipSuccess) return DSA_ERR_DEVICE;
    at.seq_offsets = nullptr;
    at.S = S;
  } else if (a->mode == DSA_MODE_PREFILL) {
    const int64_t S = prefill_keys(a);
    for (int64_t r0 = 0; r0 < R; r0 += p.chunk_rows) {
      const int64_t r1 = r0 + p.chunk_rows < R ? r0 + p.chunk_rows : R;
      e = launch_index_scores(qf, qs, a->k_idx, a->k_scale, fp8, R, S, nullptr, a->q_offset, r0, r1, sc, S,
                              st);
      if (e != hipSuccess) return DSA_ERR_DEVICE;
      TopkRows tr{sc, S, nullptr, nullptr, S, nullptr, r0, a->q_offset};
      e = launch_topk(tr, r1 - r0, S, a->topk, idx + r0 * a->topk, nullptr, nullptr, st, dyn);
      if (e != hipSuccess) return DSA_ERR_DEVICE;
    }
    at.seq_offsets = nullptr;
    at.S = S;
  } else {
    e = launch_index_scores_decode((const uint8_t*)qf, qs, (const uint8_t*)a->k_idx, a->k_scale,
                                   a->seq_offsets, R, a->total_keys, sc, st);
    if (e != hipSuccess) return DSA_ERR_DEVICE;
    TopkRows tr{sc, 0, nullptr, nullptr, 0, a->seq_offsets, 0, 0};
    e = launch_topk(tr, R, a->max_len, a->topk, idx, nullptr, p.topk_bytes ? base + p.topk_off : nullptr, st,
                    dyn);
    if (e != hipSuccess) return DSA_ERR_DEVICE;
    at.seq_offsets = a->seq_offsets;
    at.S = a->total_keys;
  }
  return from_hip(launch_attn(at, a->attn_dtype == DSA_F32, base + p.total, attn_ws, st));
}

// the workspace bytes one forward call needs (indices in the workspace
// only when idx_out is NULL)
size_t forward_bytes(const dsa_forward_args* a, const int32_t* idx_out) {
  return plan_forward(a, idx_out == nullptr).total +
         attn_workspace_bytes(a->attn_dtype == DSA_F32, a->T, a->H, a->Dv, a->topk);
}

dsa_status_t check_forward_call(const dsa_forward_args* a, const void* out) {
  DSA_TRY(check_forward(a));
  if (a->T == 0) return DSA_OK;
  if (!out) return DSA_ERR_NULL;
  if (a->attn_dtype == DSA_BF16 && !aligned(out, 8)) return DSA_ERR_SHAPE;
  return DSA_OK;
}

// ---- the static scratch of dsa_forward_static ------------------------------
// One array per device, allocated with the code object and held until the
// process ends.  Host code never uses the array's name as an address: each
// device's copy is looked up once (hipGetSymbolAddress, with that device
// current) and that address is what the kernels receive.
constexpr size_t kStaticScratchBytes = DSA_STATIC_SCRATCH_BYTES;
__device__ __align__(256) static unsigned char scratch[kStaticScratchBytes];
std::atomic<void*> g_scratch_ptr[kMaxDevices];

dsa_status_t static_scratch(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DSA_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    // a racing first call on the same device looks up the same address
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DSA_ERR_DEVICE;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return DSA_OK;
}

}  // namespace

extern "C" {

dsa_status_t dsa_forward(const dsa_forward_args* a, int32_t* idx_out, void* out, void* ws,
                         size_t ws_bytes, void* stream) {
  try {
    DSA_TRY(check_forward_call(a, out));
    if (a->T == 0) return DSA_OK;
    if (!ws || !aligned(ws, kAlign) || ws_bytes < forward_bytes(a, idx_out)) return DSA_ERR_WORKSPACE;
    DSA_TRY(check_device());
    return forward_run(a, idx_out, out, ws, ws_bytes, as_stream(stream));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

dsa_status_t dsa_forward_static(const dsa_forward_args* a, int32_t* idx_out, void* out, void* stream) {
  try {
    DSA_TRY(check_forward_call(a, out));
    if (a->T == 0) return DSA_OK;
    if (forward_bytes(a, idx_out) > kStaticScratchBytes) return DSA_ERR_WORKSPACE;
    DSA_TRY(check_device());
    void* ws = nullptr;
    DSA_TRY(static_scratch(&ws));
    return forward_run(a, idx_out, out, ws, kStaticScratchBytes, as_stream(stream));
  } catch (...) {
    return DSA_ERR_DEVICE;
  }
}

}  // extern "C"
