"""fp64 CPU oracle of the DeepSeek Sparse Attention (DSA) forward path.

Test infrastructure: only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  It is a plain, slow, step-by-step
restatement of the method; it shares no code with the HIP path and never runs
in the product path.

The method, as the DeepSeek-V3.2 write-up on intelliparadigm.com describes it
("DSA", sections 2.1-3.1):
  * a lightning indexer scores every query token against every earlier token
    with I[t,s] = ReLU(q_t . W_index . k_s) on 128-dim index vectors held in
    FP8 (section 2.2);
  * a fine-grained selection keeps, per query, the k = 2048 keys with the
    highest index score (section 2.3);
  * ordinary softmax attention then runs over the selected keys only, with all
    query heads sharing one key/value head, MLA's MQA mode (sections 2.3, 3.1).

Readings of points the pages leave open (each is a stated choice):
  R1  W is folded into the index query before the FP8 product:
      qf_t = dq(q8_t) @ W  (q a row vector, qf_j = sum_i q_i W_ij), then qf_t
      is re-quantised to e4m3 with a per-row scale amax/448 (fp32, RNE);
      amax = 0 gives scale 1.  The folded, re-quantised query is the FP8
      operand of the score product.  The fp32 workload skips the re-quantising.
  R2  keys of query t are s in [0, t] (its own token included), so a query
      keeps m_t = min(k, t+1) keys.
  R3  ties are broken by the lower key index; ReLU maps every u <= 0
      (including -0.0) to +0.0, so zero scores tie.
  R4  the selected set is reported in ascending key order, padded with -1.
  R5  V of the shared latent row is its first Dv entries unless a separate V
      is given.
  R6  -0.0 re-quantises to the +0 code.
"""
from __future__ import annotations

import numpy as np

from . import codecs

IDX_DIM = 128


# ---------------------------------------------------------------- inputs ---

def dequant_rows(codes, scale) -> np.ndarray:
    """dq(x8)[t, j] = e4m3(x8[t, j]) * scale[t], exact in fp64."""
    return codecs.e4m3_decode(codes) * np.asarray(scale, dtype=np.float32).astype(np.float64)[:, None]


def as_f64(x) -> np.ndarray:
    """fp32 / bf16(uint16 bits) / fp64 arrays -> fp64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return codecs.bf16_decode(x)
    return x.astype(np.float64)


# ------------------------------------------------------ R1: fold, requant ---

def fold(q_rows: np.ndarray, w: np.ndarray) -> np.ndarray:
    """qf = q @ W in fp64, q as row vectors (section 2.2's q_t . W_index)."""
    return np.asarray(q_rows, np.float64) @ np.asarray(w, np.float64)


def requant(qf: np.ndarray):
    """Per-row e4m3 re-quantisation of the folded query (reading R1).

    scale_t = fp32(amax_t / 448), 1 when amax_t = 0;
    code[t, j] = e4m3_RNE_sat(qf[t, j] / scale_t), quotient in fp64.
    """
    amax = np.max(np.abs(qf), axis=1)
    scale = codecs.f64_to_f32_rne(np.where(amax > 0, amax / codecs.E4M3_MAX, 1.0))
    codes = codecs.e4m3_encode(qf / scale.astype(np.float64)[:, None])
    return codes, scale


# ----------------------------------------------------- section 2.2: I[t,s] ---

def relu(u: np.ndarray) -> np.ndarray:
    """ReLU with +0.0 for every u <= 0 (reading R3)."""
    return np.where(u > 0, u, 0.0)


def index_scores_row(q_vals: np.ndarray, q_scale: float, k_vals: np.ndarray, k_scale, t: int) -> np.ndarray:
    """I[t, s] for s in [0, t], fp64 (one row, causal).

    u[s] = q_scale * k_scale[s] * sum_j q_vals[j] * k_vals[s, j];  I = ReLU(u).
    For FP8 operands q_vals / k_vals are the decoded e4m3 values (their
    128-term dot product is exact in fp64) and the scales are the per-row
    fp32 scales; for fp32 operands the scales are 1.
    """
    dots = np.asarray(k_vals[: t + 1], np.float64) @ np.asarray(q_vals, np.float64)
    ks = np.ones(t + 1) if k_scale is None else np.asarray(k_scale[: t + 1], np.float64)
    u = float(q_scale) * (ks * dots)
    return relu(u)


def index_scores(q_vals, q_scale, k_vals, k_scale, pos) -> np.ndarray:
    """Dense score matrix [T, S] with -inf where s > pos[t] (small inputs only)."""
    T, S = q_vals.shape[0], k_vals.shape[0]
    out = np.full((T, S), -np.inf)
    for t in range(T):
        p = min(int(pos[t]), S - 1)
        qs = 1.0 if q_scale is None else float(q_scale[t])
        out[t, : p + 1] = index_scores_row(q_vals[t], qs, k_vals, k_scale, p)
    return out


# ----------------------------------------------------- section 2.3: top-k ---

def topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """The min(k, n) best keys of one row under (higher score, then lower
    index), returned in ascending key order (readings R3, R4).  Full sort."""
    scores = np.asarray(scores, np.float64)
    n = scores.shape[0]
    m = min(k, n)
    order = np.lexsort((np.arange(n), -scores))   # primary: -score, secondary: index
    return np.sort(order[:m])


def dynamic_k(scores: np.ndarray, k_max: int, k_min: int, theta: float) -> int:
    """Per-query key budget for a dynamic k (reading R19 of the write-up's
    outlook on k that adapts instead of a fixed top-k, section 6): the number
    of keys whose index score exceeds theta, kept within [k_min, k_max] and
    never above the row's n keys.  theta = -inf gives the fixed min(k_max, n)."""
    n = np.asarray(scores).shape[0]
    above = int(np.count_nonzero(np.asarray(scores, np.float64) > theta))
    return min(n, k_max, max(k_min, above))


def topk_row_dynamic(scores: np.ndarray, k_max: int, k_min: int, theta: float) -> np.ndarray:
    """The dynamic_k(...) best keys of one row, under the same order and
    output convention as topk_row."""
    return topk_row(scores, dynamic_k(scores, k_max, k_min, theta))


def pad_idx(sel: np.ndarray, k: int) -> np.ndarray:
    out = np.full(k, -1, dtype=np.int32)
    out[: sel.shape[0]] = sel
    return out


# ------------------------------------------- sections 2.3 / 3.1: attention ---

def attend(q_heads: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float):
    """Softmax attention of H query heads over n shared key/value rows, fp64.

    z[h, s] = scale * q_h . k_s;  p = softmax_s(z);  o_h = sum_s p[h, s] v_s.
    Returns (o [H, Dv], lse [H]) with lse the natural-log normaliser of z.
    """
    q = np.asarray(q_heads, np.float64)
    z = scale * (q @ np.asarray(k_rows, np.float64).T)
    zmax = np.max(z, axis=1, keepdims=True)
    e = np.exp(z - zmax)
    den = np.sum(e, axis=1, keepdims=True)
    o = (e / den) @ np.asarray(v_rows, np.float64)
    return o, (zmax + np.log(den))[:, 0]


def attend_backward(q_heads: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float,
                    d_out: np.ndarray):
    """Gradients of `attend` for one query in fp64 (the sparse training stage
    of the write-up, section 4.1, trains through attention over the selected
    keys).  With z = scale q k^T, p = softmax(z), o = p v and the incoming
    gradient dO of o:
      dv = p^T dO;   dp = dO v^T;   dz = p * (dp - rowsum(dO * o));
      dq = scale dz k;   dk = scale dz^T q.
    Returns (dq [H, Dk], dk [n, Dk], dv [n, Dv])."""
    q = np.asarray(q_heads, np.float64)
    kr = np.asarray(k_rows, np.float64)
    vr = np.asarray(v_rows, np.float64)
    do = np.asarray(d_out, np.float64)
    z = scale * (q @ kr.T)
    e = np.exp(z - np.max(z, axis=1, keepdims=True))
    p = e / np.sum(e, axis=1, keepdims=True)
    o = p @ vr
    dv = p.T @ do
    dp = do @ vr.T
    dz = p * (dp - np.sum(do * o, axis=1, keepdims=True))
    return scale * (dz @ kr), scale * (dz.T @ q), dv


def sparse_attn_backward(q, kv, idx, scale: float, Dv: int, d_out, rows=None):
    """Backward of sparse MQA attention over a shared latent KV row per key
    (K = kv[:, :Dk], V = kv[:, :Dv]): dq [T, H, Dk] and dkv [S, Dk], the sum
    over every query that selected a key of its dk, plus its dv in the first
    Dv columns.  `rows` restricts the queries (dq of the others stays 0 and
    they add nothing to dkv).  Inputs in the library's storage formats."""
    qa = as_f64(q)
    kva = as_f64(kv)
    doa = as_f64(d_out)
    T = qa.shape[0]
    dq = np.zeros_like(qa)
    dkv = np.zeros_like(kva)
    for t in (range(T) if rows is None else rows):
        sel = np.asarray(idx[t])
        sel = sel[: np.argmax(sel < 0)] if np.any(sel < 0) else sel
        if sel.shape[0] == 0:
            continue
        krows = kva[sel]
        dq[t], dk, dv = attend_backward(qa[t], krows, krows[:, :Dv], scale, doa[t])
        np.add.at(dkv, sel, dk)
        np.add.at(dkv[:, :Dv], sel, dv)
    return dq, dkv


# ------------------------------------- section 4.1: indexer alignment (KL) ---

def attention_target_row(q_heads: np.ndarray, k_rows: np.ndarray, scale: float) -> np.ndarray:
    """The dense model's attention distribution of one query over its keys,
    summed over the heads and L1-normalised (reading R21): the mean over
    heads of softmax_s(scale q_h . k_s)."""
    q = np.asarray(q_heads, np.float64)
    z = scale * (q @ np.asarray(k_rows, np.float64).T)
    e = np.exp(z - np.max(z, axis=1, keepdims=True))
    return np.mean(e / np.sum(e, axis=1, keepdims=True), axis=0)


def indexer_kl(q_idx, k_idx, w, q, kv, scale: float, Dk: int, rows=None):
    """KL alignment of the lightning indexer to the dense attention (dense
    warm-up of section 4.1, reading R21), fp64, causal prefill over L tokens.

    For query t over keys s <= t: the target p_t is attention_target_row, the
    indexer distribution is q_t = softmax_s(I[t,s]) with I = ReLU(u),
    u[t,s] = (q_idx[t] W) . k_idx[s] on real-valued index vectors, and the
    loss is sum_t KL(p_t || q_t) = sum_t sum_s p (log p - log q) (0 log 0 = 0).
    Its gradient with respect to I[t,s] is q_t[s] - p_t[s]; through the ReLU
    it is kept where u > 0.  With G that gradient and qf = q_idx W:
      d qf = G k_idx;  d k_idx = G^T qf;  d q_idx = (d qf) W^T;  d W = q_idx^T (d qf).
    `rows` restricts the queries whose terms are summed.  Returns
    (loss, per-query losses [L], dq_idx [L,128], dk_idx [L,128], dW [128,128]).
    """
    qi = as_f64(q_idx)
    ki = as_f64(k_idx)
    wd = as_f64(w)
    qa = q   # rows are read one at a time (q may be a row accessor)
    kva = as_f64(kv)
    L = qi.shape[0]
    qf = fold(qi, wd)
    losses = np.zeros(L)
    dqf = np.zeros_like(qf)
    dk = np.zeros_like(ki)
    for t in (range(L) if rows is None else rows):
        u = ki[: t + 1] @ qf[t]
        i_row = relu(u)
        m = np.max(i_row)
        logq = i_row - (m + np.log(np.sum(np.exp(i_row - m))))
        p = attention_target_row(as_f64(qa[t]), kva[: t + 1, :Dk], scale)
        nz = p > 0
        losses[t] = float(np.sum(p[nz] * (np.log(p[nz]) - logq[nz])))
        g = (np.exp(logq) - p) * (u > 0)
        dqf[t] = g @ ki[: t + 1]
        dk[: t + 1] += np.outer(g, qf[t])
    return float(np.sum(losses)), losses, dqf @ wd.T, dk, qi.T @ dqf


# ---------------------------------------------------------- whole forward ---

class PrefillOracle:
    """One causal prefill over S key tokens; query row t is the token at
    position q_offset + t (q_offset = 0: queries = keys, the whole sequence;
    q_offset > 0: the last T tokens, a later chunk of a long prefill).

    Arguments are host numpy arrays in the library's storage formats:
      q_idx, k_idx : uint8 e4m3 codes [T,128] / [S,128] with fp32 scales
                     (FP8), or float32 rows with scales None (fp32)
      w            : uint16 bf16 bits or float32 [128,128]
      q            : [T,H,Dk] (uint16 bf16 bits or float32)
      kv           : [S,Dk]; v : [S,Dv] or None (then V = kv[:, :Dv])
    """

    def __init__(self, q_idx, q_scale, k_idx, k_scale, w, q, kv, v, topk, scale, Dv, q_offset=0):
        self.fp8 = q_scale is not None
        if self.fp8:
            qv = dequant_rows(q_idx, q_scale)
            self.k_vals = codecs.e4m3_decode(k_idx)
            self.k_scale = np.asarray(k_scale, np.float32).astype(np.float64)
        else:
            qv = as_f64(q_idx)
            self.k_vals = as_f64(k_idx)
            self.k_scale = None
        self.qf = fold(qv, as_f64(w))
        if self.fp8:
            self.qf8, self.qf_scale = requant(self.qf)
            self.q_vals = codecs.e4m3_decode(self.qf8)
        else:
            self.qf8, self.qf_scale = None, None
            self.q_vals = self.qf
        self.q, self.kv, self.v = q, kv, v
        self.k, self.scale, self.Dv = topk, scale, Dv
        self.q_offset = int(q_offset)

    def q_scale_of(self, t: int) -> float:
        return 1.0 if self.qf_scale is None else float(self.qf_scale[t])

    def scores_row(self, t: int) -> np.ndarray:
        return index_scores_row(self.q_vals[t], self.q_scale_of(t), self.k_vals, self.k_scale, self.q_offset + t)

    def select_row(self, t: int) -> np.ndarray:
        return topk_row(self.scores_row(t), self.k)

    def attend_row(self, t: int, sel: np.ndarray):
        k_rows = as_f64(self.kv[sel])
        v_rows = as_f64(self.v[sel]) if self.v is not None else k_rows[:, : self.Dv]
        return attend(as_f64(self.q[t]), k_rows, v_rows, self.scale)

    def row(self, t: int):
        sel = self.select_row(t)
        o, lse = self.attend_row(t, sel)
        return pad_idx(sel, self.k), o, lse


class DecodeOracle:
    """One batched decode step: sequence b owns cache rows
    [off[b], off[b+1]) and its query sits at position n_b - 1 over keys
    [0, n_b) of its own cache."""

    def __init__(self, q_idx, q_scale, k_idx, k_scale, w, q, kv, v, offsets, topk, scale, Dv):
        qv = dequant_rows(q_idx, q_scale)
        self.k_idx, self.k_scale = k_idx, k_scale
        self.qf = fold(qv, as_f64(w))
        self.qf8, self.qf_scale = requant(self.qf)
        self.q_vals = codecs.e4m3_decode(self.qf8)
        self.q, self.kv, self.v = q, kv, v
        self.off = np.asarray(offsets, np.int64)
        self.k, self.scale, self.Dv = topk, scale, Dv

    def scores_seq(self, b: int) -> np.ndarray:
        lo, hi = int(self.off[b]), int(self.off[b + 1])
        k_vals = codecs.e4m3_decode(self.k_idx[lo:hi])
        k_scale = np.asarray(self.k_scale[lo:hi], np.float32).astype(np.float64)
        return index_scores_row(self.q_vals[b], float(self.qf_scale[b]), k_vals, k_scale, hi - lo - 1)

    def seq(self, b: int):
        lo, hi = int(self.off[b]), int(self.off[b + 1])
        sel = topk_row(self.scores_seq(b), self.k)
        kv = as_f64(self.kv[lo:hi][sel])
        vv = as_f64(self.v[lo:hi][sel]) if self.v is not None else kv[:, : self.Dv]
        o, lse = attend(as_f64(self.q[b]), kv, vv, self.scale)
        return pad_idx(sel, self.k), o, lse
