"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each of them: a dropped term, a wrong sign or index, a
transposed operand, a wrong constant, a flipped tie rule."""
import numpy as np
import pytest

import oracle.codecs as oc
import oracle.dsa as od
import oracle_pins as pins

_orig = {name: getattr(od, name) for name in ("fold", "requant", "index_scores_row", "relu", "topk_row", "attend")}
_orig_c = {name: getattr(oc, name) for name in ("e4m3_decode", "e4m3_encode", "bf16_decode")}


def _fold_transposed(q, w):
    return np.asarray(q, np.float64) @ np.asarray(w, np.float64).T


def _requant_wrong_const(qf):
    amax = np.max(np.abs(qf), axis=1)
    scale = np.where(amax > 0, amax / 224.0, 1.0).astype(np.float32)
    return oc.e4m3_encode(qf / scale.astype(np.float64)[:, None]), scale


def _requant_no_f32_round(qf):
    amax = np.max(np.abs(qf), axis=1)
    scale = np.where(amax > 0, amax / 448.0, 1.0)          # kept in fp64
    return oc.e4m3_encode(qf / scale[:, None]), scale.astype(np.float32)


def _scores_no_kscale(q_vals, q_scale, k_vals, k_scale, t):
    return _orig["index_scores_row"](q_vals, q_scale, k_vals, None, t)


def _scores_exclude_self(q_vals, q_scale, k_vals, k_scale, t):
    r = _orig["index_scores_row"](q_vals, q_scale, k_vals, k_scale, t)
    r[t] = 0.0
    return r


def _scores_neg(q_vals, q_scale, k_vals, k_scale, t):
    return _orig["index_scores_row"](-np.asarray(q_vals), q_scale, k_vals, k_scale, t)


def _relu_identity(u):
    return np.asarray(u, np.float64)


def _relu_abs(u):
    return np.abs(u)


def _topk_high_index_ties(scores, k):
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    order = np.lexsort((-np.arange(n), -s))
    return np.sort(order[: min(k, n)])


def _topk_smallest(scores, k):
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), s))
    return np.sort(order[: min(k, n)])


def _topk_unsorted(scores, k):
    s = np.asarray(scores, np.float64)
    n = s.shape[0]
    return np.lexsort((np.arange(n), -s))[: min(k, n)]


def _topk_one_short(scores, k):
    return _orig["topk_row"](scores, k)[:-1] if len(scores) > 1 else _orig["topk_row"](scores, k)


def _attend_no_scale(q, k, v, scale):
    return _orig["attend"](q, k, v, 1.0)


def _attend_no_max(q, k, v, scale):
    q = np.asarray(q, np.float64)
    z = scale * (q @ np.asarray(k, np.float64).T)
    e = np.exp(z)
    den = e.sum(axis=1, keepdims=True)
    return (e / den) @ np.asarray(v, np.float64), np.log(den)[:, 0] + 1e-3


def _attend_wrong_axis(q, k, v, scale):
    q = np.asarray(q, np.float64)
    z = scale * (q @ np.asarray(k, np.float64).T)
    e = np.exp(z - z.max(axis=0, keepdims=True))
    p = e / e.sum(axis=0, keepdims=True)
    return p @ np.asarray(v, np.float64), np.zeros(q.shape[0])


def _attend_transposed_v(q, k, v, scale):
    v = np.asarray(v, np.float64)
    return _orig["attend"](q, k, v[::-1], scale)


def _decode_bias8(codes):
    return _orig_c["e4m3_decode"](codes) / 2.0


def _decode_no_subnormal(codes):
    c = np.asarray(codes, np.uint8).astype(np.int64)
    out = _orig_c["e4m3_decode"](codes)
    e = (c >> 3) & 15
    m = c & 7
    sub = (e == 0) & (m > 0)
    return np.where(sub, np.where((c >> 7) == 1, -1.0, 1.0) * np.ldexp(1.0 + m / 8.0, -7), out)


def _encode_truncate(x):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)
    step = np.ldexp(1.0, (e - 3).astype(np.int64))
    v = np.floor(a / step) * step
    return _orig_c["e4m3_encode"](np.where(np.signbit(x), -v, v))


def _encode_ties_away(x):
    x = np.asarray(x, np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)
    e = np.maximum(ex - 1, -6)
    step = np.ldexp(1.0, (e - 3).astype(np.int64))
    v = np.floor(a / step + 0.5) * step
    return _orig_c["e4m3_encode"](np.where(np.signbit(x), -v, v))


def _encode_no_saturation(x):
    x = np.asarray(x, np.float64)
    out = _orig_c["e4m3_encode"](x)
    return np.where(np.abs(x) > 448.0, np.uint8(0x7F), out).astype(np.uint8)


def _bf16_wrong_shift(bits):
    b = np.asarray(bits, np.uint16).astype(np.uint32) << 15
    return b.view(np.float32).astype(np.float64)


def _chunk_ignores_offset(self, t):
    return od.index_scores_row(self.q_vals[t], self.q_scale_of(t), self.k_vals, self.k_scale, t)


def _dynamic_k_ge(scores, k_max, k_min, theta):
    n = np.asarray(scores).shape[0]
    return min(n, k_max, max(k_min, int(np.count_nonzero(np.asarray(scores) >= theta))))


def _dynamic_k_no_floor(scores, k_max, k_min, theta):
    n = np.asarray(scores).shape[0]
    return min(n, k_max, int(np.count_nonzero(np.asarray(scores) > theta)))


def _bwd_no_rowsum(q, k, v, scale, do):
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    z = scale * (q @ k.T)
    p = np.exp(z - z.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    dz = p * (do @ v.T)
    return scale * (dz @ k), scale * (dz.T @ q), p.T @ do


def _bwd_dq_unscaled(q, k, v, scale, do):
    dq, dk, dv = _orig_bwd(q, k, v, scale, do)
    return dq / scale, dk, dv


_orig_bwd = od.attend_backward


def _sparse_bwd_no_dv(q, kv, idx, scale, Dv, d_out, rows=None):
    qa, kva, doa = od.as_f64(q), od.as_f64(kv), od.as_f64(d_out)
    dq, dkv = np.zeros_like(qa), np.zeros_like(kva)
    for t in range(qa.shape[0]):
        sel = np.asarray([s for s in idx[t] if s >= 0], np.int64)
        if sel.shape[0]:
            dq[t], dk, _ = _orig_bwd(qa[t], kva[sel], kva[sel][:, :Dv], scale, doa[t])
            np.add.at(dkv, sel, dk)
    return dq, dkv

def _target_unscaled(q_heads, k_rows, scale):
    return _orig_target(q_heads, k_rows, 1.0)


def _target_summed(q_heads, k_rows, scale):
    return _orig_target(q_heads, k_rows, scale) * np.asarray(q_heads).shape[0]


_orig_target = od.attention_target_row

MUTATIONS = {
    "kl_target_unscaled": (od, "attention_target_row", _target_unscaled),
    "kl_target_summed_not_averaged": (od, "attention_target_row", _target_summed),
    "attn_bwd_dropped_rowsum": (od, "attend_backward", _bwd_no_rowsum),
    "attn_bwd_dq_unscaled": (od, "attend_backward", _bwd_dq_unscaled),
    "sparse_bwd_dropped_dv_scatter": (od, "sparse_attn_backward", _sparse_bwd_no_dv),
    "dynamic_k_counts_ties_at_theta": (od, "dynamic_k", _dynamic_k_ge),
    "dynamic_k_ignores_k_min": (od, "dynamic_k", _dynamic_k_no_floor),
    "prefill_chunk_ignores_offset": (od.PrefillOracle, "scores_row", _chunk_ignores_offset),
    "fold_transposed": (od, "fold", _fold_transposed),
    "requant_wrong_constant": (od, "requant", _requant_wrong_const),
    "requant_scale_not_f32": (od, "requant", _requant_no_f32_round),
    "scores_dropped_key_scale": (od, "index_scores_row", _scores_no_kscale),
    "scores_exclude_self": (od, "index_scores_row", _scores_exclude_self),
    "scores_sign_flip": (od, "index_scores_row", _scores_neg),
    "relu_dropped": (od, "relu", _relu_identity),
    "relu_abs": (od, "relu", _relu_abs),
    "topk_high_index_ties": (od, "topk_row", _topk_high_index_ties),
    "topk_smallest": (od, "topk_row", _topk_smallest),
    "topk_not_ascending": (od, "topk_row", _topk_unsorted),
    "topk_one_short": (od, "topk_row", _topk_one_short),
    "attend_no_scale": (od, "attend", _attend_no_scale),
    "attend_lse_wrong": (od, "attend", _attend_no_max),
    "attend_softmax_wrong_axis": (od, "attend", _attend_wrong_axis),
    "attend_v_rows_permuted": (od, "attend", _attend_transposed_v),
    "e4m3_bias_8": (oc, "e4m3_decode", _decode_bias8),
    "e4m3_no_subnormals": (oc, "e4m3_decode", _decode_no_subnormal),
    "e4m3_encode_truncates": (oc, "e4m3_encode", _encode_truncate),
    "e4m3_encode_ties_away": (oc, "e4m3_encode", _encode_ties_away),
    "e4m3_encode_nan_on_overflow": (oc, "e4m3_encode", _encode_no_saturation),
    "bf16_wrong_shift": (oc, "bf16_decode", _bf16_wrong_shift),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(od, oc)
        except Exception as e:  # an assertion or a shape error both count as caught
            caught.append(pin.__name__)
            break
    assert caught, f"no pin caught the planted mistake {name}"
