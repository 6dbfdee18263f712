"""Parity rules between the HIP path and the oracle.

* fold codes: bit-exact; a differing code is excused only when the oracle's
  fp64 quotient lies within 1e-12 (relative) of the rounding midpoint between
  the two codes (the two sides sum 128 fp64 products in different orders).
* scores: |g - o| <= 2e-2 |o| + 2e-2 rms_t (rms_t over the oracle row), and
  exactly -inf past the causal position.
* top-k: the GPU set differs from the oracle's only inside the window
  A = {s : |o_s - o_(m)| <= 1e-3 |o_(m)| + 1e-6 max_s |o_s|} around the m-th
  best oracle score; both have m = min(k, n) distinct ascending entries.
* attention: bf16 |g - o| <= 1e-2 + 2e-2 |o| and, per (query, head),
  max |g - o| <= 2e-2 rms(o); fp32 |g - o| <= 1e-5 + 1e-5 |o|.
"""
import numpy as np

import oracle.codecs as oc


def check_fold_codes(g_codes, g_scale, o_qf, o_codes, o_scale):
    assert np.array_equal(g_scale, o_scale), np.nonzero(g_scale != o_scale)[0][:8]
    bad = np.argwhere(g_codes != o_codes)
    for t, j in bad:
        q = o_qf[t, j] / float(o_scale[t])
        a, b = oc.e4m3_decode(np.array([g_codes[t, j], o_codes[t, j]], np.uint8))
        mid = (a + b) / 2.0
        assert abs(q - mid) <= 1e-12 * abs(mid), (t, j, q, a, b)
    return len(bad)


def check_scores_row(g, o, t):
    g = np.asarray(g, np.float64)
    n = t + 1
    assert np.all(np.isneginf(g[n:])), "masked entries must be -inf"
    gv, ov = g[:n], o[:n]
    assert np.all(gv >= 0) and not np.any(np.signbit(gv)), "ReLU output must be +0 or positive"
    rms = np.sqrt(np.mean(ov ** 2)) if n else 0.0
    err = np.abs(gv - ov)
    tol = 2e-2 * np.abs(ov) + 2e-2 * rms
    assert np.all(err <= tol), (t, float(np.max(err - tol)))
    return float(np.linalg.norm(gv - ov) / max(np.linalg.norm(ov), 1e-300))


def check_topk_row(g_idx, o_scores, o_sel, k, rel=1e-3):
    """Returns the number of indices that differ (inside the window)."""
    n = o_scores.shape[0]
    m = min(k, n)
    g = np.asarray(g_idx)
    assert np.all(g[m:] == -1), "padding must be -1"
    gs = g[:m]
    assert gs.shape[0] == m and np.all(gs >= 0) and np.all(gs < n)
    assert np.all(np.diff(gs) > 0), "indices must be distinct and ascending"
    if m == n:
        assert np.array_equal(gs, np.arange(n))
        return 0
    sk = np.sort(o_scores)[::-1][m - 1]
    eps = 1e-6 * np.max(np.abs(o_scores))
    window = np.abs(o_scores - sk) <= rel * abs(sk) + eps
    gset, oset = set(gs.tolist()), set(np.asarray(o_sel).tolist())
    A = set(np.nonzero(window)[0].tolist())
    assert gset - A == oset - A, ("selection differs outside the boundary window",
                                  sorted(gset - oset)[:8], sorted(oset - gset)[:8])
    return len(gset ^ oset)


def check_attn(g, o, f32=False):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    if f32:
        err = np.abs(g - o)
        tol = 1e-5 + 1e-5 * np.abs(o)
        assert np.all(err <= tol), float(np.max(err - tol))
        return float(np.max(err))
    err = np.abs(g - o)
    assert np.all(err <= 1e-2 + 2e-2 * np.abs(o)), float(np.max(err))
    rms = np.sqrt(np.mean(o ** 2, axis=-1))
    rel = np.max(err, axis=-1) / np.maximum(rms, 1e-30)
    assert np.all(rel <= 2e-2), float(np.max(rel))
    return float(np.max(rel))


def check_forward_row(g_idx, o_scores, o_sel, k, attend, g_out, f32=False):
    """One query of a whole forward: the kept indices under the window rule,
    then its attention output.  The output is held to the oracle's fp64
    attention over the GPU's own kept set: that is the oracle's set when the
    two agree, and otherwise a set that differs only inside the boundary
    window (so every sampled row's output is checked).  `attend(sel)` returns
    the oracle's (o, lse) over the key indices `sel`.
    Returns (index differences, worst attention error)."""
    d = check_topk_row(g_idx, o_scores, o_sel, k)
    g = np.asarray(g_idx)
    m = min(k, o_scores.shape[0])
    sel = np.asarray(o_sel) if d == 0 else g[:m]
    o, _ = attend(sel)
    return d, check_attn(g_out, o, f32=f32)
