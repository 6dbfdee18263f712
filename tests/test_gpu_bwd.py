"""Backward of the sparse attention on the GPU through the C ABI, against the
fp64 oracle (oracle.dsa.sparse_attn_backward) on the same bf16 inputs and
selections: every query of a small ragged batch, and sampled queries of a
full-size batch (k = 2048, two query chunks) whose other queries select
nothing, so dkv holds only the sampled queries' share.

Tolerance, per element, from the kernels' arithmetic (error_budget below):
* P is exp2 of an fp32 logit minus the forward's fp32 log-sum-exp, stored as
  bf16 for the dkv product (unit roundoff u = 2^-8) and used unrounded in dS;
* dS = scale P (dP - Delta) in fp32, stored as bf16 (u); dP sums Dv exact
  bf16 products in fp32; Delta = dO . O takes the forward's bf16 output O,
  so it is off the exact value by at most sum |dO| |O_gpu - O_exact|;
* dq and dkv sum exact products of those bf16 operands in fp32.
Each element's bound is the sum of those per-term errors along its row
(triangle inequality, so far above the typical error); the test asserts
|g - o| <= 2 x bound + 1e-30.  A dropped term, a wrong row or a transposed
operand moves an element by the size of a whole term, which the bound (a few
u of the absolute sum) does not admit."""
import sys

import numpy as np
import pytest
import torch

import oracle.dsa as od
from helpers import to_np
from sparse_attention_long_indexer_amd import binding as B
from sparse_attention_long_indexer_amd import inputs as gen

pytestmark = pytest.mark.gpu

SPEC = gen.PREFILL_32K   # MLA shape: H = 128, Dk = 576, Dv = 512, shared latent KV


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


U = 2.0 ** -8        # bf16 unit roundoff (8 significand bits, round to nearest)
EPS32 = 2.0 ** -24   # fp32 unit roundoff


def error_budget(q, kv, idx, scale, Dv, d_out, out_gpu, rows):
    """Per-element error bounds of dq [T, H, Dk] and dkv [S, Dk] for the
    queries `rows`, from the exact fp64 quantities of each query and the
    roundings the kernels make (see the module docstring)."""
    qa, kva, doa, oga = od.as_f64(q), od.as_f64(kv), od.as_f64(d_out), od.as_f64(out_gpu)
    T, H, Dk = qa.shape
    b_dq = np.zeros_like(qa)
    b_dkv = np.zeros((kva.shape[0], Dk))
    for t in rows:
        sel = np.asarray(idx[t])
        sel = sel[: np.argmax(sel < 0)] if np.any(sel < 0) else sel
        m = sel.shape[0]
        if m == 0:
            continue
        kr = kva[sel]
        vr = kr[:, :Dv]
        z = scale * (qa[t] @ kr.T)
        e = np.exp(z - z.max(axis=1, keepdims=True))
        p = e / e.sum(axis=1, keepdims=True)
        o = p @ vr
        dp = doa[t] @ vr.T
        delta = np.sum(doa[t] * o, axis=1)
        # Delta from the bf16 output, and fp32 sums over Dv products
        d_delta = np.sum(np.abs(doa[t]) * np.abs(oga[t] - o), axis=1) + \
            (Dv + 32) * EPS32 * np.sum(np.abs(doa[t] * o), axis=1)
        d_dp = (Dv + 32) * EPS32 * (np.abs(doa[t]) @ np.abs(vr).T)
        ds = scale * p * (dp - delta[:, None])
        # dS: the logit and the forward's log-sum-exp (fp32; the forward's
        # lse is within 1e-4 relative of exact) perturb P by < 1e-4, then the
        # bf16 store, Delta and dP
        e_ds = scale * p * (d_delta[:, None] + (U + 1e-4) * np.abs(dp - delta[:, None]) + d_dp)
        e_p = p * (U + 1e-4)
        g_k = (m + 64) * EPS32
        b_dq[t] = e_ds @ np.abs(kr) + g_k * (np.abs(ds) @ np.abs(kr))
        contrib = e_ds.T @ np.abs(qa[t])                            # [m, Dk]
        contrib[:, :Dv] += e_p.T @ np.abs(doa[t])
        mag = np.abs(ds).T @ np.abs(qa[t])
        mag[:, :Dv] += np.abs(p).T @ np.abs(doa[t])
        np.add.at(b_dkv, sel, contrib + (len(rows) * H + 64) * EPS32 * mag)
    return b_dq, b_dkv


def within(g, o, bound, what):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = np.abs(g - o)
    lim = 2.0 * bound + 1e-30
    ok = err <= lim
    assert np.all(ok), (what, int(np.sum(~ok)), float(np.max(err / lim)))
    rel = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))
    return rel, float(np.max(err / lim))


def run(dev, T, S, k, seed, min_valid, keep=None):
    spec = SPEC.with_(L=S)
    x = gen.make_prefill(spec, seed=seed, device=dev)
    q = x["q"][:T].contiguous()
    kv = x["kv"]
    idx = gen.make_selection(T, S, k, seed=seed, min_valid=min_valid)
    if keep is not None:  # queries outside `keep` select nothing
        mask = torch.ones(T, dtype=torch.bool)
        mask[keep] = False
        idx[mask] = -1
    idx = idx.to(dev)
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    out = B.dsa_sparse_attn(q, kv, idx, spec.scale, Dv=spec.Dv, lse_out=lse)
    d_out = gen.make_grad((T, spec.H, spec.Dv), seed=seed, device=dev)
    dq, dkv = B.dsa_sparse_attn_bwd(q, kv, idx, spec.scale, out, lse, d_out, spec.Dv)
    torch.cuda.synchronize()
    return spec, q, kv, idx, d_out, dq, dkv, out


def check(spec, q, kv, idx, d_out, dq, dkv, out, rows, S):
    gi = idx.cpu().numpy()
    o_dq, o_dkv = od.sparse_attn_backward(to_np(q), to_np(kv), gi, spec.scale, spec.Dv, to_np(d_out), rows=rows)
    b_dq, b_dkv = error_budget(to_np(q), to_np(kv), gi, spec.scale, spec.Dv, to_np(d_out), to_np(out), rows)
    g_dq = od.as_f64(to_np(dq))
    worst = (0.0, 0.0)
    for t in rows:
        if int(np.sum(gi[t] >= 0)) == 0:
            assert np.all(g_dq[t] == 0), t
            continue
        r = within(g_dq[t], o_dq[t], b_dq[t], ("dq", t))
        worst = (max(worst[0], r[0]), max(worst[1], r[1]))
    sel_rows = np.unique(gi[rows][gi[rows] >= 0])
    g_dkv = to_np(dkv).astype(np.float64)
    r2 = within(g_dkv[sel_rows], o_dkv[sel_rows], b_dkv[sel_rows], "dkv")
    untouched = np.setdiff1d(np.arange(S), np.unique(gi[gi >= 0]))
    assert np.all(g_dkv[untouched] == 0)
    return worst, r2


def test_attn_bwd_small(dev):
    T, S, k = 37, 3000, 256
    spec, q, kv, idx, d_out, dq, dkv, out = run(dev, T, S, k, seed=41, min_valid=0)
    worst, r2 = check(spec, q, kv, idx, d_out, dq, dkv, out, list(range(T)), S)
    say(f"dq: worst normwise {worst[0]:.3g}, worst error / bound {worst[1]:.3g}; dkv: normwise {r2[0]:.3g}, "
        f"worst error / bound {r2[1]:.3g}")


def test_attn_bwd_full_k_two_chunks(dev):
    T, S, k = 4100, 8192, 2048
    keep = [0, 1, 2047, 2048, 2049, 4099]
    spec, q, kv, idx, d_out, dq, dkv, out = run(dev, T, S, k, seed=42, min_valid=1500, keep=keep)
    worst, r2 = check(spec, q, kv, idx, d_out, dq, dkv, out, keep, S)
    assert torch.all(dq[3] == 0)  # a query with no selected key
    say(f"dq: worst normwise {worst[0]:.3g}, worst error / bound {worst[1]:.3g}; dkv: normwise {r2[0]:.3g}, "
        f"worst error / bound {r2[1]:.3g}")


def test_attn_bwd_accumulates(dev):
    """Two calls into one dkv equal twice one call (to rounding); dq is
    written, not accumulated."""
    T, S, k = 64, 2000, 128
    spec, q, kv, idx, d_out, dq, dkv, _ = run(dev, T, S, k, seed=43, min_valid=1)
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    out = B.dsa_sparse_attn(q, kv, idx, spec.scale, Dv=spec.Dv, lse_out=lse)
    dq2, dkv2 = B.dsa_sparse_attn_bwd(q, kv, idx, spec.scale, out, lse, d_out, spec.Dv, dkv=dkv.clone())
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq)
    assert torch.allclose(dkv2, 2 * dkv, rtol=1e-5, atol=1e-6)
