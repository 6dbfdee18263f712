"""Backward of the sparse attention on the GPU through the C ABI, against the
fp64 oracle (oracle.dsa.sparse_attn_backward) on the same bf16 inputs and
selections: every query of a small ragged batch, and sampled queries of a
full-size batch (k = 2048, two query chunks) whose other queries select
nothing, so dkv holds only the sampled queries' share.

Tolerance, from the arithmetic: the GPU rounds P and dS to bf16 (unit
roundoff u = 2^-9) before the products and takes Delta = dO . O from the
bf16 forward output (another u-sized, per-head coherent error in dS).  So the
gradients carry a few u of normwise relative error: a query's dq and the set
of touched dkv rows must hold ||g - o|| <= 2e-2 ||o|| (about 10 u), and no
element may stray past 0.25 rms of its query (row set), which still catches a
dropped term, a wrong row or a transposed operand (errors of order 1)."""
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


def close(g, o, what):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    rel = float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))
    rms = float(np.sqrt(np.mean(o ** 2)))
    worst = float(np.max(np.abs(g - o)) / max(rms, 1e-300))
    assert rel <= 2e-2 and worst <= 0.25, (what, rel, worst)
    return rel


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
    return spec, q, kv, idx, d_out, dq, dkv


def test_attn_bwd_small(dev):
    T, S, k = 37, 3000, 256
    spec, q, kv, idx, d_out, dq, dkv = run(dev, T, S, k, seed=41, min_valid=0)
    gi = idx.cpu().numpy()
    o_dq, o_dkv = od.sparse_attn_backward(to_np(q), to_np(kv), gi, spec.scale, spec.Dv, to_np(d_out))
    g_dq = od.as_f64(to_np(dq))
    worst = 0.0
    for t in range(T):
        m = int(np.sum(gi[t] >= 0))
        if m == 0:
            assert np.all(g_dq[t] == 0), t
            continue
        worst = max(worst, close(g_dq[t], o_dq[t], ("dq", t)))
    rows = np.unique(gi[gi >= 0])
    g_dkv = to_np(dkv).astype(np.float64)
    w2 = close(g_dkv[rows], o_dkv[rows], "dkv")
    untouched = np.setdiff1d(np.arange(S), rows)
    assert np.all(g_dkv[untouched] == 0)
    say(f"valid counts {sorted(set(int(np.sum(r >= 0)) for r in gi))[:6]}...; worst dq relative error {worst:.3g}, "
        f"dkv relative error {w2:.3g}")


def test_attn_bwd_full_k_two_chunks(dev):
    T, S, k = 4100, 8192, 2048
    keep = [0, 1, 2047, 2048, 2049, 4099]
    spec, q, kv, idx, d_out, dq, dkv = run(dev, T, S, k, seed=42, min_valid=1500, keep=keep)
    gi = idx.cpu().numpy()
    o_dq, o_dkv = od.sparse_attn_backward(to_np(q), to_np(kv), gi, spec.scale, spec.Dv, to_np(d_out), rows=keep)
    g_dq = od.as_f64(to_np(dq))
    worst = max(close(g_dq[t], o_dq[t], ("dq", t)) for t in keep)
    rows = np.unique(gi[gi >= 0])
    w2 = close(to_np(dkv).astype(np.float64)[rows], o_dkv[rows], "dkv")
    assert torch.all(dq[3] == 0)  # a query with no selected key
    say(f"worst dq relative error {worst:.3g}, dkv relative error {w2:.3g}")


def test_attn_bwd_accumulates(dev):
    """Two calls into one dkv equal twice one call (to rounding); dq is
    written, not accumulated."""
    T, S, k = 64, 2000, 128
    spec, q, kv, idx, d_out, dq, dkv = run(dev, T, S, k, seed=43, min_valid=1)
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    out = B.dsa_sparse_attn(q, kv, idx, spec.scale, Dv=spec.Dv, lse_out=lse)
    dq2, dkv2 = B.dsa_sparse_attn_bwd(q, kv, idx, spec.scale, out, lse, d_out, spec.Dv, dkv=dkv.clone())
    torch.cuda.synchronize()
    assert torch.equal(dq2, dq)
    assert torch.allclose(dkv2, 2 * dkv, rtol=1e-5, atol=1e-6)
