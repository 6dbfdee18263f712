"""KL alignment of the indexer (dense warm-up) on the GPU through the C ABI,
against the fp64 oracle (oracle.dsa.indexer_kl) on the same inputs: fp32
index vectors and W, bf16 MLA-shaped attention operands.

Tolerance, per element, from the arithmetic (error_budget below): the fold
rounds qf = q_idx W to fp32; an index score sums 128 fp32 products; the
indexer softmax and the attention target (bf16 x bf16 products summed in
fp32, then exp2f) carry those errors into q and p; G = (q - p) [u > 0], where
a score within its fp32 error of 0 may take either ReLU branch; the gradient
sums run in fp32 over up to L terms.  Each gradient element's bound is the
sum of the per-term errors along its row or column; the test asserts
|g - o| <= 2 x bound + 1e-30.  A query's loss is the difference of two sums
of p log p and p log q whose terms are about log(t + 1) in size (the
distributions spread over t + 1 keys), so its error scales with that and not
with the loss: the bound is 1e-5 (1 + log(t + 1)) + 1e-4 |loss|."""
import sys

import numpy as np
import pytest
import torch

import oracle.dsa as od
from helpers import to_np
from sparse_attention_long_indexer_amd import binding as B
from sparse_attention_long_indexer_amd import inputs as gen

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


class RowsOf:
    def __init__(self, t):
        self.t = t

    def __getitem__(self, i):
        return to_np(self.t[i])


EPS32 = 2.0 ** -24


def rel(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))


def error_budget(q_idx, k_idx, w, q, kv, scale, Dk):
    """Per-element bounds of (dq_idx, dk_idx, dw) from the exact fp64
    quantities and the GPU's fp32 roundings (see the module docstring)."""
    qi, ki, wd = od.as_f64(q_idx), od.as_f64(k_idx), od.as_f64(w)
    kr = od.as_f64(kv)[:, :Dk]
    L = qi.shape[0]
    qf = od.fold(qi, wd)
    e_qf = EPS32 * np.abs(qf)
    G = np.zeros((L, L))
    eG = np.zeros((L, L))
    for t in range(L):
        n = t + 1
        u = ki[:n] @ qf[t]
        eu = 130 * EPS32 * (np.abs(ki[:n]) @ np.abs(qf[t]))
        i_row = od.relu(u)
        e = np.exp(i_row - i_row.max())
        qs = e / e.sum()
        eq = qs * (eu + eu.max() + 1e-6 + n * EPS32)
        qa = od.as_f64(q[t])
        z = scale * (qa @ kr[:n].T)                                  # [H, n]
        ez = scale * (Dk + 32) * EPS32 * (np.abs(qa) @ np.abs(kr[:n]).T)
        ph = np.exp(z - z.max(axis=1, keepdims=True))
        ph /= ph.sum(axis=1, keepdims=True)
        p = ph.mean(axis=0)
        ep = np.mean(ph * (ez + ez.max(axis=1, keepdims=True) + 1e-6 + n * EPS32), axis=0) + 160 * EPS32 * p
        g = (qs - p) * (u > 0)
        eg = eq + ep
        amb = np.abs(u) <= eu                                         # either ReLU branch
        eg = np.where(amb, np.maximum(eg, np.abs(qs - p) + eq + ep), eg)
        G[t, :n] = g
        eG[t, :n] = eg
    absk = np.abs(ki)
    dqf = G @ ki
    e_dqf = eG @ absk + (L + 32) * EPS32 * (np.abs(G) @ absk)
    b_dq = e_dqf @ np.abs(wd).T + 160 * EPS32 * (np.abs(dqf) @ np.abs(wd).T)
    b_dk = eG.T @ np.abs(qf) + np.abs(G).T @ e_qf + (L + 32) * EPS32 * (np.abs(G).T @ np.abs(qf))
    b_dw = np.abs(qi).T @ e_dqf + (L + 64) * EPS32 * (np.abs(qi).T @ np.abs(dqf))
    return b_dq, b_dk, b_dw


def within(g, o, bound, what):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    err = np.abs(g - o)
    lim = 2.0 * bound + 1e-30
    ok = err <= lim
    assert np.all(ok), (what, int(np.sum(~ok)), float(np.max(err / lim)))
    return float(np.max(err / lim))


@pytest.mark.parametrize("L", [97, 600])
def test_indexer_kl(dev, L):
    spec = gen.PREFILL_32K.with_(name=f"kl_L{L}", L=L, fp8=False)
    x = gen.make_prefill(spec, seed=51, device=dev)
    say("indexer KL", L)
    loss, dqi, dki, dw = B.dsa_indexer_kl(x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], spec.scale)
    torch.cuda.synchronize()
    o_loss, o_losses, o_dqi, o_dki, o_dw = od.indexer_kl(to_np(x["q_idx"]), to_np(x["k_idx"]), to_np(x["w"]),
                                                         RowsOf(x["q"]), to_np(x["kv"]), spec.scale, spec.Dk)
    g = to_np(loss).astype(np.float64)
    err = np.abs(g - o_losses)
    tol = 1e-5 * (1 + np.log(np.arange(L) + 1.0)) + 1e-4 * np.abs(o_losses)
    assert np.all(err <= tol), float(np.max(err / tol))
    b_dq, b_dk, b_dw = error_budget(to_np(x["q_idx"]), to_np(x["k_idx"]), to_np(x["w"]), RowsOf(x["q"]),
                                    to_np(x["kv"]), spec.scale, spec.Dk)
    worst = [within(to_np(dqi), o_dqi, b_dq, "dq_idx"), within(to_np(dki), o_dki, b_dk, "dk_idx"),
             within(to_np(dw), o_dw, b_dw, "dw")]
    r = [rel(to_np(dqi), o_dqi), rel(to_np(dki), o_dki), rel(to_np(dw), o_dw)]
    say(f"total loss {g.sum():.6g} (oracle {o_loss:.6g}); gradient relative errors {r}; worst error / bound {worst}")
