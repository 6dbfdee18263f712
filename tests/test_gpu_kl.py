"""KL alignment of the indexer (dense warm-up) on the GPU through the C ABI,
against the fp64 oracle (oracle.dsa.indexer_kl) on the same inputs: fp32
index vectors and W, bf16 MLA-shaped attention operands.

Tolerance, from the arithmetic: the GPU runs in fp32 (index scores: 128-term
fp32 dot products; the target: bf16 x bf16 products summed in fp32, exp2f;
the gradient sums: fp32 over up to L terms), so gradients carry a few 1e-6
of relative error (bound: 1e-3 normwise).  A query's loss is the difference
of two sums of p log p and p log q whose terms are about log(t + 1) in size
(the distributions spread over t + 1 keys), so its error scales with that
and not with the loss: the bound is 1e-5 (1 + log(t + 1)) + 1e-4 |loss|.  A ReLU decision
taken differently on the two sides (a score within fp32 rounding of 0) moves
one entry of G by |q - p| ~ 1/t, far inside the normwise bound."""
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


def rel(g, o):
    g = np.asarray(g, np.float64)
    o = np.asarray(o, np.float64)
    return float(np.linalg.norm(g - o) / max(np.linalg.norm(o), 1e-300))


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
    r = [rel(to_np(dqi), o_dqi), rel(to_np(dki), o_dki), rel(to_np(dw), o_dw)]
    say(f"total loss {g.sum():.6g} (oracle {o_loss:.6g}); gradient relative errors {r}")
    assert max(r) <= 1e-3
