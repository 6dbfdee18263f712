"""Poisoned workspaces and outputs: no kernel may read workspace memory it
did not write first, and every output element must be written.

Each call runs twice through the C ABI: once with its workspace zeroed and its
outputs filled with one byte pattern, once with the workspace filled with 0xFF
bytes (NaN as fp32, -1 as int32) and the outputs with another pattern.  The
results must be identical bit for bit.  Covered: the fused and materialised
prefill paths, the fp32 path, a prefill chunk, batched decode (candidate
top-k and split attention), the standalone candidate top-k, split attention
with its log-sum-exp, the attention backward (dq) and the indexer KL step."""
import sys

import numpy as np
import pytest
import torch

from sparse_attention_long_indexer_amd import binding as B
from sparse_attention_long_indexer_amd import inputs as gen

pytestmark = pytest.mark.gpu

PATTERNS = [(0x00, 0x5A), (0xFF, 0xA5)]   # (workspace byte, output byte)


def say(*a):
    print("[gpu-test]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.lib()
    return torch.device("cuda:0")


def fill(t, byte):
    t.view(torch.uint8).fill_(byte)
    return t


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def twice(run, outs, ws_bytes, dev):
    """run(ws, *outs) under both patterns; returns the two output lists."""
    res = []
    for wb, ob in PATTERNS:
        ws = fill(torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev), wb)
        o = [fill(torch.empty_like(t), ob) for t in outs]
        run(ws, *o)
        torch.cuda.synchronize()
        res.append(o)
    return res


def check_same(res, names):
    for a, b, n in zip(res[0], res[1], names):
        assert same(a, b), f"{n} depends on the prior contents of the workspace or output"


FWD = [
    ("fused_L6000_mla", gen.PREFILL_32K.with_(L=6000, topk=1024), B.DSA_FLAG_FUSED, 0),
    ("materialized_L6000_mla", gen.PREFILL_32K.with_(L=6000, topk=1024), B.DSA_FLAG_MATERIALIZE, 0),
    ("chunk_L6000_h16", gen.PREFILL_8K.with_(L=6000, topk=700), 0, 5000),
    ("tiny_f32", gen.TINY_F32.with_(L=300), 0, 0),
    ("dynamic_L5000_mla", gen.PREFILL_32K.with_(L=5000, topk=512), B.DSA_FLAG_DYNAMIC_K | B.DSA_FLAG_FUSED, 0),
]


@pytest.mark.parametrize("name,spec,flags,q0", FWD, ids=[c[0] for c in FWD])
def test_forward_prefill_poisoned(dev, name, spec, flags, q0):
    say("poison forward", name)
    x = gen.make_prefill_chunk(spec, q0, seed=31, device=dev)
    T = spec.L - q0
    fa = B.forward_args(x, spec.topk, spec.scale, spec.Dv, flags=flags, q_offset=q0)
    if flags & B.DSA_FLAG_DYNAMIC_K:
        fa.dyn_theta, fa.dyn_k_min = 0.3, 16
    wsb = B.dsa_forward_workspace_size(fa)
    out = torch.empty((T, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((T, spec.topk), dtype=torch.int32, device=dev)
    res = twice(lambda ws, o, i: B.dsa_forward(fa, o, idx_out=i, ws=ws), [out, idx], wsb, dev)
    check_same(res, ["out", "idx"])
    # the indices kept inside the workspace (idx_out NULL) give the same output
    res2 = twice(lambda ws, o: B.dsa_forward(fa, o, idx_out=None, ws=ws), [out], wsb, dev)
    check_same(res2, ["out (indices in the workspace)"])
    assert same(res2[0][0], res[0][0])


def test_forward_decode_poisoned(dev):
    spec = gen.DECODE_64.with_(name="decode_B16", B=16, n_min=16384, n_max=40000)
    x = gen.make_decode(spec, seed=32, device=dev)
    fa = B.forward_args(x, spec.topk, spec.scale, spec.Dv, mode=B.DSA_MODE_DECODE, max_len=int(x["lengths"].max()))
    wsb = B.dsa_forward_workspace_size(fa)
    out = torch.empty((spec.B, spec.H, spec.Dv), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((spec.B, spec.topk), dtype=torch.int32, device=dev)
    res = twice(lambda ws, o, i: B.dsa_forward(fa, o, idx_out=i, ws=ws), [out, idx], wsb, dev)
    check_same(res, ["out", "idx"])


def test_topk_candidates_poisoned(dev):
    T, S, k = 8, 131072, 2048
    sc = gen.make_scores(T, S, seed=33, q_pos=torch.full((T,), S - 1, dtype=torch.int64)).to(dev)
    wsb = B.lib().dsa_topk_workspace_size(T, S, k)
    assert wsb > 0, "the candidate path should take a workspace"
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    cnt = torch.empty(T, dtype=torch.int32, device=dev)
    res = twice(lambda ws, i, c: B.dsa_topk(sc, k, idx_out=i, count_out=c, ws=ws), [idx, cnt], wsb, dev)
    check_same(res, ["idx", "count"])


def test_sparse_attn_split_poisoned(dev):
    spec = gen.PREFILL_32K.with_(L=3000)
    x = gen.make_prefill(spec, seed=34, device=dev)
    T = 20
    q = x["q"][:T].contiguous()
    idx = gen.make_selection(T, spec.L, 2048, seed=35, min_valid=0).to(dev)
    wsb = B.lib().dsa_sparse_attn_workspace_size(T, spec.H, spec.Dv, 2048, B.DSA_BF16)
    assert wsb > 0, "few queries should split their keys"
    out = torch.empty((T, spec.H, spec.Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    res = twice(lambda ws, o, l: B.dsa_sparse_attn(q, x["kv"], idx, spec.scale, Dv=spec.Dv, out=o, lse_out=l, ws=ws),
                [out, lse], wsb, dev)
    check_same(res, ["out", "lse"])


def test_sparse_attn_bwd_poisoned(dev):
    spec = gen.PREFILL_32K.with_(L=2000)
    x = gen.make_prefill(spec, seed=36, device=dev)
    T, k = 40, 256
    q = x["q"][:T].contiguous()
    idx = gen.make_selection(T, spec.L, k, seed=37, min_valid=0).to(dev)
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    out = B.dsa_sparse_attn(q, x["kv"], idx, spec.scale, Dv=spec.Dv, lse_out=lse)
    d_out = gen.make_grad((T, spec.H, spec.Dv), seed=38, device=dev)
    wsb = B.lib().dsa_sparse_attn_bwd_workspace_size(T, spec.H, k)
    res = []
    for wb, ob in PATTERNS:
        ws = fill(torch.empty(wsb, dtype=torch.uint8, device=dev), wb)
        dq = fill(torch.empty_like(q), ob)
        dkv = torch.zeros((spec.L, spec.Dk), dtype=torch.float32, device=dev)
        B.dsa_sparse_attn_bwd(q, x["kv"], idx, spec.scale, out, lse, d_out, spec.Dv, dq=dq, dkv=dkv, ws=ws)
        torch.cuda.synchronize()
        res.append((dq, dkv))
    assert same(res[0][0], res[1][0]), "dq depends on prior memory contents"
    # dkv sums float atomics in no fixed order: equal to rounding
    a, b = res[0][1], res[1][1]
    assert torch.allclose(a, b, rtol=1e-5, atol=1e-7 * float(a.abs().max()))


def test_indexer_kl_poisoned(dev):
    spec = gen.PREFILL_32K.with_(name="kl_L600", L=600, fp8=False)
    x = gen.make_prefill(spec, seed=39, device=dev)
    L = spec.L
    wsb = B.lib().dsa_indexer_kl_workspace_size(L)
    res = []
    for wb, _ in PATTERNS:
        ws = fill(torch.empty(wsb, dtype=torch.uint8, device=dev), wb)
        r = B.dsa_indexer_kl(x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], spec.scale, ws=ws)
        torch.cuda.synchronize()
        res.append([t.clone() for t in r])
    for a, b, n in zip(res[0], res[1], ["loss", "dq_idx", "dk_idx", "dw"]):
        assert same(a, b), f"{n} depends on prior workspace contents"
