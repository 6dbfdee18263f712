"""Dynamic k on the GPU through the C ABI: dsa_topk_dynamic bit-exact against
the oracle's dynamic selection of the same fp32 scores (standalone radix,
candidate and long-row paths), and dsa_forward with a per-query budget
(fused equals materialised bit for bit, the materialised indices equal the
oracle's selection of the GPU's own scores, attention over the kept rows
against the oracle; decode against the fp64 oracle with the boundary
windows).  Rules in tests/parity.py."""
import sys

import numpy as np
import pytest
import torch

import oracle.dsa as od
import parity as P
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


# (theta, k_min): scores are ReLU(N(0,1)) on a grid, so 1 / 2 / 3 keep about
# 16% / 2.3% / 0.13% of a row; 1e9 keeps only k_min
DYN = [(2.0, 0), (1.0, 16), (3.0, 100), (0.0, 0), (1e9, 0), (1e9, 5)]


# radix path, short rows (n <= k), candidate path, candidate path past its bitmap
@pytest.mark.parametrize("T,S,k,levels", [(64, 5000, 64, 8), (48, 8192, 2048, 64), (30, 3000, 2048, 2),
                                           (16, 40000, 1000, 4096), (4, 300000, 4096, 64),
                                           (3, 600000, 2048, 64)])
def test_topk_dynamic_bit_exact(dev, T, S, k, levels):
    say("topk dynamic", T, S, k, levels)
    pos = torch.tensor(np.random.default_rng(T + S).integers(0, S, T), dtype=torch.int64)
    pos[0] = S - 1
    sc = gen.make_scores(T, S, seed=T * 37 + S, q_pos=pos, levels=levels)
    s64 = sc.numpy().astype(np.float64)
    scd, posd = sc.to(dev), pos.to(dev)
    for theta, k_min in DYN:
        k_min = min(k_min, k)
        cnt = torch.empty(T, dtype=torch.int32, device=dev)
        g = to_np(B.dsa_topk_dynamic(scd, k, k_min, theta, q_pos=posd, count_out=cnt))
        cnt = to_np(cnt)
        for t in range(T):
            n = int(pos[t]) + 1
            want = od.topk_row_dynamic(s64[t, :n], k, k_min, theta)
            assert np.array_equal(g[t], od.pad_idx(want, k)), (theta, k_min, t, n)
            assert cnt[t] == want.shape[0]
    # theta = -inf is the fixed top-k
    assert torch.equal(B.dsa_topk_dynamic(scd, k, 3, float("-inf"), q_pos=posd), B.dsa_topk(scd, k, q_pos=posd))


def forward(spec, x, dev, flags=0, theta=None, k_min=0):
    T = x["q"].shape[0]
    out = torch.empty((T, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((T, spec.topk), dtype=torch.int32, device=dev)
    B.dsa_forward(B.forward_args(x, spec.topk, spec.scale, spec.Dv, flags=flags, dyn_theta=theta, dyn_k_min=k_min),
                  out, idx_out=idx)
    torch.cuda.synchronize()
    return out, idx


# index scores here are ~N(0, 1/128) before ReLU: 0.2 keeps ~1.2% of a row
@pytest.mark.parametrize("theta,k_min", [(0.2, 32), (0.15, 0), (0.3, 300)])
def test_forward_dynamic_prefill(dev, theta, k_min):
    spec = gen.PREFILL_8K.with_(L=6000, topk=1024)
    say("forward dynamic", spec.L, theta, k_min)
    x = gen.make_prefill(spec, seed=31, device=dev)
    o_f, i_f = forward(spec, x, dev, B.DSA_FLAG_FUSED, theta, k_min)
    o_m, i_m = forward(spec, x, dev, B.DSA_FLAG_MATERIALIZE, theta, k_min)
    bad = (i_f != i_m).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, bad[:8].tolist()
    assert torch.equal(o_f.view(torch.int16), o_m.view(torch.int16))
    # the materialised path's indices are the oracle's dynamic selection of
    # the GPU's own fp32 scores
    qf, qs = B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"])
    sc = to_np(B.dsa_index_scores(qf, qs, x["k_idx"], x["k_scale"])).astype(np.float64)
    gi = i_m.cpu().numpy()
    counts = []
    for t in range(spec.L):
        want = od.topk_row_dynamic(sc[t, : t + 1], spec.topk, k_min, theta)
        assert np.array_equal(gi[t], od.pad_idx(want, spec.topk)), t
        counts.append(want.shape[0])
    say("kept per query: min", min(counts), "mean", float(np.mean(counts)), "max", max(counts))
    # attention over the kept rows
    orc = od.PrefillOracle(to_np(x["q_idx"]), to_np(x["q_scale"]), to_np(x["k_idx"]), to_np(x["k_scale"]),
                           to_np(x["w"]), RowsOf(x["q"]), to_np(x["kv"]), to_np(x["v"]), spec.topk, spec.scale,
                           spec.Dv)
    for t in (0, 1, 100, 2047, 2048, 4000, spec.L - 1):
        m = counts[t]
        if m == 0:
            assert torch.all(o_f[t] == 0)
            continue
        o, _ = orc.attend_row(t, gi[t][:m])
        P.check_attn(od.as_f64(to_np(o_f[t])), o)


def test_forward_dynamic_decode(dev):
    spec = gen.DECODE_64.with_(name="decode_B7_dyn", B=7, n_min=1, n_max=3000, topk=512)
    lengths = torch.tensor([1, 2, 511, 512, 513, 40000, 200000], dtype=torch.int64)
    theta, k_min = 0.25, 8
    x = gen.make_decode(spec, seed=32, device=dev, lengths=lengths)
    out = torch.empty((spec.B, spec.H, spec.Dv), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((spec.B, spec.topk), dtype=torch.int32, device=dev)
    args = B.forward_args(x, spec.topk, spec.scale, spec.Dv, mode=B.DSA_MODE_DECODE, max_len=int(lengths.max()),
                          dyn_theta=theta, dyn_k_min=k_min)
    B.dsa_forward(args, out, idx_out=idx)
    torch.cuda.synchronize()
    n = {k: to_np(v) for k, v in x.items() if k not in ("q", "kv", "lengths")}
    dec = od.DecodeOracle(n["q_idx"], n["q_scale"], n["k_idx"], n["k_scale"], n["w"], RowsOf(x["q"]),
                          RowsOf(x["kv"]), None, n["offsets"], spec.topk, spec.scale, spec.Dv)
    gi = idx.cpu().numpy()
    for b in range(spec.B):
        sc = dec.scores_seq(b)
        m_g = int((gi[b] >= 0).sum())
        # the budget may differ only by scores within the fp32-vs-fp64 margin of theta
        eps = 1e-3 * theta + 1e-6 * float(np.max(np.abs(sc)))
        lo = od.dynamic_k(sc, spec.topk, k_min, theta + eps)
        hi = od.dynamic_k(sc, spec.topk, k_min, theta - eps)
        say(f"seq {b}: n={sc.shape[0]} kept {m_g} (oracle {lo}..{hi})")
        assert lo <= m_g <= hi
        P.check_topk_row(gi[b], sc, od.topk_row(sc, m_g), m_g)
        if m_g:
            kv = to_np(x["kv"][int(n["offsets"][b]):int(n["offsets"][b + 1])])
            rows = od.as_f64(kv[gi[b][:m_g]])
            o, _ = od.attend(od.as_f64(to_np(x["q"][b])), rows, rows[:, : spec.Dv], spec.scale)
            P.check_attn(od.as_f64(to_np(out[b])), o)
