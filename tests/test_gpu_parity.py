"""GPU parity of every stage and of the whole forward pass against the fp64
oracle, through the C ABI.  Same seeded inputs on both sides; rules in
tests/parity.py."""
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
    B.lib()  # fails loudly when the library is missing
    return torch.device("cuda:0")


class RowsOf:
    """Row accessor over a device tensor (copies one row at a time)."""

    def __init__(self, t):
        self.t = t

    def __getitem__(self, i):
        return to_np(self.t[i])


def oracle_prefill(spec, x):
    return od.PrefillOracle(to_np(x["q_idx"]), to_np(x["q_scale"]), to_np(x["k_idx"]), to_np(x["k_scale"]),
                            to_np(x["w"]), RowsOf(x["q"]), to_np(x["kv"]), to_np(x["v"]), spec.topk,
                            spec.scale, spec.Dv)


def sample_rows(L, k, n=24, seed=0):
    rng = np.random.default_rng(seed)
    rows = {0, 1, 2, L - 1, L - 2, min(L - 1, k - 1), min(L - 1, k), min(L - 1, k + 1), min(L - 1, 2 * k)}
    rows |= set(rng.integers(0, L, n).tolist())
    return sorted(r for r in rows if 0 <= r < L)


SMALL_H16 = gen.PREFILL_8K.with_(name="ragged_L777_h16", L=777, topk=128)
SMALL_MLA = gen.PREFILL_32K.with_(name="ragged_L1000_mla", L=1000, topk=256)
UNIT_MLA = gen.PREFILL_32K.with_(name="unit_L1500_mla", L=1500, topk=300, qkv_unit=True)


# ------------------------------------------------------------------ fold ---

# the tiled fold: 32-row tiles with a ragged last tile (fewer tiles than
# CUs), and 64-row tiles outnumbering the grid with a ragged last tile
FOLD_T32 = gen.PREFILL_8K.with_(name="fold_L8232", L=8232)
FOLD_T64 = gen.PREFILL_8K.with_(name="fold_L16424", L=16424)


@pytest.mark.parametrize("spec", [gen.TINY_F32, gen.PREFILL_8K, SMALL_MLA, FOLD_T32, FOLD_T64],
                         ids=lambda s: s.name)
def test_fold(dev, spec):
    say("fold", spec.name)
    x = gen.make_prefill(spec, seed=1, device=dev)
    qf, qs = B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"])
    torch.cuda.synchronize()
    orc = oracle_prefill(spec, x)
    if spec.fp8:
        nbad = P.check_fold_codes(to_np(qf), to_np(qs), orc.qf, orc.qf8, orc.qf_scale)
        say("fold codes differing at a rounding midpoint:", nbad)
    else:
        g = to_np(qf).astype(np.float64)
        assert np.array_equal(g, orc.qf.astype(np.float32).astype(np.float64))


# ---------------------------------------------------------------- scores ---

@pytest.mark.parametrize("spec", [gen.TINY_F32, SMALL_H16, gen.PREFILL_8K, gen.PREFILL_32K], ids=lambda s: s.name)
def test_index_scores(dev, spec):
    say("scores", spec.name)
    x = gen.make_prefill(spec, seed=2, device=dev)
    qf, qs = B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"])
    orc = oracle_prefill(spec, x)
    rows = sample_rows(spec.L, spec.topk, n=16)
    worst = 0.0
    for t in rows:
        g = B.dsa_index_scores(qf, qs, x["k_idx"], x["k_scale"], row_begin=t, row_end=t + 1)
        worst = max(worst, P.check_scores_row(to_np(g)[0], orc.scores_row(t), t))
    # a block of rows at once, with a padded leading dimension
    r0, r1 = max(0, spec.L - 70), spec.L
    blk = B.dsa_index_scores(qf, qs, x["k_idx"], x["k_scale"], row_begin=r0, row_end=r1, ld=spec.L + 5)
    blk = to_np(blk)
    for t in range(r0, r1, 7):
        P.check_scores_row(blk[t - r0, : spec.L], orc.scores_row(t), t)
    say("worst normwise row error", worst)


def test_index_scores_q_pos(dev):
    spec = SMALL_H16
    x = gen.make_prefill(spec, seed=3, device=dev)
    qf, qs = B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"])
    pos = torch.tensor(np.random.default_rng(1).integers(0, spec.L, spec.L), dtype=torch.int64, device=dev)
    g = to_np(B.dsa_index_scores(qf, qs, x["k_idx"], x["k_scale"], q_pos=pos))
    orc = oracle_prefill(spec, x)
    pn = pos.cpu().numpy()
    for t in range(0, spec.L, 37):
        p = int(pn[t])
        o = od.index_scores_row(orc.q_vals[t], orc.q_scale_of(t), orc.k_vals, orc.k_scale, p)
        P.check_scores_row(g[t], o, p)


# ------------------------------------------------------------------ top-k ---

# few long rows (T < 512, S >= 16384) take the candidate path: sampled
# threshold, filter, select among candidates, one-block fallback; levels=1
# leaves fewer positive scores than k, so every long row falls back
@pytest.mark.parametrize("T,S,k,levels", [(64, 100, 1, 64), (64, 5000, 64, 8), (48, 8192, 2048, 64),
                                           (40, 4000, 4096, 16), (8, 131072, 2048, 64), (30, 3000, 2048, 2),
                                           (16, 40000, 1000, 4096), (6, 50000, 2048, 1),
                                           (4, 300000, 4096, 64), (3, 20000, 2048, 2)])
def test_topk_bit_exact(dev, T, S, k, levels):
    say("topk", T, S, k, levels)
    pos = torch.tensor(np.random.default_rng(T + S).integers(0, S, T), dtype=torch.int64)
    pos[0] = S - 1
    sc = gen.make_scores(T, S, seed=T * 31 + S, q_pos=pos, levels=levels)
    g = B.dsa_topk(sc.to(dev), k, q_pos=pos.to(dev))
    cnt = torch.empty(T, dtype=torch.int32, device=dev)
    g2 = B.dsa_topk(sc.to(dev), k, q_pos=pos.to(dev), count_out=cnt)
    g, g2, cnt = to_np(g), to_np(g2), to_np(cnt)
    assert np.array_equal(g, g2)
    s64 = sc.numpy().astype(np.float64)
    for t in range(T):
        n = int(pos[t]) + 1
        want = od.pad_idx(od.topk_row(s64[t, :n], k), k)
        assert np.array_equal(g[t], want), (t, n)
        assert cnt[t] == min(k, n)


# -------------------------------------------------------------- attention ---

ATTN_CASES = [
    ("f32_h4_d64", gen.TINY_F32.with_(L=300), 64),
    ("bf16_h16_d128", gen.PREFILL_8K.with_(L=3000), 2048),
    ("bf16_h16_k4096", gen.PREFILL_8K.with_(L=5000), 4096),
    ("bf16_h16_k5", gen.PREFILL_8K.with_(L=300), 5),                 # one partial 16-key tile
    ("bf16_mla_k5", gen.PREFILL_32K.with_(L=300), 5),                 # one partial 32-key tile
    ("bf16_mla", gen.PREFILL_32K.with_(L=2500), 2048),
    ("bf16_mla_unit", gen.PREFILL_32K.with_(L=2500, qkv_unit=True), 700),
    ("bf16_mla_k4096", gen.PREFILL_32K.with_(L=5000), 4096),      # the largest k
]


@pytest.mark.parametrize("name,spec,k", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
def test_sparse_attn(dev, name, spec, k):
    say("attn", name)
    x = gen.make_prefill(spec, seed=4, device=dev)
    T = 40
    q = x["q"][:T].contiguous()
    idx = gen.make_selection(T, spec.L, k, seed=5, min_valid=1)
    idx[3] = -1                                   # a query with no valid entry
    idx[5, : min(k, 33)] = torch.arange(min(k, 33), dtype=torch.int32)  # ragged tail of one tile
    idx[5, min(k, 33):] = -1
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    out = B.dsa_sparse_attn(q, x["kv"], idx.to(dev), spec.scale, v=x["v"], Dv=spec.Dv, lse_out=lse)
    g, gl = to_np(out), to_np(lse)
    if g.dtype == np.uint16:
        g = od.as_f64(g)
    kv, vv = to_np(x["kv"]), to_np(x["v"])
    qn = to_np(q)
    worst = 0.0
    for t in range(T):
        sel = idx[t].numpy()
        sel = sel[sel >= 0]
        if sel.size == 0:
            assert np.all(g[t] == 0) and np.all(np.isneginf(gl[t]))
            continue
        kr = od.as_f64(kv[sel])
        vr = od.as_f64(vv[sel]) if vv is not None else kr[:, : spec.Dv]
        o, l = od.attend(od.as_f64(qn[t]), kr, vr, spec.scale)
        worst = max(worst, P.check_attn(g[t], o, f32=spec.attn_f32))
        assert np.allclose(gl[t], l, rtol=1e-5, atol=1e-5)
    say("worst", worst)


@pytest.mark.parametrize("T", [20, 300], ids=["split", "unsplit"])
def test_sparse_attn_mla_rescale_and_ragged(dev, T):
    """The MLA kernel when a later tile raises a head's running max by far
    more than 2^8 (key rows from position 1000 on scaled by 8, exact in
    bf16, so the accumulated output must be rescaled mid-row), with valid
    counts that end inside a tile, at a tile boundary and at 0, both with the
    key splits of few queries (T = 20) and without them (T = 300); sampled
    queries and their log-sum-exp against the oracle."""
    spec = gen.PREFILL_32K.with_(L=2000)
    x = gen.make_prefill(spec, seed=8, device=dev)
    kv = x["kv"].clone()
    kv[1000:] *= 8
    q = x["q"][:T].contiguous()
    idx = gen.make_selection(T, spec.L, 2048, seed=9, min_valid=1)
    counts = {0: 2000, 1: 1, 2: 31, 3: 32, 4: 33, 5: 0, 6: 1023, 7: 1999}
    for t, m in counts.items():
        idx[t] = -1
        if m:
            idx[t, :m] = torch.arange(2000 - m, 2000, dtype=torch.int32) if t == 2 else torch.arange(m, dtype=torch.int32)
    lse = torch.empty((T, spec.H), dtype=torch.float32, device=dev)
    out = B.dsa_sparse_attn(q, kv, idx.to(dev), spec.scale, Dv=spec.Dv, lse_out=lse)
    g, gl = od.as_f64(to_np(out)), to_np(lse)
    kvn, qn, gi = to_np(kv), to_np(q), idx.numpy()
    rows = list(counts) + list(range(8, T, max(1, T // 12)))
    worst = 0.0
    for t in rows:
        sel = gi[t][gi[t] >= 0]
        if sel.size == 0:
            assert np.all(g[t] == 0) and np.all(np.isneginf(gl[t])), t
            continue
        kr = od.as_f64(kvn[sel])
        o, l = od.attend(od.as_f64(qn[t]), kr, kr[:, : spec.Dv], spec.scale)
        worst = max(worst, P.check_attn(g[t], o))
        assert np.allclose(gl[t], l, rtol=1e-5, atol=1e-4), t
    say("rows", len(rows), "worst", worst)


@pytest.mark.parametrize("L,k", [(600, 256), (5000, 4096)], ids=["k256", "k4096"])
def test_sparse_attn_separate_v_view(dev, L, k):
    """The latent-row reading (V = first Dv entries of the KV row, taken by
    the two-group MLA kernel) and the same columns passed as an explicit V
    with its own leading dimension (the separate-V kernel) both match the
    oracle, and agree with each other to one bf16 rounding: the two kernels
    accumulate in different orders, so their fp32 results differ far below
    a bf16 unit in the last place (2^-7 relative)."""
    spec = gen.PREFILL_32K.with_(L=L)
    x = gen.make_prefill(spec, seed=6, device=dev)
    idx = gen.make_selection(16, spec.L, k, seed=7, min_valid=1).to(dev)
    q = x["q"][:16].contiguous()
    a = B.dsa_sparse_attn(q, x["kv"], idx, spec.scale, v=None, Dv=512)
    b = B.dsa_sparse_attn(q, x["kv"], idx, spec.scale, v=x["kv"][:, :512], Dv=512)
    ga, gb = od.as_f64(to_np(a)), od.as_f64(to_np(b))
    kv, qn, gi = to_np(x["kv"]), to_np(q), idx.cpu().numpy()
    for t in range(16):
        sel = gi[t][gi[t] >= 0]
        kr = od.as_f64(kv[sel])
        o, _ = od.attend(od.as_f64(qn[t]), kr, kr[:, :512], spec.scale)
        P.check_attn(ga[t], o)
        P.check_attn(gb[t], o)
    assert np.all(np.abs(ga - gb) <= 2.0 ** -7 * np.maximum(np.abs(ga), np.abs(gb)) + 1e-6)
    say("differing elements", int(np.sum(ga != gb)), "of", ga.size)


# ---------------------------------------------------------- whole forward ---

def run_forward(spec, x, dev, flags=0):
    out = torch.empty((spec.L, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((spec.L, spec.topk), dtype=torch.int32, device=dev)
    args = B.forward_args(x, spec.topk, spec.scale, spec.Dv, flags=flags)
    B.dsa_forward(args, out, idx_out=idx)
    torch.cuda.synchronize()
    return out, idx


FWD_CASES = [gen.TINY_F32, SMALL_H16, SMALL_MLA, UNIT_MLA, gen.PREFILL_8K, gen.PREFILL_32K, gen.PREFILL_128K]


@pytest.mark.parametrize("spec", FWD_CASES, ids=lambda s: s.name)
def test_forward_prefill(dev, spec):
    """dsa_forward against the oracle: every row of the short prefills, and
    sampled rows (the first ones, rows around k and 2k, the last ones and a
    seeded random draw) of the 8K, 32K and 131072-token ones.  Each sampled
    row's indices obey the window rule and its attention output is held to
    the oracle's; at the largest size the indexer's materialised score rows
    are checked against the oracle's as well."""
    say("forward prefill", spec.name)
    x = gen.make_prefill(spec, seed=8, device=dev)
    out, idx = run_forward(spec, x, dev)
    orc = oracle_prefill(spec, x)
    rows = list(range(spec.L)) if spec.L <= 1000 else sample_rows(spec.L, spec.topk, n=24)
    gi = idx.cpu().numpy()
    qf, qs = B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"])
    diffs = 0
    worst = 0.0
    nrm = 0.0
    for t in rows:
        sc = orc.scores_row(t)
        # zero tolerance: the kept set is the exact top-k of the GPU's own
        # fp32 scores (materialised for this row), under the same order
        gs = to_np(B.dsa_index_scores(qf, qs, x["k_idx"], x["k_scale"], row_begin=t, row_end=t + 1))[0]
        assert np.array_equal(gi[t], od.pad_idx(od.topk_row(gs[: t + 1].astype(np.float64), spec.topk), spec.topk)), t
        nrm = max(nrm, P.check_scores_row(gs, sc, t))
        g = to_np(out[t])
        g = od.as_f64(g) if g.dtype == np.uint16 else g.astype(np.float64)
        d, e = P.check_forward_row(gi[t], sc, od.topk_row(sc, spec.topk), spec.topk,
                                   lambda sel: orc.attend_row(t, sel), g, f32=spec.attn_f32)
        diffs += d
        worst = max(worst, e)
    # indices that differ from the oracle's fp64 selection all lie inside the
    # boundary window (checked per row above): longer rows hold more keys
    # within fp32 accumulation error of their m-th score
    say(f"rows={len(rows)} window-diffs={diffs} worst-attn={worst:.3g} worst score-row error={nrm:.3g}")


@pytest.mark.parametrize("flags", [0, B.DSA_FLAG_FUSED], ids=["default", "fused"])
def test_forward_k_at_least_L_is_dense(dev, flags):
    """With k >= L every query keeps all of its causal keys, so the sparse
    forward is dense causal attention (the write-up's sparse attention
    reduces to ordinary attention when nothing is dropped)."""
    spec = gen.PREFILL_32K.with_(name="dense_L300", L=300, topk=512)
    x = gen.make_prefill(spec, seed=13, device=dev)
    out, idx = run_forward(spec, x, dev, flags)
    gi = idx.cpu().numpy()
    for t in range(spec.L):
        assert np.array_equal(gi[t, : t + 1], np.arange(t + 1)) and np.all(gi[t, t + 1:] == -1), t
    kv = od.as_f64(to_np(x["kv"]))
    q = to_np(x["q"])
    for t in (0, 1, 17, 150, 299):
        o, _ = od.attend(od.as_f64(q[t]), kv[: t + 1], kv[: t + 1, : spec.Dv], spec.scale)
        P.check_attn(od.as_f64(to_np(out[t])), o)


def test_forward_single_token(dev):
    """L = 1: the only query attends to its own key with weight 1, so the
    output is its value row (bf16, exact)."""
    spec = gen.PREFILL_32K.with_(name="single", L=1, topk=1)
    x = gen.make_prefill(spec, seed=14, device=dev)
    out, idx = run_forward(spec, x, dev)
    assert idx.cpu().tolist() == [[0]]
    want = x["kv"][0, : spec.Dv].float().expand(spec.H, spec.Dv)
    assert torch.equal(out[0].float(), want)


def test_forward_empty(dev):
    """T = 0 is a no-op through the whole forward."""
    spec = gen.PREFILL_32K.with_(name="empty", L=0, topk=64)
    x = gen.make_prefill(spec, seed=15, device=dev)
    out = torch.empty((0, spec.H, spec.Dv), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((0, spec.topk), dtype=torch.int32, device=dev)
    B.dsa_forward(B.forward_args(x, spec.topk, spec.scale, spec.Dv), out, idx_out=idx)
    torch.cuda.synchronize()


def test_forward_deterministic(dev):
    spec = SMALL_MLA
    x = gen.make_prefill(spec, seed=9, device=dev)
    o1, i1 = run_forward(spec, x, dev)
    o2, i2 = run_forward(spec, x, dev)
    assert torch.equal(i1, i2) and torch.equal(o1.view(torch.int16), o2.view(torch.int16))


# ----------------------------------------------------------------- decode ---

def run_decode(spec, x, dev):
    out = torch.empty((spec.B, spec.H, spec.Dv), dtype=torch.bfloat16, device=dev)
    idx = torch.empty((spec.B, spec.topk), dtype=torch.int32, device=dev)
    args = B.forward_args(x, spec.topk, spec.scale, spec.Dv, mode=B.DSA_MODE_DECODE,
                          max_len=int(x["lengths"].max()))
    B.dsa_forward(args, out, idx_out=idx)
    torch.cuda.synchronize()
    return out, idx


DEC_SMALL = gen.DECODE_64.with_(name="decode_B7_small", B=7, n_min=1, n_max=3000, topk=512)
# 16 heads of 128 over shared key/value rows: the 16-head attention kernel
# with per-sequence row bases and key splits
DEC_H16 = DEC_SMALL.with_(name="decode_B7_h16", H=16, Dk=128, Dv=128)


@pytest.mark.parametrize("spec", [DEC_SMALL, DEC_H16, gen.DECODE_64], ids=["small", "h16", "B64_full"])
def test_forward_decode(dev, spec):
    """Every sequence of the batch against the oracle: indices under the
    window rule, attention over the kept set."""
    say("forward decode", spec.name)
    lengths = None
    if spec.B == 7:
        lengths = torch.tensor([1, 2, 511, 512, 513, 2999, 1000], dtype=torch.int64)
    x = gen.make_decode(spec, seed=10, device=dev, lengths=lengths)
    out, idx = run_decode(spec, x, dev)
    n = {k: to_np(v) for k, v in x.items() if k not in ("q", "kv")}
    dec = od.DecodeOracle(n["q_idx"], n["q_scale"], n["k_idx"], n["k_scale"], n["w"], RowsOf(x["q"]),
                          RowsOf(x["kv"]), None, n["offsets"], spec.topk, spec.scale, spec.Dv)
    gi = idx.cpu().numpy()
    off = n["offsets"]
    kv = x["kv"]
    qf, qs = B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"])
    diffs = 0
    worst = 0.0
    for b in range(spec.B):
        sc = dec.scores_seq(b)
        lo, hi = int(off[b]), int(off[b + 1])
        # zero tolerance against the GPU's own fp32 scores of this sequence
        gs = to_np(B.dsa_index_scores(qf[b:b + 1], qs[b:b + 1], x["k_idx"][lo:hi], x["k_scale"][lo:hi],
                                      q_pos=torch.tensor([hi - lo - 1], dtype=torch.int64, device=dev)))[0]
        assert np.array_equal(gi[b], od.pad_idx(od.topk_row(gs.astype(np.float64), spec.topk), spec.topk)), b

        def attend(sel, b=b, lo=lo):
            rows = od.as_f64(to_np(kv[lo + torch.as_tensor(np.asarray(sel, np.int64))]))
            return od.attend(od.as_f64(to_np(x["q"][b])), rows, rows[:, : spec.Dv], spec.scale)

        d, e = P.check_forward_row(gi[b], sc, od.topk_row(sc, spec.topk), spec.topk, attend,
                                   od.as_f64(to_np(out[b])))
        diffs += d
        worst = max(worst, e)
    say(f"decode sequences={spec.B} window diffs={diffs} worst-attn={worst:.3g}")


# ------------------------------------------------- fused indexer + select ---

def forward_idx(spec, x, dev, flags):
    idx = torch.empty((spec.L, spec.topk), dtype=torch.int32, device=dev)
    out = torch.empty((spec.L, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    B.dsa_forward(B.forward_args(x, spec.topk, spec.scale, spec.Dv, flags=flags), out, idx_out=idx)
    torch.cuda.synchronize()
    return idx, out


FUSED_CASES = [gen.PREFILL_8K.with_(L=5000, topk=700), gen.PREFILL_8K.with_(L=6001, topk=2048),
               gen.PREFILL_8K, gen.PREFILL_32K, gen.PREFILL_128K]


@pytest.mark.parametrize("spec", FUSED_CASES, ids=lambda s: f"L{s.L}_k{s.topk}")
def test_fused_select_equals_materialized(dev, spec):
    """The fused scores + select path returns exactly what materialised
    scores + the standalone radix select return (same fp32 scores)."""
    say("fused vs materialized", spec.L, spec.topk)
    x = gen.make_prefill(spec, seed=11, device=dev)
    i_f, o_f = forward_idx(spec, x, dev, B.DSA_FLAG_FUSED)
    i_m, o_m = forward_idx(spec, x, dev, B.DSA_FLAG_MATERIALIZE)
    bad = (i_f != i_m).any(dim=1).nonzero().flatten()
    assert bad.numel() == 0, bad[:10].tolist()
    assert torch.equal(o_f.view(torch.int16), o_m.view(torch.int16))
    if spec.L >= 131072:
        # full-size sampled rows against the oracle as well
        orc = oracle_prefill(spec, x)
        gi = i_f.cpu().numpy()
        for t in sample_rows(spec.L, spec.topk, n=6, seed=3):
            sc = orc.scores_row(t)
            P.check_topk_row(gi[t], sc, od.topk_row(sc, spec.topk), spec.topk)


def test_fused_forced_fallback(dev):
    spec = gen.PREFILL_8K.with_(L=6000, topk=1024)
    x = gen.make_prefill(spec, seed=12, device=dev)
    i_f, _ = forward_idx(spec, x, dev, B.DSA_FLAG_FUSED | B.DSA_FLAG_FORCE_FALLBACK)
    i_m, _ = forward_idx(spec, x, dev, B.DSA_FLAG_MATERIALIZE)
    assert torch.equal(i_f, i_m)
