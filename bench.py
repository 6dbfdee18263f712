"""Throughput of the DSA forward path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one dsa_forward call over the whole synthetic workload (fold,
indexer scores, top-k selection and sparse MQA attention), inputs resident in
HBM.  The headline is the 131072-token causal prefill with k = 2048 and
MLA-shaped attention (128 heads, key 576, value 512); the 64-sequence batched
decode step is timed after it.  Prints one JSON line.

--workload prefill_L1048576_mla times the 2^20-token prefill instead, as
chunks of --chunk queries over the growing key prefix (a step is all the
chunks), and a 64-sequence decode over caches of 2^19 .. 2^20 keys.

The dominant kernel's duration is measured live with HIP events on the stream
the kernel runs on; its roofline uses algorithmic FLOPs (or bytes) only.  The
CPU baseline times the fp64 oracle on a bounded random sample of query rows of
the same workload, on this host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0      # MI355X dense fp8 MFMA
PEAK_HBM_GBPS = 8000.0        # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def attn_flops(L, k, H, Dk, Dv):
    pairs = sum(min(k, t + 1) for t in range(min(L, k))) + max(0, L - k) * k
    return 2.0 * H * (Dk + Dv) * pairs, pairs


def indexer_flops(L):
    return 2.0 * 128 * L * (L + 1) / 2


def kernel_source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "sparse_attention_long_indexer_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, sha):
    """HBM bytes per launch from the committed rocprofv3 counter runs, valid
    only while the kernel source is unchanged."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    e = d.get(kernel)
    if not e or e.get("source_sha") != sha:
        return None
    return e.get("bytes_per_launch")


def cpu_baseline(spec, x, budget_s=15.0, max_rows=4096, seed=0):
    """Time the fp64 oracle on query rows drawn uniformly from the workload
    until about `budget_s` seconds of row work have run; the per-row mean
    (plus the one-off setup) estimates the whole prefill's CPU time."""
    import numpy as np
    import torch

    import oracle.dsa as od

    def np_(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    class Rows:
        def __init__(self, t):
            self.t = t

        def __getitem__(self, i):
            return np_(self.t[i])

    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    rng = np.random.default_rng(seed)
    sample = rng.integers(0, spec.L, max_rows)
    t0 = time.perf_counter()
    orc = od.PrefillOracle(np_(x["q_idx"]), np_(x["q_scale"]), np_(x["k_idx"]), np_(x["k_scale"]), np_(x["w"]),
                           Rows(x["q"]), np_(x["kv"]), None if x["v"] is None else np_(x["v"]), spec.topk,
                           spec.scale, spec.Dv)
    t_setup = time.perf_counter() - t0
    t1 = time.perf_counter()
    rows = 0
    for t in sample:
        orc.row(int(t))
        rows += 1
        if time.perf_counter() - t1 >= budget_s:
            break
    t_rows = time.perf_counter() - t1
    per_row = t_rows / rows
    total = t_setup + per_row * spec.L
    return {"value": round(spec.L / total, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{rows} query rows drawn uniformly from the {spec.L}-token prefill "
                      f"(oracle setup {t_setup:.1f} s + {t_rows:.1f} s for the rows; the whole prefill "
                      f"extrapolated as setup + L x row mean)",
            "seconds": round(t_setup + t_rows, 2)}


def profile_attention(spec, x, reps):
    """Launch sequence for the rocprofv3 counter runs: one known-size copy
    (2 GiB read + 2 GiB written, the scale for FETCH_SIZE / WRITE_SIZE) and
    `reps` sparse-attention launches of the prefill workload."""
    import torch

    from sparse_attention_long_indexer_amd import binding as B

    dev = x["q"].device
    L, k = spec.L, spec.topk
    out = torch.empty((L, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((L, k), dtype=torch.int32, device=dev)
    fa = B.forward_args(x, k, spec.scale, spec.Dv)
    ws = torch.empty(max(B.dsa_forward_workspace_size(fa), 256), dtype=torch.uint8, device=dev)
    B.dsa_forward(fa, out, idx_out=idx, ws=ws)
    del ws
    n = 1 << 31
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    for _ in range(reps):
        B.dsa_sparse_attn(x["q"], x["kv"], idx, spec.scale, v=x["v"], Dv=spec.Dv, out=out)
    torch.cuda.synchronize()
    log(f"profiled: 1 copy of {n} bytes, {reps} attention launches")


def decode_step_stats(B, gen, torch, dev, ds, lengths=None, reps=20):
    """Time whole decode steps (fold, scores, top-k, attention) with HIP
    events on the stream the library launches on."""
    xd = gen.make_decode(ds, seed=0, device=dev, lengths=lengths)
    dout = torch.empty((ds.B, ds.H, ds.Dv), dtype=torch.bfloat16, device=dev)
    didx = torch.empty((ds.B, ds.topk), dtype=torch.int32, device=dev)
    da = B.forward_args(xd, ds.topk, ds.scale, ds.Dv, mode=B.DSA_MODE_DECODE, max_len=int(xd["lengths"].max()))
    dws = torch.empty(max(B.dsa_forward_workspace_size(da), 256), dtype=torch.uint8, device=dev)
    for _ in range(3):
        B.dsa_forward(da, dout, idx_out=didx, ws=dws)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(st)
    for _ in range(reps):
        B.dsa_forward(da, dout, idx_out=didx, ws=dws)
    ev1.record(st)
    torch.cuda.synchronize()
    dms = ev0.elapsed_time(ev1) / reps
    n = xd["lengths"]
    byts = float(n.sum()) * 132 + float(torch.clamp(n, max=ds.topk).sum()) * ds.Dk * 2 \
        + ds.B * ds.H * (ds.Dk + ds.Dv) * 2 + 2 * ds.B * ds.topk * 4
    del xd, dout, didx, dws
    return {"workload": ds.name, "queries_per_s": round(ds.B / (dms * 1e-3), 1),
            "ms_per_step": round(dms, 4), "keys": int(n.sum()), "algorithmic_bytes": byts,
            "roofline": {"bound": "hbm", "achieved": round(byts / (dms * 1e-3) / 1e9, 1),
                         "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                         "frac": round(byts / (dms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4),
                         "note": "warm caches; whole decode step"}}


def backward_stats(B, torch, spec, x, idx, out, pairs, reps=3):
    """Time dsa_sparse_attn_bwd over the forward's selection with HIP events
    on the launch stream; algorithmic FLOPs per selected pair: S and dP
    recomputed, dq, dk and dv, 2 H (3 Dk + 2 Dv)."""
    from sparse_attention_long_indexer_amd import inputs as gen
    L = x["q"].shape[0]
    dev = x["q"].device
    lse = torch.empty((L, spec.H), dtype=torch.float32, device=dev)
    B.dsa_sparse_attn(x["q"], x["kv"], idx, spec.scale, Dv=spec.Dv, out=out, lse_out=lse)
    d_out = gen.make_grad((L, spec.H, spec.Dv), seed=5, device=dev)
    dq = torch.empty_like(x["q"])
    dkv = torch.zeros((x["kv"].shape[0], spec.Dk), dtype=torch.float32, device=dev)
    B.dsa_sparse_attn_bwd(x["q"], x["kv"], idx, spec.scale, out, lse, d_out, spec.Dv, dq=dq, dkv=dkv)
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(st)
    for _ in range(reps):
        B.dsa_sparse_attn_bwd(x["q"], x["kv"], idx, spec.scale, out, lse, d_out, spec.Dv, dq=dq, dkv=dkv)
    ev1.record(st)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    flops = 2.0 * spec.H * (3 * spec.Dk + 2 * spec.Dv) * pairs
    achieved = flops / (ms * 1e-3) / 1e12
    log(f"backward {ms:.2f} ms = {achieved:.1f} TFLOP/s")
    del d_out, dq, dkv, lse
    return {"ms": round(ms, 3), "selected_pairs": pairs, "algorithmic_flops": flops,
            "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}}


def bench_kl(args, B, gen, torch, dev):
    """The indexer's KL alignment step (dense warm-up) on an L-token
    MLA-shaped prefill with fp32 index vectors: HIP events around whole
    dsa_indexer_kl calls on the launch stream."""
    L = args.kl
    spec = gen.PREFILL_32K.with_(name=f"kl_L{L}", L=L, fp8=False)
    log("KL alignment, L =", L)
    x = gen.make_prefill(spec, seed=0, device=dev)
    B.dsa_indexer_kl(x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], spec.scale)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(args.warmup):
        B.dsa_indexer_kl(x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], spec.scale)
    ev0.record(st)
    for _ in range(args.steps):
        loss = B.dsa_indexer_kl(x["q_idx"], x["k_idx"], x["w"], x["q"], x["kv"], spec.scale)[0]
    ev1.record(st)
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / args.steps
    pairs = L * (L + 1) // 2
    flops_target = 2 * 2.0 * spec.H * spec.Dk * pairs     # two passes of q . k over the heads
    flops = flops_target + 3 * 2.0 * 128 * pairs         # index scores, G k, G^T qf
    achieved = flops / (ms * 1e-3) / 1e12
    log(f"KL step {ms:.2f} ms = {achieved:.1f} TFLOP/s")
    print(json.dumps({
        "metric": "indexer KL alignment step (loss + gradients), causal L-token prefill",
        "value": round(L / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 3), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "dtype_detail": "attention target bf16 MFMA; indexer and gradients fp32",
        "data": "synthetic", "config": {"workload": spec.name, "L": L, "heads": spec.H, "dk": spec.Dk},
        "total_loss": float(loss.sum()),
        "roofline": {"bound": "mfma", "kernel": "kl_target_kernel<576>", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "algorithmic_flops": flops, "note": "whole step over its dominant FLOPs"}}), flush=True)


def bench_long(args, B, gen, torch, dev):
    """The 2^20-token prefill as chunks of C queries (each chunk attends over
    the keys of every earlier chunk and its own), then a 64-sequence decode
    step over caches of 2^19 .. 2^20 keys.  All queries, keys and the latent
    KV of the whole sequence are resident; one output buffer of C rows is
    rewritten by every chunk (the 2^20-row output and the queries do not fit
    in HBM together)."""
    spec = gen.PREFILL_1M
    L, k, C = spec.L, spec.topk, args.chunk
    if L % C:
        raise SystemExit("--chunk must divide 2^20")
    log("workload", spec.name, f"generating inputs (chunks of {C})")
    x = gen.make_prefill_chunk(spec, 0, seed=0, device=dev)
    out = torch.empty((C, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((L // C, C, k), dtype=torch.int32, device=dev)
    fas = []
    for c in range(L // C):
        y = dict(x)
        for key in ("q_idx", "q_scale", "q"):
            y[key] = x[key][c * C:(c + 1) * C]
        for key in ("k_idx", "k_scale", "kv"):
            y[key] = x[key][:(c + 1) * C]
        fas.append(B.forward_args(y, k, spec.scale, spec.Dv, q_offset=c * C))
    ws = torch.empty(max(B.dsa_forward_workspace_size(fa) for fa in fas), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        for c, fa in enumerate(fas):
            B.dsa_forward(fa, out, idx_out=idx[c], ws=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    log(f"prefill {dt * 1e3:.1f} ms/step, {L / dt:.4g} tokens/s")

    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fas) + 1)]
    evs[0].record(st)
    for c, fa in enumerate(fas):
        B.dsa_forward(fa, out, idx_out=idx[c], ws=ws)
        evs[c + 1].record(st)
    torch.cuda.synchronize()
    chunk_ms = [round(evs[c].elapsed_time(evs[c + 1]), 2) for c in range(len(fas))]
    # attention of the last chunk alone: C queries over the whole 2^20 keys
    qc = x["q"][L - C:]
    B.dsa_sparse_attn(qc, x["kv"], idx[-1], spec.scale, Dv=spec.Dv, out=out)
    reps = 3
    evs[0].record(st)
    for _ in range(reps):
        B.dsa_sparse_attn(qc, x["kv"], idx[-1], spec.scale, Dv=spec.Dv, out=out)
    evs[1].record(st)
    torch.cuda.synchronize()
    attn_ms = evs[0].elapsed_time(evs[1]) / reps
    flops = 2.0 * spec.H * (spec.Dk + spec.Dv) * C * k
    achieved = flops / (attn_ms * 1e-3) / 1e12
    log(f"chunks {chunk_ms} ms; last-chunk attention {attn_ms:.2f} ms = {achieved:.1f} TFLOP/s")
    result = {
        "metric": "DSA prefill tokens/s at L=1M (query chunks over the growing key prefix), k=2048",
        "value": round(L / dt, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "dtype_detail": "indexer e4m3 x e4m3 -> fp32 MFMA; attention bf16 -> fp32 MFMA",
        "data": "synthetic",
        "config": {"workload": spec.name, "L": L, "chunk": C, "topk": k, "heads": spec.H, "dk": spec.Dk,
                   "dv": spec.Dv, "batch": 1, "index_dim": 128},
        "chunk_ms": chunk_ms,
        "roofline": {"bound": "mfma", "kernel": "attn_mla_kernel", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": None, "ms_per_launch": round(attn_ms, 3), "algorithmic_flops_per_launch": flops,
                     "note": "last chunk: the chunk's queries over all 2^20 keys"},
    }
    del out, ws
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(spec, x, budget_s=args.cpu_seconds)
    del x, idx, fas
    torch.cuda.empty_cache()
    if not args.no_decode:
        ds = gen.DECODE_64.with_(name="decode_B64_ctx512k_1m", wid=8, n_min=1 << 19, n_max=1 << 20)
        log("decode: generating inputs")
        result["decode"] = decode_step_stats(B, gen, torch, dev, ds)
        log(f"decode {result['decode']['ms_per_step']:.3f} ms/step")
    print(json.dumps(result), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="prefill_L131072_mla")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="row-time budget of the CPU baseline")
    ap.add_argument("--chunk", type=int, default=131072, help="queries per chunk of the 2^20-token prefill")
    ap.add_argument("--dynamic-theta", type=float, default=None,
                    help="per-query k: keep the keys scoring above this (within [--dynamic-kmin, k])")
    ap.add_argument("--dynamic-kmin", type=int, default=0)
    ap.add_argument("--kl", type=int, default=0, metavar="L",
                    help="time only the indexer KL alignment step (loss and gradients) on an L-token MLA prefill")
    ap.add_argument("--backward", action="store_true",
                    help="also time the sparse attention backward (dq, dkv) over the prefill's selection")
    ap.add_argument("--profile-attn", type=int, default=0, metavar="N",
                    help="only run the counter-profile sequence (a 2 GiB copy, then N attention launches)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(a prefill would shard by query rows, a decode batch by sequence).", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_attention_long_indexer_amd import binding as B
    from sparse_attention_long_indexer_amd import inputs as gen

    B.lib()
    dev = torch.device("cuda:0")
    if args.kl:
        bench_kl(args, B, gen, torch, dev)
        return
    if args.workload == gen.PREFILL_1M.name:
        bench_long(args, B, gen, torch, dev)
        return
    spec = gen.WORKLOADS[args.workload]
    log("workload", spec.name, "generating inputs")
    x = gen.make_prefill(spec, seed=0, device=dev)
    if args.profile_attn:
        profile_attention(spec, x, args.profile_attn)
        return
    L, k = spec.L, spec.topk
    out = torch.empty((L, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((L, k), dtype=torch.int32, device=dev)
    fa = B.forward_args(x, k, spec.scale, spec.Dv, dyn_theta=args.dynamic_theta, dyn_k_min=args.dynamic_kmin)
    ws = torch.empty(max(B.dsa_forward_workspace_size(fa), 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        B.dsa_forward(fa, out, idx_out=idx, ws=ws)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    tok_s = L / dt
    log(f"prefill {dt * 1e3:.2f} ms/step, {tok_s:.4g} tokens/s")

    # dominant kernel (sparse attention) timed alone with HIP events on the
    # stream it is launched on (torch's current stream, passed to the library)
    st = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = max(2, args.steps)
    B.dsa_sparse_attn(x["q"], x["kv"], idx, spec.scale, v=x["v"], Dv=spec.Dv, out=out)
    ev0.record(st)
    for _ in range(reps):
        B.dsa_sparse_attn(x["q"], x["kv"], idx, spec.scale, v=x["v"], Dv=spec.Dv, out=out)
    ev1.record(st)
    torch.cuda.synchronize()
    attn_ms = ev0.elapsed_time(ev1) / reps
    flops, pairs = attn_flops(L, k, spec.H, spec.Dk, spec.Dv)
    if args.dynamic_theta is not None:  # the pairs the per-query budgets kept
        pairs = int((idx >= 0).sum())
        flops = 2.0 * spec.H * (spec.Dk + spec.Dv) * pairs
    achieved = flops / (attn_ms * 1e-3) / 1e12
    sha = kernel_source_sha(["attn.hip", "common.h", "kernels.h"])
    traffic = load_traffic("attn_mla_kernel", sha)
    roof = {"bound": "mfma", "kernel": "attn_mla_kernel", "achieved": round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic, "ms_per_launch": round(attn_ms, 3),
            "algorithmic_flops_per_launch": flops, "selected_pairs": pairs}
    idx_ms = dt * 1e3 - attn_ms
    ifl = indexer_flops(L)
    roof_idx = {"bound": "mfma", "stage": "fold + indexer scores + top-k (forward minus attention)",
                "ms": round(idx_ms, 3), "achieved": round(ifl / (idx_ms * 1e-3) / 1e12, 2),
                "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ifl / (idx_ms * 1e-3) / 1e12 / PEAK_FP8_TFLOPS, 4)}
    log(f"attention {attn_ms:.2f} ms/launch = {achieved:.1f} TFLOP/s; indexer+select {idx_ms:.2f} ms")

    result = {
        "metric": "DSA prefill tokens/s at L=128K, k=2048",
        "value": round(tok_s, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(dt * 1e3, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "dtype_detail": "indexer e4m3 x e4m3 -> fp32 MFMA; attention bf16 -> fp32 MFMA",
        "data": "synthetic",
        "config": {"workload": spec.name, "L": L, "topk": k, "heads": spec.H, "dk": spec.Dk, "dv": spec.Dv,
                   "batch": 1, "index_dim": 128},
        "roofline": roof, "roofline_indexer": roof_idx,
    }
    if args.dynamic_theta is not None:
        result["metric"] = "DSA prefill tokens/s at L=128K, dynamic k (theta, k_min .. 2048)"
        result["config"]["dynamic_k"] = {"theta": args.dynamic_theta, "k_min": args.dynamic_kmin,
                                         "mean_kept": round(pairs / L, 2)}
    if args.backward:
        result["backward"] = backward_stats(B, torch, spec, x, idx, out, pairs, reps=max(2, args.steps))
    del out, idx, ws

    if not args.no_decode:
        log("decode: generating inputs")
        result["decode"] = decode_step_stats(B, gen, torch, dev, gen.DECODE_64)
        log(f"decode {result['decode']['ms_per_step']:.3f} ms/step")

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(spec, x, budget_s=args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
