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
the kernel runs on; its roofline uses algorithmic FLOPs (or bytes) only, and
is stated against both the published peak and the peak measured in the same
run by the probe library (an MFMA issue loop and a streaming HBM read).  GPU
clocks and power are read before the timed region, during (sampled while
about 5 s of further, untimed steps of the same workload run right after
it) and after.  The 8K and 32K prefills are timed as extra
lines; decode is timed warm (one cache set) and
cold (four cache sets in rotation, 24 GB, far past the 256 MB last-level
cache).  The CPU baseline times the fp64 oracle on a stratified sample of
query rows of the same workload with one single-threaded worker process per
available core, and extrapolates the whole prefill from a per-row cost model.
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


def source_tree_sha():
    """Hash of every kernel and library source (any change invalidates the
    committed per-kernel profile)."""
    d = os.path.join(ROOT, "sparse_attention_long_indexer_amd", "csrc")
    return kernel_source_sha(sorted(f for f in os.listdir(d) if f.endswith((".hip", ".h", ".cpp"))))


def load_kernel_breakdown(workload):
    """Per-kernel average durations of one workload from the committed
    rocprofv3 kernel trace (profiles/kernel_times.json), each with its
    algorithmic work and roofline fraction where one applies; None once any
    library source has changed since the trace was taken."""
    path = os.path.join(ROOT, "profiles", "kernel_times.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha") != source_tree_sha():
        return None
    w = d.get("workloads", {}).get(workload)
    if w is None:
        return None
    return {"source": "profiles/kernel_times.json (rocprofv3 kernel trace of this source tree)",
            "clocks_mhz": d.get("clocks_mhz"), "kernels": w}


def gpu_clocks():
    """Shader and memory clocks and power of GPU 0 as the system tools report
    them (amd-smi, else rocm-smi); the raw fields are kept as reported."""
    import subprocess
    cmds = [["amd-smi", "metric", "-g", "0", "-c", "-p", "--json"],
            ["rocm-smi", "-d", "0", "--showclocks", "--showpower", "--json"]]
    for cmd in cmds:
        try:
            r = subprocess.run(cmd, capture_output=True, text=True, timeout=30)
        except Exception:  # pragma: no cover - tool missing or hung
            continue
        if r.returncode != 0 or not r.stdout.strip():
            continue
        try:
            d = json.loads(r.stdout[r.stdout.index(r.stdout.lstrip()[0]):])
        except Exception:
            continue
        flat = {}

        def walk(v, key):
            if isinstance(v, dict):
                for k2, v2 in v.items():
                    walk(v2, f"{key}.{k2}" if key else str(k2))
            elif isinstance(v, list):
                for i, v2 in enumerate(v):
                    walk(v2, f"{key}[{i}]")
            else:
                low = key.lower()
                if any(w in low for w in ("sclk", "mclk", "gfx", "mem", "power", "socket", "clk")):
                    flat[key] = v
        walk(d, "")
        if flat:
            return {"tool": cmd[0], **clock_summary(flat)}
    return None


def clock_summary(flat):
    """Shader clocks (MHz, per XCD), memory clock (MHz) and socket power (W)
    picked out of the tool's flattened fields."""
    gfx, mem, power = [], None, None
    for k, v in flat.items():
        low = k.lower()
        if not isinstance(v, (int, float)):
            continue
        if "gfx_" in low and low.endswith("clk.value") and "min_clk" not in low and "max_clk" not in low:
            gfx.append(v)
        elif ("mem_0" in low or "mclk" in low) and low.endswith("clk.value") and "min" not in low and "max" not in low:
            mem = v
        elif "socket_power.value" in low:
            power = v
    return {"gfx_mhz": gfx, "mem_mhz": mem, "power_w": power}


class ClockSampler:
    """Reads the clocks once on a helper thread, `delay` seconds after it
    starts, while the GPU runs queued work (the caller queues enough work to
    outlast the delay and the tool's start-up).  The delay also keeps the
    read apart from an earlier one: a read within about a second of the
    previous one can return the same cached metrics."""

    def __init__(self, delay=1.5):
        import threading
        self.result = None
        self.delay = delay
        self.t = threading.Thread(target=self._run, daemon=True)

    def _run(self):
        time.sleep(self.delay)
        self.result = gpu_clocks()

    def start(self):
        self.t.start()
        return self

    def join(self):
        self.t.join(timeout=60)
        return self.result


def probe_peaks(torch, dev):
    """Achievable peaks measured with the probe library on this GPU: the FP8
    and bf16 MFMA issue rates (whole chip, 2 blocks of 4 waves per CU) and a
    streaming read of 4 GiB (16 times the last-level cache), each the best of
    a few launches timed with HIP events on the stream they run on."""
    import ctypes

    from sparse_attention_long_indexer_amd import build as b
    lib = ctypes.CDLL(b.PROBE_LIB)
    lib.dsa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    lib.dsa_probe_mfma_flops.restype = ctypes.c_double
    lib.dsa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    st = torch.cuda.current_stream()
    sp = ctypes.c_void_p(st.cuda_stream)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus
    sink = torch.empty(blocks * 256 * 4, dtype=torch.float32, device=dev)

    def timed(launch, reps=3):
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            if launch() != 0:
                raise RuntimeError("probe launch rejected")
            e1.record(st)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best

    out = {"method": "probe library: MFMA issue loops (8 independent accumulators per wave, 2 workgroups of "
                     "4 waves per CU) and a streaming read of 4 GiB (2 workgroups per CU, each a contiguous "
                     "slice, 16-byte non-temporal loads, 8 in flight per thread); best of 3 launches"}
    iters = 4096
    for kind, key in ((0, "fp8_tflops"), (1, "bf16_16x16x32_tflops"), (2, "bf16_32x32x16_tflops")):
        lib.dsa_probe_mfma(kind, 16, blocks, ctypes.c_void_p(sink.data_ptr()), sp)   # warm-up
        ms = timed(lambda: lib.dsa_probe_mfma(kind, iters, blocks, ctypes.c_void_p(sink.data_ptr()), sp))
        out[key] = round(lib.dsa_probe_mfma_flops(kind, iters, blocks) / (ms * 1e-3) / 1e12, 1)
    out["bf16_tflops"] = max(out["bf16_16x16x32_tflops"], out["bf16_32x32x16_tflops"])
    nbytes = 4 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.int32, device=dev)
    rblocks = 2 * cus
    rsink = torch.empty(rblocks * 256, dtype=torch.float32, device=dev)
    lib.dsa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rblocks, ctypes.c_void_p(rsink.data_ptr()), sp)
    ms = timed(lambda: lib.dsa_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, rblocks,
                                          ctypes.c_void_p(rsink.data_ptr()), sp))
    out["hbm_read_gbps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    del buf, rsink, sink
    torch.cuda.empty_cache()
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for ln in fh:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def stratified_rows(L, k, n, seed=0):
    """At least n query rows of an L-token prefill: every row below 64, the
    rows around k and 2k (where the selection stops taking every key), the
    last 64 rows, and a seeded uniform draw for the rest."""
    import numpy as np
    rows = set(range(min(L, 64)))
    for c in (k, 2 * k):
        rows |= set(range(max(0, c - 16), min(L, c + 16)))
    rows |= set(range(max(0, L - 64), L))
    rng = np.random.default_rng(seed)
    while len(rows) < min(n, L):
        rows |= set(rng.integers(0, L, n - len(rows)).tolist())
    return sorted(rows)


_W = {}   # per-worker state of the CPU-baseline pool


def _cpu_worker_init(data_dir, topk, scale, Dv):
    """Pool worker set-up: one BLAS thread, then the oracle of the whole
    prefill from memory-mapped host copies of the inputs."""
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        os.environ[v] = "1"
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        _W["limit"] = threadpool_limits(1)
    except Exception:  # pragma: no cover
        pass
    import oracle.dsa as od

    def ld(name):
        return np.load(os.path.join(data_dir, name + ".npy"), mmap_mode="r")

    rows = ld("rows")
    qrows = ld("q_rows")
    where = {int(t): i for i, t in enumerate(rows)}

    class Q:
        def __getitem__(self, t):
            return np.asarray(qrows[where[int(t)]])

    t0 = time.perf_counter()
    _W["orc"] = od.PrefillOracle(np.asarray(ld("q_idx")), np.asarray(ld("q_scale")), np.asarray(ld("k_idx")),
                                 np.asarray(ld("k_scale")), np.asarray(ld("w")), Q(), ld("kv"), None, topk, scale, Dv)
    _W["setup"] = time.perf_counter() - t0


def _cpu_worker_rows(rows):
    out = []
    for t in rows:
        t0 = time.perf_counter()
        _W["orc"].row(int(t))
        out.append((int(t), time.perf_counter() - t0))
    return out, _W.get("setup", 0.0)


def cpu_baseline_pool(spec, x, min_rows=4096, seed=0, timeout_s=600):
    """The fp64 oracle timed on this host's cores: N = the available cores
    (at most 16, the host share of one GPU) single-threaded worker processes
    (BLAS threads 1) run a stratified sample of >= min_rows query rows.  The
    whole prefill's time is extrapolated from a least-squares per-row cost
    model cost(t) = a + b (t + 1) + c m_t (scoring grows with the row's keys,
    attention with its kept keys m_t = min(k, t + 1)), summed over all L rows
    and divided over the N workers, plus the worker set-up."""
    import multiprocessing as mp
    import shutil
    import tempfile
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np
    import torch

    def np_(t):
        t = t.detach().cpu().contiguous()
        return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()

    ncores = len(os.sched_getaffinity(0))
    nworkers = max(1, min(ncores, 16))
    rows = stratified_rows(spec.L, spec.topk, min_rows, seed)
    tmp = tempfile.mkdtemp(prefix="dsa_cpu_baseline_")
    try:
        ridx = torch.tensor(rows, dtype=torch.int64, device=x["q"].device)
        np.save(os.path.join(tmp, "rows.npy"), np.asarray(rows, np.int64))
        np.save(os.path.join(tmp, "q_rows.npy"), np_(x["q"].index_select(0, ridx)))
        for name in ("q_idx", "q_scale", "k_idx", "k_scale", "w", "kv"):
            np.save(os.path.join(tmp, name + ".npy"), np_(x[name]))
        chunks = [rows[i::nworkers * 4] for i in range(nworkers * 4)]
        # fresh interpreters (spawn): the workers never touch the GPU; a
        # worker that dies fails the pool instead of hanging it
        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ProcessPoolExecutor(nworkers, mp_context=ctx, initializer=_cpu_worker_init,
                                 initargs=(tmp, spec.topk, spec.scale, spec.Dv)) as pool:
            res = list(pool.map(_cpu_worker_rows, chunks, timeout=timeout_s))
        wall = time.perf_counter() - t0
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    per = [r for part, _ in res for r in part]
    setup = max(s for _, s in res)
    t = np.array([p[0] for p in per], np.float64)
    sec = np.array([p[1] for p in per], np.float64)
    m = np.minimum(spec.topk, t + 1)
    A = np.stack([np.ones_like(t), t + 1, m], axis=1)
    coef, *_ = np.linalg.lstsq(A, sec, rcond=None)
    coef = np.maximum(coef, 0.0)
    L = spec.L
    allt = np.arange(L, dtype=np.float64)
    total_cpu = float(coef[0] * L + coef[1] * np.sum(allt + 1) + coef[2] * np.sum(np.minimum(spec.topk, allt + 1)))
    est_wall = setup + total_cpu / nworkers
    return {"value": round(L / est_wall, 3), "unit": "tokens/s", "cores": nworkers, "kind": "oracle",
            "sample": f"{len(rows)} stratified query rows of the {L}-token prefill (rows 0-63, rows around k and "
                      f"2k, the last 64, the rest uniform) on {nworkers} single-threaded worker processes; "
                      f"whole prefill extrapolated from the per-row cost model a + b (t+1) + c min(k, t+1) "
                      f"fitted to the sample (extrapolated)",
            "cpu_model": cpu_model(), "cores_available": ncores, "blas_threads_per_worker": 1,
            "sample_wall_s": round(wall, 2), "worker_setup_s": round(setup, 2),
            "row_cost_model_s": [float(c) for c in coef], "extrapolated_cpu_s": round(total_cpu, 1),
            "extrapolated_wall_s": round(est_wall, 1)}


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


def decode_bytes(n, ds):
    """Algorithmic HBM bytes of one decode step: every cached index key and
    its scale (132 B), the kept latent rows (Dk bf16 each), Q and O, and the
    indices written and read once."""
    import torch
    return float(n.sum()) * 132 + float(torch.clamp(n, max=ds.topk).sum()) * ds.Dk * 2 \
        + ds.B * ds.H * (ds.Dk + ds.Dv) * 2 + 2 * ds.B * ds.topk * 4


def decode_step_stats(B, gen, torch, dev, ds, lengths=None, reps=20, cold_copies=4):
    """Time whole decode steps (fold, scores, top-k, attention) with HIP
    events on the stream the library launches on.  Warm: one cache set,
    stepped `reps` times.  Cold: `cold_copies` independent cache sets of the
    same lengths (different contents and addresses, together far larger than
    the last-level cache), stepped in rotation, so every step reads its
    cache from HBM."""
    if lengths is None:
        lengths = gen.decode_lengths(ds, 0)
    sets = []
    for c in range(max(1, cold_copies)):
        xd = gen.make_decode(ds, seed=c, device=dev, lengths=lengths)
        dout = torch.empty((ds.B, ds.H, ds.Dv), dtype=torch.bfloat16, device=dev)
        didx = torch.empty((ds.B, ds.topk), dtype=torch.int32, device=dev)
        da = B.forward_args(xd, ds.topk, ds.scale, ds.Dv, mode=B.DSA_MODE_DECODE, max_len=int(lengths.max()))
        sets.append((xd, dout, didx, da))
    dws = torch.empty(max(max(B.dsa_forward_workspace_size(s[3]) for s in sets), 256), dtype=torch.uint8,
                      device=dev)
    for xd, dout, didx, da in sets:
        B.dsa_forward(da, dout, idx_out=didx, ws=dws)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()

    def run(order):
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(st)
        for i in order:
            xd, dout, didx, da = sets[i]
            B.dsa_forward(da, dout, idx_out=didx, ws=dws)
        ev1.record(st)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / len(order)

    warm_ms = run([0] * reps)
    cold_ms = run([i % len(sets) for i in range(max(reps, 4 * len(sets)))]) if len(sets) > 1 else None
    byts = decode_bytes(lengths, ds)

    def roof(ms, note):
        gbps = byts / (ms * 1e-3) / 1e9
        return {"bound": "hbm", "achieved": round(gbps, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": round(gbps / PEAK_HBM_GBPS, 4), "note": note}

    ms = cold_ms if cold_ms is not None else warm_ms
    res = {"workload": ds.name, "queries_per_s": round(ds.B / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "keys": int(lengths.sum()), "algorithmic_bytes": byts,
           "cache_bytes_per_set": float(lengths.sum()) * (132 + ds.Dk * 2),
           "roofline": roof(ms, f"cold: {len(sets)} cache sets in rotation" if cold_ms is not None
                            else "warm caches")}
    res["warm"] = {"ms_per_step": round(warm_ms, 4), "queries_per_s": round(ds.B / (warm_ms * 1e-3), 1),
                   "roofline": roof(warm_ms, "warm: one cache set stepped repeatedly")}
    del sets, dws
    torch.cuda.empty_cache()
    return res


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
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="row-time budget of the CPU baseline of the 2^20-token workload")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak probes")
    ap.add_argument("--no-extra-configs", action="store_true", help="skip the 8K and 32K prefill lines")
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
    peaks = None
    if not args.no_peaks:
        log("measured peaks (probe library)")
        peaks = probe_peaks(torch, dev)
        log(f"peaks: fp8 {peaks['fp8_tflops']} TF, bf16 {peaks['bf16_tflops']} TF, read {peaks['hbm_read_gbps']} GB/s")
    log("workload", spec.name, "generating inputs")
    x = gen.make_prefill(spec, seed=0, device=dev)
    if args.profile_attn:
        profile_attention(spec, x, args.profile_attn)
        return
    clocks = {"before": gpu_clocks()}
    line, idx, out = time_prefill(B, torch, dev, spec, x, args.steps, args.warmup, peaks,
                                  dyn_theta=args.dynamic_theta, dyn_k_min=args.dynamic_kmin, keep=True)
    clocks["during"] = line.pop("clocks_during", None)
    clocks["after"] = gpu_clocks()
    pairs = line["roofline"]["selected_pairs"]
    result = {
        "metric": "DSA prefill tokens/s at L=128K, k=2048",
        "value": line["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": line["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "dtype_detail": "indexer e4m3 x e4m3 -> fp32 MFMA; attention bf16 -> fp32 MFMA", "data": "synthetic",
        "config": {"workload": spec.name, "L": spec.L, "topk": spec.topk, "heads": spec.H, "dk": spec.Dk,
                   "dv": spec.Dv, "batch": 1, "index_dim": 128},
        "roofline": line["roofline"], "roofline_indexer": line["roofline_indexer"],
        "measured_peaks": peaks, "clocks": clocks,
    }
    if args.dynamic_theta is None:
        result["roofline_indexer"]["kernels"] = load_kernel_breakdown(spec.name)
    if args.dynamic_theta is not None:
        result["metric"] = "DSA prefill tokens/s at L=128K, dynamic k (theta, k_min .. 2048)"
        result["config"]["dynamic_k"] = {"theta": args.dynamic_theta, "k_min": args.dynamic_kmin,
                                         "mean_kept": round(pairs / spec.L, 2)}
    if args.backward:
        result["backward"] = backward_stats(B, torch, spec, x, idx, out, pairs, reps=max(2, args.steps))
    del out, idx
    torch.cuda.empty_cache()

    if not args.no_extra_configs and args.dynamic_theta is None and spec is gen.PREFILL_128K:
        result["other_prefills"] = {}
        for extra in (gen.PREFILL_8K, gen.PREFILL_32K):
            log("workload", extra.name, "generating inputs")
            xe = gen.make_prefill(extra, seed=0, device=dev)
            result["other_prefills"][extra.name] = time_prefill(B, torch, dev, extra, xe, max(args.steps, 5),
                                                                args.warmup, peaks)[0]
            del xe
            torch.cuda.empty_cache()

    if not args.no_decode:
        log("decode: generating inputs (warm: one cache set; cold: four in rotation)")
        result["decode"] = decode_step_stats(B, gen, torch, dev, gen.DECODE_64, cold_copies=4)
        if peaks:
            r = result["decode"]["roofline"]
            r["frac_measured_peak"] = round(r["achieved"] / peaks["hbm_read_gbps"], 4)
        result["decode"]["kernels"] = load_kernel_breakdown(gen.DECODE_64.name)
        log(f"decode cold {result['decode']['ms_per_step']:.3f} ms/step, "
            f"warm {result['decode']['warm']['ms_per_step']:.3f} ms/step")

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle, process pool)")
        result["cpu_baseline"] = cpu_baseline_pool(spec, x)
        log(f"cpu baseline {result['cpu_baseline']['value']} tokens/s on {result['cpu_baseline']['cores']} workers")
    print(json.dumps(result), flush=True)


def time_prefill(B, torch, dev, spec, x, steps, warmup, peaks, dyn_theta=None, dyn_k_min=0, keep=False):
    """Whole dsa_forward steps on one prefill workload (wall clock around
    `steps` steps between synchronisations), then the dominant kernel alone
    (sparse attention over the step's selection) and the fold alone, each
    timed with HIP events on the stream the library launches on.  The
    indexer stage is the step minus attention; its FLOPs are the causal
    pairs' 2 x 128 each."""
    L, k = spec.L, spec.topk
    out = torch.empty((L, spec.H, spec.Dv), dtype=x["q"].dtype, device=dev)
    idx = torch.empty((L, k), dtype=torch.int32, device=dev)
    fa = B.forward_args(x, k, spec.scale, spec.Dv, dyn_theta=dyn_theta, dyn_k_min=dyn_k_min)
    ws = torch.empty(max(B.dsa_forward_workspace_size(fa), 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def step():
        B.dsa_forward(fa, out, idx_out=idx, ws=ws)

    log(f"{spec.name}: warmup {warmup}")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    log(f"{spec.name}: timing {steps} steps")
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / steps
    clocks_during = None
    if keep:
        # the sampler reads the clocks 1.5 s after it starts (the tool itself
        # takes about a second); meanwhile ~5 s of further untimed steps of
        # the same workload keep the GPU busy (the launches may block once the
        # queue is full, so the sampler starts first)
        sampler = ClockSampler().start()
        for _ in range(max(1, int(math.ceil(5.0 / dt)))):
            step()
        torch.cuda.synchronize()
        clocks_during = sampler.join()
    log(f"{spec.name}: prefill {dt * 1e3:.2f} ms/step, {L / dt:.4g} tokens/s")
    del ws

    st = torch.cuda.current_stream()

    def events(fn, reps):
        fn()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ev0.record(st)
        for _ in range(reps):
            fn()
        ev1.record(st)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / reps

    reps = max(2, steps)
    attn_ms = events(lambda: B.dsa_sparse_attn(x["q"], x["kv"], idx, spec.scale, v=x["v"], Dv=spec.Dv, out=out),
                     reps)
    qf = torch.empty_like(x["q_idx"])
    qs = torch.empty(L, dtype=torch.float32, device=dev)
    fold_ms = events(lambda: B.dsa_fold_index_query(x["q_idx"], x["q_scale"], x["w"], qf, qs), reps)
    del qf, qs
    flops, pairs = attn_flops(L, k, spec.H, spec.Dk, spec.Dv)
    if dyn_theta is not None:  # the pairs the per-query budgets kept
        pairs = int((idx >= 0).sum())
        flops = 2.0 * spec.H * (spec.Dk + spec.Dv) * pairs
    achieved = flops / (attn_ms * 1e-3) / 1e12
    kern = ("attn_mla_kernel" if (spec.H, spec.Dk, spec.Dv) == (128, 576, 512) and x["v"] is None
            else "attn_h16_kernel" if (spec.H, spec.Dk, spec.Dv) == (16, 128, 128) else "attn_bf16_kernel")
    sha = kernel_source_sha(["attn.hip", "common.h", "kernels.h"])
    traffic = load_traffic(kern, sha) if spec is not None and L == 131072 else None
    roof = {"bound": "mfma", "kernel": kern, "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": traffic,
            "ms_per_launch": round(attn_ms, 3), "algorithmic_flops_per_launch": flops, "selected_pairs": pairs}
    idx_ms = dt * 1e3 - attn_ms
    ifl = indexer_flops(L)
    idx_tf = ifl / (idx_ms * 1e-3) / 1e12
    roof_idx = {"bound": "mfma", "stage": "fold + indexer scores + top-k (step minus attention)",
                "ms": round(idx_ms, 3), "fold_ms": round(fold_ms, 3), "scores_and_select_ms": round(idx_ms - fold_ms, 3),
                "achieved": round(idx_tf, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                "frac": round(idx_tf / PEAK_FP8_TFLOPS, 4), "algorithmic_flops": ifl,
                "note": "step minus attention, timed live; per-kernel times under 'kernels' (committed trace)"}
    # the rows the attention gathers: one latent row per pair (shared K/V), else
    # a key row and a value row; for few heads this, not the MFMA work, bounds it
    row_bytes = 2 * (spec.Dk + (spec.Dv if x["v"] is not None else 0))
    gathered = pairs * row_bytes
    roof["gathered_bytes_per_launch"] = gathered
    roof["gather_gbps"] = round(gathered / (attn_ms * 1e-3) / 1e9, 1)
    if peaks:
        roof["frac_measured_peak"] = round(achieved / peaks["bf16_tflops"], 4)
        roof_idx["frac_measured_peak"] = round(idx_tf / peaks["fp8_tflops"], 4)
    log(f"{spec.name}: attention {attn_ms:.2f} ms/launch = {achieved:.1f} TFLOP/s; indexer stage {idx_ms:.2f} ms "
        f"(fold {fold_ms:.3f} ms)")
    line = {"tokens_per_s": round(L / dt, 1), "ms_per_step": round(dt * 1e3, 3), "L": L, "topk": k,
            "heads": spec.H, "dk": spec.Dk, "dv": spec.Dv, "roofline": roof, "roofline_indexer": roof_idx}
    if clocks_during is not None:
        line["clocks_during"] = clocks_during
    if keep:
        return line, idx, out
    del idx, out
    return line, None, None

if __name__ == "__main__":
    main()
