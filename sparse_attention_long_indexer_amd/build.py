"""Build libdsa.so (HIP kernels + C ABI) for gfx950, in-tree.

    python -m sparse_attention_long_indexer_amd.build

Every source is compiled by hipcc for --offload-arch=gfx950 only, with packed
fp32 instructions disabled, then linked into one shared library next to this
file.
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libdsa.so")
PROBE_LIB = os.path.join(PKG, "libdsa_probe.so")

SOURCES = ["fold.hip", "index_scores.hip", "topk.hip", "index_select.hip", "attn.hip", "attn_bwd.hip", "indexer_kl.hip", "api.cpp"]
# achievable-peak probes for the benchmark's roofline fractions (not the DSA path)
PROBE_SOURCES = ["probe.hip"]
SOURCE_FLAGS = {}   # per-source extra hipcc flags
ARCH = "gfx950"
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def hipcc() -> str:
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.isabs(c) and os.path.exists(c):
            return c
    return "hipcc"


def _compile(src: str, obj: str) -> None:
    lang = ["-x", "hip"]
    extra = os.environ.get("DSA_EXTRA_HIPCC_FLAGS", "").split()   # tuning experiments only
    cmd = [hipcc()] + FLAGS + SOURCE_FLAGS.get(src, []) + extra + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")


def _link(objs, out: str) -> None:
    out_tmp = out + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-fPIC", "-o", out_tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(out_tmp, out)


def build(verbose: bool = False, out: str = LIB, probe_out: str = PROBE_LIB) -> str:
    """Compile every source and link libdsa.so (or `out`) and the probe
    library libdsa_probe.so (or `probe_out`); returns the libdsa path."""
    srcs = SOURCES + PROBE_SOURCES
    with tempfile.TemporaryDirectory(prefix="dsa_build_") as tmp:
        objs = [os.path.join(tmp, s.replace(".", "_") + ".o") for s in srcs]
        with ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            list(ex.map(_compile, srcs, objs))
        _link(objs[: len(SOURCES)], out)
        _link(objs[len(SOURCES):], probe_out)
    if verbose:
        print(f"built {out} and {probe_out}")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
