"""The library's host side under sanitizers, on the CPU (no GPU needed).

Every library source is compiled host-only (kernel bodies are not built for
the device) with -DDSA_DEBUG, which turns on the launch-plan checks, and with
AddressSanitizer and UndefinedBehaviorSanitizer on the host code.  The
result is linked with tests/host/abi_host_check.cpp, which stands in for the
HIP runtime calls the host side makes, and run: every entry point with
invalid arguments (documented status, nothing launched) and with valid ones
over the supported shapes (every launch within the device's grid, block and
LDS limits; every workspace carve-up inside its size query).
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_attention_long_indexer_amd", "csrc")
HARNESS = os.path.join(ROOT, "tests", "host", "abi_host_check.cpp")


def _hipcc():
    p = "/opt/rocm/bin/hipcc"
    return p if os.path.exists(p) else shutil.which("hipcc")


@pytest.fixture(scope="module")
def host_check_exe(tmp_path_factory):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not found")
    from sparse_attention_long_indexer_amd import build as b
    tmp = tmp_path_factory.mktemp("host_check")
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
    common = ["-O1", "-g", "-std=c++17", "-DDSA_DEBUG", f"-I{b.INCLUDE}", f"-I{CSRC}"] + san
    objs = []
    for src in b.SOURCES + [HARNESS]:
        path = src if os.path.isabs(src) else os.path.join(CSRC, src)
        obj = str(tmp / (os.path.basename(src).replace(".", "_") + ".o"))
        cmd = [hipcc, "-x", "hip", "--cuda-host-only"] + common + ["-c", path, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
        objs.append(obj)
    # host-only objects still name the device code objects their kernels
    # would be registered from; the stand-in runtime ignores them
    syms = set()
    for o in objs:
        out = subprocess.run(["nm", "-u", o], capture_output=True, text=True, check=True).stdout
        syms |= {ln.split()[-1] for ln in out.splitlines() if ln.split() and ln.split()[-1].startswith("__hip_fatbin")}
    stub = tmp / "fatbin_stubs.c"
    stub.write_text("".join(f"const char {s}[8] = {{0}};\n" for s in sorted(syms)))
    stub_o = str(tmp / "fatbin_stubs.o")
    subprocess.run(["gcc", "-c", str(stub), "-o", stub_o], check=True)
    exe = str(tmp / "abi_host_check")
    cmd = [hipcc, "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-o", exe,
           stub_o] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"{' '.join(cmd)}\n{r.stdout}\n{r.stderr}"
    return exe


def test_abi_host_check_under_sanitizers(host_check_exe):
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([host_check_exe], capture_output=True, text=True, env=env, timeout=300)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "0 failures" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
