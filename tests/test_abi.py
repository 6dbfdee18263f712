"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every entry point include/dsa.h declares, and rejects invalid arguments with
the documented status before touching the device."""
import ctypes
import os
import re

import pytest

from sparse_attention_long_indexer_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return B.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) >= 10
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTED) == names


def test_probe_library_exports(lib):
    """The achievable-peak probe library exports what include/dsa_probe.h
    declares, and rejects invalid arguments without launching."""
    from sparse_attention_long_indexer_amd import build as b
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "dsa_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(dsa_probe_[a-z_]+)\s*\(", src)))
    assert names == ["dsa_probe_mfma", "dsa_probe_mfma_flops", "dsa_probe_read"]
    probe = ctypes.CDLL(b.PROBE_LIB)
    for n in names:
        assert hasattr(probe, n), n
    probe.dsa_probe_mfma_flops.restype = ctypes.c_double
    probe.dsa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64]
    assert probe.dsa_probe_mfma_flops(0, 10, 2) == 65536.0 * 8 * 4 * 10 * 2
    assert probe.dsa_probe_mfma_flops(3, 10, 2) == 0.0
    probe.dsa_probe_mfma.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p]
    assert probe.dsa_probe_mfma(7, 10, 2, _vp(), None) == -1
    assert probe.dsa_probe_mfma(0, 10, 2, None, None) == -1
    assert probe.dsa_probe_mfma(1, 11, 2, _vp(), None) == -1   # odd round count
    probe.dsa_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p,
                                     ctypes.c_void_p]
    assert probe.dsa_probe_read(_vp(), 4096 * 3 + 8, 1, _vp(), None) == -1     # not a multiple of 16
    assert probe.dsa_probe_read(_vp(), 4096 * 3, 2, _vp(), None) == -1        # not whole rounds of the grid


def test_abi_version_and_status_strings(lib):
    assert lib.dsa_abi_version() == 6
    for s in range(7):
        assert lib.dsa_status_str(s)
    assert lib.dsa_status_str(99) == b"unknown status"


def _vp(x=0x1000):
    return ctypes.c_void_p(x)


def test_fold_validation(lib):
    f = lib.dsa_fold_index_query
    # bad dtypes
    assert f(_vp(), _vp(), 7, _vp(), B.DSA_BF16, 4, _vp(), _vp(), None) == 3
    assert f(_vp(), None, B.DSA_F32, _vp(), B.DSA_BF16, 4, _vp(), None, None) == 3
    # null pointers
    assert f(None, _vp(), B.DSA_FP8_E4M3, _vp(), B.DSA_BF16, 4, _vp(), _vp(), None) == 1
    assert f(_vp(), None, B.DSA_FP8_E4M3, _vp(), B.DSA_BF16, 4, _vp(), _vp(), None) == 1
    # negative size
    assert f(_vp(), _vp(), B.DSA_FP8_E4M3, _vp(), B.DSA_BF16, -1, _vp(), _vp(), None) == 2
    # empty input is a no-op
    assert f(None, None, B.DSA_FP8_E4M3, None, B.DSA_BF16, 0, None, None, None) == 0


def test_scores_validation(lib):
    f = lib.dsa_index_scores
    a = _vp(0x10000)
    assert f(a, a, a, a, B.DSA_FP8_E4M3, 10, 10, None, 5, 4, a, 10, None) == 2       # row_begin > row_end
    assert f(a, a, a, a, B.DSA_FP8_E4M3, 10, 10, None, 0, 11, a, 10, None) == 2      # row_end > T
    assert f(a, a, a, a, B.DSA_FP8_E4M3, 10, 10, None, 0, 10, a, 9, None) == 2       # ld < S
    assert f(a, None, a, a, B.DSA_FP8_E4M3, 10, 10, None, 0, 10, a, 10, None) == 1   # no scale
    assert f(_vp(0x10008), a, a, a, B.DSA_FP8_E4M3, 10, 10, None, 0, 10, a, 10, None) == 2  # misaligned
    assert f(a, a, a, a, B.DSA_BF16, 10, 10, None, 0, 10, a, 10, None) == 3
    assert f(a, a, a, a, B.DSA_FP8_E4M3, 10, 10, None, 3, 3, a, 10, None) == 0       # empty range


def test_topk_validation(lib):
    f = lib.dsa_topk
    a = _vp(0x10000)
    assert f(a, 10, 4, 10, None, 0, a, None, None, 0, None) == 2           # k = 0
    assert f(a, 10, 4, 10, None, 4097, a, None, None, 0, None) == 2        # k > max
    assert f(a, 9, 4, 10, None, 8, a, None, None, 0, None) == 2            # ld < S
    assert f(a, 10, 4, 10, None, 8, None, None, None, 0, None) == 1        # no output
    assert f(a, 10, 0, 10, None, 8, None, None, None, 0, None) == 0        # no rows


def test_topk_dynamic_validation(lib):
    f = lib.dsa_topk_dynamic
    a = _vp(0x10000)
    nan = ctypes.c_float(float("nan"))
    th = ctypes.c_float(0.5)
    assert f(a, 10, 4, 10, None, 8, 9, th, a, None, None, 0, None) == 2     # k_min > k_max
    assert f(a, 10, 4, 10, None, 8, -1, th, a, None, None, 0, None) == 2    # k_min < 0
    assert f(a, 10, 4, 10, None, 8, 2, nan, a, None, None, 0, None) == 2    # theta NaN
    assert f(a, 10, 4, 10, None, 0, 0, th, a, None, None, 0, None) == 2     # k_max = 0
    assert f(a, 10, 4, 10, None, 8, 2, th, None, None, None, 0, None) == 1  # no output
    assert f(a, 10, 0, 10, None, 8, 2, th, None, None, None, 0, None) == 0  # no rows


def test_attn_bwd_validation(lib):
    f = lib.dsa_sparse_attn_bwd
    p = _vp(0x100000)
    sc = ctypes.c_float(0.04)
    args = dict(q=p, T=4, H=128, Dk=576, dt=B.DSA_BF16, kv=p, ldkv=576, Dv=512, S=100, idx=p, k=64, sc=sc, out=p,
                lse=p, do=p, dq=p, dkv=p, lddkv=576, ws=p, wsb=1 << 30, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())
    assert call(dt=B.DSA_F32) == 4          # fp32 not supported
    assert call(dt=7) == 3                  # not a dtype
    assert call(H=64) == 4                  # head count
    assert call(k=100) == 4                 # k not a multiple of 32
    assert call(ldkv=500) == 2              # ld_kv < Dk
    assert call(dq=None) == 1
    assert call(wsb=16) == 5
    assert call(T=0) == 0
    assert lib.dsa_sparse_attn_bwd_workspace_size(4, 128, 64) > 0


def test_indexer_kl_validation(lib):
    f = lib.dsa_indexer_kl
    p = _vp(0x100000)
    sc = ctypes.c_float(0.04)
    args = dict(qi=p, ki=p, w=p, q=p, H=128, Dk=576, dt=B.DSA_BF16, kv=p, ldkv=576, L=64, sc=sc, loss=p, dqi=p,
                dki=p, dw=p, ws=p, wsb=1 << 30, st=None)

    def call(**kw):
        a = dict(args, **kw)
        return f(*a.values())
    assert call(dt=B.DSA_F32) == 4
    assert call(H=16) == 4
    assert call(L=1 << 17) == 4
    assert call(ldkv=100) == 2
    assert call(dw=None) == 1
    assert call(wsb=16) == 5
    assert call(L=0) == 0
    assert lib.dsa_indexer_kl_workspace_size(64) >= 64 * 64 * 4


def test_attn_validation(lib):
    f = lib.dsa_sparse_attn
    a = _vp(0x10000)
    args = lambda **kw: [kw.get("q", a), kw.get("T", 4), kw.get("H", 16), kw.get("Dk", 128),
                         kw.get("dt", B.DSA_BF16), kw.get("kv", a), kw.get("ldkv", 128), kw.get("v", a),
                         kw.get("ldv", 128), kw.get("Dv", 128), kw.get("S", 10), kw.get("idx", a),
                         kw.get("k", 8), ctypes.c_float(0.1), kw.get("out", a), None, None, 0, None]
    assert f(*args(H=8)) == 4                      # unsupported head shape for bf16
    assert f(*args(dt=B.DSA_FP8_E4M3)) == 3
    assert f(*args(k=0)) == 2
    assert f(*args(ldkv=100)) == 2                 # ld_kv < Dk
    assert f(*args(ldkv=136 + 4)) == 2             # ld not a multiple of 8 bf16
    assert f(*args(idx=None)) == 1
    assert f(*args(q=_vp(0x10008))) == 2           # misaligned Q
    assert f(*args(S=0)) == 2
    assert f(*args(T=0)) == 0
    # bf16 rows are gathered through 32-bit byte offsets: S * ld * 2 <= 4 GiB
    # (only failing cases here: a call that passes validation would launch)
    assert f(*args(S=(1 << 32) // 256 + 1)) == 4
    assert f(*args(S=(1 << 31) // 128 + 1, ldkv=256, v=None)) == 4
    assert f(*args(S=(1 << 31) // 128 + 1, ldv=256)) == 4


def test_forward_validation(lib):
    a = B.ForwardArgs()
    a.mode = 5
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(), _vp(0x10000), 1 << 20, None) == 4
    assert lib.dsa_forward(None, None, _vp(), _vp(0x10000), 1 << 20, None) == 1
    a.mode = B.DSA_MODE_PREFILL
    a.T = 16
    a.topk = 0
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(), _vp(0x10000), 1 << 20, None) == 2
    assert lib.dsa_forward_workspace_size(ctypes.byref(a)) == 0
    # a valid prefill description: workspace grows with T, and a too-small one is rejected
    p = 0x100000
    a.topk = 64
    a.idx_dtype, a.w_dtype, a.attn_dtype = B.DSA_FP8_E4M3, B.DSA_BF16, B.DSA_BF16
    a.q_idx = a.q_scale = a.w_index = a.k_idx = a.k_scale = a.q = a.kv = p
    a.H, a.Dk, a.Dv, a.ld_kv = 16, 128, 128, 128
    a.v, a.ld_v, a.scale = p, 128, 0.1
    n16 = lib.dsa_forward_workspace_size(ctypes.byref(a))
    a.T = 4096
    n4k = lib.dsa_forward_workspace_size(ctypes.byref(a))
    assert 0 < n16 < n4k
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), n4k - 1, None) == 5
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p + 8), n4k, None) == 5
    # a later chunk of a prefill sees more keys: a larger workspace
    a.q_offset = 1 << 20
    assert lib.dsa_forward_workspace_size(ctypes.byref(a)) > n4k
    a.q_offset = -1
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), 1 << 40, None) == 2
    a.q_offset = (1 << 31) - 4096    # positions past int32
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), 1 << 40, None) == 2
    a.q_offset = 0
    a.flags = B.DSA_FLAG_DYNAMIC_K
    a.dyn_theta, a.dyn_k_min = 0.5, 65           # k_min above topk
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), 1 << 40, None) == 2
    a.dyn_theta, a.dyn_k_min = float("nan"), 1
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), 1 << 40, None) == 2
    a.flags = 0
    a.mode = B.DSA_MODE_DECODE
    a.seq_offsets = None
    a.T, a.total_keys, a.max_len = 4, 100, 50
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), 1 << 30, None) == 1
    a.q_offset = 3                               # decode takes no query offset
    assert lib.dsa_forward(ctypes.byref(a), None, _vp(p), _vp(p), 1 << 30, None) == 2
    a.q_offset = 0
