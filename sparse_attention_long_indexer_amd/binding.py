"""ctypes binding of libdsa.so.

Argument marshalling only: each function takes torch tensors (device memory
owned by the caller), passes their pointers and the current HIP stream to the
C entry point of the same name and turns a non-zero status into DsaError.
Every step of the path runs in the library's HIP kernels; there is no
fallback, and importing this module fails loudly if the library is missing.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdsa.so")

DSA_F32, DSA_BF16, DSA_FP8_E4M3 = 0, 1, 2
DSA_MODE_PREFILL, DSA_MODE_DECODE = 0, 1
DSA_FLAG_MATERIALIZE = 1
DSA_FLAG_FUSED = 2
DSA_FLAG_FORCE_FALLBACK = 4
DSA_FLAG_DYNAMIC_K = 8
INDEX_DIM = 128
MAX_TOPK = 4096
ABI_VERSION = 6
STATIC_SCRATCH_BYTES = 128 << 20

EXPORTED = [
    "dsa_abi_version", "dsa_status_str", "dsa_fold_index_query", "dsa_index_scores",
    "dsa_topk_workspace_size", "dsa_topk", "dsa_topk_dynamic", "dsa_sparse_attn_workspace_size", "dsa_sparse_attn",
    "dsa_sparse_attn_bwd_workspace_size", "dsa_sparse_attn_bwd", "dsa_indexer_kl_workspace_size", "dsa_indexer_kl",
    "dsa_forward_workspace_size", "dsa_forward", "dsa_forward_static",
]


class DsaError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: status {status} ({msg})")
        self.status = status


class ForwardArgs(ctypes.Structure):
    _fields_ = [
        ("mode", ctypes.c_int32), ("flags", ctypes.c_uint32), ("T", ctypes.c_int64),
        ("seq_offsets", ctypes.c_void_p), ("total_keys", ctypes.c_int64), ("max_len", ctypes.c_int64),
        ("idx_dtype", ctypes.c_int), ("q_idx", ctypes.c_void_p), ("q_scale", ctypes.c_void_p),
        ("w_index", ctypes.c_void_p), ("w_dtype", ctypes.c_int), ("k_idx", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p), ("attn_dtype", ctypes.c_int), ("q", ctypes.c_void_p),
        ("H", ctypes.c_int64), ("Dk", ctypes.c_int64), ("Dv", ctypes.c_int64), ("kv", ctypes.c_void_p),
        ("ld_kv", ctypes.c_int64), ("v", ctypes.c_void_p), ("ld_v", ctypes.c_int64),
        ("topk", ctypes.c_int64), ("scale", ctypes.c_float), ("q_offset", ctypes.c_int64),
        ("dyn_theta", ctypes.c_float), ("dyn_k_min", ctypes.c_int64),
    ]


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m sparse_attention_long_indexer_amd.build`")
    lib = ctypes.CDLL(path)
    c_i64, c_vp, c_int, c_sz, c_f = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    sig = {
        "dsa_abi_version": ([], c_int),
        "dsa_status_str": ([c_int], ctypes.c_char_p),
        "dsa_fold_index_query": ([c_vp, c_vp, c_int, c_vp, c_int, c_i64, c_vp, c_vp, c_vp], c_int),
        "dsa_index_scores": ([c_vp, c_vp, c_vp, c_vp, c_int, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp, c_i64, c_vp],
                             c_int),
        "dsa_topk_workspace_size": ([c_i64, c_i64, c_i64], c_sz),
        "dsa_topk": ([c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp, c_vp, c_sz, c_vp], c_int),
        "dsa_topk_dynamic": ([c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_f, c_vp, c_vp, c_vp, c_sz, c_vp],
                             c_int),
        "dsa_sparse_attn_workspace_size": ([c_i64, c_i64, c_i64, c_i64, c_int], c_sz),
        "dsa_sparse_attn": ([c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_i64, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64,
                             c_f, c_vp, c_vp, c_vp, c_sz, c_vp], c_int),
        "dsa_sparse_attn_bwd_workspace_size": ([c_i64, c_i64, c_i64], c_sz),
        "dsa_sparse_attn_bwd": ([c_vp, c_i64, c_i64, c_i64, c_int, c_vp, c_i64, c_i64, c_i64, c_vp, c_i64, c_f,
                                 c_vp, c_vp, c_vp, c_vp, c_vp, c_i64, c_vp, c_sz, c_vp], c_int),
        "dsa_indexer_kl_workspace_size": ([c_i64], c_sz),
        "dsa_indexer_kl": ([c_vp, c_vp, c_vp, c_vp, c_i64, c_i64, c_int, c_vp, c_i64, c_i64, c_f, c_vp, c_vp, c_vp,
                            c_vp, c_vp, c_sz, c_vp], c_int),
        "dsa_forward_workspace_size": ([ctypes.POINTER(ForwardArgs)], c_sz),
        "dsa_forward": ([ctypes.POINTER(ForwardArgs), c_vp, c_vp, c_vp, c_sz, c_vp], c_int),
        "dsa_forward_static": ([ctypes.POINTER(ForwardArgs), c_vp, c_vp, c_vp], c_int),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    if lib.dsa_abi_version() != ABI_VERSION:
        raise ImportError(f"{path} has ABI {lib.dsa_abi_version()}, this binding expects {ABI_VERSION}: rebuild it")
    return lib


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = load()
    return _lib


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, st: int):
    if st != 0:
        raise DsaError(fn, st, lib().dsa_status_str(st).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    if t.dtype == torch.uint8:
        return DSA_FP8_E4M3
    raise TypeError(f"unsupported dtype {t.dtype}")


def abi_version() -> int:
    return lib().dsa_abi_version()


# ---- entry points --------------------------------------------------------

def dsa_fold_index_query(q_idx, q_scale, w, qf_out=None, qf_scale_out=None, stream=None):
    T = q_idx.shape[0]
    qd = _dtype_code(q_idx)
    if qf_out is None:
        qf_out = torch.empty_like(q_idx)
    if qf_scale_out is None and qd == DSA_FP8_E4M3:
        qf_scale_out = torch.empty(T, dtype=torch.float32, device=q_idx.device)
    _check("dsa_fold_index_query", lib().dsa_fold_index_query(
        _p(q_idx), _p(q_scale), qd, _p(w), _dtype_code(w), T, _p(qf_out), _p(qf_scale_out), _stream(stream)))
    return qf_out, qf_scale_out


def dsa_index_scores(qf, qf_scale, k_idx, k_scale, q_pos=None, row_begin=0, row_end=None, out=None,
                     ld=None, stream=None):
    T, S = qf.shape[0], k_idx.shape[0]
    row_end = T if row_end is None else row_end
    ld = S if ld is None else ld
    if out is None:
        out = torch.empty((row_end - row_begin, ld), dtype=torch.float32, device=qf.device)
    _check("dsa_index_scores", lib().dsa_index_scores(
        _p(qf), _p(qf_scale), _p(k_idx), _p(k_scale), _dtype_code(qf), T, S, _p(q_pos), row_begin, row_end,
        _p(out), ld, _stream(stream)))
    return out


def _workspace(ws, nbytes, device, minimum=1):
    """The caller's workspace tensor, or a fresh one of the queried size."""
    if ws is None:
        ws = torch.empty(max(nbytes, minimum), dtype=torch.uint8, device=device)
    return ws


def dsa_topk(scores, k, S=None, q_pos=None, idx_out=None, count_out=None, stream=None, ws=None):
    T, ld = scores.shape
    S = ld if S is None else S
    if idx_out is None:
        idx_out = torch.empty((T, k), dtype=torch.int32, device=scores.device)
    wsb = lib().dsa_topk_workspace_size(T, S, k)
    ws = _workspace(ws, wsb, scores.device)
    _check("dsa_topk", lib().dsa_topk(_p(scores), ld, T, S, _p(q_pos), k, _p(idx_out), _p(count_out), _p(ws),
                                      wsb, _stream(stream)))
    return idx_out


def dsa_topk_dynamic(scores, k_max, k_min, theta, S=None, q_pos=None, idx_out=None, count_out=None, stream=None,
                     ws=None):
    T, ld = scores.shape
    S = ld if S is None else S
    if idx_out is None:
        idx_out = torch.empty((T, k_max), dtype=torch.int32, device=scores.device)
    wsb = lib().dsa_topk_workspace_size(T, S, k_max)
    ws = _workspace(ws, wsb, scores.device)
    _check("dsa_topk_dynamic", lib().dsa_topk_dynamic(_p(scores), ld, T, S, _p(q_pos), k_max, k_min,
                                                      ctypes.c_float(theta), _p(idx_out), _p(count_out), _p(ws),
                                                      wsb, _stream(stream)))
    return idx_out


def dsa_sparse_attn(q, kv, idx, scale, v=None, Dv=None, out=None, lse_out=None, stream=None, ws=None):
    T, H, Dk = q.shape
    S = kv.shape[0]
    Dv = (v.shape[1] if v is not None else Dk) if Dv is None else Dv
    k = idx.shape[1]
    dt = _dtype_code(q)
    if out is None:
        out = torch.empty((T, H, Dv), dtype=q.dtype, device=q.device)
    wsb = lib().dsa_sparse_attn_workspace_size(T, H, Dv, k, dt)
    ws = _workspace(ws, wsb, q.device)
    _check("dsa_sparse_attn", lib().dsa_sparse_attn(
        _p(q), T, H, Dk, dt, _p(kv), kv.stride(0), _p(v), v.stride(0) if v is not None else 0, Dv, S, _p(idx), k,
        ctypes.c_float(scale), _p(out), _p(lse_out), _p(ws), wsb, _stream(stream)))
    return out


def dsa_sparse_attn_bwd(q, kv, idx, scale, out, lse, d_out, Dv, dq=None, dkv=None, stream=None, ws=None):
    """dq (bf16, written) and dkv (fp32, accumulated; zeroed here when not
    given) of the shared-latent sparse attention."""
    T, H, Dk = q.shape
    S = kv.shape[0]
    k = idx.shape[1]
    if dq is None:
        dq = torch.empty_like(q)
    if dkv is None:
        dkv = torch.zeros((S, Dk), dtype=torch.float32, device=q.device)
    wsb = lib().dsa_sparse_attn_bwd_workspace_size(T, H, k)
    ws = _workspace(ws, wsb, q.device, 256)
    _check("dsa_sparse_attn_bwd", lib().dsa_sparse_attn_bwd(
        _p(q), T, H, Dk, _dtype_code(q), _p(kv), kv.stride(0), Dv, S, _p(idx), k, ctypes.c_float(scale), _p(out),
        _p(lse), _p(d_out), _p(dq), _p(dkv), dkv.stride(0), _p(ws), ws.numel(), _stream(stream)))
    return dq, dkv


def dsa_indexer_kl(q_idx, k_idx, w, q, kv, scale, stream=None, ws=None):
    """Per-query KL losses and the gradients (dq_idx, dk_idx, dw) of the
    indexer alignment; all fp32 except the bf16 attention operands."""
    L, H, Dk = q.shape
    dev = q.device
    loss = torch.empty(L, dtype=torch.float32, device=dev)
    dq_idx = torch.empty((L, 128), dtype=torch.float32, device=dev)
    dk_idx = torch.empty((L, 128), dtype=torch.float32, device=dev)
    dw = torch.empty((128, 128), dtype=torch.float32, device=dev)
    wsb = lib().dsa_indexer_kl_workspace_size(L)
    ws = _workspace(ws, wsb, dev, 256)
    _check("dsa_indexer_kl", lib().dsa_indexer_kl(
        _p(q_idx), _p(k_idx), _p(w), _p(q), H, Dk, _dtype_code(q), _p(kv), kv.stride(0), L, ctypes.c_float(scale),
        _p(loss), _p(dq_idx), _p(dk_idx), _p(dw), _p(ws), ws.numel(), _stream(stream)))
    return loss, dq_idx, dk_idx, dw


def forward_args(x: dict, topk: int, scale: float, Dv: int, mode: int = DSA_MODE_PREFILL, flags: int = 0,
                 max_len: int = 0, q_offset: int = 0, dyn_theta: Optional[float] = None, dyn_k_min: int = 0):
    """Build the dsa_forward argument struct from an input dict of device
    tensors (keys as produced by the input generators).  For a prefill chunk
    (q_offset > 0) the query tensors hold the chunk's rows and the key
    tensors the first q_offset + T rows of the sequence."""
    q = x["q"]
    a = ForwardArgs()
    a.mode = mode
    a.flags = flags
    a.T = q.shape[0]
    a.idx_dtype = _dtype_code(x["q_idx"])
    a.q_idx = x["q_idx"].data_ptr()
    a.q_scale = x["q_scale"].data_ptr() if x.get("q_scale") is not None else None
    a.w_index = x["w"].data_ptr()
    a.w_dtype = _dtype_code(x["w"])
    a.k_idx = x["k_idx"].data_ptr()
    a.k_scale = x["k_scale"].data_ptr() if x.get("k_scale") is not None else None
    a.attn_dtype = _dtype_code(q)
    a.q = q.data_ptr()
    a.H, a.Dk, a.Dv = q.shape[1], q.shape[2], Dv
    a.kv = x["kv"].data_ptr()
    a.ld_kv = x["kv"].stride(0)
    v = x.get("v")
    a.v = v.data_ptr() if v is not None else None
    a.ld_v = v.stride(0) if v is not None else 0
    a.topk = topk
    a.scale = scale
    a.q_offset = q_offset
    if dyn_theta is not None:
        a.flags |= DSA_FLAG_DYNAMIC_K
        a.dyn_theta = dyn_theta
        a.dyn_k_min = dyn_k_min
    if mode == DSA_MODE_DECODE:
        a.seq_offsets = x["offsets"].data_ptr()
        a.total_keys = x["k_idx"].shape[0]
        a.max_len = max_len
    return a


def dsa_forward_workspace_size(args: ForwardArgs) -> int:
    return lib().dsa_forward_workspace_size(ctypes.byref(args))


def dsa_forward(args: ForwardArgs, out, idx_out=None, ws=None, stream=None):
    wsb = dsa_forward_workspace_size(args)
    if wsb == 0:
        # invalid arguments: let the call report the status
        wsb = 0
    if ws is None:
        ws = torch.empty(max(wsb, 256), dtype=torch.uint8, device=out.device)
    _check("dsa_forward", lib().dsa_forward(ctypes.byref(args), _p(idx_out), _p(out), _p(ws), ws.numel(),
                                            _stream(stream)))
    return out, idx_out


def dsa_forward_static(args: ForwardArgs, out, idx_out=None, stream=None):
    """dsa_forward on the library's static scratch (no workspace, nothing
    allocated by the call)."""
    _check("dsa_forward_static", lib().dsa_forward_static(ctypes.byref(args), _p(idx_out), _p(out),
                                                          _stream(stream)))
    return out, idx_out
