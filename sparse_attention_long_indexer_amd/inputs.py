"""Seeded synthetic inputs for the DSA forward path.

This module only draws random tensors and stores them in the byte formats the
library consumes; it holds none of the method's arithmetic (no fold, no score,
no selection, no softmax).  Both the HIP path and the CPU oracle are fed from
the tensors it returns, and neither imports the other.

Recipe (DeepSeek-V3.2 write-up on intelliparadigm.com, sections 2.2-3.1: a
128-dim index key per token kept in FP8, one bilinear projection W_index,
k = 2048 selected keys, MQA over one shared latent KV head):

* index query / key rows: N(0,1)/sqrt(128) in fp64-free float32 draws; for
  the FP8 workloads each row is stored as OCP e4m3fn codes with a per-row
  fp32 scale amax/448 (torch's own saturating round-to-nearest-even cast);
* W_index: N(0,1)/sqrt(128), stored as bf16 (fp32 for the tiny workload);
* attention Q/K/V: N(0,1) (tiny and 8K workloads) or N(0,1)/sqrt(dim)
  (MLA-shaped workloads), stored as bf16 (fp32 for the tiny workload);
* planted heavy tail: every 64th key gets +3/sqrt(128) added to all 128
  coordinates of its index key before quantisation;
* decode: 64 ragged sequences with lengths uniform in [16384, 131072].

Every tensor has its own generator, seeded from (workload id, seed, tensor
id), so a workload is reproducible on one device.  Draws on different devices
differ; a test always feeds the very same tensors to both sides.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

IDX_DIM = 128
E4M3_MAX = 448.0

# tensor ids used to derive per-tensor seeds
_T_QIDX, _T_KIDX, _T_W, _T_Q, _T_K, _T_V, _T_LEN = range(7)


@dataclasses.dataclass(frozen=True)
class PrefillSpec:
    name: str
    wid: int            # workload id (seed domain)
    L: int              # tokens: queries = keys = L, causal
    topk: int
    fp8: bool           # index inputs stored as e4m3 + per-row scale (else fp32)
    H: int
    Dk: int
    Dv: int
    attn_f32: bool      # attention tensors in fp32 (else bf16)
    shared_kv: bool     # one latent row per key: K = KV[:, :Dk], V = KV[:, :Dv]
    qkv_unit: bool      # Q/K/V ~ N(0,1) (else N(0,1)/sqrt(dim))
    planted_every: int  # 0: none; else every n-th key gets a +3 sigma index-key bias
    batch: int = 1

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dk)

    def with_(self, **kw) -> "PrefillSpec":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    name: str
    wid: int
    B: int
    n_min: int
    n_max: int
    topk: int
    H: int
    Dk: int
    Dv: int
    qkv_unit: bool = False

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dk)

    def with_(self, **kw) -> "DecodeSpec":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 case, an 8K prefill, MLA-shaped 32K and 128K
# prefills with a planted heavy tail, and a 64-sequence batched decode.
TINY_F32 = PrefillSpec("tiny_f32_L512", 1, 512, 64, False, 4, 64, 64, True, False, True, 0)
PREFILL_8K = PrefillSpec("prefill_L8192_h16", 2, 8192, 2048, True, 16, 128, 128, False, False, True, 0)
PREFILL_32K = PrefillSpec("prefill_L32768_mla", 3, 32768, 2048, True, 128, 576, 512, False, True, False, 64)
PREFILL_128K = PrefillSpec("prefill_L131072_mla", 4, 131072, 2048, True, 128, 576, 512, False, True, False, 64)
DECODE_64 = DecodeSpec("decode_B64_ctx16k_128k", 5, 64, 16384, 131072, 2048, 128, 576, 512)

WORKLOADS = {s.name: s for s in (TINY_F32, PREFILL_8K, PREFILL_32K, PREFILL_128K, DECODE_64)}

# Million-token context (the write-up's closing outlook): the MLA-shaped
# prefill at L = 2^20, run as chunks of queries over the growing key prefix,
# and decode caches of up to 2^20 + a few entries.
PREFILL_1M = PREFILL_128K.with_(name="prefill_L1048576_mla", wid=6, L=1 << 20)
DECODE_1M = DecodeSpec("decode_B4_ctx1m", 7, 4, 65536, (1 << 20) + 64, 2048, 128, 576, 512)


def _gen(device, wid: int, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + wid * 7_919 + tid * 104_729 + 20260000) % (2 ** 63))
    return g


def _randn(shape, g, device, std: float, dtype, chunk_rows: int = 1 << 14) -> torch.Tensor:
    """N(0, std^2) draws cast to `dtype`, made in row chunks to bound fp32 temporaries."""
    out = torch.empty(shape, dtype=dtype, device=device)
    rows = shape[0]
    row_elems = max(1, math.prod(shape[1:]))
    step = max(1, min(rows, (1 << 26) // row_elems)) if rows else 1
    step = max(step, 1)
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0,) + tuple(shape[1:]), generator=g, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        out[r0:r1] = x.to(dtype)
    return out


def quantize_rows_e4m3(x: torch.Tensor):
    """Store fp32 rows as e4m3fn codes with a per-row fp32 scale amax/448.

    Input recipe only (how the cached index keys and index queries arrive in
    FP8); uses torch's saturating round-to-nearest-even cast.
    """
    amax = x.abs().amax(dim=1)
    scale = torch.where(amax > 0, amax / E4M3_MAX, torch.ones_like(amax)).to(torch.float32)
    y = (x / scale[:, None]).clamp_(-E4M3_MAX, E4M3_MAX)
    codes = y.to(torch.float8_e4m3fn).view(torch.uint8).contiguous()
    return codes, scale.contiguous()


def _index_rows(n: int, g, device, planted_every: int, fp8: bool):
    x = torch.randn((n, IDX_DIM), generator=g, device=device, dtype=torch.float32) / math.sqrt(IDX_DIM)
    if planted_every:
        x[::planted_every] += 3.0 / math.sqrt(IDX_DIM)
    if fp8:
        return quantize_rows_e4m3(x)
    return x.contiguous(), None


def make_prefill(spec: PrefillSpec, seed: int = 0, device="cpu") -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of one causal prefill: queries and keys are the same L tokens."""
    return make_prefill_chunk(spec, 0, seed, device)


def make_prefill_chunk(spec: PrefillSpec, q_offset: int, seed: int = 0, device="cpu",
                       queries: bool = True) -> Dict[str, Optional[torch.Tensor]]:
    """Inputs of the last chunk of one causal prefill: keys for all L tokens,
    index queries and attention queries only for tokens q_offset .. L-1 (the
    whole prefill when q_offset = 0).  With queries=False only the key side
    is drawn (q_idx, q_scale and q are None)."""
    dev = torch.device(device)
    L = spec.L
    T = L - q_offset
    if not 0 <= q_offset <= L:
        raise ValueError("q_offset outside [0, L]")
    q_idx = q_scale = q = None
    if queries:
        q_idx, q_scale = _index_rows(T, _gen(dev, spec.wid, seed, _T_QIDX), dev, 0, spec.fp8)
    k_idx, k_scale = _index_rows(L, _gen(dev, spec.wid, seed, _T_KIDX), dev, spec.planted_every, spec.fp8)
    wdt = torch.float32 if not spec.fp8 else torch.bfloat16
    w = _randn((IDX_DIM, IDX_DIM), _gen(dev, spec.wid, seed, _T_W), dev, 1.0 / math.sqrt(IDX_DIM), wdt)
    adt = torch.float32 if spec.attn_f32 else torch.bfloat16
    q_std = 1.0 if spec.qkv_unit else 1.0 / math.sqrt(spec.Dk)
    if queries:
        q = _randn((T, spec.H, spec.Dk), _gen(dev, spec.wid, seed, _T_Q), dev, q_std, adt)
    if spec.shared_kv:
        kv = _randn((L, spec.Dk), _gen(dev, spec.wid, seed, _T_K), dev, q_std, adt)
        v = None
    else:
        kv = _randn((L, spec.Dk), _gen(dev, spec.wid, seed, _T_K), dev, q_std, adt)
        v_std = 1.0 if spec.qkv_unit else 1.0 / math.sqrt(spec.Dv)
        v = _randn((L, spec.Dv), _gen(dev, spec.wid, seed, _T_V), dev, v_std, adt)
    return dict(q_idx=q_idx, q_scale=q_scale, k_idx=k_idx, k_scale=k_scale, w=w, q=q, kv=kv, v=v)


def decode_lengths(spec: DecodeSpec, seed: int = 0) -> torch.Tensor:
    g = _gen(torch.device("cpu"), spec.wid, seed, _T_LEN)
    return torch.randint(spec.n_min, spec.n_max + 1, (spec.B,), generator=g, dtype=torch.int64)


def make_decode(spec: DecodeSpec, seed: int = 0, device="cpu", lengths: Optional[torch.Tensor] = None):
    """Inputs of one batched decode step over ragged per-sequence caches.

    Sequence b owns cache rows [offsets[b], offsets[b+1]); its one new query
    sits at position n_b - 1 and its own key is the last cached row.
    """
    dev = torch.device(device)
    n = decode_lengths(spec, seed) if lengths is None else lengths.to(torch.int64).cpu()
    offsets = torch.zeros(spec.B + 1, dtype=torch.int64)
    offsets[1:] = torch.cumsum(n, 0)
    total = int(offsets[-1])
    q_idx, q_scale = _index_rows(spec.B, _gen(dev, spec.wid, seed, _T_QIDX), dev, 0, True)
    k_idx, k_scale = _index_rows(total, _gen(dev, spec.wid, seed, _T_KIDX), dev, 0, True)
    w = _randn((IDX_DIM, IDX_DIM), _gen(dev, spec.wid, seed, _T_W), dev, 1.0 / math.sqrt(IDX_DIM), torch.bfloat16)
    std = 1.0 if spec.qkv_unit else 1.0 / math.sqrt(spec.Dk)
    q = _randn((spec.B, spec.H, spec.Dk), _gen(dev, spec.wid, seed, _T_Q), dev, std, torch.bfloat16)
    kv = _randn((total, spec.Dk), _gen(dev, spec.wid, seed, _T_K), dev, std, torch.bfloat16)
    return dict(q_idx=q_idx, q_scale=q_scale, k_idx=k_idx, k_scale=k_scale, w=w, q=q, kv=kv, v=None,
                lengths=n, offsets=offsets.to(dev))


# ---- stage-level inputs (each stage can be fed on its own) ----------------

def make_scores(T: int, S: int, seed: int = 0, device="cpu", q_pos: Optional[torch.Tensor] = None,
                levels: int = 64) -> torch.Tensor:
    """fp32 score rows shaped like lightning-indexer output: about half exact
    zeros (some stored as -0.0), positive values quantised to `levels` steps so
    that exact ties are common, and -inf past each row's causal position."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 7_777 + 31)
    x = torch.randn((T, S), generator=g, dtype=torch.float32)
    x = torch.clamp(torch.round(x * (levels / 4.0)) / (levels / 4.0), min=0.0)
    negz = torch.rand((T, S), generator=g) < 0.1
    x = torch.where((x == 0) & negz, torch.full_like(x, -0.0), x)
    if q_pos is None:
        q_pos = torch.arange(T, dtype=torch.int64)
    s = torch.arange(S)[None, :]
    x = torch.where(s <= q_pos.cpu()[:, None], x, torch.full_like(x, float("-inf")))
    return x.to(device)


def make_grad(shape, seed: int = 0, device="cpu", dtype=torch.bfloat16) -> torch.Tensor:
    """An incoming gradient (dLoss/dout) for the backward pass: N(0,1)
    entries stored as `dtype`."""
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(seed * 6_151 + 101)
    return _randn(tuple(shape), g, torch.device(device), 1.0, dtype)


def make_selection(T: int, S: int, k: int, seed: int = 0, device="cpu", min_valid: int = 0) -> torch.Tensor:
    """int32 [T][k] rows of ascending distinct key indices in [0, S), each row
    holding a random number (>= min_valid) of valid entries followed by -1."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed * 9_973 + 17)
    out = torch.full((T, k), -1, dtype=torch.int32)
    cap = min(k, S)
    for t in range(T):
        m = int(torch.randint(min(min_valid, cap), cap + 1, (1,), generator=g))
        if t == 0:
            m = cap
        sel = torch.randperm(S, generator=g)[:m].sort().values
        out[t, :m] = sel.to(torch.int32)
    return out.to(device)
