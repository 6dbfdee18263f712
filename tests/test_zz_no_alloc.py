"""dsa_forward_static (no workspace, nothing allocated by the call) against
dsa_forward with a caller workspace, through the C ABI: the same kernels run,
so outputs and indices must be identical bit for bit.  Two calls in a row on
the static scratch, the second with a smaller input, then a short prefill,
then an input too large for the scratch (DSA_ERR_WORKSPACE)."""
import sys

import pytest
import torch

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


def same(a, b):
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def decode_case(spec, dev, seed, lengths=None):
    x = gen.make_decode(spec, seed=seed, device=dev, lengths=lengths)
    fa = B.forward_args(x, spec.topk, spec.scale, spec.Dv, mode=B.DSA_MODE_DECODE, max_len=int(x["lengths"].max()))
    return x, fa, (spec.B, spec.H, spec.Dv), (spec.B, spec.topk)


def prefill_case(spec, dev, seed):
    x = gen.make_prefill(spec, seed=seed, device=dev)
    fa = B.forward_args(x, spec.topk, spec.scale, spec.Dv)
    return x, fa, (spec.L, spec.H, spec.Dv), (spec.L, spec.topk)


def compare(fa, out_shape, idx_shape, dev, with_idx=True):
    out_ref = torch.empty(out_shape, dtype=torch.bfloat16, device=dev)
    idx_ref = torch.empty(idx_shape, dtype=torch.int32, device=dev)
    B.dsa_forward(fa, out_ref, idx_out=idx_ref)
    out = torch.full(out_shape, float("nan"), dtype=torch.bfloat16, device=dev)
    idx = torch.full(idx_shape, -7, dtype=torch.int32, device=dev) if with_idx else None
    B.dsa_forward_static(fa, out, idx_out=idx)
    torch.cuda.synchronize()
    assert same(out, out_ref), "output differs from dsa_forward's"
    if with_idx:
        assert torch.equal(idx, idx_ref), "indices differ from dsa_forward's"


def test_static_scratch_two_calls_then_smaller(dev):
    # 1: the 64-sequence decode step over caches of 16K..128K keys
    spec = gen.DECODE_64
    x, fa, so, si = decode_case(spec, dev, seed=41)
    need = B.dsa_forward_workspace_size(fa)
    say(f"decode B=64: workspace {need / 2**20:.1f} MiB of {B.STATIC_SCRATCH_BYTES / 2**20:.0f} MiB")
    assert need <= B.STATIC_SCRATCH_BYTES
    compare(fa, so, si, dev)
    del x
    # 2: a smaller decode right after (the scratch keeps the first call's
    # contents; nothing may depend on them)
    small = gen.DECODE_64.with_(name="decode_B7", B=7, n_min=1, n_max=3000, topk=512)
    x2, fa2, so2, si2 = decode_case(small, dev, seed=42,
                                    lengths=torch.tensor([1, 2, 511, 512, 513, 2999, 1000], dtype=torch.int64))
    compare(fa2, so2, si2, dev)
    compare(fa2, so2, si2, dev, with_idx=False)
    # 3: a short prefill on the same scratch
    x3, fa3, so3, si3 = prefill_case(gen.PREFILL_32K.with_(name="prefill_L1000", L=1000, topk=256), dev, seed=43)
    compare(fa3, so3, si3, dev)


def test_static_scratch_rejects_too_large(dev):
    spec = gen.PREFILL_32K.with_(name="prefill_L6000", L=6000, topk=2048)
    x, fa, so, si = prefill_case(spec, dev, seed=44)
    assert B.dsa_forward_workspace_size(fa) > B.STATIC_SCRATCH_BYTES
    out = torch.empty(so, dtype=torch.bfloat16, device=dev)
    idx = torch.empty(si, dtype=torch.int32, device=dev)
    with pytest.raises(B.DsaError) as e:
        B.dsa_forward_static(fa, out, idx_out=idx)
    assert e.value.status == 5
