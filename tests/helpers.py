"""Test helpers: host copies of input tensors in the oracle's storage formats
and the parity rules for each stage."""
import numpy as np
import torch


def to_np(t):
    """torch tensor -> numpy in storage format (bf16 -> uint16 bits)."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return t.cpu().contiguous().numpy()


def inputs_np(d):
    return {k: (to_np(v) if isinstance(v, torch.Tensor) else v) for k, v in d.items()}


def prefill_oracle(oracle_dsa, spec, x):
    n = inputs_np(x)
    return oracle_dsa.PrefillOracle(n["q_idx"], n["q_scale"], n["k_idx"], n["k_scale"], n["w"], n["q"],
                                    n["kv"], n["v"], spec.topk, spec.scale, spec.Dv)


def decode_oracle(oracle_dsa, spec, x):
    n = inputs_np(x)
    return oracle_dsa.DecodeOracle(n["q_idx"], n["q_scale"], n["k_idx"], n["k_scale"], n["w"], n["q"],
                                   n["kv"], n["v"], n["offsets"], spec.topk, spec.scale, spec.Dv)
