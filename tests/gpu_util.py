"""Helpers for the GPU parity tests: seeded inputs to the device, calls through
the C ABI (via the thin binding), results back to numpy."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import precision_flash_attention_attn_amd as pfa

DEV = "cuda:0"


def dev_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(torch.bfloat16).contiguous()


def dev_f32(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).contiguous()


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def run(inp, mode, causal=True, scale=None, bwd=True, beta=2.0, eps=1e-3):
    """Forward (and backward) of a synthetic Inputs object on the GPU.
    Returns a dict of float64 numpy arrays (o, lse, flags, dq, dk, dv, delta)."""
    q, k, v = dev_bf16(inp.q), dev_bf16(inp.k), dev_bf16(inp.v)
    o, lse, fl = pfa.forward(q, k, v, causal=causal, scale=scale, mode=mode, beta=beta, eps=eps)
    out = dict(o=host(o), lse=host(lse), flags=fl.cpu().numpy().astype(bool))
    if bwd:
        do = dev_f32(inp.do_f32) if mode == "fp32_out" else dev_bf16(inp.do_bf16)
        dq, dk, dv, delta = pfa.backward(q, k, v, o, do, lse, causal=causal, scale=scale, mode=mode,
                                         want_delta=True)
        out.update(dq=host(dq), dk=host(dk), dv=host(dv), delta=host(delta))
    torch.cuda.synchronize()
    return out


def record(section: str, key: str, value) -> None:
    """Add a measured figure to the JSON file named by PFA_PARITY_REPORT (if
    set): {section: {key: value}}, merged with what is already there."""
    path = os.environ.get("PFA_PARITY_REPORT")
    if not path:
        return
    data = {}
    if os.path.exists(path):
        with open(path) as f:
            data = json.load(f)
    data.setdefault(section, {})[key] = value
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
