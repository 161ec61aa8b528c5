"""Harness helpers shared by the tests, the smoke check and the benchmark.

Device placement of the seeded inputs (numpy storage layout of ``synth`` -> torch device tensors of the binding's
types) and the parity measure (max |got - want| / rms(want)).  No arithmetic of the layer is here.
"""
from __future__ import annotations

import numpy as np

from synth import BF16, F32, W8

# the parity bar: max|gpu - oracle| <= TOL * rms(oracle)
TOL = {F32: 1e-4, BF16: 1e-2, W8: 1e-2}


def dev_inputs(inp: dict, dtype: int, device="cuda") -> dict:
    """numpy inputs (synth layout) -> device tensors of the binding's types."""
    import torch

    def bf(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(
            torch.bfloat16).to(device)

    def raw(a):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device)

    out = {}
    if dtype == F32:
        for n in ("x", "router_w", "w1", "wv", "w2"):
            out[n] = raw(inp[n])
        out["scales"] = None
    elif dtype == BF16:
        for n in ("x", "router_w", "w1", "wv", "w2"):
            out[n] = bf(inp[n])
        out["scales"] = None
    elif dtype == W8:
        out["x"], out["router_w"] = bf(inp["x"]), bf(inp["router_w"])
        for n in ("w1", "wv", "w2"):
            out[n] = raw(inp[n])
        out["scales"] = (bf(inp["s1"]), bf(inp["sv"]), bf(inp["s2"]))
    else:
        raise ValueError(f"unknown dtype {dtype}")
    b = inp.get("router_bias")
    out["router_bias"] = None if b is None else torch.from_numpy(np.asarray(b, np.float32)).to(device)
    return out


def rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """max |got - want| / rms(want)."""
    rms = float(np.sqrt(np.mean(want.astype(np.float64) ** 2)))
    return float(np.max(np.abs(got.astype(np.float64) - want))) / rms


def rms_rel_err(got: np.ndarray, want: np.ndarray) -> float:
    """rms(got - want) / rms(want)."""
    want = want.astype(np.float64)
    rms = float(np.sqrt(np.mean(want ** 2)))
    return float(np.sqrt(np.mean((got.astype(np.float64) - want) ** 2))) / rms
