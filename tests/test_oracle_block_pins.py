"""Pins of the oracle's MoE block (pre-MoE RMSNorm -> MoE -> post-MoE RMSNorm -> residual add)."""
import math

import numpy as np
import pytest
import torch
from scipy.special import ndtr

import oracle
import synth

F32, BF16 = synth.F32, synth.BF16


def test_rmsnorm_3_4_5_triangle():
    """x = (3, 4): mean of squares 12.5, so x / rms = x sqrt(2) / 5 = (0.6 sqrt 2, 0.8 sqrt 2)."""
    x = torch.tensor([[3.0, 4.0]], dtype=torch.float64)
    y = oracle.rmsnorm(x, torch.ones(2, dtype=torch.float64), 0.0)
    assert torch.allclose(y, torch.tensor([[0.6 * math.sqrt(2), 0.8 * math.sqrt(2)]], dtype=torch.float64),
                          rtol=1e-15)


def test_rmsnorm_constant_rows_and_scale_invariance():
    g = torch.tensor([0.5, -2.0, 3.0, 1.0], dtype=torch.float64)
    for c in (2.0, -7.5, 1e-3):
        y = oracle.rmsnorm(torch.full((1, 4), c, dtype=torch.float64), g, 0.0)
        assert torch.allclose(y, math.copysign(1.0, c) * g[None, :], rtol=1e-15)
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal((5, 16)))
    g1 = torch.ones(16, dtype=torch.float64)
    for a in (0.01, 3.0, 1e4):
        assert torch.allclose(oracle.rmsnorm(a * x, g1, 0.0), oracle.rmsnorm(x, g1, 0.0), rtol=1e-13)


def test_rmsnorm_eps_closed_form_and_zero_row():
    rng = np.random.default_rng(1)
    x = torch.from_numpy(rng.standard_normal((6, 32)))
    g = torch.ones(32, dtype=torch.float64)
    eps = 0.25
    y = oracle.rmsnorm(x, g, eps)
    ms = (x * x).mean(dim=1)
    assert torch.allclose((y * y).mean(dim=1), ms / (ms + eps), rtol=1e-13)
    z = oracle.rmsnorm(torch.zeros((1, 32), dtype=torch.float64), g, 1e-5)
    assert torch.equal(z, torch.zeros_like(z))


def _f32_block_inputs(rng, T, d, f, E):
    x = rng.standard_normal((T, d)).astype(np.float32)
    rw = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    w1 = (rng.standard_normal((E, d, f)) / math.sqrt(d)).astype(np.float32)
    wv = (rng.standard_normal((E, d, f)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((E, f, d)) / math.sqrt(f)).astype(np.float32)
    return {"x": x, "router_w": rw, "w1": w1, "wv": wv, "w2": w2, "s1": None, "sv": None, "s2": None,
            "router_bias": None}


def test_block_zero_post_scale_is_identity():
    rng = np.random.default_rng(2)
    inp = _f32_block_inputs(rng, 10, 8, 12, 8)
    g = (1 + rng.random(8)).astype(np.float32)
    r = oracle.block_forward(inp, F32, g, np.zeros(8, np.float32), 1e-5)
    assert torch.equal(r["out"], oracle.as_f64(inp["x"], "f32"))


def test_block_against_numpy():
    """Block = x + RMSNorm_post(MoE(RMSNorm_pre(x))) with numpy/scipy: zero router (experts 0 and 1, p = 1/8),
    so MoE(v) = (E0(v) + E1(v)) / 8 with E_e(v) = (v W1 Phi(v W1)) * (v Wv) W2."""
    rng = np.random.default_rng(3)
    T, d, f, E = 9, 8, 12, 8
    inp = _f32_block_inputs(rng, T, d, f, E)
    inp["router_w"] = np.zeros_like(inp["router_w"])
    gp = (0.5 + rng.random(d)).astype(np.float32)
    gq = (0.5 + rng.random(d)).astype(np.float32)
    eps = 1e-3
    r = oracle.block_forward(inp, F32, gp, gq, eps)
    x = inp["x"].astype(np.float64)
    xn = x / np.sqrt((x * x).mean(axis=1, keepdims=True) + eps) * gp.astype(np.float64)
    xn = xn.astype(np.float32).astype(np.float64)  # the fp32 layer stores the normed input in float32
    def expert(e):
        a = xn @ inp["w1"][e].astype(np.float64)
        return (a * ndtr(a) * (xn @ inp["wv"][e].astype(np.float64))) @ inp["w2"][e].astype(np.float64)
    moe = (expert(0) + expert(1)) / 8
    want = x + moe / np.sqrt((moe * moe).mean(axis=1, keepdims=True) + eps) * gq.astype(np.float64)
    assert np.allclose(r["out"].numpy(), want, rtol=1e-12, atol=1e-12)


def test_block_bf16_normed_input_is_rounded_once():
    rng = np.random.default_rng(4)
    w = synth.Workload("blk", T=6, d=256, f=256, w_std=0.1)
    inp = synth.make_inputs(w)
    g = synth.f32_to_bf16_bits((0.5 + rng.random(256)).astype(np.float32))
    r = oracle.block_forward(inp, BF16, g, g, 1e-5)
    x = oracle.as_f64(inp["x"], "bf16")
    exact = oracle.rmsnorm(x, oracle.as_f64(g, "bf16"), 1e-5)
    assert torch.equal(r["xn"], oracle.bf16_round(exact))
