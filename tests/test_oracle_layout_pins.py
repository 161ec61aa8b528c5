"""Pins of the oracle's [out, in] weight layout (page "Grok-1-BF16", section "Conversion Details": the conversion
transposes the weights from JAX [in, out] to the PyTorch [out, in] convention).

A closed form with selection matrices (d != f, so a transpose in the wrong place cannot even be shaped right),
and the identity that storing every weight transposed and declaring the layout leaves the layer unchanged, for
bf16, int8 with grouped scales and fp32."""
import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_selection_matrices_closed_form():
    """W1t[e, n, k] = Wvt[e, n, k] = [k == s1(n)], W2t[e, m, n] = [n == s2(m)] for every expert (stored [out, in]).
    Then h[n] = GELU(x[s1(n)]) x[s1(n)] (rounded to bf16), y[m] = h[s2(m)], and with identical experts
    out = (p1 + p2) y."""
    T, d, f, E = 3, 8, 12, 4
    rng = np.random.default_rng(11)
    s1 = rng.integers(0, d, size=f)   # input coordinate read by up-projection column n
    s2 = rng.integers(0, f, size=d)   # h coordinate read by output column m
    w1t = np.zeros((E, f, d), np.float32)
    w2t = np.zeros((E, d, f), np.float32)
    for e in range(E):
        w1t[e, np.arange(f), s1] = 1.0
        w2t[e, np.arange(d), s2] = 1.0
    x = rng.standard_normal((T, d)).astype(np.float32)
    rw = rng.standard_normal((E, d)).astype(np.float32) * 0.3
    inp = {"x": _bf16(x), "router_w": _bf16(rw), "w1": _bf16(w1t), "wv": _bf16(w1t), "w2": _bf16(w2t),
           "s1": None, "sv": None, "s2": None, "router_bias": None}
    got = oracle.forward(inp, synth.BF16, layout=oracle.OUT_IN)
    xb = synth.bf16_bits_to_f32(inp["x"]).astype(np.float64)
    for t in range(T):
        z = xb[t, s1]
        h = np.array([0.5 * v * (1 + math.erf(v / math.sqrt(2))) * v for v in z])
        m_, ex = np.frexp(h)
        h = np.ldexp(np.round(np.ldexp(m_, 8)), ex - 8)  # one rounding to bf16 (nearest even)
        y = h[s2]
        p = got["p"][t].numpy()
        assert np.allclose(got["out"][t].numpy(), (p[0] + p[1]) * y, rtol=1e-13, atol=1e-300)


def _transposed(inp):
    out = dict(inp)
    for n in ("w1", "wv", "w2"):
        out[n] = np.ascontiguousarray(np.swapaxes(inp[n], 1, 2))
    return out


@pytest.mark.parametrize("dtype,g1,g2", [(synth.BF16, 1, 1), (synth.W8, 4, 2), (synth.W8, 1, 1), (synth.F32, 1, 1)])
def test_transposed_storage_is_the_same_layer(dtype, g1, g2):
    w = synth.Workload("lay", T=20, d=128, f=256, E=4, dtype=dtype, groups_up=g1, groups_down=g2)
    inp = synth.make_inputs(w)
    ref = oracle.forward(inp, dtype)
    got = oracle.forward(_transposed(inp), dtype, layout=oracle.OUT_IN)
    assert torch.equal(got["out"], ref["out"])
    assert torch.equal(got["idx"], ref["idx"])


def test_grouped_scales_follow_the_input_axis_in_out_in_storage():
    """Grouping along the stored rows (the out axis of [out, in] storage) instead of the input axis changes the
    layer: a closed-form check of one expert, q = 1 stored [out, in], s[g, n] = 2^g, x_k = k + 1."""
    K, N, G = 16, 4, 4
    qt = np.ones((N, K), np.int8)          # [out, in]
    s = _bf16([[2.0 ** g] * N for g in range(G)])
    w = oracle.dequant(oracle.stored_in_out(qt, oracle.OUT_IN), s)  # [in, out]
    y = torch.arange(1, K + 1, dtype=torch.float64) @ w
    assert torch.equal(y, torch.full((N,), 694.0, dtype=torch.float64))


def test_unknown_layout_rejected():
    with pytest.raises(ValueError):
        oracle.stored_in_out(np.zeros((2, 2)), "rows")
