"""Pins of the oracle's int8 dequantisation with grouped scales.

Page "Grok-1-BF16", section "Conversion Details": int8 weights times bf16 scales, the scales broadcast over
groups, with scale shapes (1,N), (8,N), (8,1,N) and (8,8,N).  Reading: a weight [E, K, N] takes scales
[Es, G, N] (Es = E per expert, Es = 1 shared; G contiguous groups of K/G input rows); the two-dimensional forms
are [Es, N] with one group.  Each pin below is a fact that holds independently of the oracle's code: a closed
form, a brute-force loop, or an identity between two layouts that describe the same weights."""
import numpy as np
import pytest
import torch

import oracle
import synth


def _bf16_bits(v):
    return synth.f32_to_bf16_bits(np.asarray(v, dtype=np.float32))


def test_group_index_closed_form():
    """q = 1, x_k = k + 1, s[g, n] = 2^g (n + 1), K = 16 in G = 4 groups of 4:
    y[n] = (n + 1) * (1*(1+2+3+4) + 2*(5+..+8) + 4*(9+..+12) + 8*(13+..+16)) = 694 (n + 1).
    Taking the group as k mod G instead of k // (K/G) would give 556 (n + 1)."""
    K, N, G = 16, 3, 4
    q = np.ones((K, N), dtype=np.int8)
    s = _bf16_bits([[2.0 ** g * (n + 1) for n in range(N)] for g in range(G)])
    w = oracle.dequant(q, s)
    x = torch.arange(1, K + 1, dtype=torch.float64)
    y = x @ w
    assert torch.equal(y, torch.tensor([694.0 * (n + 1) for n in range(N)], dtype=torch.float64))


def test_dequant_brute_force_loops():
    """Element by element with explicit loops over (k, n): W[k, n] = q[k, n] * s[k // (K/G), n]."""
    rng = np.random.default_rng(3)
    K, N, G = 12, 5, 3
    q = rng.integers(-127, 128, size=(K, N)).astype(np.int8)
    s = _bf16_bits(rng.uniform(1e-4, 5e-4, size=(G, N)))
    sf = synth.bf16_bits_to_f32(s).astype(np.float64)
    w = oracle.dequant(q, s).numpy()
    for k in range(K):
        for n in range(N):
            assert w[k, n] == float(q[k, n]) * sf[k // (K // G), n]


def test_dequant_rejects_groups_not_dividing_k():
    with pytest.raises(ValueError):
        oracle.dequant(np.ones((10, 2), dtype=np.int8), _bf16_bits(np.ones((3, 2))))


def _tiny_w8(G1=1, G2=1, Es=None, T=24, seed=0):
    w = synth.Workload("tiny_w8", T=T, d=128, f=256, E=4, dtype=synth.W8, groups_up=G1, groups_down=G2,
                       scale_experts=Es, seed=seed)
    return w, synth.make_inputs(w)


def test_groups_with_equal_scales_equal_one_group():
    """Scales repeated across G groups describe the same weights as one group: identical layer output."""
    w, inp = _tiny_w8()
    ref = oracle.forward(inp, synth.W8)
    g = dict(inp)
    g["s1"] = np.repeat(inp["s1"], 4, axis=1)
    g["sv"] = np.repeat(inp["sv"], 4, axis=1)
    g["s2"] = np.repeat(inp["s2"], 8, axis=1)
    got = oracle.forward(g, synth.W8)
    assert torch.equal(got["out"], ref["out"])


def test_shared_scales_equal_repeated_per_expert_scales():
    """A shared [1, G, N] tensor describes the same weights as that tensor repeated for every expert."""
    w, inp = _tiny_w8(G1=2, G2=4, Es=1)
    assert inp["s1"].shape == (1, 2, 256) and inp["s2"].shape == (1, 4, 128)
    ref = oracle.forward(inp, synth.W8)
    rep = dict(inp)
    for n in ("s1", "sv", "s2"):
        rep[n] = np.repeat(inp[n], 4, axis=0)
    assert torch.equal(oracle.forward(rep, synth.W8)["out"], ref["out"])


def test_two_dimensional_forms():
    """(1, N) is [1, 1, N]; (8, N) is [8, 1, N] for the expert weights."""
    w, inp = _tiny_w8()
    ref = oracle.forward(inp, synth.W8)
    per_expert_2d = dict(inp)
    for n in ("s1", "sv", "s2"):
        per_expert_2d[n] = inp[n][:, 0, :]
    assert torch.equal(oracle.forward(per_expert_2d, synth.W8)["out"], ref["out"])
    w1, inp1 = _tiny_w8(Es=1)
    shared_2d = dict(inp1)
    for n in ("s1", "sv", "s2"):
        shared_2d[n] = inp1[n][0]
        assert shared_2d[n].ndim == 2 and shared_2d[n].shape[0] == 1
    assert torch.equal(oracle.forward(shared_2d, synth.W8)["out"], oracle.forward(inp1, synth.W8)["out"])


def test_grouped_layer_against_numpy_brute_force():
    """Whole layer with (E, G, N) scales against a numpy evaluation: dequantise by explicit group slices, route by
    sorting, per-token expert evaluation with scipy's erf, h rounded to bf16."""
    from scipy.special import erf

    w, inp = _tiny_w8(G1=4, G2=2, T=10, seed=5)
    got = oracle.forward(inp, synth.W8)
    f32 = lambda b: synth.bf16_bits_to_f32(b).astype(np.float64)
    x = f32(inp["x"])
    rw = f32(inp["router_w"])
    E, d, f = inp["w1"].shape

    def deq(q, s):
        K = q.shape[0]
        G = s.shape[0]
        out = np.empty(q.shape)
        for g in range(G):
            sl = slice(g * (K // G), (g + 1) * (K // G))
            out[sl] = q[sl].astype(np.float64) * f32(s[g])[None, :]
        return out

    for t in range(x.shape[0]):
        lg = rw @ x[t]
        order = sorted(range(E), key=lambda e: (-lg[e], e))
        pr = np.exp(lg - lg.max())
        pr /= pr.sum()
        o = np.zeros(d)
        for e in order[:2]:
            a = x[t] @ deq(inp["w1"][e], inp["s1"][e])
            b = x[t] @ deq(inp["wv"][e], inp["sv"][e])
            h = 0.5 * a * (1 + erf(a / np.sqrt(2))) * b
            m, ex = np.frexp(h)  # one round-to-nearest-even step to 8 significant bits
            h = np.ldexp(np.round(np.ldexp(m, 8)), ex - 8)
            o += pr[e] * (h @ deq(inp["w2"][e], inp["s2"][e]))
        assert np.allclose(got["out"][t].numpy(), o, rtol=1e-12, atol=1e-12 * np.abs(o).max())
