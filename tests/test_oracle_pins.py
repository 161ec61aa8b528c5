"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test states what it pins.  Together they are chosen so that a plausible slip in the oracle (a dropped term,
a wrong sign, a swapped GELU branch, a transposed weight, renormalised gates, a reversed tie-break, a missing
max-subtraction, a wrong rounding step) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import ndtr, softmax

import oracle
import synth

F32, BF16, W8 = synth.F32, synth.BF16, synth.W8


def _phi_gelu(z):
    """GELU(z) = z * Phi(z) with scipy's normal CDF (a separate library from the oracle's torch erf)."""
    z = np.asarray(z, dtype=np.float64)
    return z * ndtr(z)


def _dense_geglu(x, w1, wv, w2, round_h=False):
    """One expert evaluated with numpy + scipy only (rows of x through [in,out] weights)."""
    h = _phi_gelu(x @ w1) * (x @ wv)
    if round_h:
        h = oracle.bf16_round(torch.from_numpy(h)).numpy()
    return h @ w2


def _f32_inputs(x, rw, w1, wv, w2, bias=None):
    return {"x": np.asarray(x, np.float32), "router_w": np.asarray(rw, np.float32),
            "w1": np.asarray(w1, np.float32), "wv": np.asarray(wv, np.float32), "w2": np.asarray(w2, np.float32),
            "s1": None, "sv": None, "s2": None,
            "router_bias": None if bias is None else np.asarray(bias, np.float32)}


def _rand_layer(rng, T, d, f, E, scale=1.0):
    x = rng.standard_normal((T, d)).astype(np.float32)
    rw = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    w1 = (scale * rng.standard_normal((E, d, f)) / math.sqrt(d)).astype(np.float32)
    wv = (scale * rng.standard_normal((E, d, f)) / math.sqrt(d)).astype(np.float32)
    w2 = (rng.standard_normal((E, f, d)) / math.sqrt(f)).astype(np.float32)
    return x, rw, w1, wv, w2


# --------------------------------------------------------------------------------------------- GELU

def test_gelu_matches_normal_cdf_table(golden_dir):
    """GELU(z) = z Phi(z): textbook table values of Phi (tests/golden/normal_cdf.json)."""
    tab = json.load(open(os.path.join(golden_dir, "normal_cdf.json")))["phi"]
    z = torch.tensor([float(k) for k in tab], dtype=torch.float64)
    want = z * torch.tensor(list(tab.values()), dtype=torch.float64)
    got = oracle.gelu(z)
    assert torch.allclose(got, want, rtol=1e-12, atol=1e-16)


def test_gelu_identities_and_not_tanh():
    z = torch.linspace(-8, 8, 4001, dtype=torch.float64)
    g = oracle.gelu(z)
    assert oracle.gelu(torch.zeros(1, dtype=torch.float64)).item() == 0.0
    # GELU(z) - GELU(-z) = z  (Phi(z) + Phi(-z) = 1): pins the sign inside erf and the 0.5 factor
    assert torch.allclose(g - oracle.gelu(-z), z, atol=1e-14)
    # GELU(z)/z -> 1 for large z, -> 0 for very negative z
    assert abs(oracle.gelu(torch.tensor([40.0], dtype=torch.float64)).item() / 40.0 - 1) < 1e-15
    assert abs(oracle.gelu(torch.tensor([-40.0], dtype=torch.float64)).item()) < 1e-300
    # agrees with scipy's Phi everywhere; the tanh approximation misses by up to ~4.7e-4 near z = -2.7
    assert np.max(np.abs(g.numpy() - _phi_gelu(z.numpy()))) < 1e-14
    tanh_form = 0.5 * z * (1 + torch.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))
    assert (g - tanh_form).abs().max().item() > 4e-4


# --------------------------------------------------------------------------------------------- bf16 rounding

def test_bf16_round_golden(golden_dir):
    """Hand-derived round-to-nearest-even cases, including one where rounding via float32 would differ."""
    cases = json.load(open(os.path.join(golden_dir, "bf16_rne.json")))["cases"]
    x = torch.tensor([c["in"] for c in cases], dtype=torch.float64)
    want = torch.tensor([c["out"] for c in cases], dtype=torch.float64)
    assert torch.equal(oracle.bf16_round(x), want)


def test_bf16_round_matches_torch_on_float32_values():
    """On values exactly representable in float32, a single rounding equals torch's float32->bfloat16 (RNE)."""
    rng = np.random.default_rng(5)
    v = np.concatenate([rng.standard_normal(200000), rng.standard_normal(2000) * 1e-3,
                        rng.standard_normal(2000) * 1e4]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).to(torch.float64)
    got = oracle.bf16_round(torch.from_numpy(v).to(torch.float64))
    assert torch.equal(got, want)


# --------------------------------------------------------------------------------------------- routing

def test_zero_router_uniform_probs_and_tie_break():
    """router_w = 0: all logits tie, p = 1/8 each, and the lower-index rule picks (0, 1) for every token."""
    rng = np.random.default_rng(0)
    x, rw, w1, wv, w2 = _rand_layer(rng, 16, 8, 16, 8)
    r = oracle.forward(_f32_inputs(x, np.zeros_like(rw), w1, wv, w2), F32)
    assert torch.equal(r["idx"], torch.tensor([[0, 1]] * 16))
    assert torch.allclose(r["p"], torch.full((16, 2), 1 / 8, dtype=torch.float64), rtol=0, atol=1e-16)
    assert torch.equal(r["counts"], torch.tensor([16, 16, 0, 0, 0, 0, 0, 0]))


def test_uniform_routing_entropy_is_ln8():
    """Uniform routing over 8 experts has entropy ln 8 = 2.079, the maximum the bridge README's demo prints
    (page "A functional bridge between openai/grok and xai-org/grok-1", the expected --demo output)."""
    x = np.ones((4, 8), np.float32)
    r = oracle.route(torch.from_numpy(x).double(), torch.zeros((8, 8), dtype=torch.float64))
    pr = r["probs"]
    ent = -(pr * pr.log()).sum(dim=1)
    assert torch.allclose(ent, torch.full((4,), math.log(8), dtype=torch.float64))
    assert round(math.log(8), 3) == 2.079


def test_bias_only_router_is_softmax_of_bias():
    """router_w = 0 and a bias b: probabilities are softmax(b) (scipy), selection is the two largest b."""
    b = np.array([0.3, -1.0, 2.5, 0.0, 1.25, -0.5, 2.0, 0.1], np.float32)
    x = np.ones((3, 4), np.float32)
    r = oracle.route(torch.from_numpy(x).double(), torch.zeros((8, 4), dtype=torch.float64),
                     torch.from_numpy(b).double())
    sm = softmax(b.astype(np.float64))
    assert np.allclose(r["probs"].numpy(), np.tile(sm, (3, 1)), rtol=1e-15, atol=0)
    assert torch.equal(r["idx"], torch.tensor([[2, 6]] * 3))
    assert np.allclose(r["p"].numpy(), np.tile(sm[[2, 6]], (3, 1)), rtol=1e-15)


def test_partial_ties_keep_lower_index_first():
    x = torch.ones((1, 2), dtype=torch.float64)
    z = torch.zeros((8, 2), dtype=torch.float64)
    for bias, want in [([0, 5, 5, 5, 0, 0, 0, 0], [1, 2]), ([5, 0, 5, 0, 0, 0, 0, 0], [0, 2]),
                       ([0, 0, 0, 0, 0, 0, 0, 5], [7, 0]), ([0, 0, 0, 0, 0, 0, 5, 5], [6, 7])]:
        r = oracle.route(x, z, torch.tensor(bias, dtype=torch.float64))
        assert r["idx"][0].tolist() == want, bias


def test_saturated_router_selects_known_experts():
    """Bias +60 on expert a and +50 on b (router_w = 0): idx = (a, b), p_a = 1/(1+e^-10+6e^-60), p_b = e^-10 p_a."""
    a, bb = 5, 2
    bias = np.zeros(8)
    bias[a], bias[bb] = 60.0, 50.0
    x = torch.ones((2, 3), dtype=torch.float64)
    r = oracle.route(x, torch.zeros((8, 3), dtype=torch.float64), torch.from_numpy(bias))
    pa = 1.0 / (1.0 + math.exp(-10) + 6 * math.exp(-60))
    assert r["idx"].tolist() == [[a, bb]] * 2
    assert abs(r["p"][0, 0].item() - pa) < 1e-15
    assert abs(r["p"][0, 1].item() - math.exp(-10) * pa) < 1e-18


def test_huge_logits_do_not_overflow():
    """A logit of 1000 would overflow exp() without subtracting the maximum first."""
    bias = torch.zeros(8, dtype=torch.float64)
    bias[3] = 1000.0
    r = oracle.route(torch.ones((1, 2), dtype=torch.float64), torch.zeros((8, 2), dtype=torch.float64), bias)
    assert torch.isfinite(r["probs"]).all()
    assert r["idx"][0].tolist() == [3, 0]
    assert r["p"][0, 0].item() == 1.0


def test_routing_brute_force_tiny():
    """Per-token brute force: logits by explicit sums, all experts sorted by (-logit, index), softmax by math.exp."""
    rng = np.random.default_rng(11)
    T, d, E = 40, 12, 8
    x = rng.standard_normal((T, d))
    rw = rng.standard_normal((E, d)) / math.sqrt(d)
    r = oracle.route(torch.from_numpy(x), torch.from_numpy(rw))
    for t in range(T):
        logits = [sum(x[t, i] * rw[e, i] for i in range(d)) for e in range(E)]
        order = sorted(range(E), key=lambda e: (-logits[e], e))
        m = max(logits)
        den = sum(math.exp(v - m) for v in logits)
        assert r["idx"][t].tolist() == order[:2]
        for j in range(2):
            assert abs(r["p"][t, j].item() - math.exp(logits[order[j]] - m) / den) < 1e-14
        p1, p2 = r["p"][t].tolist()
        assert p1 >= p2 and 0 < p1 + p2 <= 1


def test_gate_sum_bounds_on_tiny_workload():
    inp = synth.make_inputs(synth.WORKLOADS["tiny_f32"])
    r = oracle.forward(inp, F32)
    s = r["p"].sum(dim=1)
    assert (s > 0).all() and (s <= 1).all() and (r["p"][:, 0] >= r["p"][:, 1]).all()
    assert (r["idx"][:, 0] != r["idx"][:, 1]).all()
    assert r["counts"].sum().item() == 2 * 64


# --------------------------------------------------------------------------------------------- expert FFN

def test_identity_experts_closed_form():
    """d = f, W1 = Wv = W2 = I: each expert returns GELU(x) * x elementwise."""
    rng = np.random.default_rng(2)
    d = 6
    x = rng.standard_normal((5, d))
    eye = np.eye(d)
    _, y = oracle.expert_ffn(torch.from_numpy(x), *(torch.from_numpy(eye),) * 3, round_h=False)
    assert np.allclose(y.numpy(), _phi_gelu(x) * x, rtol=1e-14, atol=1e-15)


def test_gelu_goes_on_the_w1_branch():
    """W1 = I, Wv = 2I: h = GELU(x) * 2x; with the branches swapped it would be GELU(2x) * x."""
    rng = np.random.default_rng(3)
    d = 5
    x = rng.standard_normal((4, d))
    eye = np.eye(d)
    _, y = oracle.expert_ffn(torch.from_numpy(x), torch.from_numpy(eye), torch.from_numpy(2 * eye),
                             torch.from_numpy(eye), round_h=False)
    assert np.allclose(y.numpy(), _phi_gelu(x) * 2 * x, rtol=1e-14, atol=1e-15)
    assert not np.allclose(y.numpy(), _phi_gelu(2 * x) * x, rtol=1e-3)


def test_weights_are_in_out_layout():
    """d = 3, f = 7 selection matrices: W1[i, 2i] = 1, Wv[i, 2i] = 3, W2[2i, i] = 1 give y_i = 3 GELU(x_i) x_i.
    Reading any weight as [out, in] breaks the shapes or the values."""
    d, f = 3, 7
    w1 = np.zeros((d, f))
    wv = np.zeros((d, f))
    w2 = np.zeros((f, d))
    for i in range(d):
        w1[i, 2 * i] = 1.0
        wv[i, 2 * i] = 3.0
        w2[2 * i, i] = 1.0
    w1[0, 5] = 7.0  # column 5 is never read back by W2: must not leak into the output
    x = np.array([[0.5, -1.0, 2.0], [1.0, 0.0, -0.5]])
    h, y = oracle.expert_ffn(torch.from_numpy(x), torch.from_numpy(w1), torch.from_numpy(wv), torch.from_numpy(w2),
                             round_h=False)
    assert h.shape == (2, f)
    assert np.allclose(y.numpy(), 3 * _phi_gelu(x) * x, rtol=1e-14, atol=1e-15)


def test_h_rounding_closed_form():
    """bf16 layer with identity weights and x = 1: h = Phi(1) = 0.84134..., rounded once to bf16 = 215/256."""
    one = np.float32(1.0)
    d = 8
    x = np.full((1, d), one, np.float32)
    eye = np.eye(d, dtype=np.float32)
    bits = synth.f32_to_bf16_bits
    inp = {"x": bits(x), "router_w": bits(np.zeros((8, d), np.float32)),
           "w1": bits(np.stack([eye] * 8)), "wv": bits(np.stack([eye] * 8)), "w2": bits(np.stack([eye] * 8)),
           "s1": None, "sv": None, "s2": None, "router_bias": None}
    r = oracle.forward(inp, BF16, return_h=True)
    assert torch.all(r["h"] == 215 / 256)
    assert torch.allclose(r["out"], torch.full((1, d), 2 * (215 / 256) / 8, dtype=torch.float64), rtol=1e-15)
    r32 = oracle.forward({k: (v if v is None or k == "router_bias" else synth.bf16_bits_to_f32(v))
                          for k, v in inp.items()}, F32, return_h=True)
    assert torch.allclose(r32["h"], torch.full_like(r32["h"], 0.8413447460685429), rtol=1e-15)


# --------------------------------------------------------------------------------------------- combine

def test_identical_experts_scale_by_gate_sum():
    """All experts equal: out = expert(x) * (p1 + p2), expert(x) from numpy/scipy."""
    rng = np.random.default_rng(4)
    T, d, f, E = 24, 10, 14, 8
    x, rw, w1, wv, w2 = _rand_layer(rng, T, d, f, E)
    w1[:] = w1[0]
    wv[:] = wv[0]
    w2[:] = w2[0]
    r = oracle.forward(_f32_inputs(x, rw, w1, wv, w2), F32)
    y = _dense_geglu(x.astype(np.float64), w1[0].astype(np.float64), wv[0].astype(np.float64),
                     w2[0].astype(np.float64))
    want = y * r["p"].sum(dim=1, keepdim=True).numpy()
    assert np.allclose(r["out"].numpy(), want, rtol=1e-12, atol=1e-13)


def test_zero_router_combine_is_one_eighth_of_first_two_experts():
    """router_w = 0: out = (E0(x) + E1(x)) / 8 -- renormalised gates would give / 2, a reversed tie-break E6+E7."""
    rng = np.random.default_rng(6)
    T, d, f, E = 9, 6, 10, 8
    x, rw, w1, wv, w2 = _rand_layer(rng, T, d, f, E)
    r = oracle.forward(_f32_inputs(x, np.zeros_like(rw), w1, wv, w2), F32)
    x64 = x.astype(np.float64)
    e = [_dense_geglu(x64, w1[i].astype(np.float64), wv[i].astype(np.float64), w2[i].astype(np.float64))
         for i in range(E)]
    assert np.allclose(r["out"].numpy(), (e[0] + e[1]) / 8, rtol=1e-12, atol=1e-13)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(7)
    x, rw, w1, wv, w2 = _rand_layer(rng, 30, 8, 12, 8)
    perm = rng.permutation(30)
    r = oracle.forward(_f32_inputs(x, rw, w1, wv, w2), F32)
    rp = oracle.forward(_f32_inputs(x[perm], rw, w1, wv, w2), F32)
    assert torch.equal(rp["idx"], r["idx"][perm])
    assert torch.allclose(rp["out"], r["out"][perm], rtol=1e-13, atol=1e-14)


def test_linearity_in_wv_and_w2():
    """fp32 layer: scaling Wv or W2 by c scales the output by c (GELU sees only x W1)."""
    rng = np.random.default_rng(8)
    x, rw, w1, wv, w2 = _rand_layer(rng, 20, 8, 12, 8)
    base = oracle.forward(_f32_inputs(x, rw, w1, wv, w2), F32)["out"]
    for c in (2.0, -0.5):
        o1 = oracle.forward(_f32_inputs(x, rw, w1, c * wv, w2), F32)["out"]
        o2 = oracle.forward(_f32_inputs(x, rw, w1, wv, c * w2), F32)["out"]
        assert torch.allclose(o1, c * base, rtol=1e-12, atol=1e-13)
        assert torch.allclose(o2, c * base, rtol=1e-12, atol=1e-13)
    # not linear in W1
    o3 = oracle.forward(_f32_inputs(x, rw, 2 * w1, wv, w2), F32)["out"]
    assert not torch.allclose(o3, 2 * base, rtol=1e-3)


def test_whole_layer_brute_force_tiny():
    """Brute force with numpy/scipy: evaluate all 8 experts on every token, sort experts per token by
    (-logit, index), weight the top two by their full-softmax probability."""
    rng = np.random.default_rng(9)
    T, d, f, E = 17, 8, 12, 8
    x, rw, w1, wv, w2 = _rand_layer(rng, T, d, f, E)
    r = oracle.forward(_f32_inputs(x, rw, w1, wv, w2), F32)
    x64 = x.astype(np.float64)
    all_y = np.stack([_dense_geglu(x64, w1[e].astype(np.float64), wv[e].astype(np.float64),
                                   w2[e].astype(np.float64)) for e in range(E)], axis=1)  # [T, E, d]
    logits = x64 @ rw.astype(np.float64).T
    probs = softmax(logits, axis=1)
    want = np.zeros((T, d))
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:2]
        assert r["idx"][t].tolist() == order
        want[t] = sum(probs[t, e] * all_y[t, e] for e in order)
    assert np.allclose(r["out"].numpy(), want, rtol=1e-12, atol=1e-13)


def test_sampled_rows_equal_full_rows():
    inp = synth.make_inputs(synth.WORKLOADS["tiny_f32"])
    full = oracle.forward(inp, F32)
    rows = synth.sampled_rows(64, 13)
    part = oracle.forward(inp, F32, rows=rows)
    assert torch.equal(part["idx"], full["idx"])
    assert torch.allclose(part["out"], full["out"][torch.from_numpy(rows)], rtol=1e-13, atol=1e-15)


def test_worked_example_by_hand():
    """T = 1, d = f = 1, E = 3: x = 1, gate rows (2, 1, 0) -> logits (2, 1, 0); W1 = W2 = 1, Wv_e = e + 1.
    Selected (0, 1) with p = e^2/S and e/S, S = e^2 + e + 1; out = Phi(1) (p0 + 2 p1).
    Phi(1) from the normal table, exponentials from math."""
    phi1 = 0.8413447460685429
    inp = _f32_inputs([[1.0]], [[2.0], [1.0], [0.0]], np.ones((3, 1, 1)), np.array([1.0, 2.0, 3.0]).reshape(3, 1, 1),
                      np.ones((3, 1, 1)))
    r = oracle.forward(inp, F32)
    S = math.e ** 2 + math.e + 1
    p0, p1 = math.e ** 2 / S, math.e / S
    assert r["idx"].tolist() == [[0, 1]]
    assert abs(r["p"][0, 0].item() - p0) < 1e-15 and abs(r["p"][0, 1].item() - p1) < 1e-15
    assert abs(r["out"][0, 0].item() - phi1 * (p0 + 2 * p1)) < 1e-15


# --------------------------------------------------------------------------------------------- int8 weights

def _w8_layer(rng, T, d, f, E, unit_scales):
    bits = synth.f32_to_bf16_bits
    x = bits(rng.standard_normal((T, d)).astype(np.float32))
    rw = bits((rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32))
    q = [rng.integers(-127, 128, size=s, dtype=np.int8) for s in ((E, d, f), (E, d, f), (E, f, d))]
    if unit_scales:
        sc = [np.full(s, 0x3F80, np.uint16) for s in ((E, 1, f), (E, 1, f), (E, 1, d))]
    else:
        sc = [bits(rng.uniform(1e-4, 5e-4, size=s).astype(np.float32)) for s in ((E, 1, f), (E, 1, f), (E, 1, d))]
    return {"x": x, "router_w": rw, "w1": q[0], "wv": q[1], "w2": q[2], "s1": sc[0], "sv": sc[1], "s2": sc[2],
            "router_bias": None}


def test_int8_unit_scales_equal_bf16_layer():
    """Scales all 1.0: the int8 layer equals the bf16 layer whose weights are the same integers (|q| <= 127 is
    exact in bf16)."""
    rng = np.random.default_rng(12)
    inp = _w8_layer(rng, 20, 16, 24, 8, unit_scales=True)
    r8 = oracle.forward(inp, W8)
    as_bf16 = dict(inp)
    for n in ("w1", "wv", "w2"):
        as_bf16[n] = synth.f32_to_bf16_bits(inp[n].astype(np.float32))
    rb = oracle.forward(as_bf16, BF16)
    assert torch.equal(r8["idx"], rb["idx"])
    assert torch.equal(r8["out"], rb["out"])


def test_int8_scales_per_output_channel():
    """General scales: equals a numpy evaluation with W[e, i, n] = q[e, i, n] * s[e, 0, n] (broadcast over the
    input axis), h rounded once to bf16."""
    rng = np.random.default_rng(13)
    T, d, f, E = 12, 16, 24, 8
    inp = _w8_layer(rng, T, d, f, E, unit_scales=False)
    r = oracle.forward(inp, W8)
    f32 = synth.bf16_bits_to_f32
    x = f32(inp["x"]).astype(np.float64)
    W = {n: inp[n].astype(np.float64) * f32(inp[s]).astype(np.float64) for n, s in
         (("w1", "s1"), ("wv", "sv"), ("w2", "s2"))}
    want = np.zeros((T, 16))
    p = r["p"].numpy()
    for t in range(T):
        for j, e in enumerate(r["idx"][t].tolist()):
            want[t] += p[t, j] * _dense_geglu(x[t:t + 1], W["w1"][e], W["wv"][e], W["w2"][e], round_h=True)[0]
    assert np.allclose(r["out"].numpy(), want, rtol=1e-12, atol=1e-12)
    # scales applied on the output axis: swapping in a transposed broadcast changes the result
    assert not np.allclose(W["w1"][0], inp["w1"][0].astype(np.float64) * f32(inp["s1"][0]).reshape(-1)[:d, None])


# --------------------------------------------------------------------------------------------- shapes

def test_grok1_shapes_reproduce_printed_counts(golden_dir):
    """The page's per-layer shapes give 4,919,992,320 parameters ('4,920M'), 33 tensors, and 4-layer shards of
    39.36 GB in bf16; the Grok-1-shape workloads use the same d, f and E."""
    g = json.load(open(os.path.join(golden_dir, "grok1_layer_shapes.json")))
    shp = g["torch_out_in_shapes"]
    E = g["experts"]
    n_params = 0
    n_tensors = 0
    for name, s in shp.items():
        mult = E if ".experts.E." in name else 1
        n_params += mult * int(np.prod(s))
        n_tensors += mult
    pr = g["printed"]
    assert n_tensors == pr["tensors_per_layer"]
    assert round(n_params / 1e6) == pr["parameters_per_layer_millions"]
    per_shard = pr["layers"] // pr["layer_shards"]
    assert round(per_shard * n_params * 2 / 1e9, 2) == pr["layer_shard_gigabytes"]
    f, d = shp["moe_block.experts.E.linear.weight"]
    for wname in ("decode_bf16", "prefill_bf16", "int8_w8", "skew_bf16"):
        w = synth.WORKLOADS[wname]
        assert (w.d, w.f, w.E) == (d, f, E) == (pr["hidden"], 32768, 8)


def test_round_h_switch_is_the_plain_definition():
    """forward(round_h=False) on a bf16 layer is the unrounded definition (numpy/scipy evaluation of the exact
    stored values, no rounding anywhere); round_h=True on the same inputs rounds each h value to bf16, which the
    closed form of test_h_rounding_closed_form pins; the default keeps the rounding for bf16 and int8 and not for
    fp32."""
    rng = np.random.default_rng(31)
    T, d, f, E = 11, 8, 16, 8
    x, rw, w1, wv, w2 = _rand_layer(rng, T, d, f, E, scale=2.0)
    bits = synth.f32_to_bf16_bits
    inp = {"x": bits(x), "router_w": bits(rw), "w1": bits(w1), "wv": bits(wv), "w2": bits(w2),
           "s1": None, "sv": None, "s2": None, "router_bias": None}
    val = {n: synth.bf16_bits_to_f32(inp[n]).astype(np.float64) for n in ("x", "router_w", "w1", "wv", "w2")}
    plain = oracle.forward(inp, BF16, round_h=False)
    rounded = oracle.forward(inp, BF16, round_h=True)
    default = oracle.forward(inp, BF16)
    assert torch.equal(default["out"], rounded["out"])
    logits = val["x"] @ val["router_w"].T
    probs = softmax(logits, axis=1)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-logits[t, e], e))[:2]
        want = sum(probs[t, e] * _dense_geglu(val["x"][t:t + 1], val["w1"][e], val["wv"][e], val["w2"][e])[0]
                   for e in order)
        want_r = sum(probs[t, e] * _dense_geglu(val["x"][t:t + 1], val["w1"][e], val["wv"][e], val["w2"][e],
                                                round_h=True)[0] for e in order)
        assert np.allclose(plain["out"][t].numpy(), want, rtol=1e-12, atol=1e-13)
        assert np.allclose(rounded["out"][t].numpy(), want_r, rtol=1e-12, atol=1e-13)
    assert not torch.allclose(plain["out"], rounded["out"], rtol=1e-6, atol=0)  # the rounding is visible
    # fp32 layer: the default does not round, round_h=True does
    f32 = _f32_inputs(x, rw, w1, wv, w2)
    assert torch.equal(oracle.forward(f32, F32)["out"], oracle.forward(f32, F32, round_h=False)["out"])
    assert not torch.equal(oracle.forward(f32, F32)["out"], oracle.forward(f32, F32, round_h=True)["out"])
