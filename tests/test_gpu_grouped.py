"""GPU parity of the int8 layer with grouped scales ([Es, G, out]: per-expert or shared, G groups along the input
axis) against the oracle, through the C ABI.

Bar as for the other layers: routing and counts bit-exact, out within 1e-2 rms(oracle).  Where two layouts
describe the same weights the kernels must agree bit for bit (equal scales in every group change the
accumulators' unit by exactly 1)."""
import dataclasses

import numpy as np
import pytest
import torch

import synth
from tests._helpers import dev_inputs, say
from tests.test_gpu_parity import check_layer

pytestmark = pytest.mark.gpu

W8 = synth.W8


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


def _w(name, T, d, f, E=8, g1=1, g2=1, es=None, seed=0):
    return synth.Workload(name, T=T, d=d, f=f, E=E, dtype=W8, groups_up=g1, groups_down=g2, scale_experts=es,
                          seed=seed)


CASES = [
    # streaming kernels (int8: T <= 128): one and two 16-row tiles per pass, 64-row groups, chunks of the down
    # projection that start inside a group (f = 8192 in 4 chunks of 2048, groups of 4096)
    _w("g_T10_gs64", 10, 512, 1024, g1=8, g2=16),
    _w("g_T40", 40, 512, 2048, g1=2, g2=4),
    _w("g_T40_midchunk", 40, 256, 8192, g1=4, g2=2),
    _w("g_T64_shared", 64, 512, 1024, g1=2, g2=4, es=1),
    _w("g_T128", 128, 512, 1024, g1=4, g2=8),          # the largest int8 streaming batch: several passes
    _w("g_T40_straddle", 40, 1024, 1024, g1=2, g2=2),  # d split in 4 quarters; a 512-row group spans two
    _w("g_T40_uneven", 40, 256, 6400, g1=2, g2=5),      # down chunks 2048, 2176, 2176: one ends inside a group
    # LDS-tiled kernels: 128-row tiles, several tiles and ragged tails, E = 4, group counts 3 and 6
    _w("g_T300", 300, 512, 1024, g1=4, g2=8),
    _w("g_T700_E4", 700, 768, 1536, E=4, g1=3, g2=6),
    _w("g_T200_shared", 200, 512, 1024, g1=2, g2=2, es=1),
    # one group, shared by all experts: the (1, N) form on both kernel families
    _w("g_T24_shared1", 24, 512, 1024, es=1),
    _w("g_T300_shared1", 300, 512, 1024, es=1),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_grouped_layer(gm, w):
    check_layer(gm, w)


def _zero_some(inp, seed):
    """Zero whole scale groups of some columns: the first, a middle and the last group."""
    rng = np.random.default_rng(seed)
    out = dict(inp)
    for n in ("s1", "sv", "s2"):
        s = inp[n].copy()
        Es, G, N = s.shape
        cols = rng.choice(N, size=max(1, N // 16), replace=False)
        for j, c in enumerate(cols):
            s[:, [0, G // 2, G - 1][j % 3], c] = 0
        s[:, :, cols[0]] = 0  # one column with every group zero
        out[n] = s
    return out


@pytest.mark.parametrize("w", [_w("g_zero_T40", 40, 512, 1024, g1=4, g2=4),
                               _w("g_zero_T300", 300, 512, 1024, g1=4, g2=4)], ids=lambda w: w.name)
def test_zero_scales(gm, w):
    inp = _zero_some(synth.make_inputs(w), 7)
    check_layer(gm, w, inp=inp)


@pytest.mark.parametrize("T", [40, 300])
def test_equal_group_scales_match_ungrouped_bitwise(gm, T):
    """Scales repeated over G groups: the grouped kernels give the per-channel path's bits."""
    w = _w(f"g_eq_T{T}", T, 512, 1024)
    inp = synth.make_inputs(w)
    dv = dev_inputs(inp, W8)
    ref = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"])
    s1, sv, s2 = dv["scales"]
    rep = (s1.repeat(1, 4, 1).contiguous(), sv.repeat(1, 4, 1).contiguous(), s2.repeat(1, 8, 1).contiguous())
    got = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=rep)
    torch.cuda.synchronize()
    say(f"[result] equal-group scales T={T}: max |diff| = {(got - ref).abs().max().item():.3e}")
    assert torch.equal(got, ref)


def test_two_dimensional_per_expert_form_is_the_default(gm):
    """(E, N) scales are the per-(expert, channel) layout: same bits as [E, 1, N]."""
    w = _w("g_2d", 40, 512, 1024)
    dv = dev_inputs(synth.make_inputs(w), W8)
    ref = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"])
    flat = tuple(s[:, 0, :].contiguous() for s in dv["scales"])
    got = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=flat)
    torch.cuda.synchronize()
    assert torch.equal(got, ref)


def test_grok_int8_group_scales(gm):
    """Grok-1 shape, T = 64, int8 weights with (8, 8, N) scales, every row against the oracle."""
    check_layer(gm, synth.WORKLOADS["int8_w8_g8"])


def test_grok_int8_group_scales_prefill_sampled(gm):
    """Grok-1 shape, T = 2048 (the direct-to-LDS 128-row tiles with grouped scales), int8 weights with (8, 8, N)
    scales, 64 seeded rows against the oracle."""
    w = dataclasses.replace(synth.WORKLOADS["int8_w8_g8"], T=2048, name="int8_w8_g8_T2048", sampled_rows=64)
    check_layer(gm, w, rows=synth.sampled_rows(w.T, 64))
