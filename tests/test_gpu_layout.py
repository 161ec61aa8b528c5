"""GPU parity of the [E, out, in] weight layout (the converted PyTorch layout) through the C ABI.

The kernels for [out, in] storage multiply the same operands in the same order as those for [in, out] storage,
so on the same weights the two layer outputs must be bit-identical; each case also meets the oracle's bar
(routing exact, out within 1e-2 rms, 1e-4 for fp32) with the oracle reading the [out, in] storage itself."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import TOL, dev_inputs, rel_err, say

pytestmark = pytest.mark.gpu

F32, BF16, W8 = synth.F32, synth.BF16, synth.W8


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


def _t(w):
    return w.transpose(1, 2).contiguous()


def _np_t(a):
    return np.ascontiguousarray(np.swapaxes(a, 1, 2))


def check_layout(gm, w, rows=None, oracle_check=True, inp=None, dv=None):
    say(f"[case] out_in {w.name}: T={w.T} d={w.d} f={w.f} E={w.E} dtype={synth.DTYPE_NAMES[w.dtype]} "
        f"groups=({w.groups_up},{w.groups_down}) scale_experts={w.scale_experts}")
    inp = inp if inp is not None else synth.make_inputs(w)
    dv = dv if dv is not None else dev_inputs(inp, w.dtype)
    ref = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"],
                     router_bias=dv["router_bias"])
    w1t, wvt, w2t = _t(dv["w1"]), _t(dv["wv"]), _t(dv["w2"])
    out, idx, p, cnt = gm.forward(dv["x"], dv["router_w"], w1t, wvt, w2t, scales=dv["scales"],
                                  router_bias=dv["router_bias"], return_routing=True, weight_layout=gm.OUT_IN)
    torch.cuda.synchronize()
    same = torch.equal(out, ref)
    say(f"[result] out_in {w.name}: bit-identical to in_out = {same}")
    assert same
    del w1t, wvt, w2t
    if oracle_check:
        tin = dict(inp)
        for n in ("w1", "wv", "w2"):
            tin[n] = _np_t(inp[n])
        want = oracle.forward(tin, w.dtype, rows=rows, layout=oracle.OUT_IN)
        rows_t = want["rows"].numpy()
        err = rel_err(out.cpu().numpy()[rows_t], want["out"].numpy())
        say(f"[result] out_in {w.name}: vs oracle max_err/rms={err:.3e}")
        assert np.array_equal(idx.cpu().numpy(), want["idx"].numpy())
        assert np.array_equal(cnt.cpu().numpy(), want["counts"].numpy())
        assert err <= TOL[w.dtype]


def _w(name, T, d, f, E=8, dtype=BF16, g1=1, g2=1, es=None):
    return synth.Workload(name, T=T, d=d, f=f, E=E, dtype=dtype, groups_up=g1, groups_down=g2, scale_experts=es)


CASES = [
    _w("oi_bf16_T10", 10, 512, 1024),                      # streaming, one 16-row tile per pass
    _w("oi_bf16_T40", 40, 256, 8192),                      # streaming, two tiles, 4 down chunks
    _w("oi_bf16_T96", 96, 512, 1024),                      # streaming, several passes (largest bf16 batch)
    _w("oi_bf16_T8_share", 8, 6144, 4096),                 # a d_ff share: d split over the waves, both layouts
    _w("oi_bf16_T24_uneven", 24, 256, 6400),               # down chunks of 2048, 2176 and 2176 rows
    _w("oi_bf16_T300", 300, 512, 1024),                    # direct-to-LDS tiles, down K split in 2
    _w("oi_bf16_T700_E4", 700, 768, 1536, E=4),
    _w("oi_bf16_T16_E64_nb8", 16, 256, 8192, E=64),        # 8 column blocks per workgroup, 16-row tiles
    _w("oi_bf16_T40_E64_nb8", 40, 256, 4096, E=64),        # 8 column blocks per workgroup, 32-row tiles
    synth.Workload("oi_bf16_T96_skew_nb8", T=96, d=256, f=32768, router_bias=(4.0, 4.0, 0, 0, 0, 0, 0, 0)),
    # ... 8 blocks, two busy experts in three passes of 32 rows, the other experts few or no rows
    _w("oi_w8_T40", 40, 512, 2048, dtype=W8),              # int8 streaming
    _w("oi_w8_T128", 128, 512, 1024, dtype=W8),            # int8 streaming, several passes
    _w("oi_w8_T300", 300, 512, 1024, dtype=W8),            # int8 register-staged tiles
    _w("oi_w8g_T40", 40, 512, 2048, dtype=W8, g1=4, g2=4),  # grouped scales, streaming
    _w("oi_w8g_T40_straddle", 40, 1024, 1024, dtype=W8, g1=2, g2=2),  # quarters of d inside a scale group
    _w("oi_w8g_T40_uneven", 40, 256, 6400, dtype=W8, g1=2, g2=5),  # a down chunk ends inside a 1280-row group
    _w("oi_w8g_T300_shared", 300, 512, 1024, dtype=W8, g1=2, g2=8, es=1),  # grouped + shared, tiles
    _w("oi_f32_T64", 64, 128, 512, dtype=F32),
    _w("oi_f32_T200", 200, 192, 320, dtype=F32),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
def test_out_in_layer(gm, w):
    check_layout(gm, w)


def test_out_in_steps(gm):
    """The step entry points with [out, in] weights give the [in, out] steps' bits."""
    w = _w("oi_steps", 40, 512, 1024, dtype=W8, g1=2, g2=2)
    inp = synth.make_inputs(w)
    dv = dev_inputs(inp, W8)
    idx, p = gm.route(dv["x"], dv["router_w"])
    counts, offsets, perm, inv = gm.bin_tokens(idx, w.E)
    sc = dv["scales"]
    h_ref = gm.expert_up(dv["x"], dv["w1"], dv["wv"], counts, offsets, perm, scales=sc)
    h = gm.expert_up(dv["x"], _t(dv["w1"]), _t(dv["wv"]), counts, offsets, perm, scales=sc, weight_layout=gm.OUT_IN)
    y_ref = gm.expert_down(h_ref, dv["w2"], counts, offsets, w.T, dv["x"].dtype, s2=sc[2])
    y = gm.expert_down(h_ref, _t(dv["w2"]), counts, offsets, w.T, dv["x"].dtype, s2=sc[2], weight_layout=gm.OUT_IN)
    torch.cuda.synchronize()
    assert torch.equal(h, h_ref) and torch.equal(y, y_ref)


def test_bad_layout_rejected(gm):
    w = _w("oi_bad", 8, 256, 256)
    dv = dev_inputs(synth.make_inputs(w), BF16)
    with pytest.raises(gm.GrokMoeError):
        gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], weight_layout="rows")
    with pytest.raises(gm.GrokMoeError):  # [in, out] shapes declared as [out, in] (d != f)
        w2 = _w("oi_bad2", 8, 256, 512)
        dv2 = dev_inputs(synth.make_inputs(w2), BF16)
        gm.forward(dv2["x"], dv2["router_w"], dv2["w1"], dv2["wv"], dv2["w2"], weight_layout=gm.OUT_IN)


@pytest.mark.parametrize("name", ["decode_bf16", "prefill_bf16", "int8_w8"])
def test_out_in_grok_shape(gm, name):
    """Grok-1 shapes in the launch configuration the benchmark times: [out, in] bit-identical to [in, out]."""
    w = synth.WORKLOADS[name]
    check_layout(gm, w, oracle_check=False)
