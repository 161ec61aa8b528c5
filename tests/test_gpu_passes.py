"""GPU parity of a batch that the bf16 and int8 layers run as two passes (h [2 T, f] would pass 2^31 bytes in one).

d = 256, f = 2^18, E = 4: one pass holds at most 2047 tokens, so T = 2100 runs as two passes of 1050 tokens.
Checked: routing and summed counts bit-exact and sampled rows (both passes, both sides of the boundary) within
1e-2 rms(oracle) for the layer and its block form, and every output row bit-identical to running each pass's
tokens as a batch of its own (tokens are independent).  The int8 layer (LDS-tiled int8 kernels on the same 32-bit
offsets) is checked the same way."""
import numpy as np
import pytest
import torch

import synth
from tests._helpers import dev_inputs, say
from tests.test_gpu_block import check_block
from tests.test_gpu_parity import check_layer

pytestmark = pytest.mark.gpu

W = synth.Workload("passes_T2100_f256k", T=2100, d=256, f=1 << 18, E=4)
ROWS = np.array([0, 1, 517, 1048, 1049, 1050, 1051, 1500, 2098, 2099])


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


@pytest.fixture(scope="module")
def data():
    inp = synth.make_inputs(W)
    return inp, dev_inputs(inp, W.dtype)


def test_layout_needs_two_passes(gm):
    assert gm.workspace_size(W.T, W.d, W.f, W.E) == gm.workspace_size(W.T // 2, W.d, W.f, W.E)


def test_forward_in_passes(gm, data):
    inp, dv = data
    check_layer(gm, W, inp=inp, dv=dv, rows=ROWS)


def test_block_forward_in_passes(gm, data):
    inp, dv = data
    check_block(gm, W, inp=inp, dv=dv, rows=ROWS)


def test_passes_equal_separate_batches(gm, data):
    _, dv = data
    args = (dv["router_w"], dv["w1"], dv["wv"], dv["w2"])
    out, idx, p, cnt = gm.forward(dv["x"], *args, return_routing=True)
    half = W.T // 2
    parts = [gm.forward(dv["x"][a:b].contiguous(), *args, return_routing=True) for a, b in ((0, half), (half, W.T))]
    torch.cuda.synchronize()
    say(f"[result] passes: counts {cnt.tolist()} = {parts[0][3].tolist()} + {parts[1][3].tolist()}")
    assert torch.equal(out, torch.cat([parts[0][0], parts[1][0]]))
    assert torch.equal(idx, torch.cat([parts[0][1], parts[1][1]]))
    assert torch.equal(p, torch.cat([parts[0][2], parts[1][2]]))
    assert torch.equal(cnt, parts[0][3] + parts[1][3])


W8 = synth.Workload("passes_w8_T2100_f256k", T=2100, d=256, f=1 << 18, E=4, dtype=synth.W8)


def test_int8_forward_in_passes(gm):
    assert gm.workspace_size(W8.T, W8.d, W8.f, W8.E, 2, gm.W8) == gm.workspace_size(W8.T // 2, W8.d, W8.f, W8.E, 2,
                                                                                     gm.W8)
    inp = synth.make_inputs(W8)
    dv = dev_inputs(inp, W8.dtype)
    check_layer(gm, W8, inp=inp, dv=dv, rows=ROWS)
    args = (dv["router_w"], dv["w1"], dv["wv"], dv["w2"])
    out, idx, p, cnt = gm.forward(dv["x"], *args, scales=dv["scales"], return_routing=True)
    half = W8.T // 2
    parts = [gm.forward(dv["x"][a:b].contiguous(), *args, scales=dv["scales"], return_routing=True)
             for a, b in ((0, half), (half, W8.T))]
    torch.cuda.synchronize()
    assert torch.equal(out, torch.cat([parts[0][0], parts[1][0]]))
    assert torch.equal(cnt, parts[0][3] + parts[1][3])
