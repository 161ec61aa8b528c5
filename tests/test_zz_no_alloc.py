"""The allocation-free entry point grok_moe_forward_noalloc, through the C ABI, against grok_moe_forward.

For callers that cannot allocate (graph capture, tight serving loops): the workspace is the library's static
scratch array.  Each case makes two calls in a row on the same GPU, the second with a smaller batch (the array keeps
the first call's contents), and checks routing, counts, probabilities and the output bit-identical to
grok_moe_forward on the same inputs, which the parity tests hold to the oracle; one case is also checked against
the oracle directly.  A batch beyond the array is rejected on the host with nothing written."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import TOL, dev_inputs, rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(gm, dv, T, d, f, E, dt):
    """One call of grok_moe_forward_noalloc through ctypes; outputs start as sentinels."""
    out = torch.full((T, d), 7.0, dtype=torch.float32, device="cuda")
    idx = torch.full((T, 2), -9, dtype=torch.int32, device="cuda")
    pr = torch.full((T, 2), -1.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((E,), -9, dtype=torch.int32, device="cuda")
    s1, sv, s2 = dv["scales"] if dv["scales"] is not None else (None, None, None)
    st = gm.lib().grok_moe_forward_noalloc(_p(dv["x"]), _p(dv["router_w"]), _p(dv["w1"]), _p(dv["wv"]), _p(dv["w2"]),
                                           _p(s1), _p(sv), _p(s2), T, d, f, E, 2, dt, _p(out),
                                           _p(dv["router_bias"]), _p(idx), _p(pr), _p(cnt),
                                           ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return st, out, idx, pr, cnt


def _check_pair(gm, name, w_big, w_small, against_oracle=False):
    results = []
    for w in (w_big, w_small):
        say(f"[case] noalloc {name}: T={w.T} d={w.d} f={w.f} E={w.E} dtype={synth.DTYPE_NAMES[w.dtype]}")
        inp = synth.make_inputs(w)
        dv = dev_inputs(inp, w.dtype)
        st, out, idx, pr, cnt = _noalloc(gm, dv, w.T, w.d, w.f, w.E, w.dtype)
        assert st == 0, gm.strerror(st)
        results.append((w, inp, dv, out, idx, pr, cnt))
    torch.cuda.synchronize()
    for w, inp, dv, out, idx, pr, cnt in results:
        ref = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"],
                         router_bias=dv["router_bias"], return_routing=True)
        torch.cuda.synchronize()
        same = [torch.equal(a, b) for a, b in zip((out, idx, pr, cnt), ref)]
        say(f"[result] noalloc {name} T={w.T}: equal to grok_moe_forward (out, idx, p, counts) = {same}")
        assert all(same)
        if against_oracle:
            o = oracle.forward(inp, w.dtype)
            assert np.array_equal(idx.cpu().numpy(), o["idx"].numpy())
            assert np.array_equal(cnt.cpu().numpy(), o["counts"].numpy())
            err = rel_err(out.cpu().numpy(), o["out"].numpy())
            say(f"[result] noalloc {name} T={w.T}: max err / rms against the oracle {err:.2e}")
            assert err <= TOL[w.dtype]


def test_noalloc_streaming_bf16(gm):
    _check_pair(gm, "stream_bf16", synth.Workload("na1", T=40, d=256, f=4096, w_std=0.1),
                synth.Workload("na2", T=8, d=256, f=4096, w_std=0.1), against_oracle=True)


def test_noalloc_tiled_bf16(gm):
    _check_pair(gm, "tiled_bf16", synth.Workload("na3", T=300, d=256, f=512, w_std=0.1,
                                                 router_bias=(3, 0, 0, 0, 0, 1.5, 0, 0)),
                synth.Workload("na4", T=100, d=256, f=512, w_std=0.1))


def test_noalloc_int8(gm):
    _check_pair(gm, "int8", synth.Workload("na5", T=200, d=256, f=768, dtype=synth.W8),
                synth.Workload("na6", T=24, d=256, f=768, dtype=synth.W8))


def test_noalloc_fp32(gm):
    _check_pair(gm, "fp32", synth.Workload("na7", T=64, d=128, f=512, dtype=synth.F32),
                synth.Workload("na8", T=5, d=128, f=512, dtype=synth.F32))


def test_noalloc_grok_share(gm):
    """d = 6144 (Grok-1's d_model) at one GPU's d_ff share f = 4096: T = 64, then a decode batch of T = 8."""
    _check_pair(gm, "grok_share", synth.Workload("na9", T=64, d=6144, f=4096),
                synth.Workload("na10", T=8, d=6144, f=4096))


def test_noalloc_rejects_batches_beyond_the_scratch_array(gm):
    d, f, E, T = 256, 65536, 8, 300
    assert gm.workspace_size(T, d, f, E, 2, gm.BF16) > gm.SCRATCH_BYTES
    assert gm.workspace_size(16, d, f, E, 2, gm.BF16) <= gm.SCRATCH_BYTES
    x = torch.zeros((T, d), dtype=torch.bfloat16, device="cuda")
    rw = torch.zeros((E, d), dtype=torch.bfloat16, device="cuda")
    w1 = torch.zeros((E, d, f), dtype=torch.bfloat16, device="cuda")
    w2 = torch.zeros((E, f, d), dtype=torch.bfloat16, device="cuda")
    dv = {"x": x, "router_w": rw, "w1": w1, "wv": w1, "w2": w2, "scales": None, "router_bias": None}
    st, out, idx, pr, cnt = _noalloc(gm, dv, T, d, f, E, gm.BF16)
    torch.cuda.synchronize()
    assert st == -5 and "scratch" in gm.strerror(st)
    assert (out == 7.0).all() and (idx == -9).all() and (cnt == -9).all()  # nothing written
    # a batch that fits, on the same tensors, right after
    st, out, idx, pr, cnt = _noalloc(gm, {**dv, "x": x[:16]}, 16, d, f, E, gm.BF16)
    torch.cuda.synchronize()
    assert st == 0
    assert (idx[:, 0] == 0).all() and (idx[:, 1] == 1).all() and (out == 0).all()
