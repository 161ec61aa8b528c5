"""GPU check of the largest batch the boundary accepts: T = 2^24 tokens (d = f = 256, E = 8, bf16).

One pass holds at most min((2^31 - 1) / (2 d), (2^31 - 1) / (4 f)) = 2,097,151 tokens at f = 256, so the layer runs
as 9 passes of near-equal size (1,864,136 and 1,864,135 tokens).  The activations are drawn on the device from a
seeded generator (16.8M x 256 values would take minutes on the host); the weights come from ``synth``.  Checked:
the expert counts sum to 2T and equal the histogram of the returned indices; on 47 rows that include the first and
last token of every pass, the routing is bit-exact and the output within 1e-2 rms(oracle) of the oracle (which
routes only those rows: routing is per token).  Memory: about 55 GB of HBM at peak."""
import numpy as np
import pytest
import torch

import oracle
import synth
from synth.harness import TOL, dev_inputs, rel_err
from tests._helpers import say

pytestmark = pytest.mark.gpu

W = synth.Workload("max_tokens_T16M", T=1 << 24, d=256, f=256, E=8)
PASS_MAX = min((2 ** 31 - 1) // (2 * W.d), (2 ** 31 - 1) // (4 * W.f))


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


def pass_starts(T: int, P: int) -> list:
    n = -(-T // P)
    base, rem = T // n, T % n
    return [i * base + min(i, rem) for i in range(n)] + [T]


def test_largest_batch(gm):
    T, d = W.T, W.d
    starts = pass_starts(T, PASS_MAX)
    assert len(starts) - 1 == 9
    assert gm.workspace_size(T, d, W.f, W.E) == gm.workspace_size(starts[1] - starts[0], d, W.f, W.E)
    say(f"[case] {W.name}: T={T} d={d} f={W.f} E={W.E} passes={len(starts) - 1}")
    wts = synth.make_weights(W)
    dv = dev_inputs({**wts, "x": np.zeros((1, d), np.uint16), "router_bias": None}, W.dtype)
    g = torch.Generator(device="cuda")
    g.manual_seed(20241)
    x = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    for a in range(0, T, 1 << 22):  # in slices: the float32 draws of all rows would take 17 GB
        b = min(T, a + (1 << 22))
        x[a:b] = torch.randn((b - a, d), generator=g, device="cuda").to(torch.bfloat16)
    out, idx, p, cnt = gm.forward(x, dv["router_w"], dv["w1"], dv["wv"], dv["w2"], return_routing=True)
    torch.cuda.synchronize()
    assert int(cnt.sum()) == 2 * T
    assert torch.equal(cnt.to(torch.int64), torch.bincount(idx.reshape(-1).to(torch.int64), minlength=W.E))
    rows = sorted({r for s in starts[:-1] for r in (s, s + 1)} | {s - 1 for s in starts[1:]} |
                  set(np.random.default_rng(1).choice(T, 20, replace=False).tolist()))
    rt = torch.tensor(rows, device="cuda")
    xs = x[rt].cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.forward({**wts, "x": xs, "router_bias": None}, W.dtype)
    idx_g, p_g, out_g = idx[rt].cpu().numpy(), p[rt].cpu().numpy(), out[rt].cpu().numpy()
    err = rel_err(out_g, ref["out"].numpy())
    say(f"[result] {W.name}: rows={len(rows)} counts={cnt.tolist()} idx_exact="
        f"{np.array_equal(idx_g, ref['idx'].numpy())} max_err/rms={err:.3e}")
    assert np.array_equal(idx_g, ref["idx"].numpy())
    assert np.allclose(p_g, ref["p"].numpy(), rtol=1e-6, atol=0)
    assert err <= TOL[W.dtype]
