"""GPU parity over a seeded sweep of layer shapes inside the boundary's limits, through the C ABI.

The other GPU tests pick their shapes to reach each kernel path on purpose; this sweep draws shapes the same way a
user might pass them: any expert count from 2 to 64 (odd ones included), d and f multiples of 256, batches from 1
to 1200 tokens (so the streaming kernels, the LDS-tiled kernels and the switch between them are all reached), both
weight layouts, per-channel and grouped int8 scales, shared scales, and a skewing router bias.  Each case meets the
bar of the parity tests: routing indices and expert counts exact, probabilities within 1e-6 relative, the output
within 1e-2 rms (1e-4 for fp32) of the oracle on up to 48 sampled rows.  The shapes come from a fixed seed, so the
list is the same on every run."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import TOL, dev_inputs, rel_err, say

pytestmark = pytest.mark.gpu

F32, BF16, W8 = synth.F32, synth.BF16, synth.W8


def _groups(rng, n):
    """A group count along an axis of n values: each group a multiple of 64 values."""
    return int(rng.choice([g for g in (1, 2, 3, 4, 8) if n % g == 0 and (n // g) % 64 == 0]))


def _cases(count=60, seed=20240601):
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < count:
        dtype = [BF16, W8, F32][int(rng.choice(3, p=[0.5, 0.35, 0.15]))]
        E = int(rng.choice([2, 3, 4, 5, 6, 7, 8, 8, 8, 12, 16, 24, 32, 64]))
        d = 256 * int(rng.integers(1, 7 if dtype != F32 else 3))
        f = 256 * int(rng.integers(1, 17 if dtype != F32 else 5))
        if E * d * f > (1 << 24):
            continue
        T = int([rng.integers(1, 17), rng.integers(17, 129), rng.integers(129, 1201)][int(rng.integers(0, 3))])
        layout = "out_in" if rng.random() < 0.5 else "in_out"
        g1 = g2 = 1
        es = None
        if dtype == W8:
            g1, g2 = _groups(rng, d), _groups(rng, f)
            es = 1 if rng.random() < 0.25 else None
        bias = None
        if rng.random() < 0.3:
            bias = tuple(float(v) for v in rng.normal(0.0, 1.5, E))
        name = (f"sw{len(out)}_{synth.DTYPE_NAMES[dtype]}_T{T}_d{d}_f{f}_E{E}_{layout}"
                + (f"_g{g1}x{g2}" if (g1, g2) != (1, 1) else "") + ("_shared" if es else "") + ("_bias" if bias else ""))
        out.append((synth.Workload(name, T=T, d=d, f=f, E=E, dtype=dtype, groups_up=g1, groups_down=g2,
                                   scale_experts=es, router_bias=bias, seed=len(out)), layout))
    return out


CASES = _cases()


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


def _t(a):
    return np.ascontiguousarray(np.swapaxes(a, 1, 2))


@pytest.mark.parametrize("w,layout", CASES, ids=[c[0].name for c in CASES])
def test_sweep(gm, w, layout):
    say(f"[case] {w.name}")
    inp = synth.make_inputs(w)
    oi = layout == "out_in"
    dv_in = dict(inp)
    if oi:
        for n in ("w1", "wv", "w2"):
            dv_in[n] = _t(inp[n])
    dv = dev_inputs(dv_in, w.dtype)
    out, idx, p, cnt = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"],
                                  router_bias=dv["router_bias"], return_routing=True,
                                  weight_layout=gm.OUT_IN if oi else gm.IN_OUT)
    torch.cuda.synchronize()
    rows = synth.sampled_rows(w.T, 48, seed=w.seed)
    ref = oracle.forward(dv_in, w.dtype, rows=rows, layout=oracle.OUT_IN if oi else oracle.IN_OUT)
    rows_t = ref["rows"].numpy()
    err = rel_err(out.cpu().numpy()[rows_t], ref["out"].numpy())
    p_g = p.cpu().numpy()
    perr = float(np.max(np.abs(p_g - ref["p"].numpy()) / ref["p"].numpy()))
    ok_idx = np.array_equal(idx.cpu().numpy(), ref["idx"].numpy())
    ok_cnt = np.array_equal(cnt.cpu().numpy(), ref["counts"].numpy())
    say(f"[result] {w.name}: idx_exact={ok_idx} counts_exact={ok_cnt} counts={cnt.cpu().tolist()} "
        f"max_err/rms={err:.3e} (tol {TOL[w.dtype]:.0e}) p_rel_err={perr:.2e}")
    assert ok_idx and ok_cnt
    assert perr < 1e-6
    assert err <= TOL[w.dtype]
