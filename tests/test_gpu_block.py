"""GPU parity of the MoE block (pre-MoE RMSNorm -> MoE -> post-MoE RMSNorm -> residual) against the oracle.

Bar: normed input xn bit-exact (both sides round it once from float64), routing and counts bit-exact, block
output within max|gpu - oracle| <= 1e-2 rms(oracle) (bf16, int8) / 1e-4 rms(oracle) (fp32)."""
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


def _scales_dev(ns, dtype):
    if dtype == F32:
        return (torch.from_numpy(ns["pre_scale"]).cuda(), torch.from_numpy(ns["post_scale"]).cuda())
    bf = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return bf(ns["pre_scale"]), bf(ns["post_scale"])


def check_block(gm, w, inp=None, dv=None, rows=None):
    say(f"[case] block {w.name}: T={w.T} d={w.d} f={w.f} E={w.E} dtype={synth.DTYPE_NAMES[w.dtype]}")
    inp = inp if inp is not None else synth.make_inputs(w)
    dv = dv if dv is not None else dev_inputs(inp, w.dtype)
    ns = synth.make_norm_scales(w)
    g_pre, g_post = _scales_dev(ns, w.dtype)
    out, idx, p, cnt = gm.block_forward(dv["x"], g_pre, g_post, ns["eps"], dv["router_w"], dv["w1"], dv["wv"],
                                        dv["w2"], scales=dv["scales"], router_bias=dv["router_bias"],
                                        return_routing=True)
    torch.cuda.synchronize()
    ref = oracle.block_forward(inp, w.dtype, ns["pre_scale"], ns["post_scale"], ns["eps"], rows=rows)
    rows_t = ref["rows"].numpy()
    err = rel_err(out.cpu().numpy()[rows_t], ref["out"].numpy())
    ok_idx = np.array_equal(idx.cpu().numpy(), ref["idx"].numpy())
    ok_cnt = np.array_equal(cnt.cpu().numpy(), ref["counts"].numpy())
    say(f"[result] block {w.name}: idx_exact={ok_idx} counts_exact={ok_cnt} max_err/rms={err:.3e}")
    assert ok_idx and ok_cnt
    assert err <= TOL[w.dtype]
    return out, ref


@pytest.mark.parametrize("T,d,E,dtype", [(1, 256, 8, BF16), (37, 512, 8, BF16), (300, 256, 16, BF16),
                                         (64, 128, 8, F32), (20, 256, 8, W8)])
def test_route_norm_step(gm, T, d, E, dtype):
    """xn bit-exact against the oracle's single rounding; routing on xn bit-exact."""
    w = synth.Workload("rn", T=T, d=d, f=256, E=E, dtype=dtype)
    inp = synth.make_inputs(w)
    ns = synth.make_norm_scales(w)
    dv = dev_inputs(inp, dtype)
    g_pre, _ = _scales_dev(ns, dtype)
    xn, idx, p = gm.route_norm(dv["x"], g_pre, ns["eps"], dv["router_w"])
    torch.cuda.synchronize()
    kind = "f32" if dtype == F32 else "bf16"
    x = oracle.as_f64(inp["x"], kind)
    want = oracle.rmsnorm(x, oracle.as_f64(ns["pre_scale"], kind), ns["eps"])
    xn_ref = want.to(torch.float32).to(torch.float64) if dtype == F32 else oracle.bf16_round(want)
    assert torch.equal(xn.cpu().to(torch.float64), xn_ref)
    r = oracle.route(xn_ref, oracle.as_f64(inp["router_w"], kind))  # the oracle's own normed input
    assert np.array_equal(idx.cpu().numpy(), r["idx"].numpy())
    assert np.allclose(p.cpu().numpy(), r["p"].numpy(), rtol=1e-6, atol=0)


def test_combine_norm_step(gm):
    """Against a float64 numpy evaluation on synthetic partial sums (S = 3)."""
    rng = np.random.default_rng(0)
    T, d, S = 5, 1024, 3
    y = rng.standard_normal((S, 2 * T, d)).astype(np.float32)
    perm = rng.permutation(2 * T).reshape(T, 2).astype(np.int32)
    p = np.sort(rng.random((T, 2)), axis=1)[:, ::-1].astype(np.float32) * 0.5
    x = rng.standard_normal((T, d)).astype(np.float32)
    g = (1 + 0.1 * rng.standard_normal(d)).astype(np.float32)
    out = gm.combine_norm(torch.from_numpy(y).cuda(), torch.from_numpy(np.ascontiguousarray(p)).cuda(),
                          torch.from_numpy(perm).cuda(), torch.from_numpy(x).cuda(), torch.from_numpy(g).cuda(), 1e-5)
    torch.cuda.synchronize()
    ys = y.astype(np.float64).sum(axis=0)
    o = p[:, 0:1] * ys[perm[:, 0]] + p[:, 1:2] * ys[perm[:, 1]]
    want = x + o / np.sqrt((o * o).mean(axis=1, keepdims=True) + 1e-5) * g
    assert np.max(np.abs(out.cpu().numpy() - want)) < 1e-5


SMALL = [synth.Workload("blk_bf16_T8", T=8, d=256, f=512, w_std=0.1),
         synth.Workload("blk_bf16_T300", T=300, d=512, f=768, w_std=0.07),
         synth.Workload("blk_w8_T40", T=40, d=256, f=512, dtype=W8),
         synth.Workload("blk_f32_T64", T=64, d=128, f=512, dtype=F32)]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_block_small(gm, w):
    check_block(gm, w)


def test_block_grok_decode(gm):
    say("[setup] drawing Grok-1-shape bf16 weights")
    w = synth.WORKLOADS["decode_bf16"]
    check_block(gm, w)


@pytest.mark.parametrize("dtype,T,g", [(BF16, 24, 1), (W8, 40, 4), (W8, 300, 2)])
def test_block_out_in_and_grouped(gm, dtype, T, g):
    """The block with [out, in] weights (and grouped int8 scales): bit-identical to the [in, out] block on the same
    weights, and against the oracle reading the [out, in] storage."""
    w = synth.Workload(f"blk_oi_T{T}", T=T, d=512, f=1024, E=8, dtype=dtype, groups_up=g, groups_down=g)
    say(f"[case] block out_in {w.name} dtype={synth.DTYPE_NAMES[dtype]} groups={g}")
    inp = synth.make_inputs(w)
    dv = dev_inputs(inp, dtype)
    ns = synth.make_norm_scales(w)
    g_pre, g_post = _scales_dev(ns, dtype)
    ref = gm.block_forward(dv["x"], g_pre, g_post, ns["eps"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"],
                           scales=dv["scales"])
    tr = lambda t: t.transpose(1, 2).contiguous()
    out = gm.block_forward(dv["x"], g_pre, g_post, ns["eps"], dv["router_w"], tr(dv["w1"]), tr(dv["wv"]),
                           tr(dv["w2"]), scales=dv["scales"], weight_layout=gm.OUT_IN)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    tin = dict(inp)
    for n in ("w1", "wv", "w2"):
        tin[n] = np.ascontiguousarray(np.swapaxes(inp[n], 1, 2))
    want = oracle.block_forward(tin, dtype, ns["pre_scale"], ns["post_scale"], ns["eps"], layout=oracle.OUT_IN)
    err = rel_err(out.cpu().numpy(), want["out"].numpy())
    say(f"[result] block out_in {w.name}: max_err/rms={err:.3e}")
    assert err <= TOL[dtype]
