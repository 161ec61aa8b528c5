"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Bar: routing indices, per-expert counts, the permutation and its inverse bit-exact; the layer output within
max|gpu - oracle| <= 1e-2 rms(oracle) for bf16 and int8 layers and 1e-4 rms(oracle) for the fp32 layer.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._helpers import TOL, dev_inputs, dump, rel_err, rms_rel_err, say

pytestmark = pytest.mark.gpu

F32, BF16, W8 = synth.F32, synth.BF16, synth.W8


@pytest.fixture(scope="module")
def gm():
    import mixture_experts_transformer_gemv_amd as gm
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    gm.lib()
    return gm


def _forward(gm, dv):
    return gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"],
                      router_bias=dv["router_bias"], return_routing=True)


def check_layer(gm, w: synth.Workload, inp=None, rows=None, name=None, dv=None, unrounded=False):
    """The layer through grok_moe_forward against the oracle on `rows` (all rows if None).  unrounded: also log the
    error against the oracle without the bf16 rounding of h (the plain float64 definition), which has no bar."""
    name = name or w.name
    say(f"[case] {name}: T={w.T} d={w.d} f={w.f} E={w.E} dtype={synth.DTYPE_NAMES[w.dtype]}")
    inp = inp if inp is not None else synth.make_inputs(w)
    dv = dv if dv is not None else dev_inputs(inp, w.dtype)
    out, idx, p, cnt = _forward(gm, dv)
    torch.cuda.synchronize()
    ref = oracle.forward(inp, w.dtype, rows=rows)
    idx_g, p_g, cnt_g = idx.cpu().numpy(), p.cpu().numpy(), cnt.cpu().numpy()
    rows_t = ref["rows"].numpy()
    out_g = out.cpu().numpy()[rows_t]
    ok_idx = np.array_equal(idx_g, ref["idx"].numpy())
    ok_cnt = np.array_equal(cnt_g, ref["counts"].numpy())
    err = rel_err(out_g, ref["out"].numpy())
    perr = float(np.max(np.abs(p_g - ref["p"].numpy()) / ref["p"].numpy()))
    say(f"[result] {name}: idx_exact={ok_idx} counts_exact={ok_cnt} counts={cnt_g.tolist()} "
        f"max_err/rms={err:.3e} rms_err/rms={rms_rel_err(out_g, ref['out'].numpy()):.3e} (tol {TOL[w.dtype]:.0e}) "
        f"p_rel_err={perr:.2e} min_gap_cut={ref['min_gap_cut']:.3e}")
    if unrounded and w.dtype != F32:
        plain = oracle.forward(inp, w.dtype, rows=rows, round_h=False)["out"].numpy()
        say(f"[result] {name}: against the unrounded definition max_err/rms={rel_err(out_g, plain):.3e} "
            f"rms_err/rms={rms_rel_err(out_g, plain):.3e}")
    if not (ok_idx and ok_cnt and err <= TOL[w.dtype] and perr < 1e-6):
        dump(name, out=out_g, want=ref["out"].numpy(), idx=idx_g, want_idx=ref["idx"].numpy(), p=p_g,
             want_p=ref["p"].numpy(), counts=cnt_g, rows=rows_t)
    assert ok_idx, "routing indices differ"
    assert ok_cnt, "expert counts differ"
    assert perr < 1e-6
    assert err <= TOL[w.dtype]
    return out, ref


# ------------------------------------------------------------------------------------------------ steps

@pytest.mark.parametrize("T,d,E,dtype,bias", [
    (1, 256, 8, BF16, False), (77, 512, 8, BF16, True), (1000, 256, 8, BF16, False), (50, 256, 16, BF16, False),
    (30, 256, 64, BF16, True), (64, 128, 8, F32, False), (129, 192, 8, F32, True), (20, 6144, 8, BF16, False),
    # batches above 256 tokens, ragged sizes, 2 and 4 experts
    (1003, 256, 8, BF16, True), (300, 512, 4, F32, True), (777, 6144, 8, BF16, False), (260, 256, 2, BF16, False),
    # larger batches
    (2048, 256, 8, BF16, True), (2051, 6144, 8, BF16, False), (3001, 192, 8, F32, True), (2500, 256, 4, BF16, True)])
def test_router_step(gm, T, d, E, dtype, bias):
    say(f"[case] router T={T} d={d} E={E} dtype={dtype} bias={bias}")
    w = synth.Workload("r", T=T, d=d, f=256, E=E, dtype=dtype)
    inp = synth.make_inputs(w)
    if bias:
        inp["router_bias"] = np.linspace(-1, 2, E).astype(np.float32)
    dv = dev_inputs(inp, dtype)
    idx, p = gm.route(dv["x"], dv["router_w"], dv["router_bias"])
    torch.cuda.synchronize()
    kind = "f32" if dtype == F32 else "bf16"
    b = None if inp["router_bias"] is None else torch.from_numpy(inp["router_bias"]).double()
    ref = oracle.route(oracle.as_f64(inp["x"], kind), oracle.as_f64(inp["router_w"], kind), b)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"].numpy())
    assert np.allclose(p.cpu().numpy(), ref["p"].numpy(), rtol=1e-6, atol=0)


@pytest.mark.parametrize("dtype", [BF16, F32])
def test_router_batch_forms_agree(gm, dtype):
    """Routing is per token: a token's indices and probabilities are bit-identical whether it is routed in a batch
    of 2051 tokens or in a smaller batch holding it."""
    say(f"[case] router forms dtype={dtype}")
    w = synth.Workload("rf", T=2051, d=6144 if dtype == BF16 else 512, f=256, dtype=dtype)
    inp = synth.make_inputs(w)
    inp["router_bias"] = np.linspace(-1, 2, 8).astype(np.float32)
    dv = dev_inputs(inp, dtype)
    idx, p = gm.route(dv["x"], dv["router_w"], dv["router_bias"])
    for a, b in ((0, 1000), (1000, 2000), (2000, 2051)):
        idx_s, p_s = gm.route(dv["x"][a:b].contiguous(), dv["router_w"], dv["router_bias"])
        assert torch.equal(idx_s, idx[a:b])
        assert torch.equal(p_s.view(torch.int32), p[a:b].view(torch.int32))


@pytest.mark.parametrize("T", [40, 603, 2049])
def test_router_ties_take_lower_index(gm, T):
    x = torch.randn(T, 256, device="cuda").to(torch.bfloat16)
    rw = torch.zeros(8, 256, device="cuda", dtype=torch.bfloat16)
    bias = torch.tensor([0, 0, 1, 1, 1, 0, 0, 0], dtype=torch.float32, device="cuda")
    idx, p = gm.route(x, rw, bias)
    assert (idx.cpu() == torch.tensor([2, 3], dtype=torch.int32)).all()
    idx0, p0 = gm.route(x, rw, None)
    assert (idx0.cpu() == torch.tensor([0, 1], dtype=torch.int32)).all()
    assert torch.allclose(p0.cpu(), torch.full((T, 2), 0.125))


def _random_assignments(T, E, rng):
    a = rng.integers(0, E, size=T)
    b = (a + 1 + rng.integers(0, E - 1, size=T)) % E
    return np.stack([a, b], axis=1).astype(np.int32)


@pytest.mark.parametrize("T,E", [(1, 8), (8, 8), (1023, 8), (1024, 8), (1025, 8), (5000, 64), (8192, 8), (300, 2)])
def test_bin_step(gm, T, E):
    say(f"[case] bin T={T} E={E}")
    rng = np.random.default_rng(T * 131 + E)
    idx = _random_assignments(T, E, rng)
    counts, offsets, perm, inv = gm.bin_tokens(torch.from_numpy(idx).cuda(), E)
    torch.cuda.synchronize()
    flat = idx.reshape(-1)
    want_counts = np.bincount(flat, minlength=E)
    order = np.argsort(flat, kind="stable")  # slot -> flat (token, j) index, grouped by expert, token ascending
    want_perm = order // 2
    want_inv = np.empty(2 * T, np.int64)
    want_inv[order] = np.arange(2 * T)
    assert np.array_equal(counts.cpu().numpy(), want_counts)
    assert np.array_equal(offsets.cpu().numpy(), np.concatenate([[0], np.cumsum(want_counts)]))
    assert np.array_equal(perm.cpu().numpy(), want_perm)
    assert np.array_equal(inv.cpu().numpy().reshape(-1), want_inv)


@pytest.mark.parametrize("T,d,f,dtype", [(8, 256, 512, BF16), (40, 512, 768, BF16), (200, 256, 512, BF16),
                                         (24, 256, 512, W8), (150, 256, 768, W8), (64, 128, 512, F32)])
def test_up_step_matches_oracle_h(gm, T, d, f, dtype):
    """h per slot against the oracle's h (bf16 layers: a one-ulp rounding flip is allowed)."""
    say(f"[case] up T={T} d={d} f={f} dtype={dtype}")
    w = synth.Workload("u", T=T, d=d, f=f, dtype=dtype, w_std=1.5 / np.sqrt(d))
    inp = synth.make_inputs(w)
    dv = dev_inputs(inp, dtype)
    idx, p = gm.route(dv["x"], dv["router_w"], None)
    counts, offsets, perm, inv = gm.bin_tokens(idx, 8)
    h = gm.expert_up(dv["x"], dv["w1"], dv["wv"], counts, offsets, perm, scales=dv["scales"])
    torch.cuda.synchronize()
    ref = oracle.forward(inp, dtype, return_h=True)
    hg = h.float().cpu().numpy()
    inv_n = inv.cpu().numpy()
    want = ref["h"].numpy()  # [T, 2, f]
    got = hg[inv_n.reshape(-1)].reshape(T, 2, f)
    rms = np.sqrt(np.mean(want ** 2))
    if dtype == F32:
        assert np.max(np.abs(got - want)) <= 1e-5 * rms
    else:
        assert np.all(np.abs(got - want) <= 2.0 ** -7 * np.abs(want) + 1e-5 * rms)


# ------------------------------------------------------------------------------------------------ whole layer, small

SMALL = [
    # streaming kernels (T <= 96 for bf16, <= 128 for int8), one and two 16-row tiles per pass
    synth.Workload("bf16_T1", T=1, d=256, f=512, w_std=0.1),
    synth.Workload("bf16_T8", T=8, d=256, f=512, w_std=0.1),
    synth.Workload("bf16_T13_f768", T=13, d=512, f=768, w_std=0.07),
    synth.Workload("bf16_T40", T=40, d=256, f=1024, w_std=0.1),
    synth.Workload("bf16_T64_E16", T=64, d=256, f=512, E=16, w_std=0.1),
    synth.Workload("bf16_T8_split2", T=8, d=256, f=4096, w_std=0.1),
    synth.Workload("bf16_T5_split4", T=5, d=512, f=8192, w_std=0.05),
    # one GPU's d_ff share of a Grok-1 layer (d = 6144, f = 4096): the up-projection splits d over the 4 waves
    synth.Workload("bf16_T8_d6144_f4096", T=8, d=6144, f=4096, w_std=0.02),
    # streaming kernels above 32 rows per expert: several passes over the weights (bf16 T = 65, 96)
    synth.Workload("bf16_T96", T=96, d=256, f=512, w_std=0.1),
    # LDS-tiled grouped GEMM (bf16 T > 96), ragged row tiles
    synth.Workload("bf16_T65", T=65, d=256, f=512, w_std=0.1),
    synth.Workload("bf16_T300", T=300, d=512, f=768, w_std=0.07),
    synth.Workload("bf16_T1000_E4", T=1000, d=256, f=512, E=4, w_std=0.1),
    synth.Workload("bf16_T700_E64", T=700, d=256, f=512, E=64, w_std=0.1),
    synth.Workload("bf16_T500_skew", T=500, d=256, f=512, w_std=0.1, router_bias=(3, 0, 0, 0, 0, 1.5, 0, 0)),
    # int8 weights
    synth.Workload("w8_T8", T=8, d=256, f=512, dtype=W8),
    synth.Workload("w8_T64", T=64, d=512, f=1024, dtype=W8),
    synth.Workload("w8_T33_split2", T=33, d=256, f=4096, dtype=W8),
    synth.Workload("w8_T128", T=128, d=256, f=768, dtype=W8),     # int8 streaming, the largest batch
    synth.Workload("w8_T200", T=200, d=256, f=768, dtype=W8),     # int8 LDS tiles
    # fp32
    synth.Workload("f32_T1", T=1, d=64, f=64, E=2, dtype=F32),
    synth.Workload("f32_T200", T=200, d=192, f=320, dtype=F32),
    synth.Workload("f32_T70_E16", T=70, d=128, f=256, E=16, dtype=F32),
]


@pytest.mark.parametrize("w", SMALL, ids=[w.name for w in SMALL])
def test_layer_small(gm, w):
    check_layer(gm, w)


def test_tiny_fp32_workload(gm):
    """The tiny fp32 layer: T=64, d=128, f=512, E=8, top-2, seed 0."""
    check_layer(gm, synth.WORKLOADS["tiny_f32"])


def test_layer_all_tokens_to_two_experts(gm):
    """router_w = 0: every token ties and goes to experts (0, 1); 64 rows per expert exercise several passes of
    the streaming kernels and leave six experts empty."""
    for T, dtype in ((64, BF16), (64, W8), (200, BF16)):
        w = synth.Workload(f"zero_router_T{T}_{dtype}", T=T, d=256, f=512, dtype=dtype, w_std=0.1)
        inp = synth.make_inputs(w)
        inp["router_w"] = np.zeros_like(inp["router_w"])
        _, ref = check_layer(gm, w, inp=inp)
        assert ref["counts"].tolist() == [T, T, 0, 0, 0, 0, 0, 0]


def test_layer_tile_heights(gm):
    """router_w = 0 puts all T tokens on experts 0 and 1, so each has exactly T slots.  The tiled kernels pick the
    tile height from the count: T = 150, 315, 384 and 550 run as 1, 2, 2 and 3 tiles of 192 rows; T = 420, 600 and
    1230 as 2, 3 and 5 tiles of 256 rows, the last partly filled; T = 1100 and 1152 as 4 full 256-row tiles plus a
    last tile of 76 / 128 rows run as a 128-row tile; T = 1153 keeps its 129-row last tile in the 256-row launch.
    Both weight types, and the [out, in] layout."""
    from tests.test_gpu_layout import check_layout
    cases = [(150, BF16), (315, BF16), (384, BF16), (420, BF16), (550, BF16), (600, BF16), (1100, BF16),
             (1152, BF16), (1153, BF16), (1230, BF16), (315, W8), (600, W8), (1100, W8), (1153, W8)]
    for T, dtype in cases:
        w = synth.Workload(f"tiles_T{T}_{dtype}", T=T, d=256, f=512, dtype=dtype, w_std=0.1)
        inp = synth.make_inputs(w)
        inp["router_w"] = np.zeros_like(inp["router_w"])
        _, ref = check_layer(gm, w, inp=inp)
        assert ref["counts"].tolist() == [T, T, 0, 0, 0, 0, 0, 0]
    for T in (315, 600, 1100, 1153):
        w = synth.Workload(f"oi_tiles_T{T}", T=T, d=256, f=512, w_std=0.1)
        inp = synth.make_inputs(w)
        inp["router_w"] = np.zeros_like(inp["router_w"])
        check_layout(gm, w, inp=inp)


def test_steps_compose_to_forward(gm):
    """grok_moe_forward equals the five step entry points called in order (bit-identical)."""
    for w in (synth.Workload("c1", T=8, d=256, f=4096, w_std=0.1), synth.Workload("c2", T=300, d=256, f=512),
              synth.Workload("c3", T=40, d=256, f=512, dtype=W8), synth.Workload("c4", T=50, d=64, f=128, dtype=F32)):
        inp = synth.make_inputs(w)
        dv = dev_inputs(inp, w.dtype)
        out = gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"])
        idx, p = gm.route(dv["x"], dv["router_w"], None)
        counts, offsets, perm, inv = gm.bin_tokens(idx, w.E)
        h = gm.expert_up(dv["x"], dv["w1"], dv["wv"], counts, offsets, perm, scales=dv["scales"])
        y = gm.expert_down(h, dv["w2"], counts, offsets, w.T, dv["x"].dtype,
                           s2=None if dv["scales"] is None else dv["scales"][2])
        out2 = gm.combine(y, p, inv)
        torch.cuda.synchronize()
        assert torch.equal(out, out2), w.name


def test_zero_tokens_is_a_noop(gm):
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    rw = torch.randn(8, 256, device="cuda").to(torch.bfloat16)
    w1 = torch.zeros(8, 256, 512, device="cuda", dtype=torch.bfloat16)
    w2 = torch.zeros(8, 512, 256, device="cuda", dtype=torch.bfloat16)
    out = gm.forward(x, rw, w1, w1, w2)
    assert out.shape == (0, 256)


def test_short_workspace_is_rejected(gm):
    w = synth.Workload("ws", T=8, d=256, f=512)
    dv = dev_inputs(synth.make_inputs(w), BF16)
    import ctypes
    out = torch.full((8, 256), 7.0, device="cuda")
    ws = torch.empty(1024, dtype=torch.uint8, device="cuda")
    L = gm.lib()
    st = L.grok_moe_forward(*(ctypes.c_void_p(t.data_ptr()) for t in (dv["x"], dv["router_w"], dv["w1"], dv["wv"],
                                                                       dv["w2"])), None, None, None, 8, 256, 512, 8,
                            2, 1, ctypes.c_void_p(out.data_ptr()), None, None, None, None,
                            ctypes.c_void_p(ws.data_ptr()), 1024, None)
    assert st == -3
    torch.cuda.synchronize()
    assert (out == 7.0).all()  # untouched


def test_deterministic_small(gm):
    for w in (synth.Workload("det1", T=8, d=256, f=4096), synth.Workload("det2", T=500, d=256, f=512)):
        dv = dev_inputs(synth.make_inputs(w), BF16)
        a = _forward(gm, dv)[0]
        b = _forward(gm, dv)[0]
        torch.cuda.synchronize()
        assert torch.equal(a, b)


# ------------------------------------------------------------------------------------------------ Grok-1 shape

@pytest.fixture(scope="module")
def grok_bf16():
    say("[setup] drawing Grok-1-shape bf16 weights (9.66 GB)")
    w = synth.WORKLOADS["decode_bf16"]
    wts = synth.make_weights(w)
    dvw = dev_inputs({**wts, "x": np.zeros((1, w.d), np.uint16), "router_bias": None}, BF16)
    say("[setup] done")
    yield wts, dvw
    del dvw
    torch.cuda.empty_cache()


def _grok_case(gm, grok_bf16, name):
    w = synth.WORKLOADS[name] if isinstance(name, str) else name
    wts, dvw = grok_bf16
    inp = synth.make_inputs(w, weights=wts)
    dv = dict(dvw)
    dv["x"] = dev_inputs({"x": inp["x"], "router_w": inp["router_w"], "w1": None, "wv": None, "w2": None,
                          "router_bias": inp["router_bias"]}, BF16)["x"]
    dv["router_bias"] = None if inp["router_bias"] is None else torch.from_numpy(inp["router_bias"]).cuda()
    rows = None if w.sampled_rows is None else synth.sampled_rows(w.T, w.sampled_rows)
    return check_layer(gm, w, inp=inp, rows=rows, dv=dv, unrounded=isinstance(name, str)), dv


def test_grok_decode_bf16(gm, grok_bf16):
    (out, ref), dv = _grok_case(gm, grok_bf16, "decode_bf16")
    again = _forward(gm, dv)[0]
    torch.cuda.synchronize()
    assert torch.equal(out, again)


@pytest.mark.parametrize("T", [1, 3])
def test_grok_decode_few_tokens(gm, grok_bf16, T):
    """One and three tokens at Grok-1 shape, every row against the oracle: at most 2 T experts are hit, the others
    are empty (their streaming workgroups return at once), and the down-projection runs in 5 chunks of f."""
    w = dataclasses.replace(synth.WORKLOADS["decode_bf16"], T=T, name=f"decode_bf16_T{T}")
    (out, ref), _ = _grok_case(gm, grok_bf16, w)
    assert int((ref["counts"].numpy() == 0).sum()) >= 8 - 2 * T
    assert gm.down_splits(T, w.d, w.f) == 5


def test_grok_prefill_bf16_sampled(gm, grok_bf16):
    (out, ref), dv = _grok_case(gm, grok_bf16, "prefill_bf16")
    again = _forward(gm, dv)[0]
    torch.cuda.synchronize()
    assert torch.equal(out, again)


def test_grok_skew_bf16_sampled(gm, grok_bf16):
    (out, ref), _ = _grok_case(gm, grok_bf16, "skew_bf16")
    c = ref["counts"].numpy()
    assert c[0] > 0.4 * c.sum() and c[5] > 0.2 * c.sum()


@pytest.mark.parametrize("T", [72, 256, 600])
def test_grok_mid_batch_bf16_sampled(gm, grok_bf16, T):
    """Batches of a few hundred tokens at Grok-1 shape: T = 72 on the streaming kernels (11-23 slots per expert,
    one pass of 32 rows); at T = 256 every expert has at most 128 slots and runs as 128-row tiles with
    nontemporal weight copies; at T = 600 one expert does, the others (149-160 slots) run as 192-row tiles."""
    w = dataclasses.replace(synth.WORKLOADS["prefill_bf16"], T=T, name=f"mid_bf16_T{T}", sampled_rows=64)
    (out, ref), _ = _grok_case(gm, grok_bf16, w)
    c = ref["counts"].numpy()
    if T <= 256:
        assert c.max() <= 128
    else:
        assert c.min() <= 128 < c.max()


@pytest.fixture(scope="module")
def grok_int8():
    say("[setup] drawing Grok-1-shape int8 weights (4.83 GB)")
    w = synth.WORKLOADS["int8_w8"]
    wts = synth.make_weights(w)
    dvw = dev_inputs({**wts, "x": np.zeros((1, w.d), np.uint16), "router_bias": None}, W8)
    say("[setup] done")
    yield wts, dvw
    del dvw
    torch.cuda.empty_cache()


def _grok_int8_case(gm, grok_int8, T, sampled):
    w = dataclasses.replace(synth.WORKLOADS["int8_w8"], T=T, name=f"int8_w8_T{T}", sampled_rows=sampled)
    wts, dvw = grok_int8
    inp = synth.make_inputs(w, weights=wts)
    dv = dict(dvw)
    dv["x"] = dev_inputs({"x": inp["x"], "router_w": inp["router_w"], "w1": None, "wv": None, "w2": None,
                          "s1": None, "sv": None, "s2": None, "router_bias": None}, W8)["x"]
    rows = None if sampled is None else synth.sampled_rows(T, sampled)
    return check_layer(gm, w, inp=inp, rows=rows, dv=dv, unrounded=T == 64)


def test_grok_int8(gm, grok_int8):
    """The int8 workload (T = 64, weight-streaming kernels), every row."""
    _grok_int8_case(gm, grok_int8, 64, None)


def test_grok_int8_two_tokens(gm, grok_int8):
    """int8 weights, T = 2 at Grok-1 shape, every row: at most 4 experts hit, the down-projection in 5 chunks."""
    _grok_int8_case(gm, grok_int8, 2, None)


@pytest.mark.parametrize("T", [128, 192])
def test_grok_int8_mid_batch_sampled(gm, grok_int8, T):
    """int8 weights at T = 128 (the largest int8 streaming batch, several passes) and T = 192 (every expert in
    the 128-row tiles), 64 seeded rows."""
    _grok_int8_case(gm, grok_int8, T, 64)


def test_grok_int8_prefill_sampled(gm, grok_int8):
    """int8 weights at prefill size (T = 8192: the direct-to-LDS int8 tile kernels), 64 seeded rows."""
    _grok_int8_case(gm, grok_int8, 8192, 64)
