"""Plant plausible mistakes in the oracle (on the CPU, via monkeypatch) and check that a pin catches each one."""
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.grok_moe_oracle as om
import synth
from tests import test_oracle_pins as pins


def _tanh_gelu(z):
    return 0.5 * z * (1 + torch.tanh(math.sqrt(2 / math.pi) * (z + 0.044715 * z ** 3)))


def _swapped_branches(x, w1, wv, w2, round_h):
    a = x @ w1
    b = x @ wv
    h = om.gelu(b) * a
    if round_h:
        h = om.bf16_round(h)
    return h, h @ w2


def _round_via_f32(v):
    return v.to(torch.float32).to(torch.bfloat16).to(torch.float64)


def _transposed_w2(x, w1, wv, w2, round_h):
    a = x @ w1
    b = x @ wv
    h = om.gelu(a) * b
    if round_h:
        h = om.bf16_round(h)
    return h, h @ w2.T.reshape(w2.shape)


_orig_route = om.route


def _renormalised_route(x, rw, bias=None, k=2):
    r = _orig_route(x, rw, bias, k)
    r["p"] = r["p"] / r["p"].sum(dim=1, keepdim=True)
    return r


def _reversed_tie_route(x, rw, bias=None, k=2):
    E = rw.shape[0]
    flip = torch.arange(E - 1, -1, -1)
    r = _orig_route(x, rw[flip], None if bias is None else bias[flip], k)
    r["idx"] = flip[r["idx"]]
    r["probs"] = r["probs"][:, flip]
    r["logits"] = r["logits"][:, flip]
    return r


def _no_max_route(x, rw, bias=None, k=2):
    logits = x @ rw.T
    if bias is not None:
        logits = logits + bias[None, :]
    ex = torch.exp(logits)
    r = _orig_route(x, rw, bias, k)
    r["probs"] = ex / ex.sum(dim=1, keepdim=True)
    r["p"] = r["probs"].gather(1, r["idx"])
    return r


def _no_bias_route(x, rw, bias=None, k=2):
    return _orig_route(x, rw, None, k)


MUTANTS = [
    ("gelu", _tanh_gelu, [pins.test_gelu_matches_normal_cdf_table]),
    ("gelu", lambda z: 0.5 * z * (1 - torch.special.erf(z / math.sqrt(2))), [pins.test_gelu_identities_and_not_tanh]),
    ("expert_ffn", _swapped_branches, [pins.test_gelu_goes_on_the_w1_branch]),
    ("expert_ffn", _transposed_w2, [pins.test_weights_are_in_out_layout]),
    ("bf16_round", _round_via_f32, [pins.test_bf16_round_golden]),
    ("route", _renormalised_route, [pins.test_zero_router_combine_is_one_eighth_of_first_two_experts,
                                    pins.test_whole_layer_brute_force_tiny]),
    ("route", _reversed_tie_route, [pins.test_zero_router_uniform_probs_and_tie_break,
                                    pins.test_partial_ties_keep_lower_index_first]),
    ("route", _no_max_route, [pins.test_huge_logits_do_not_overflow]),
    ("route", _no_bias_route, [pins.test_bias_only_router_is_softmax_of_bias]),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)))
def test_pin_catches_planted_mistake(i, monkeypatch, golden_dir):
    name, fn, catching = MUTANTS[i]
    monkeypatch.setattr(om, name, fn)
    monkeypatch.setattr(oracle, name, fn)
    for t in catching:
        args = [golden_dir] if "golden_dir" in t.__code__.co_varnames[:t.__code__.co_argcount] else []
        with pytest.raises((AssertionError, RuntimeError)):
            t(*args)


def test_dropped_combine_term_is_caught(monkeypatch):
    """Combine with only the first expert: the identical-experts pin fails."""
    orig = om.forward

    def one_term(inp, dtype, rows=None, k=2, return_h=False):
        r = orig(inp, dtype, rows, k, return_h)
        r["out"] = r["out"] * (r["p"][r["rows"], 0:1] / r["p"][r["rows"]].sum(dim=1, keepdim=True))
        return r

    monkeypatch.setattr(om, "forward", one_term)
    monkeypatch.setattr(oracle, "forward", one_term)
    with pytest.raises(AssertionError):
        pins.test_identical_experts_scale_by_gate_sum()


from tests import test_oracle_block_pins as bpins


@pytest.mark.parametrize("bad", [
    lambda v, g, eps: v / ((v * v).mean(dim=-1, keepdim=True) + eps) * g,            # no square root
    lambda v, g, eps: v / (torch.sqrt((v * v).mean(dim=-1, keepdim=True)) + eps) * g,  # eps outside the root
    lambda v, g, eps: v / torch.sqrt((v * v).sum(dim=-1, keepdim=True) + eps) * g,     # sum instead of mean
])
def test_rmsnorm_mistakes_are_caught(bad, monkeypatch):
    monkeypatch.setattr(om, "rmsnorm", bad)
    monkeypatch.setattr(oracle, "rmsnorm", bad)
    caught = 0
    for t in (bpins.test_rmsnorm_3_4_5_triangle, bpins.test_rmsnorm_eps_closed_form_and_zero_row,
              bpins.test_block_against_numpy):
        try:
            t()
        except AssertionError:
            caught += 1
    assert caught >= 1


def test_dropped_residual_is_caught(monkeypatch):
    orig = om.block_forward

    def no_residual(inp, dtype, pre, post, eps, rows=None, k=2):
        r = orig(inp, dtype, pre, post, eps, rows, k)
        r["out"] = r["out"] - om.as_f64(inp["x"], "f32" if dtype == om.F32 else "bf16")[r["rows"]]
        return r

    monkeypatch.setattr(om, "block_forward", no_residual)
    monkeypatch.setattr(oracle, "block_forward", no_residual)
    with pytest.raises(AssertionError):
        bpins.test_block_against_numpy()


def _dequant_group_mod(q, s):
    """Planted mistake: group of row k taken as k mod G."""
    qq = om.as_f64(q, "i8")
    sc = om.as_f64(s, "bf16")
    G = sc.shape[0]
    return qq * sc[torch.arange(qq.shape[0]) % G]


def _dequant_first_group(q, s):
    """Planted mistake: the first group's scales used for every row."""
    return om.as_f64(q, "i8") * om.as_f64(s, "bf16")[0:1]


@pytest.mark.parametrize("bad", [_dequant_group_mod, _dequant_first_group])
def test_grouped_scale_mistakes_are_caught(bad, monkeypatch):
    from tests import test_oracle_scale_pins as sp
    monkeypatch.setattr(om, "dequant", bad)
    monkeypatch.setattr(oracle, "dequant", bad)
    caught = 0
    for pin in (sp.test_group_index_closed_form, sp.test_dequant_brute_force_loops,
                sp.test_grouped_layer_against_numpy_brute_force):
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught >= 1


def _reshaped_not_transposed(w, layout):
    """Planted mistake: the [out, in] storage reshaped to [in, out] instead of transposed."""
    w = np.asarray(w)
    return w if layout == om.IN_OUT else w.reshape(w.shape[::-1])


def test_out_in_layout_mistake_is_caught(monkeypatch):
    from tests import test_oracle_layout_pins as lp
    monkeypatch.setattr(om, "stored_in_out", _reshaped_not_transposed)
    monkeypatch.setattr(oracle, "stored_in_out", _reshaped_not_transposed)
    with pytest.raises(AssertionError):
        lp.test_selection_matrices_closed_form()
    with pytest.raises(AssertionError):
        lp.test_transposed_storage_is_the_same_layer(synth.BF16, 1, 1)
