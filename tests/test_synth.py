"""The seeded input generators: determinism, storage conversion and the distributions they promise."""
import math

import numpy as np
import pytest
import torch

import synth


def test_bf16_storage_conversion_matches_torch():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(100000), rng.standard_normal(1000) * 1e-30,
                        rng.standard_normal(1000) * 1e30]).astype(np.float32)
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(synth.f32_to_bf16_bits(v), want)
    back = synth.bf16_bits_to_f32(want)
    assert np.array_equal(back, torch.from_numpy(v).to(torch.bfloat16).float().numpy())


def test_deterministic_and_thread_independent(monkeypatch):
    a = synth.normal("t", (3, synth.CHUNK // 2 + 7), 0.5, synth.BF16, seed=0)
    monkeypatch.setattr(synth, "_threads", lambda: 1)
    b = synth.normal("t", (3, synth.CHUNK // 2 + 7), 0.5, synth.BF16, seed=0)
    assert np.array_equal(a, b)
    c = synth.normal("t", (3, synth.CHUNK // 2 + 7), 0.5, synth.BF16, seed=1)
    assert not np.array_equal(a, c)
    d = synth.normal("u", (3, synth.CHUNK // 2 + 7), 0.5, synth.BF16, seed=0)
    assert not np.array_equal(a, d)


def test_tiny_workload_distributions():
    w = synth.WORKLOADS["tiny_f32"]
    inp = synth.make_inputs(w)
    assert inp["x"].dtype == np.float32 and inp["x"].shape == (64, 128)
    assert abs(inp["x"].std() - 1) < 0.05
    assert abs(inp["router_w"].std() * math.sqrt(128) - 1) < 0.1
    assert abs(inp["w1"].std() * math.sqrt(128) - 1) < 0.02
    assert abs(inp["w2"].std() * math.sqrt(512) - 1) < 0.02
    assert inp["w1"].shape == (8, 128, 512) and inp["w2"].shape == (8, 512, 128)


def test_int8_and_scale_ranges():
    q = synth.uniform_int8("q", (1 << 20,), -127, 127)
    assert q.min() == -127 and q.max() == 127
    assert abs(q.astype(np.float64).mean()) < 0.5
    s = synth.bf16_bits_to_f32(synth.uniform_bf16("s", (1 << 16,), 1e-4, 5e-4))
    assert s.min() >= 1e-4 * (1 - 2 ** -8) and s.max() <= 5e-4 * (1 + 2 ** -8)


def test_weights_shared_across_token_counts():
    w = synth.Workload("small", T=8, d=64, f=128)
    wts = synth.make_weights(w)
    a = synth.make_inputs(w, T=8, weights=wts)
    b = synth.make_inputs(w, T=16, weights=wts)
    assert a["w1"] is b["w1"]
    assert a["x"].shape == (8, 64) and b["x"].shape == (16, 64)
    assert np.array_equal(synth.make_weights(w)["w2"], wts["w2"])


def test_sampled_rows():
    r = synth.sampled_rows(8192, 256)
    assert len(r) == 256 and len(set(r.tolist())) == 256 and np.all(np.diff(r) > 0)
    assert np.array_equal(r, synth.sampled_rows(8192, 256))
    assert np.array_equal(synth.sampled_rows(10, 256), np.arange(10))
