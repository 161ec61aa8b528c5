"""Seeded synthetic inputs for the Grok-1 MoE FFN layer.

This module only draws random numbers and stores them in the layer's storage types (fp32, bf16 bit patterns,
int8).  It holds none of the layer's arithmetic, so both the HIP path and the CPU oracle can take their inputs
from it without sharing any of the method.

Shapes follow the Grok-1 architecture as the pages list it:
  * d_model = 6144, 8 experts, 2 selected per token (page "Grok-1 by torrent: 314 billion parameters,
    Apache 2.0, no paper", section "What was released");
  * expert tensors linear / linear_v of [32768, 6144] and linear_1 of [6144, 32768] in the PyTorch [out, in]
    convention, router gate.weight [8, 6144] (page "Grok-1-BF16", section "Verification", weight listing).
This module stores expert weights in the JAX [in, out] convention: W1, Wv as [E, d, f] and W2 as [E, f, d]
(page "Grok-1-BF16", section "Conversion Details", which states that the original checkpoint is [in, out]).

Every tensor has its own random stream: numpy SeedSequence(seed, spawn_key=(crc32(name), chunk)).  Large tensors
are drawn in fixed-size chunks on a thread pool, so the values do not depend on the number of threads.
"""
from __future__ import annotations

import math
import os
import zlib
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

CHUNK = 1 << 22  # elements per independently seeded chunk

F32, BF16, W8 = 0, 1, 2  # storage dtypes; same numbering as the C ABI's grok_moe_dtype
DTYPE_NAMES = {F32: "f32", BF16: "bf16", W8: "w8"}


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def f32_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even) and return the 16-bit patterns.

    This is a storage conversion of drawn samples, applied identically for every consumer of the inputs.
    """
    u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _key(name: str) -> int:
    return zlib.crc32(name.encode())


def _rng(seed: int, name: str, chunk: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(_key(name), chunk))))


def _chunked(n: int, out: np.ndarray, fill) -> np.ndarray:
    nchunks = max(1, math.ceil(n / CHUNK))

    def work(c):
        lo = c * CHUNK
        hi = min(n, lo + CHUNK)
        out[lo:hi] = fill(c, hi - lo)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def normal(name: str, shape, std: float, dtype: int, seed: int = 0) -> np.ndarray:
    """N(0, std^2) samples: float32 array for F32, bf16 bit patterns (uint16) otherwise."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == F32 else np.uint16)
    s = np.float32(std)

    def fill(c, m):
        v = _rng(seed, name, c).standard_normal(m, dtype=np.float32)
        if std != 1.0:
            v *= s
        return v if dtype == F32 else f32_to_bf16_bits(v)

    return _chunked(n, out, fill).reshape(shape)


def uniform_int8(name: str, shape, lo: int, hi: int, seed: int = 0) -> np.ndarray:
    """Integers uniform on [lo, hi] (inclusive), stored as int8."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.int8)

    def fill(c, m):
        return _rng(seed, name, c).integers(lo, hi + 1, size=m, dtype=np.int8)

    return _chunked(n, out, fill).reshape(shape)


def uniform_bf16(name: str, shape, lo: float, hi: float, seed: int = 0) -> np.ndarray:
    """U(lo, hi) samples rounded to bf16 bit patterns."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)

    def fill(c, m):
        v = _rng(seed, name, c).uniform(lo, hi, size=m).astype(np.float32)
        return f32_to_bf16_bits(v)

    return _chunked(n, out, fill).reshape(shape)


@dataclass
class Workload:
    """One synthetic layer configuration (shapes, storage type, distributions)."""

    name: str
    T: int
    d: int
    f: int
    E: int = 8
    k: int = 2
    dtype: int = BF16
    router_bias: tuple | None = None
    sampled_rows: int | None = None  # check the expert path on this many seeded rows (None = all rows)
    seed: int = 0
    w_std: float = 0.02  # std of bf16 expert weights
    # int8 scale layout [Es, G, out]: Es = E (per expert) or 1 (shared by all experts); G contiguous groups along
    # the input axis of W1/Wv (groups_up) and of W2 (groups_down)
    scale_experts: int | None = None
    groups_up: int = 1
    groups_down: int = 1
    note: str = ""
    tags: dict = field(default_factory=dict)


# The five workloads of the layer: shapes and distributions as described above; bf16 weights have std 0.02,
# the router N(0, 1/d) (variance), the tiny fp32 layer N(0, 1/fan_in) (variance).
WORKLOADS = {
    "tiny_f32": Workload("tiny_f32", T=64, d=128, f=512, dtype=F32,
                         note="tiny fp32 layer: T=64, d=128, f=512, E=8, top-2"),
    "decode_bf16": Workload("decode_bf16", T=8, d=6144, f=32768, dtype=BF16,
                            note="Grok-1 shape decode step: T=8, bf16 weights and activations"),
    "prefill_bf16": Workload("prefill_bf16", T=8192, d=6144, f=32768, dtype=BF16, sampled_rows=256,
                             note="Grok-1 shape prefill: T=8192 (maximum context), bf16"),
    "int8_w8": Workload("int8_w8", T=64, d=6144, f=32768, dtype=W8,
                        note="Grok-1 shape, int8 weights with per-(expert, channel) bf16 scales, T=64"),
    "int8_w8_g8": Workload("int8_w8_g8", T=64, d=6144, f=32768, dtype=W8, groups_up=8, groups_down=8,
                           note="Grok-1 shape, int8 weights with (8, 8, N) group-wise bf16 scales, T=64"),
    "skew_bf16": Workload("skew_bf16", T=4096, d=6144, f=32768, dtype=BF16, sampled_rows=256,
                          router_bias=(3.0, 0.0, 0.0, 0.0, 0.0, 1.5, 0.0, 0.0),
                          note="skewed routing: logit bias +3 on expert 0, +1.5 on expert 5, T=4096"),
}


def make_inputs(w: Workload, T: int | None = None, weights: dict | None = None) -> dict:
    """Draw every input tensor of workload ``w`` (optionally at another token count ``T``).

    ``weights`` may carry already drawn weight tensors (they do not depend on T) to avoid drawing them twice.
    Returns a dict of numpy arrays: x, router_w, w1, wv, w2, s1, sv, s2 (None unless int8), router_bias (or None).
    """
    T = w.T if T is None else T
    d, f, E, dt, seed = w.d, w.f, w.E, w.dtype, w.seed
    out = {}
    act_dt = F32 if dt == F32 else BF16
    out["x"] = normal(f"x/T={T}/d={d}", (T, d), 1.0, act_dt, seed)
    if weights is None:
        weights = make_weights(w)
    out.update(weights)
    out["router_bias"] = None if w.router_bias is None else np.asarray(w.router_bias, dtype=np.float32)
    return out


def make_weights(w: Workload) -> dict:
    d, f, E, dt, seed = w.d, w.f, w.E, w.dtype, w.seed
    out = {}
    if dt == F32:
        out["router_w"] = normal(f"router_w/{d}/E={E}", (E, d), 1.0 / math.sqrt(d), F32, seed)
        out["w1"] = normal(f"w1/{d}x{f}/E={E}", (E, d, f), 1.0 / math.sqrt(d), F32, seed)
        out["wv"] = normal(f"wv/{d}x{f}/E={E}", (E, d, f), 1.0 / math.sqrt(d), F32, seed)
        out["w2"] = normal(f"w2/{f}x{d}/E={E}", (E, f, d), 1.0 / math.sqrt(f), F32, seed)
        out["s1"] = out["sv"] = out["s2"] = None
    elif dt == BF16:
        out["router_w"] = normal(f"router_w/{d}/E={E}", (E, d), 1.0 / math.sqrt(d), BF16, seed)
        out["w1"] = normal(f"w1/{d}x{f}/E={E}", (E, d, f), w.w_std, BF16, seed)
        out["wv"] = normal(f"wv/{d}x{f}/E={E}", (E, d, f), w.w_std, BF16, seed)
        out["w2"] = normal(f"w2/{f}x{d}/E={E}", (E, f, d), w.w_std, BF16, seed)
        out["s1"] = out["sv"] = out["s2"] = None
    elif dt == W8:
        out["router_w"] = normal(f"router_w/{d}/E={E}", (E, d), 1.0 / math.sqrt(d), BF16, seed)
        out["w1"] = uniform_int8(f"q1/{d}x{f}/E={E}", (E, d, f), -127, 127, seed)
        out["wv"] = uniform_int8(f"qv/{d}x{f}/E={E}", (E, d, f), -127, 127, seed)
        out["w2"] = uniform_int8(f"q2/{f}x{d}/E={E}", (E, f, d), -127, 127, seed)
        Es = E if w.scale_experts is None else w.scale_experts
        g1, g2 = w.groups_up, w.groups_down
        tag1 = "" if (Es, g1) == (E, 1) else f"/G={g1}"
        tag2 = "" if (Es, g2) == (E, 1) else f"/G={g2}"
        out["s1"] = uniform_bf16(f"s1/{f}/E={Es}{tag1}", (Es, g1, f), 1e-4, 5e-4, seed)
        out["sv"] = uniform_bf16(f"sv/{f}/E={Es}{tag1}", (Es, g1, f), 1e-4, 5e-4, seed)
        out["s2"] = uniform_bf16(f"s2/{d}/E={Es}{tag2}", (Es, g2, d), 1e-4, 5e-4, seed)
    else:
        raise ValueError(f"unknown dtype {dt}")
    return out


def sampled_rows(T: int, n: int, seed: int = 1) -> np.ndarray:
    """The seeded subset of token rows on which prefill-sized runs are checked (sorted)."""
    if n >= T:
        return np.arange(T, dtype=np.int64)
    return np.sort(np.random.default_rng(seed).choice(T, n, replace=False)).astype(np.int64)


def make_norm_scales(w: Workload, eps: float = 1e-5) -> dict:
    """Scales of the pre-MoE and post-MoE RMSNorms, [d] each, drawn as 1 + 0.1 N(0, 1) in the activation type,
    and the eps used with them (the pages give no eps; 1e-5 is a common choice)."""
    act = F32 if w.dtype == F32 else BF16
    out = {}
    for name in ("pre_scale", "post_scale"):
        v = normal(f"{name}/{w.d}", (w.d,), 0.1, F32, w.seed) + np.float32(1.0)
        out[name] = v if act == F32 else f32_to_bf16_bits(v)
    out["eps"] = eps
    return out
