"""Plain CPU oracle of the forward pass of one Grok-1 mixture-of-experts FFN layer.

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's CPU-baseline leg may import this module.
It shares no code with the HIP library and never imports it; both sides take their inputs from ``synth``.

Everything is evaluated in float64 on the exact values of the stored inputs, with plain PyTorch CPU operations
(a float64 matrix product is the only library primitive used as a step).  Pages followed:

* [bridge] "A functional bridge between openai/grok and xai-org/grok-1" (github.com/Jah-yee/grok README),
  architecture diagram: each expert is GELU(x W1) ⊙ (x Wv) W2; 8 experts, top-2 routing.
* [moe] "Grok-1: 314B Total Parameters, 25B Active Per Token (MoE Explained)",
  section "Expert Routing Details": logits = gate(x) (a Dense layer to the expert count), gates = softmax(logits),
  then top_k(gates, k=2) returns (top-k gates, top-k indices); no gating noise outside training.
  Section "How MoE Works in Practice": the layer output is the sum, over the selected experts, of each expert's
  output times that expert's router weight.
* [card] "Grok-1-BF16" (TevunahAi conversion notes), section "Conversion Details": int8 weights times bf16 scales,
  scales broadcast over the grouped axis, JAX [in, out] layout; section "Verification": tensor shapes and the
  four RMSNorms of a layer (pre_moe_norm and post_moe_norm around moe_block); section "Architecture": "Four norms
  per layer".
* [bridge] lists RMSNorm among Grok-1's components; [moe] section "Why JAX Instead of PyTorch" shows the block as
  x = x + moe(norm(x)).

Readings where the pages leave a step open (each is also listed in the design notes):
  * GELU is the exact erf form (the pages name GELU without saying which).
  * The two combine weights are the softmax probabilities of the selected experts over all E experts, not
    renormalised over the two ([moe] returns top_k of the full softmax and multiplies by it).
  * Selection is by descending logit with the lower expert index first on equal logits (softmax is strictly
    increasing, so this equals selecting on the probabilities, without ties created by rounding them).
  * Weights are stored [E, in, out]: W1, Wv are [E, d, f], W2 is [E, f, d] (the checkpoint's JAX layout), or, on
    request, [E, out, in] (the PyTorch layout [card] converts to); int8 scales are [Es, G, out] with Es = E (per
    expert) or 1 (shared) and G contiguous groups along the in axis (G = 1: per output channel).
  * In the bf16 and int8 layers the intermediate h = GELU(a) ⊙ b is rounded once to bf16 (round to nearest
    even, directly from float64) before the down projection; the fp32 layer keeps h unrounded.
  * The optional per-expert router bias is added to the logits before the softmax.
  * The MoE block: out = x + RMSNorm_post(MoE(RMSNorm_pre(x))), RMSNorm(v) = v / sqrt(mean(v^2) + eps) * scale
    (pre-norm output rounded once to the layer's activation type, post-norm on the fp32 MoE output); eps is not
    on the pages and is an argument.
"""
from __future__ import annotations

import math

import numpy as np
import torch

F32, BF16, W8 = 0, 1, 2

__all__ = [
    "F32", "BF16", "W8", "IN_OUT", "OUT_IN", "as_f64", "bf16_round", "gelu", "route", "expert_ffn", "dequant",
    "expert_scales", "stored_in_out", "forward", "rmsnorm", "block_forward",
]


def as_f64(a, kind: str) -> torch.Tensor:
    """Exact float64 value of a stored tensor.  kind: 'f32' (float32), 'bf16' (uint16 bit patterns), 'i8'."""
    a = np.ascontiguousarray(a)
    if kind == "f32":
        return torch.from_numpy(a.astype(np.float32, copy=False)).to(torch.float64)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(torch.float64)
    if kind == "i8":
        return torch.from_numpy(a.astype(np.int8, copy=False)).to(torch.float64)
    raise ValueError(kind)


def bf16_round(v: torch.Tensor) -> torch.Tensor:
    """Round float64 values to the bfloat16 grid (8 significant bits) with one round-to-nearest-even step.

    Uses frexp: v = m * 2**e with 0.5 <= |m| < 1, so m * 2**8 carries exactly the 8 significant bits plus the
    fraction to be rounded.  The values met here are far inside bf16's normal range.
    """
    m, e = torch.frexp(v)
    return torch.ldexp(torch.round(torch.ldexp(m, torch.full_like(e, 8))), e - 8)


def gelu(z: torch.Tensor) -> torch.Tensor:
    """Exact GELU: z * Phi(z) = 0.5 z (1 + erf(z / sqrt 2))."""
    return 0.5 * z * (1.0 + torch.special.erf(z / math.sqrt(2.0)))


def route(x: torch.Tensor, router_w: torch.Tensor, bias: torch.Tensor | None = None, k: int = 2) -> dict:
    """Router of [moe] "Expert Routing Details": gate logits, softmax over all experts, top-k.

    x [T, d] and router_w [E, d] in float64.  Returns logits [T, E], probs [T, E], idx [T, k] (int64, descending
    logit, lower index first on ties), p [T, k] = probs at idx, and the smallest logit gaps (diagnostics).
    """
    logits = x @ router_w.T
    if bias is not None:
        logits = logits + bias[None, :]
    T, E = logits.shape
    mx = logits.max(dim=1, keepdim=True).values
    ex = torch.exp(logits - mx)
    probs = ex / ex.sum(dim=1, keepdim=True)
    idx = torch.empty((T, k), dtype=torch.int64)
    taken = torch.zeros((T, E), dtype=torch.bool)
    rows = torch.arange(T)
    for j in range(k):
        best = torch.full((T,), -1, dtype=torch.int64)
        bestv = torch.full((T,), -math.inf, dtype=torch.float64)
        for e in range(E):  # ascending e with strict '>' keeps the lower index on equal logits
            le = logits[:, e]
            better = (~taken[:, e]) & ((best < 0) | (le > bestv))
            best = torch.where(better, torch.full_like(best, e), best)
            bestv = torch.where(better, le, bestv)
        idx[:, j] = best
        taken[rows, best] = True
    p = probs.gather(1, idx)
    srt = torch.sort(logits, dim=1, descending=True).values
    gap12 = (srt[:, 0] - srt[:, 1]).min().item() if E > 1 else math.inf
    gap_k = (srt[:, k - 1] - srt[:, k]).min().item() if E > k else math.inf
    return {"logits": logits, "probs": probs, "idx": idx, "p": p, "min_gap_top": gap12, "min_gap_cut": gap_k}


def expert_ffn(x: torch.Tensor, w1: torch.Tensor, wv: torch.Tensor, w2: torch.Tensor, round_h: bool) -> tuple:
    """One expert of [bridge]'s diagram on rows x [n, d]: h = GELU(x W1) ⊙ (x Wv); y = h W2.

    w1, wv [d, f] and w2 [f, d] in float64 ([in, out]).  Returns (h, y).
    """
    a = x @ w1
    b = x @ wv
    h = gelu(a) * b
    if round_h:
        h = bf16_round(h)
    return h, h @ w2


def dequant(q, s) -> torch.Tensor:
    """[card] "Conversion Details": weight = int8 value times its bf16 scale, the scale broadcast over its group.

    q [in, out] int8 (numpy); s [G, out] bf16 bits (numpy), G >= 1 dividing `in`: rows k of q take the scales of
    group k // (in / G) (G = 1: one scale per output channel).  Exact in float64.
    """
    q = as_f64(q, "i8")
    sc = as_f64(s, "bf16")
    K = q.shape[0]
    G = sc.shape[0]
    if K % G:
        raise ValueError(f"{G} scale groups do not divide the input size {K}")
    return q * torch.repeat_interleave(sc, K // G, dim=0)


def expert_scales(s, e: int) -> np.ndarray:
    """The [G, out] scales of expert e from a scale tensor of one of the shapes [card] lists: [Es, G, out]
    ((8,1,N), (8,8,N)) or [Es, out] ((1,N), (8,N), read as one group).  Es = 1 means shared by all experts."""
    s = np.asarray(s)
    if s.ndim == 2:
        s = s[:, None, :]
    if s.ndim != 3:
        raise ValueError(f"scale tensor of rank {s.ndim}")
    return s[e if s.shape[0] > 1 else 0]


IN_OUT, OUT_IN = "in_out", "out_in"


def stored_in_out(w, layout: str):
    """Expert e's weight as [in, out] from its stored form: [in, out] as in the checkpoint (JAX), or [out, in] as
    after [card]'s conversion to the PyTorch convention (then it is the transpose)."""
    if layout == IN_OUT:
        return w
    if layout == OUT_IN:
        return np.asarray(w).T
    raise ValueError(layout)


def _expert_weights(inp: dict, dtype: int, e: int, layout: str = IN_OUT):
    w = {n: stored_in_out(inp[n][e], layout) for n in ("w1", "wv", "w2")}
    if dtype == F32:
        return tuple(as_f64(w[n], "f32") for n in ("w1", "wv", "w2"))
    if dtype == BF16:
        return tuple(as_f64(w[n], "bf16") for n in ("w1", "wv", "w2"))
    if dtype == W8:
        return tuple(dequant(w[n], expert_scales(inp[sn], e)) for n, sn in (("w1", "s1"), ("wv", "sv"), ("w2", "s2")))
    raise ValueError(dtype)


def forward(inp: dict, dtype: int, rows=None, k: int = 2, return_h: bool = False, layout: str = IN_OUT,
            round_h: bool | None = None) -> dict:
    """The whole layer: routing on every token, expert FFNs and combine on ``rows`` (all rows if None).

    layout: how the expert weights are stored, IN_OUT (W1, Wv [E, d, f], W2 [E, f, d]) or OUT_IN (W1, Wv
    [E, f, d], W2 [E, d, f]); int8 scales are [Es, G, out] either way.

    round_h: whether h is rounded once to bf16 before the down projection.  None (the default) takes the reading
    above: rounded in the bf16 and int8 layers, not in the fp32 layer.  False gives the plain float64 definition
    of the architecture diagram ([bridge]) for any storage type, the reference against which the rounding of h
    itself is measured.

    inp: dict of numpy arrays as produced by ``synth.make_inputs`` (x, router_w, w1, wv, w2, s1, sv, s2,
    router_bias).  Returns float64 tensors: out [len(rows), d]; idx [T, k]; p [T, k]; counts [E]; logits; probs;
    and, if asked, h [len(rows), k, f] and y [len(rows), k, d] per (row, selected expert).
    """
    akind = "f32" if dtype == F32 else "bf16"
    x = as_f64(inp["x"], akind)
    rw = as_f64(inp["router_w"], akind)
    bias = inp.get("router_bias")
    bias = None if bias is None else torch.from_numpy(np.asarray(bias, dtype=np.float32)).to(torch.float64)
    T, d = x.shape
    E = rw.shape[0]
    r = route(x, rw, bias, k)
    idx, p = r["idx"], r["p"]
    counts = torch.bincount(idx.reshape(-1), minlength=E)
    rows = torch.arange(T) if rows is None else torch.as_tensor(np.asarray(rows), dtype=torch.int64)
    n = rows.numel()
    sel = idx[rows]  # [n, k]
    out = torch.zeros((n, d), dtype=torch.float64)
    f = inp["w1"].shape[2] if layout == IN_OUT else inp["w1"].shape[1]
    hs = torch.zeros((n, k, f), dtype=torch.float64) if return_h else None
    ys = torch.zeros((n, k, d), dtype=torch.float64) if return_h else None
    round_h = (dtype != F32) if round_h is None else bool(round_h)
    ys_all = torch.zeros((n, k, d), dtype=torch.float64)
    for e in range(E):
        hit = (sel == e).nonzero()  # (row position, slot j) pairs choosing expert e
        if hit.numel() == 0:
            continue
        w1, wv, w2 = _expert_weights(inp, dtype, e, layout)
        h, y = expert_ffn(x[rows[hit[:, 0]]], w1, wv, w2, round_h)
        del w1, wv, w2
        ys_all[hit[:, 0], hit[:, 1]] = y
        if return_h:
            hs[hit[:, 0], hit[:, 1]] = h
    # combine of [moe] "How MoE Works in Practice": sum over the k selected experts of p_j * y_j
    pr = p[rows]
    for j in range(k):
        out += pr[:, j:j + 1] * ys_all[:, j]
    res = {"out": out, "idx": idx, "p": p, "counts": counts, "logits": r["logits"], "probs": r["probs"],
           "rows": rows, "min_gap_top": r["min_gap_top"], "min_gap_cut": r["min_gap_cut"]}
    if return_h:
        res["h"] = hs
        res["y"] = ys_all
    return res


def rmsnorm(v: torch.Tensor, scale: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm over the last axis: v / sqrt(mean(v^2) + eps) * scale, in float64."""
    return v / torch.sqrt((v * v).mean(dim=-1, keepdim=True) + eps) * scale


def block_forward(inp: dict, dtype: int, pre_scale, post_scale, eps: float, rows=None, k: int = 2,
                  layout: str = IN_OUT) -> dict:
    """The MoE part of a Grok-1 layer with its two norms and the residual:
    out = x + RMSNorm_post(MoE(RMSNorm_pre(x))).

    pre_scale, post_scale: [d] arrays in the activation type (float32 for the fp32 layer, bf16 bits otherwise).
    The pre-norm output is what the router and the experts see, stored in the activation type: rounded once to
    bf16 (nearest even, from float64) in the bf16 and int8 layers, rounded to float32 in the fp32 layer.
    Returns the forward() dict of the MoE on the normed input, with 'out' replaced by the block output and the
    normed input under 'xn' (float64)."""
    akind = "f32" if dtype == F32 else "bf16"
    x = as_f64(inp["x"], akind)
    g_pre = as_f64(np.asarray(pre_scale), akind)
    g_post = as_f64(np.asarray(post_scale), akind)
    xn = rmsnorm(x, g_pre, eps)
    if dtype == F32:
        xn_stored = xn.to(torch.float32).numpy()  # the fp32 layer stores its activations in float32
    else:
        xn_stored = _to_bf16_bits(bf16_round(xn))
    inner = dict(inp)
    inner["x"] = xn_stored
    r = forward(inner, dtype, rows=rows, k=k, layout=layout)
    rows_t = r["rows"]
    moe = r["out"]
    r["moe_out"] = moe
    r["out"] = x[rows_t] + rmsnorm(moe, g_post, eps)
    r["xn"] = as_f64(xn_stored, akind)
    return r


def _to_bf16_bits(v: torch.Tensor) -> np.ndarray:
    """float64 values already on the bf16 grid -> their bf16 bit patterns (exact)."""
    f32 = v.to(torch.float32).numpy()  # exact: bf16 values are float32 values
    return (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
