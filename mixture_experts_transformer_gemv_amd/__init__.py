"""Python binding of libgrokmoe.so: the gfx950 forward pass of one Grok-1 mixture-of-experts FFN layer.

Argument marshalling only.  Every step of the layer runs in the HIP kernels behind the C ABI of
include/grok_moe.h; torch supplies device memory and the current stream.  There is no fallback: if the library
is missing or a call fails, a RuntimeError is raised.

Tensors are torch tensors on the current HIP device, contiguous.  bf16 data is torch.bfloat16; int8 weights are
torch.int8 with torch.bfloat16 scales of shape [E, 1, out].  Weights are [E, in, out]: W1, Wv [E, d, f] and
W2 [E, f, d].
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "F32", "BF16", "W8", "LIB_PATH", "lib", "forward", "route", "bin_tokens", "expert_up", "expert_down",
    "combine", "workspace_size", "down_splits", "strerror", "dtype_of", "GrokMoeError", "block_forward",
    "block_workspace_size", "route_norm", "combine_norm", "IN_OUT", "OUT_IN", "scale_layout", "forward_noalloc",
    "SCRATCH_BYTES",
]

F32, BF16, W8 = 0, 1, 2
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgrokmoe.so")

_c_void_p, _i64, _int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
_SIGS = {
    "grok_moe_strerror": (ctypes.c_char_p, [_int]),
    "grok_moe_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, _int, _int, _int]),
    "grok_moe_down_splits": (_int, [_i64, _i64, _i64, _int, _int, _int]),
    "grok_moe_forward": (_int, [_c_void_p] * 8 + [_i64, _i64, _i64, _int, _int, _int] + [_c_void_p] * 6
                         + [ctypes.c_size_t, _c_void_p]),
    "grok_moe_forward_ex": (_int, [_c_void_p] * 8 + [_int, _int, _int, _int, _i64, _i64, _i64, _int, _int, _int]
                            + [_c_void_p] * 6 + [ctypes.c_size_t, _c_void_p]),
    "grok_moe_route": (_int, [_c_void_p] * 3 + [_i64, _i64, _int, _int, _int] + [_c_void_p] * 3),
    "grok_moe_bin": (_int, [_c_void_p, _i64, _int, _int] + [_c_void_p] * 5),
    "grok_moe_expert_up": (_int, [_c_void_p] * 5 + [_int, _int, _int] + [_c_void_p] * 3
                           + [_i64, _i64, _i64, _int, _int, _int, _c_void_p, _c_void_p]),
    "grok_moe_expert_down": (_int, [_c_void_p] * 3 + [_int, _int, _int] + [_c_void_p] * 2
                             + [_i64, _i64, _i64, _int, _int, _int, _int, _c_void_p, _c_void_p]),
    "grok_moe_combine": (_int, [_c_void_p, _int, _c_void_p, _c_void_p, _i64, _i64, _int, _c_void_p, _c_void_p]),
    "grok_moe_block_workspace_size": (ctypes.c_size_t, [_i64, _i64, _i64, _int, _int, _int]),
    "grok_moe_block_forward": (_int, [_c_void_p, _c_void_p, _c_void_p, ctypes.c_double] + [_c_void_p] * 7
                               + [_int, _int, _int, _int, _i64, _i64, _i64, _int, _int, _int] + [_c_void_p] * 6
                               + [ctypes.c_size_t, _c_void_p]),
    "grok_moe_route_norm": (_int, [_c_void_p, _c_void_p, ctypes.c_double, _c_void_p, _c_void_p, _i64, _i64, _int,
                                   _int, _int, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "grok_moe_combine_norm": (_int, [_c_void_p, _int, _c_void_p, _c_void_p, _c_void_p, _c_void_p, ctypes.c_double,
                                     _i64, _i64, _int, _int, _c_void_p, _c_void_p]),
    "grok_moe_forward_noalloc": (_int, [_c_void_p] * 8 + [_i64, _i64, _i64, _int, _int, _int] + [_c_void_p] * 6),
}

# bytes of the static scratch array behind forward_noalloc (GROK_MOE_SCRATCH_BYTES)
SCRATCH_BYTES = 64 << 20

# weight storage: [E, in, out] (the checkpoint's JAX layout) or [E, out, in] (the converted PyTorch layout)
IN_OUT, OUT_IN = "in_out", "out_in"
_LAYOUT = {IN_OUT: 0, OUT_IN: 1}


def _layout_code(weight_layout: str) -> int:
    if weight_layout not in _LAYOUT:
        raise GrokMoeError(f"weight_layout must be {IN_OUT!r} or {OUT_IN!r}, not {weight_layout!r}")
    return _LAYOUT[weight_layout]

_lib = None


class GrokMoeError(RuntimeError):
    pass


def lib() -> ctypes.CDLL:
    """The loaded HIP library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise GrokMoeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m mixture_experts_transformer_gemv_amd.build` (there is no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def strerror(status: int) -> str:
    return lib().grok_moe_strerror(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise GrokMoeError(f"{what}: {strerror(status)} (status {status})")


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def dtype_of(x: torch.Tensor, w1: torch.Tensor) -> int:
    if x.dtype == torch.float32 and w1.dtype == torch.float32:
        return F32
    if x.dtype == torch.bfloat16 and w1.dtype == torch.bfloat16:
        return BF16
    if x.dtype == torch.bfloat16 and w1.dtype == torch.int8:
        return W8
    raise GrokMoeError(f"unsupported combination x {x.dtype}, weights {w1.dtype}")


def _need(t: torch.Tensor, name: str, dtype=None, shape=None):
    if not t.is_cuda:
        raise GrokMoeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise GrokMoeError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise GrokMoeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise GrokMoeError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def workspace_size(T: int, d: int, f: int, E: int = 8, k: int = 2, dtype: int = BF16) -> int:
    return int(lib().grok_moe_workspace_size(T, d, f, E, k, dtype))


def down_splits(T: int, d: int, f: int, E: int = 8, k: int = 2, dtype: int = BF16) -> int:
    return int(lib().grok_moe_down_splits(T, d, f, E, k, dtype))


def _layer_shapes(x, router_w, w1, wv, w2, weight_layout=IN_OUT):
    T, d = x.shape
    if _layout_code(weight_layout) == 0:
        E, d2, f = w1.shape
        up, down = (E, d, f), (E, f, d)
    else:
        E, f, d2 = w1.shape
        up, down = (E, f, d), (E, d, f)
    if (router_w.shape != (E, d) or d2 != d or tuple(w1.shape) != up or tuple(wv.shape) != up
            or tuple(w2.shape) != down):
        raise GrokMoeError(f"inconsistent shapes x{tuple(x.shape)} router_w{tuple(router_w.shape)} "
                           f"w1{tuple(w1.shape)} wv{tuple(wv.shape)} w2{tuple(w2.shape)}")
    return T, d, f, E


def scale_layout(s, E: int, n: int, name: str):
    """(scale_experts, groups) of an int8 scale tensor [Es, G, n] or [Es, n] (one group); Es is 1 or E."""
    if s is None:
        raise GrokMoeError(f"{name}: int8 weights need scales")
    if s.dim() == 2:
        s = s.unsqueeze(1)
    if s.dim() != 3 or s.shape[2] != n or s.shape[0] not in (1, E):
        raise GrokMoeError(f"{name}: scale shape {tuple(s.shape)} is not [1 or {E}, G, {n}] or [1 or {E}, {n}]")
    _need(s, name, torch.bfloat16)
    return int(s.shape[0]), int(s.shape[1])


def _grouped(scales, E, d, f):
    """Scale layout of (s1, sv, s2): None for the per-(expert, channel) layout [E, 1, out], else
    (scale_experts, groups_up, groups_down)."""
    s1, sv, s2 = scales
    l1, lv, l2 = scale_layout(s1, E, f, "s1"), scale_layout(sv, E, f, "sv"), scale_layout(s2, E, d, "s2")
    if l1 != lv or l1[0] != l2[0]:
        raise GrokMoeError("s1 and sv need the same layout, and s2 the same expert count")
    if l1 == (E, 1) and l2 == (E, 1):
        return None
    return l1[0], l1[1], l2[1]


def forward(x, router_w, w1, wv, w2, scales=None, router_bias=None, return_routing=False, workspace=None,
            weight_layout=IN_OUT):
    """The whole layer.  Returns out [T, d] fp32, or (out, topk_idx [T,2] int32, topk_p [T,2] fp32,
    expert_counts [E] int32) if return_routing.  scales = (s1, sv, s2) for int8 weights, each [Es, G, out] or
    [Es, out] bf16 (Es = E or 1 shared; G groups along the input axis).  weight_layout: IN_OUT (W1, Wv [E, d, f],
    W2 [E, f, d]) or OUT_IN (W1, Wv [E, f, d], W2 [E, d, f])."""
    T, d, f, E = _layer_shapes(x, router_w, w1, wv, w2, weight_layout)
    lay = _layout_code(weight_layout)
    dt = dtype_of(x, w1)
    for t, n in ((x, "x"), (router_w, "router_w"), (w1, "w1"), (wv, "wv"), (w2, "w2")):
        _need(t, n)
    s1 = sv = s2 = None
    grouped = None
    if dt == W8:
        if scales is None:
            raise GrokMoeError("int8 weights need scales (s1, sv, s2)")
        s1, sv, s2 = scales
        grouped = _grouped(scales, E, d, f)
    if router_bias is not None:
        _need(router_bias, "router_bias", torch.float32, (E,))
    dev = x.device
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    idx = torch.empty((T, 2), dtype=torch.int32, device=dev) if return_routing else None
    pr = torch.empty((T, 2), dtype=torch.float32, device=dev) if return_routing else None
    cnt = torch.empty((E,), dtype=torch.int32, device=dev) if return_routing else None
    need = workspace_size(T, d, f, E, 2, dt)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    wsb = workspace.numel() * workspace.element_size()
    if lay == 0 and grouped is None:
        st = lib().grok_moe_forward(_p(x), _p(router_w), _p(w1), _p(wv), _p(w2), _p(s1), _p(sv), _p(s2),
                                    T, d, f, E, 2, dt, _p(out), _p(router_bias), _p(idx), _p(pr), _p(cnt),
                                    _p(workspace), wsb, _stream())
        _check(st, "grok_moe_forward")
    else:
        es, g1, g2 = grouped if grouped is not None else (E, 1, 1)
        st = lib().grok_moe_forward_ex(_p(x), _p(router_w), _p(w1), _p(wv), _p(w2), _p(s1), _p(sv), _p(s2), lay, es,
                                       g1, g2, T, d, f, E, 2, dt, _p(out), _p(router_bias), _p(idx), _p(pr), _p(cnt),
                                       _p(workspace), wsb, _stream())
        _check(st, "grok_moe_forward_ex")
    if return_routing:
        return out, idx, pr, cnt
    return out


def forward_noalloc(x, router_w, w1, wv, w2, scales=None, router_bias=None, out=None, routing=None):
    """The whole layer through grok_moe_forward_noalloc: no workspace; the library's static scratch array on the
    current device serves as one (calls that overlap on one GPU race).  [E, in, out] weights, scales [E, 1, out] for
    int8.  out [T, d] fp32 and routing = (topk_idx, topk_p, expert_counts) may be given preallocated; returns out,
    or (out, idx, p, counts) if routing is given."""
    T, d, f, E = _layer_shapes(x, router_w, w1, wv, w2)
    dt = dtype_of(x, w1)
    for t, n in ((x, "x"), (router_w, "router_w"), (w1, "w1"), (wv, "wv"), (w2, "w2")):
        _need(t, n)
    s1 = sv = s2 = None
    if dt == W8:
        if scales is None or _grouped(scales, E, d, f) is not None:
            raise GrokMoeError("forward_noalloc takes int8 scales of layout [E, 1, out]")
        s1, sv, s2 = scales
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=x.device)
    idx, pr, cnt = routing if routing is not None else (None, None, None)
    _check(lib().grok_moe_forward_noalloc(_p(x), _p(router_w), _p(w1), _p(wv), _p(w2), _p(s1), _p(sv), _p(s2),
                                          T, d, f, E, 2, dt, _p(out), _p(router_bias), _p(idx), _p(pr), _p(cnt),
                                          _stream()), "grok_moe_forward_noalloc")
    return out if routing is None else (out, idx, pr, cnt)


def route(x, router_w, router_bias=None):
    """Router step: (topk_idx [T,2] int32, topk_p [T,2] fp32)."""
    T, d = x.shape
    E = router_w.shape[0]
    _need(x, "x")
    _need(router_w, "router_w", x.dtype, (E, d))
    dt = F32 if x.dtype == torch.float32 else BF16
    idx = torch.empty((T, 2), dtype=torch.int32, device=x.device)
    pr = torch.empty((T, 2), dtype=torch.float32, device=x.device)
    _check(lib().grok_moe_route(_p(x), _p(router_w), _p(router_bias), T, d, E, 2, dt, _p(idx), _p(pr), _stream()),
           "grok_moe_route")
    return idx, pr


def bin_tokens(topk_idx, E: int):
    """Binning step: (counts [E], offsets [E+1], perm [2T], inv [T,2]), all int32."""
    T = topk_idx.shape[0]
    _need(topk_idx, "topk_idx", torch.int32, (T, 2))
    dev = topk_idx.device
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    perm = torch.empty((max(2 * T, 1),), dtype=torch.int32, device=dev)[: 2 * T]
    inv = torch.empty((T, 2), dtype=torch.int32, device=dev)
    _check(lib().grok_moe_bin(_p(topk_idx), T, E, 2, _p(counts), _p(offsets), _p(perm), _p(inv), _stream()),
           "grok_moe_bin")
    return counts, offsets, perm, inv


def expert_up(x, w1, wv, counts, offsets, perm, scales=None, h=None, weight_layout=IN_OUT):
    """Fused up-projection step: h [2T, f] (bf16, or fp32 for an fp32 layer) in slot order."""
    T, d = x.shape
    lcode = _layout_code(weight_layout)
    E, f = (w1.shape[0], w1.shape[2]) if lcode == 0 else (w1.shape[0], w1.shape[1])
    dt = dtype_of(x, w1)
    s1 = sv = None
    lay = (E, 1)
    if dt == W8:
        s1, sv = scales[0], scales[1]
        lay = scale_layout(s1, E, f, "s1")
        if scale_layout(sv, E, f, "sv") != lay:
            raise GrokMoeError("s1 and sv need the same layout")
    if h is None:
        h = torch.empty((2 * T, f), dtype=torch.float32 if dt == F32 else torch.bfloat16, device=x.device)
    _check(lib().grok_moe_expert_up(_p(x), _p(w1), _p(wv), _p(s1), _p(sv), lcode, *lay, _p(counts), _p(offsets),
                                    _p(perm), T, d, f, E, 2, dt, _p(h), _stream()), "grok_moe_expert_up")
    return h


def expert_down(h, w2, counts, offsets, T: int, x_dtype, s2=None, y=None, weight_layout=IN_OUT):
    """Down-projection step: y [S, 2T, d] fp32 partial sums (S = down_splits)."""
    lcode = _layout_code(weight_layout)
    E, f, d = w2.shape if lcode == 0 else (w2.shape[0], w2.shape[2], w2.shape[1])
    dt = F32 if w2.dtype == torch.float32 else (W8 if w2.dtype == torch.int8 else BF16)
    S = down_splits(T, d, f, E, 2, dt)
    if y is None:
        y = torch.empty((S, 2 * T, d), dtype=torch.float32, device=h.device)
    lay = scale_layout(s2, E, d, "s2") if dt == W8 else (E, 1)
    _check(lib().grok_moe_expert_down(_p(h), _p(w2), _p(s2), lcode, *lay, _p(counts), _p(offsets), T, d, f, E, 2,
                                      dt, S, _p(y), _stream()), "grok_moe_expert_down")
    return y


def combine(y, topk_p, inv, out=None):
    """Combine step: out [T, d] fp32."""
    S, slots, d = y.shape
    T = topk_p.shape[0]
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=y.device)
    _check(lib().grok_moe_combine(_p(y), S, _p(topk_p), _p(inv), T, d, 2, _p(out), _stream()), "grok_moe_combine")
    return out


def block_workspace_size(T: int, d: int, f: int, E: int = 8, k: int = 2, dtype: int = BF16) -> int:
    return int(lib().grok_moe_block_workspace_size(T, d, f, E, k, dtype))


def block_forward(x, pre_scale, post_scale, eps, router_w, w1, wv, w2, scales=None, router_bias=None,
                  return_routing=False, workspace=None, weight_layout=IN_OUT):
    """The MoE part of a Grok-1 layer with its norms and residual: out = x + RMSNorm(MoE(RMSNorm(x; pre_scale));
    post_scale), fp32 [T, d].  pre_scale, post_scale: [d] in the activation type of x.  Weights, scales and
    weight_layout as for forward()."""
    T, d, f, E = _layer_shapes(x, router_w, w1, wv, w2, weight_layout)
    lay = _layout_code(weight_layout)
    dt = dtype_of(x, w1)
    for t, n in ((x, "x"), (router_w, "router_w"), (w1, "w1"), (wv, "wv"), (w2, "w2")):
        _need(t, n)
    _need(pre_scale, "pre_scale", x.dtype, (d,))
    _need(post_scale, "post_scale", x.dtype, (d,))
    s1 = sv = s2 = None
    grouped = None
    if dt == W8:
        if scales is None:
            raise GrokMoeError("int8 weights need scales (s1, sv, s2)")
        s1, sv, s2 = scales
        grouped = _grouped(scales, E, d, f)
    dev = x.device
    out = torch.empty((T, d), dtype=torch.float32, device=dev)
    idx = torch.empty((T, 2), dtype=torch.int32, device=dev) if return_routing else None
    pr = torch.empty((T, 2), dtype=torch.float32, device=dev) if return_routing else None
    cnt = torch.empty((E,), dtype=torch.int32, device=dev) if return_routing else None
    need = block_workspace_size(T, d, f, E, 2, dt)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty((max(need, 256),), dtype=torch.uint8, device=dev)
    es, g1, g2 = grouped if grouped is not None else (E, 1, 1)
    st = lib().grok_moe_block_forward(_p(x), _p(pre_scale), _p(post_scale), float(eps), _p(router_w), _p(w1),
                                      _p(wv), _p(w2), _p(s1), _p(sv), _p(s2), lay, es, g1, g2, T, d, f, E, 2, dt,
                                      _p(out), _p(router_bias), _p(idx), _p(pr), _p(cnt), _p(workspace),
                                      workspace.numel() * workspace.element_size(), _stream())
    _check(st, "grok_moe_block_forward")
    if return_routing:
        return out, idx, pr, cnt
    return out


def route_norm(x, pre_scale, eps, router_w, router_bias=None):
    """Pre-MoE RMSNorm fused with the router step: (xn [T,d], topk_idx [T,2], topk_p [T,2])."""
    T, d = x.shape
    E = router_w.shape[0]
    dt = F32 if x.dtype == torch.float32 else BF16
    xn = torch.empty_like(x)
    idx = torch.empty((T, 2), dtype=torch.int32, device=x.device)
    pr = torch.empty((T, 2), dtype=torch.float32, device=x.device)
    _check(lib().grok_moe_route_norm(_p(x), _p(pre_scale), float(eps), _p(router_w), _p(router_bias), T, d, E, 2,
                                     dt, _p(xn), _p(idx), _p(pr), _stream()), "grok_moe_route_norm")
    return xn, idx, pr


def combine_norm(y, topk_p, inv, x, post_scale, eps, out=None):
    """Combine fused with the post-MoE RMSNorm and the residual add: out [T, d] fp32."""
    S, slots, d = y.shape
    T = topk_p.shape[0]
    dt = F32 if x.dtype == torch.float32 else BF16
    if out is None:
        out = torch.empty((T, d), dtype=torch.float32, device=y.device)
    _check(lib().grok_moe_combine_norm(_p(y), S, _p(topk_p), _p(inv), _p(x), _p(post_scale), float(eps), T, d, 2, dt,
                                       _p(out), _stream()), "grok_moe_combine_norm")
    return out
