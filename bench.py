#!/usr/bin/env python3
"""Throughput of the Grok-1 MoE FFN layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload decode_bf16|prefill_bf16|int8_w8|int8_w8_g8|skew_bf16|tiny_f32]
                    [--weight-layout in_out|out_in] [--block] [--no-prefill] [--no-cpu-baseline]
    python bench.py --library-gemm      (torch.mm / hipBLASLt on the prefill's per-expert shapes, for context)

A step is one pass of the whole layer (router, binning, fused up-projection with GELU product, down-projection,
combine) over one batch of seeded synthetic tokens, with weights and inputs already resident in HBM.  The step
calls the library's five step entry points in order (bit-identical to grok_moe_forward) on the current stream,
so that HIP events can time the expert kernels inside the timed region.  Prints one JSON line.

The default workload is the Grok-1-shape decode step (T=8, d=6144, f=32768, E=8, top-2, bf16).  Unless
--no-prefill is given, the same run also times the T=8192 prefill on the same weights and reports it under
"prefill".  The CPU oracle is timed on a bounded sample of the same workload ("cpu_baseline").
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "Grok-1 MoE layer tokens/s (T=8 decode, T=8192 prefill); % of roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_VALU_TFLOPS = 157.3       # MI355X fp32 vector ALU (published)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_hash(files) -> str:
    h = hashlib.sha256()
    for n in files:
        with open(os.path.join(ROOT, "mixture_experts_transformer_gemv_amd", "csrc", n), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_bf16")
    ap.add_argument("--no-prefill", action="store_true", help="skip the companion T=8192 prefill measurement")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--prefill-steps", type=int, default=10, help="timed prefill steps (0: no prefill, as --no-prefill)")
    ap.add_argument("--block", action="store_true",
                    help="time the MoE block (pre-MoE RMSNorm, MoE, post-MoE RMSNorm, residual) instead of the layer")
    ap.add_argument("--weight-layout", choices=["in_out", "out_in"], default="in_out",
                    help="expert weights stored [E, in, out] (checkpoint) or [E, out, in] (converted); same values")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time torch.matmul (hipBLASLt) bf16 on the prefill's per-expert GEMM shapes, for context")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the workload at this many tokens instead of its own T (e.g. int8_w8 at 8192)")
    ap.add_argument("--d-ff", type=int, default=0,
                    help="run the workload at this d_ff instead of its own (e.g. 4096: one GPU's share of a layer "
                         "split over 8 GPUs along d_ff)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration under rocprofv3)")
    a = ap.parse_args()
    if a.steps < 1 or a.warmup < 0 or a.prefill_steps < 0 or a.tokens < 0 or a.d_ff < 0:
        ap.error("--steps must be >= 1; --warmup, --prefill-steps, --tokens and --d-ff >= 0")
    return a


class Layer:
    """Device-resident inputs and preallocated buffers of one workload, and the timed step."""

    def __init__(self, gm, w, inp, dv, norms=None, weight_layout="in_out", transpose=True):
        import torch
        self.outin = weight_layout == "out_in"
        if self.outin and transpose:  # the same weights stored [E, out, in] (transposed on the device, untimed)
            dv = dict(dv)
            for n in ("w1", "wv", "w2"):
                dv[n] = dv[n].transpose(1, 2).contiguous()
        self.gm, self.w, self.inp, self.dv = gm, w, inp, dv
        self.norms = norms  # (pre_scale, post_scale, eps) device tensors for the block form
        T, d, f, E = w.T, w.d, w.f, w.E
        dev = dv["x"].device
        self.S = gm.down_splits(T, d, f, E, 2, w.dtype)
        i32 = torch.int32
        self.idx = torch.empty((T, 2), dtype=i32, device=dev)
        self.p = torch.empty((T, 2), dtype=torch.float32, device=dev)
        self.counts = torch.empty((E,), dtype=i32, device=dev)
        self.offsets = torch.empty((E + 1,), dtype=i32, device=dev)
        self.perm = torch.empty((2 * T,), dtype=i32, device=dev)
        self.inv = torch.empty((T, 2), dtype=i32, device=dev)
        self.h = torch.empty((2 * T, f), dtype=torch.float32 if w.dtype == gm.F32 else torch.bfloat16, device=dev)
        self.y = torch.empty((self.S, 2 * T, d), dtype=torch.float32, device=dev)
        self.out = torch.empty((T, d), dtype=torch.float32, device=dev)
        self.xn = torch.empty_like(dv["x"]) if norms is not None else None
        self.s1 = self.sv = self.s2 = None
        self.grouped = None  # (scale_experts, groups_up, groups_down) of grouped int8 scales
        if dv["scales"] is not None:
            self.s1, self.sv, self.s2 = dv["scales"]
            es = E if w.scale_experts is None else w.scale_experts
            if (es, w.groups_up, w.groups_down) != (E, 1, 1):
                self.grouped = (es, w.groups_up, w.groups_down)
        mk = lambda: torch.cuda.Event(enable_timing=True)
        self.ev = [mk() for _ in range(6)]
        self.lib = gm.lib()

    def step(self, timed=False):
        import ctypes
        gm, dv, L, w = self.gm, self.dv, self.lib, self.w
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        s = ctypes.c_void_p(__import__("torch").cuda.current_stream().cuda_stream)
        T, d, f, E, dt = w.T, w.d, w.f, w.E, w.dtype
        ev = self.ev
        if timed:
            ev[0].record()
        if self.norms is None:
            xa = dv["x"]
            st = L.grok_moe_route(P(dv["x"]), P(dv["router_w"]), P(dv["router_bias"]), T, d, E, 2, dt, P(self.idx),
                                  P(self.p), s)
        else:
            xa = self.xn
            st = L.grok_moe_route_norm(P(dv["x"]), P(self.norms[0]), self.norms[2], P(dv["router_w"]),
                                       P(dv["router_bias"]), T, d, E, 2, dt, P(self.xn), P(self.idx), P(self.p), s)
        st |= L.grok_moe_bin(P(self.idx), T, E, 2, P(self.counts), P(self.offsets), P(self.perm), P(self.inv), s)
        if timed:
            ev[1].record()
        es, g1, g2 = self.grouped if self.grouped is not None else (E, 1, 1)
        if self.outin:
            st |= L.grok_moe_expert_up_ex(P(xa), P(dv["w1"]), P(dv["wv"]), P(self.s1), P(self.sv), 1, es, g1,
                                          P(self.counts), P(self.offsets), P(self.perm), T, d, f, E, 2, dt, P(self.h),
                                          s)
        elif self.grouped is None:
            st |= L.grok_moe_expert_up(P(xa), P(dv["w1"]), P(dv["wv"]), P(self.s1), P(self.sv), P(self.counts),
                                       P(self.offsets), P(self.perm), T, d, f, E, 2, dt, P(self.h), s)
        else:
            st |= L.grok_moe_expert_up_w8_grouped(P(xa), P(dv["w1"]), P(dv["wv"]), P(self.s1), P(self.sv),
                                                  self.grouped[0], self.grouped[1], P(self.counts), P(self.offsets),
                                                  P(self.perm), T, d, f, E, 2, P(self.h), s)
        if timed:
            ev[2].record()
        if self.outin:
            st |= L.grok_moe_expert_down_ex(P(self.h), P(dv["w2"]), P(self.s2), 1, es, g2, P(self.counts),
                                            P(self.offsets), T, d, f, E, 2, dt, self.S, P(self.y), s)
        elif self.grouped is None:
            st |= L.grok_moe_expert_down(P(self.h), P(dv["w2"]), P(self.s2), P(self.counts), P(self.offsets), T, d,
                                         f, E, 2, dt, self.S, P(self.y), s)
        else:
            st |= L.grok_moe_expert_down_w8_grouped(P(self.h), P(dv["w2"]), P(self.s2), self.grouped[0],
                                                    self.grouped[2], P(self.counts), P(self.offsets), T, d, f, E, 2,
                                                    self.S, P(self.y), s)
        if timed:
            ev[3].record()
        if self.norms is None:
            st |= L.grok_moe_combine(P(self.y), self.S, P(self.p), P(self.inv), T, d, 2, P(self.out), s)
        else:
            st |= L.grok_moe_combine_norm(P(self.y), self.S, P(self.p), P(self.inv), P(dv["x"]), P(self.norms[1]),
                                          self.norms[2], T, d, 2, dt, P(self.out), s)
        if timed:
            ev[4].record()
        if st != 0:
            raise RuntimeError(f"library call failed (status bits {st})")

    def run_with_kernel_times(self, steps, warmup):
        """Time `steps` steps (wall, bracketed by synchronize) and the average per-launch duration of each expert
        kernel (HIP events on the launch stream, read after the timed region)."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        mk = lambda: torch.cuda.Event(enable_timing=True)
        evs = [[mk() for _ in range(5)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.ev = evs[i]
            self.step(timed=True)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        k = np.array([[e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]), e[0].elapsed_time(e[1]),
                       e[3].elapsed_time(e[4])] for e in evs])
        per_step = np.array([e[0].elapsed_time(e[4]) for e in evs])  # first to last event of each step, ms
        self.step_stats = {"median": float(np.median(per_step)), "min": float(per_step.min()),
                           "p90": float(np.percentile(per_step, 90)), "n": int(steps)}
        return wall, k.mean(axis=0)  # ms: up, down, route+bin, combine


def n_hit(layer) -> int:
    return int((layer.counts.cpu().numpy() > 0).sum())


def up_bytes(w, nh, T):
    wb = 1 if w.dtype == 2 else (4 if w.dtype == 0 else 2)
    b = nh * 2 * w.d * w.f * wb + T * w.d * 2 + 2 * T * w.f * 2
    if w.dtype == 2:  # scales: [Es, G, f] for W1 and Wv, read for every hit expert (once if shared)
        b += (nh if w.scale_experts is None else 1) * 2 * w.groups_up * w.f * 2
    return b


def down_bytes(w, nh, T, S):
    wb = 1 if w.dtype == 2 else (4 if w.dtype == 0 else 2)
    b = nh * w.f * w.d * wb + 2 * T * w.f * 2 + S * 2 * T * w.d * 4
    if w.dtype == 2:
        b += (nh if w.scale_experts is None else 1) * w.groups_down * w.d * 2
    return b


def up_flops(w, T):
    return 2.0 * (2 * T) * w.d * w.f * 2


def load_traffic(workload: str, kernel: str):
    """HBM-side bytes per launch of a kernel from its committed counter record (profiles/traffic_*.json:
    FETCH_SIZE and WRITE_SIZE scaled by the same counters on a plain copy of known size), or None if there is no
    record or the kernel's sources changed since the counters were taken."""
    p = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
        if rec.get("source_hash") != source_hash(rec["source_files"]):
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def cpu_baseline(w, inp, oracle, synth, block=False):
    """The oracle as it stands, on a bounded sample of the workload (routing for all tokens, expert path on a few
    rows), timed on this host's cores; and the same for one row on a single thread."""
    import torch

    def run(rows):
        t0 = time.perf_counter()
        if block:
            ns = synth.make_norm_scales(w)
            oracle.block_forward(inp, w.dtype, ns["pre_scale"], ns["post_scale"], ns["eps"], rows=rows)
        else:
            oracle.forward(inp, w.dtype, rows=rows)
        return time.perf_counter() - t0

    # up to 8 seeded rows (every row of the decode batch), passes repeated until about 10 s of CPU work
    rows = synth.sampled_rows(w.T, min(w.T, 8))
    threads = torch.get_num_threads()
    dt, reps = 0.0, 0
    while reps < 20 and (reps == 0 or dt < 10.0):
        dt += run(rows)
        reps += 1
    res = {"value": reps * len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} of {w.T} token rows of {w.name} through the float64 oracle (routing on all "
                     f"{w.T} tokens, both selected experts per row), {reps} passes, {dt:.1f} s"}
    torch.set_num_threads(1)
    try:
        dt1 = run(rows[:1])
    finally:
        torch.set_num_threads(threads)
    res["single_thread"] = {"value": 1 / dt1, "unit": "tokens/s", "cores": 1,
                            "sample": f"1 token row of {w.name} (routing on all {w.T} tokens), {dt1:.1f} s"}
    return res


def library_gemm(steps, warmup):
    """torch.matmul (hipBLASLt) on dense bf16 GEMMs of the shapes one expert sees in the T=8192 prefill
    (2T/E = 2048 rows): one of the two up-projection matrices, and the down-projection with bf16 and fp32 output;
    plus the whole up-projection's rows as one dense GEMM.  Context for the grouped kernels' TFLOP/s, not part of
    the layer."""
    import torch
    d, f, M = 6144, 32768, 2048
    g = torch.Generator(device="cuda").manual_seed(0)
    res = {}
    for name, m, k, n, odt in (("up_one_matrix", M, d, f, torch.bfloat16), ("down_bf16_out", M, f, d, torch.bfloat16),
                               ("down_f32_out", M, f, d, torch.float32), ("up_all_rows_one_matrix", 8 * M, d, f,
                                                                          torch.bfloat16)):
        a = torch.randn(m, k, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(k, n, device="cuda", dtype=torch.bfloat16, generator=g) * 0.02
        if odt == torch.float32:
            fn = lambda: torch.mm(a, b, out_dtype=torch.float32)
        else:
            c = torch.empty(m, n, device="cuda", dtype=odt)
            fn = lambda: torch.mm(a, b, out=c)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / steps
        res[name] = {"M": m, "K": k, "N": n, "ms": ms, "TFLOP/s": 2 * m * k * n / (ms * 1e-3) / 1e12}
        log(f"{name}: {ms:.3f} ms, {res[name]['TFLOP/s']:.0f} TFLOP/s")
        del a, b
    print(json.dumps({"library_gemm": res, "library": "torch.mm (hipBLASLt)", "dtype": "bf16"}))


def main():
    a = parse()
    if a.library_gemm:
        library_gemm(a.steps, a.warmup)
        return
    if a.gpus != 1:
        print(json.dumps({"error": "this layer runs on one GPU; multi-GPU sharding is designed but not implemented "
                                   "(tensor-parallel over d_ff with a reduce-scatter of the fp32 output)",
                          "n_gpus": a.gpus}))
        sys.exit(2)
    import torch

    import mixture_experts_transformer_gemv_amd as gm
    import synth
    from tests._helpers import dev_inputs

    gm.lib()
    torch.cuda.set_device(0)
    w = synth.WORKLOADS[a.workload]
    if a.tokens or a.d_ff:
        import dataclasses
        if a.tokens:
            w = dataclasses.replace(w, T=a.tokens, name=f"{w.name}_T{a.tokens}")
        if a.d_ff:
            w = dataclasses.replace(w, f=a.d_ff, name=f"{w.name}_f{a.d_ff}")
    log(f"workload {w.name}: drawing weights")
    t0 = time.perf_counter()
    wts = synth.make_weights(w)
    inp = synth.make_inputs(w, weights=wts)
    dv = dev_inputs(inp, w.dtype)
    log(f"inputs resident ({time.perf_counter() - t0:.1f} s)")

    if a.copy_probe_mib:
        src = torch.empty(a.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    norms = None
    if a.block:
        ns = synth.make_norm_scales(w)
        if w.dtype == synth.F32:
            conv = lambda v: torch.from_numpy(v).cuda()
        else:
            conv = lambda v: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
        norms = (conv(ns["pre_scale"]), conv(ns["post_scale"]), ns["eps"])
    layer = Layer(gm, w, inp, dv, norms, a.weight_layout)
    wall, kms = layer.run_with_kernel_times(a.steps, a.warmup)
    ms = wall * 1e3 / a.steps
    nh = n_hit(layer)
    T = w.T
    tname = w.name + ("_out_in" if a.weight_layout == "out_in" else "")  # the expert kernels' workload
    wname = tname + ("_block" if a.block else "")
    res = {"metric": METRIC, "value": T / (ms / 1e3), "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": {0: "f32", 1: "bf16", 2: "bf16 x int8-weight"}[w.dtype], "data": "synthetic",
           "config": {"workload": wname, "T": T, "d_model": w.d, "d_ff": w.f,
                      "experts": w.E, "top_k": 2, "experts_hit": nh, "down_splits": layer.S,
                      "rmsnorm_residual": bool(a.block), "weight_layout": a.weight_layout}}
    kernels = {"expert_up_ms": kms[0], "expert_down_ms": kms[1], "route_bin_ms": kms[2], "combine_ms": kms[3]}
    if w.dtype == 0:  # the fp32 layer: vector-ALU kernels (tiny shapes: launch latency in practice)
        fl = up_flops(w, T)
        ach = fl / (kms[0] * 1e-3) / 1e12
        res["roofline"] = {"bound": "alu", "kernel": "f32_tiled_kernel<2>", "achieved": ach,
                           "peak": FP32_VALU_TFLOPS, "unit": "TFLOP/s", "frac": ach / FP32_VALU_TFLOPS,
                           "traffic": None, "algorithmic_flops": fl}
    elif w.T <= (128 if w.dtype == synth.W8 else 96):  # weight-streaming kernels: HBM-bound, the up-projection
        # (W1 and Wv) is the dominant kernel
        ub = up_bytes(w, nh, T)
        ach = ub / (kms[0] * 1e-3) / 1e9
        kname = "oi_stream_kernel<2>" if a.weight_layout == "out_in" else "up_stream_kernel"
        res["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": ach, "peak": HBM_PEAK_GBS,
                           "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                           "traffic": load_traffic(tname, "up"), "algorithmic_bytes": ub}
        db = down_bytes(w, nh, T, layer.S)
        kernels["expert_down_GBps"] = db / (kms[1] * 1e-3) / 1e9
        kernels["layer_GBps"] = (ub + db) / (ms * 1e-3) / 1e9
    else:
        fl = up_flops(w, T)
        ach = fl / (kms[0] * 1e-3) / 1e12
        oi = "true" if a.weight_layout == "out_in" else "false"
        grouped = w.groups_up > 1 or w.groups_down > 1
        if w.dtype == 1 or (not grouped and oi == "false"):  # 256-row tiles, then 128-row last tiles
            kname = f"tiled_dma_kernel<2, {oi}, {'true' if w.dtype == 2 else 'false'}, 256> + tiled_dma_small_kernel"
        elif grouped and oi == "false" and w.groups_up <= 8:  # grouped scales on the 128-row direct-to-LDS tiles
            kname = "tiled_dma_grouped_kernel<2>"
        else:
            kname = f"tiled_reg_kernel<2, {'true' if grouped else 'false'}, {oi}>"
        res["roofline"] = {"bound": "mfma", "kernel": kname, "achieved": ach, "peak": BF16_PEAK_TFLOPS,
                           "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                           "traffic": load_traffic(tname, "up"), "algorithmic_flops": fl}
        kernels["layer_TFLOPs"] = 3 * fl / 2 / (ms * 1e-3) / 1e12
    res["kernels"] = kernels
    res["step_ms"] = layer.step_stats  # per step, first to last event on the stream: median, min, p90
    log(f"{w.name}: {ms:.3f} ms/step, {res['value']:.1f} tokens/s, up {kms[0]:.3f} ms, down {kms[1]:.3f} ms")

    if not a.no_prefill and a.prefill_steps > 0 and w.name == "decode_bf16" and not a.block:
        pw = synth.WORKLOADS["prefill_bf16"]
        pinp = synth.make_inputs(pw, weights=wts)
        pdv = dict(layer.dv)  # the decode layer's weights, already in the chosen layout
        pdv["x"] = dev_inputs({**pinp, "w1": None, "wv": None, "w2": None}, synth.BF16)["x"]
        pl = Layer(gm, pw, pinp, pdv, None, a.weight_layout, transpose=False)
        pname = pw.name + ("_out_in" if a.weight_layout == "out_in" else "")
        pwall, pk = pl.run_with_kernel_times(a.prefill_steps, 2)
        pms = pwall * 1e3 / a.prefill_steps
        fl = up_flops(pw, pw.T)
        res["prefill"] = {"workload": pname, "T": pw.T, "value": pw.T / (pms / 1e3), "unit": "tokens/s",
                          "ms_per_step": pms, "steps": a.prefill_steps,
                          "layer_TFLOPs": 3 * fl / 2 / (pms * 1e-3) / 1e12,
                          "roofline": {"bound": "mfma",
                                       "kernel": f"tiled_dma_kernel<2, {str(a.weight_layout == 'out_in').lower()}, false, 256> + tiled_dma_small_kernel",
                                       "achieved": fl / (pk[0] * 1e-3) / 1e12, "peak": BF16_PEAK_TFLOPS,
                                       "unit": "TFLOP/s", "frac": fl / (pk[0] * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
                                       "traffic": load_traffic(pname, "up"), "algorithmic_flops": fl},
                          "kernels": {"expert_up_ms": pk[0], "expert_down_ms": pk[1], "route_bin_ms": pk[2],
                                      "combine_ms": pk[3],
                                      "expert_down_TFLOPs": fl / 2 / (pk[1] * 1e-3) / 1e12},
                          "step_ms": pl.step_stats}
        log(f"prefill: {pms:.3f} ms/step, {res['prefill']['value']:.0f} tokens/s")
        del pl, pdv
        torch.cuda.empty_cache()

    if not a.no_cpu_baseline:
        import oracle
        log("timing the CPU oracle on a bounded sample")
        res["cpu_baseline"] = cpu_baseline(w, inp, oracle, synth, a.block)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
