#!/usr/bin/env python3
"""Throughput of the Grok-1 MoE FFN layer forward on one MI355X, on every workload of the layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--configs LIST | --configs none]
                    [--workload decode_bf16|prefill_bf16|int8_w8|int8_w8_g8|skew_bf16|tiny_f32]
                    [--weight-layout in_out|out_in] [--block] [--tokens T] [--d-ff F]
                    [--no-parity] [--no-cpu-baseline] [--no-ceilings]
    python bench.py --library-gemm      (torch.mm / hipBLASLt on the prefill's per-expert shapes, for context)

A step is one pass of the whole layer (router, binning, fused up-projection with GELU product, down-projection,
combine) over one batch of seeded synthetic tokens, with weights and inputs already resident in HBM.  The timed
step calls the library's five step entry points in order (bit-identical to grok_moe_forward) on the current
stream, so that HIP events on that stream time the dominant kernel (the up-projection) inside the timed region;
the other kernels are timed by as many untimed steps with events between every launch (each event costs a few
microseconds of GPU time, which the timed steps do not carry).  The whole-layer entry point grok_moe_forward is
timed as well ("entry_point_ms_per_step").

The headline workload (--workload, default the Grok-1-shape decode step T=8, d=6144, f=32768, E=8, top-2, bf16)
is timed for exactly --steps steps after --warmup untimed ones; its numbers are the top-level fields.  The other
workloads of the layer (--configs, default all: prefill T=8192, skewed routing T=4096, int8 weights T=64, tiny
fp32) follow under "configs", each with its own step count.  For every workload the same run reports:
  * tokens/s, per-step median/min/p90, the per-kernel times and the roofline of the dominant kernel (HBM GB/s or
    MFMA TFLOP/s against the published peaks and the measured ceilings), the shader clock during extra untimed
    steps (a sampler kernel beside them), and the per-expert token counts;
  * parity of that run's output against the CPU oracle (tests-only code, run here only as the check and the CPU
    baseline): routing indices and counts bit for bit, max|gpu - oracle| / rms(oracle) on every row (256 seeded
    rows for prefill and skewed routing), and the same against the oracle without the bf16 rounding of h;
  * the oracle's own time on those rows (routing of all T tokens timed separately), on this host's cores.
"ceilings" holds the practical limits measured by the probe library: a streaming HBM read and dense bf16 MFMA on
random register operands (result checked), with the clock it ran at, and the same MFMA loop with the A operands zero
and in two other issue orders (what the MFMA rate depends on).  One JSON line on stdout.
"""
from __future__ import annotations

import argparse
import ctypes
import dataclasses
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
CONFIG_STEPS = {"decode_bf16": 50, "prefill_bf16": 10, "skew_bf16": 10, "int8_w8": 50, "int8_w8_g8": 50,
                "tiny_f32": 100}
ALL_CONFIGS = ("decode_bf16", "prefill_bf16", "skew_bf16", "int8_w8", "tiny_f32")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="decode_bf16", help="the headline workload (top-level fields)")
    ap.add_argument("--configs", default="all",
                    help="comma-separated workloads reported under 'configs' besides the headline one, 'all' "
                         f"({', '.join(ALL_CONFIGS)}) or 'none'")
    ap.add_argument("--config-steps", type=int, default=0, help="timed steps of every config (0: their defaults)")
    ap.add_argument("--no-parity", action="store_true", help="skip the oracle check (and the CPU baseline)")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the single-thread oracle timing")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the HBM-read and MFMA ceiling probes")
    ap.add_argument("--block", action="store_true",
                    help="time the MoE block (pre-MoE RMSNorm, MoE, post-MoE RMSNorm, residual) instead of the layer")
    ap.add_argument("--weight-layout", choices=["in_out", "out_in"], default="in_out",
                    help="expert weights stored [E, in, out] (checkpoint) or [E, out, in] (converted); same values")
    ap.add_argument("--library-gemm", action="store_true",
                    help="only time torch.matmul (hipBLASLt) bf16 on the prefill's per-expert GEMM shapes, for context")
    ap.add_argument("--tokens", type=int, default=0,
                    help="run the headline workload at this many tokens instead of its own T (e.g. int8_w8 at 8192)")
    ap.add_argument("--d-ff", type=int, default=0,
                    help="run the headline workload at this d_ff instead of its own (e.g. 4096: one GPU's share of a "
                         "layer split over 8 GPUs along d_ff)")
    ap.add_argument("--trace", action="store_true",
                    help="also run the headline workload's 256-row tile launches once with per-tile timestamps (bf16 "
                         "[in, out] weights, LDS-tiled batches) and report where their cycles go")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration under rocprofv3)")
    a = ap.parse_args()
    if a.steps < 1 or a.warmup < 0 or a.tokens < 0 or a.d_ff < 0 or a.config_steps < 0:
        ap.error("--steps must be >= 1; --warmup, --tokens, --d-ff and --config-steps >= 0")
    return a


# ------------------------------------------------------------------------------------------------ the timed step

class FenceFreeEvent:
    """A HIP event created with hipEventDisableSystemFence in the HIP runtime torch has loaded, recorded on torch's
    current stream: unlike torch.cuda.Event, recording it adds no system-scope release (a write-back of the caches)
    between the launches around it.  Same interface as the two torch.cuda.Event methods used here."""
    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    @classmethod
    def _lib(cls):
        if cls._hip is None:
            L = ctypes.CDLL("libamdhip64.so.7", mode=os.RTLD_NOLOAD)  # the runtime already in the process
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._hip = L
        return cls._hip

    def __init__(self):
        self.h = ctypes.c_void_p()
        if self._lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.FLAGS) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self):
        import torch
        if self._lib().hipEventRecord(self.h, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_time(self, end) -> float:
        ms = ctypes.c_float()
        if self._lib().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        if self.h and self._hip is not None:
            self._hip.hipEventDestroy(self.h)


class Layer:
    """Device-resident inputs and preallocated buffers of one workload, and the timed step."""

    def __init__(self, gm, w, inp, dv, norms=None, weight_layout="in_out"):
        import torch
        self.outin = weight_layout == "out_in"  # dv holds the weights in this storage already
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
        self.scale_spec = (E, 1, 1)  # (scale_experts, groups_up, groups_down)
        if dv["scales"] is not None:
            self.s1, self.sv, self.s2 = dv["scales"]
            es = E if w.scale_experts is None else w.scale_experts
            self.scale_spec = (es, w.groups_up, w.groups_down)
        self.lib = gm.lib()
        mk = lambda: torch.cuda.Event(enable_timing=True)
        self.ev = [mk() for _ in range(5)]

    def step(self, marks=()):
        """One step; records the events whose indices are in marks (0 before the router, 1 after binning, 2 after the
        up-projection, 3 after the down-projection, 4 after the combine)."""
        import torch
        dv, L, w = self.dv, self.lib, self.w
        P = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        T, d, f, E, dt = w.T, w.d, w.f, w.E, w.dtype
        lay = 1 if self.outin else 0
        es, g1, g2 = self.scale_spec
        ev = self.ev
        if 0 in marks:
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
        if 1 in marks:
            ev[1].record()
        st |= L.grok_moe_expert_up(P(xa), P(dv["w1"]), P(dv["wv"]), P(self.s1), P(self.sv), lay, es, g1,
                                   P(self.counts), P(self.offsets), P(self.perm), T, d, f, E, 2, dt, P(self.h), s)
        if 2 in marks:
            ev[2].record()
        st |= L.grok_moe_expert_down(P(self.h), P(dv["w2"]), P(self.s2), lay, es, g2, P(self.counts),
                                     P(self.offsets), T, d, f, E, 2, dt, self.S, P(self.y), s)
        if 3 in marks:
            ev[3].record()
        if self.norms is None:
            st |= L.grok_moe_combine(P(self.y), self.S, P(self.p), P(self.inv), T, d, 2, P(self.out), s)
        else:
            st |= L.grok_moe_combine_norm(P(self.y), self.S, P(self.p), P(self.inv), P(dv["x"]), P(self.norms[1]),
                                          self.norms[2], T, d, 2, dt, P(self.out), s)
        if 4 in marks:
            ev[4].record()
        if st != 0:
            raise RuntimeError(f"library call failed (status bits {st})")

    def forward_entry(self):
        """The whole layer through the binding's entry point (grok_moe_forward, or its general form)."""
        gm, dv = self.gm, self.dv
        lay = gm.OUT_IN if self.outin else gm.IN_OUT
        if self.norms is None:
            return gm.forward(dv["x"], dv["router_w"], dv["w1"], dv["wv"], dv["w2"], scales=dv["scales"],
                              router_bias=dv["router_bias"], return_routing=True, weight_layout=lay)
        return gm.block_forward(dv["x"], self.norms[0], self.norms[1], self.norms[2], dv["router_w"], dv["w1"],
                                dv["wv"], dv["w2"], scales=dv["scales"], router_bias=dv["router_bias"],
                                return_routing=True, weight_layout=lay)

    def run_with_kernel_times(self, steps, warmup):
        """Time `steps` steps (wall, bracketed by synchronize) with HIP events on the launch stream around the
        up-projection only (the dominant kernel: its average per-launch duration comes from the timed steps); then,
        untimed, as many steps with events between every launch give the other kernels' times and the per-step
        spread.  A torch event between launches costs a few microseconds of GPU time (its system-scope release
        writes the caches back), so every event here is a FenceFreeEvent, and the timed steps carry only the two
        that the dominant kernel needs."""
        import torch
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        evs = [[None, FenceFreeEvent(), FenceFreeEvent(), None, None] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            self.ev = evs[i]
            self.step(marks=(1, 2))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        up = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
        evs = [[FenceFreeEvent() for _ in range(5)] for _ in range(steps)]
        for i in range(steps):
            self.ev = evs[i]
            self.step(marks=(0, 1, 2, 3, 4))
        torch.cuda.synchronize()
        k = np.array([[e[2].elapsed_time(e[3]), e[0].elapsed_time(e[1]), e[3].elapsed_time(e[4])] for e in evs])
        per_step = np.array([e[0].elapsed_time(e[4]) for e in evs])  # first to last event of each step, ms
        self.step_stats = {"median": float(np.median(per_step)), "min": float(per_step.min()),
                           "p90": float(np.percentile(per_step, 90)), "n": int(steps),
                           "with_events_between_every_launch": True}
        down, rb, comb = k.mean(axis=0)
        return wall, np.array([up, down, rb, comb])  # ms: up, down, route+bin, combine

    def time_entry_point(self, steps):
        """ms per call of the whole-layer entry point (allocations of its outputs included)."""
        import torch
        self.forward_entry()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            self.forward_entry()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / steps


# ------------------------------------------------------------------------------------------------ rooflines

def n_hit(counts) -> int:
    return int((np.asarray(counts) > 0).sum())


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
        from mixture_experts_transformer_gemv_amd.rocprof_summary import source_hash
        if rec.get("source_hash") != source_hash(rec["source_files"]):
            return None
        return rec.get("bytes_per_launch")
    except Exception:
        return None


def stream_path(w) -> bool:
    return w.dtype != 0 and w.T <= (128 if w.dtype == 2 else 96)


def stream_up_kernel(w) -> str:
    """The library's choice of streaming up-projection kernel for [in, out] weights (the rule of
    up_stream_narrow in csrc/expert_stream.hip: bf16, 16-row token tiles, the whole d axis per wave, and
    min(2T, E) * f / 256 >= 1024)."""
    ksplit4 = w.d % 512 == 0 and ((w.f + 511) // 512) * w.E < 256
    if (w.dtype == 1 and w.T <= 16 and w.f % 256 == 0 and not ksplit4
            and min(2 * w.T, w.E) * (w.f // 256) >= 1024):
        return "up_stream_narrow_kernel"
    return "up_stream_kernel"


def roofline(w, layer, kms, ms, weight_layout, ceilings):
    """Roofline of the dominant kernel (the up-projection) and the per-kernel rates."""
    T, nh = w.T, n_hit(layer.counts.cpu().numpy())
    oi = weight_layout == "out_in"
    tname = w.name + ("_out_in" if oi else "")
    kernels = {"expert_up_ms": kms[0], "expert_down_ms": kms[1], "route_bin_ms": kms[2], "combine_ms": kms[3]}
    if w.dtype == 0:  # the fp32 layer: vector-ALU kernels (tiny shapes: launch latency in practice)
        fl = up_flops(w, T)
        ach = fl / (kms[0] * 1e-3) / 1e12
        rl = {"bound": "alu", "kernel": "f32_tiled_kernel<2>", "achieved": ach, "peak": FP32_VALU_TFLOPS,
              "unit": "TFLOP/s", "frac": ach / FP32_VALU_TFLOPS, "traffic": None, "algorithmic_flops": fl}
    elif stream_path(w):  # weight-streaming kernels: HBM-bound
        ub = up_bytes(w, nh, T)
        ach = ub / (kms[0] * 1e-3) / 1e9
        rl = {"bound": "hbm", "kernel": "oi_stream_kernel<2>" if oi else stream_up_kernel(w), "achieved": ach,
              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
              "traffic": load_traffic(tname, "up"), "algorithmic_bytes": ub}
        if ceilings and ceilings.get("hbm_read_GBps"):
            rl["frac_of_measured_read_ceiling"] = ach / ceilings["hbm_read_GBps"]
        db = down_bytes(w, nh, T, layer.S)
        kernels["expert_up_GBps"] = ach
        kernels["expert_down_GBps"] = db / (kms[1] * 1e-3) / 1e9
        kernels["layer_GBps"] = (ub + db) / (ms * 1e-3) / 1e9
    else:  # LDS-tiled grouped GEMMs: MFMA-bound
        fl = up_flops(w, T)
        ach = fl / (kms[0] * 1e-3) / 1e12
        grouped = w.groups_up > 1 or w.groups_down > 1
        if w.dtype == 1 and not oi:
            kname = "tiled_up_persist_kernel + tiled_dma_small_kernel"
        elif w.dtype == 1 or (not grouped and not oi):
            kname = (f"tiled_dma_kernel<2, {str(oi).lower()}, {'true' if w.dtype == 2 else 'false'}, 256> + "
                     "tiled_dma_small_kernel")
        elif grouped and not oi and w.groups_up <= 8:
            kname = "tiled_dma_grouped_kernel<2>"
        else:
            kname = f"tiled_reg_kernel<2, {'true' if grouped else 'false'}, {str(oi).lower()}>"
        rl = {"bound": "mfma", "kernel": kname, "achieved": ach, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
              "frac": ach / BF16_PEAK_TFLOPS, "traffic": load_traffic(tname, "up"), "algorithmic_flops": fl}
        if ceilings and ceilings.get("mfma_sustained_TFLOPs"):
            rl["frac_of_measured_mfma_ceiling"] = ach / ceilings["mfma_sustained_TFLOPs"]
        kernels["expert_up_TFLOPs"] = ach
        kernels["expert_down_TFLOPs"] = fl / 2 / (kms[1] * 1e-3) / 1e12
        kernels["layer_TFLOPs"] = 3 * fl / 2 / (ms * 1e-3) / 1e12
    return rl, kernels


# ------------------------------------------------------------------------------------------------ probes

class Probe:
    """The measurement probes of libgrokmoe_probe.so (include/grok_moe_probe.h)."""

    def __init__(self, gm):
        path = os.path.join(os.path.dirname(gm.LIB_PATH), "libgrokmoe_probe.so")
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build with `python -m mixture_experts_transformer_gemv_amd.build`")
        L = ctypes.CDLL(path)
        vp, i, u64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_size_t
        i64 = ctypes.c_int64
        for name, args in (("grok_moe_probe_read", [vp, sz, i, i, vp, vp]),
                           ("grok_moe_probe_mfma", [vp, i, i, vp, vp, vp]),
                           ("grok_moe_probe_mfma_feed", [vp, i64, i, i, vp, vp, vp]),
                           ("grok_moe_probe_clock", [i, u64, vp, vp]),
                           ("grok_moe_probe_tile_trace", [i, vp, vp, vp, vp, vp, vp, i64, i, i, i, i, i, vp, vp, i64,
                                                          vp]),
                           ("grok_moe_probe_wall_clock_khz", [])):
            fn = getattr(L, name)
            fn.restype = ctypes.c_int
            fn.argtypes = args
        self.L = L
        self.wall_khz = L.grok_moe_probe_wall_clock_khz() or 100000

    def ghz(self, clocks: np.ndarray) -> float:
        c = clocks.reshape(-1, 4).astype(np.float64)
        dc, dw = (c[:, 1] - c[:, 0]).sum(), (c[:, 3] - c[:, 2]).sum()
        return float(dc / dw * self.wall_khz * 1e3 / 1e9) if dw > 0 else float("nan")

    def clock_during(self, run, expected_ms: float) -> float | None:
        """Shader clock (GHz) read by 8 single-wave sampler workgroups (one per XCD) on a second stream while
        run() enqueues work on the current one, over 60% of the work's expected duration."""
        import torch
        out = torch.zeros(8 * 4, dtype=torch.int64, device="cuda")
        side = torch.cuda.Stream()
        ticks = int(0.6 * expected_ms * 1e-3 * self.wall_khz * 1e3)
        if ticks < 1000:
            return None
        torch.cuda.synchronize()
        run()
        with torch.cuda.stream(side):
            st = self.L.grok_moe_probe_clock(8, ticks, ctypes.c_void_p(out.data_ptr()),
                                             ctypes.c_void_p(side.cuda_stream))
        torch.cuda.synchronize()
        if st != 0:
            return None
        return self.ghz(out.cpu().numpy().view(np.uint64))

    def hbm_read(self, buf, reps=4):
        """Streaming read of a resident tensor: the best rate over grids of 1024, 2048 and 4096 workgroups, for
        default and nontemporal loads (median of `reps` timed reads each)."""
        import torch
        nbytes = buf.numel() * buf.element_size()
        nbytes -= nbytes % 16
        sink = torch.zeros(4096 * 4, dtype=torch.int32, device="cuda")
        res = {}
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        for nt in (0, 1):
            best = 0.0
            for wgs in (1024, 2048, 4096):
                times = []
                for _ in range(reps + 1):
                    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    e0.record()
                    st = self.L.grok_moe_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, wgs, nt,
                                                    ctypes.c_void_p(sink.data_ptr()), s)
                    e1.record()
                    torch.cuda.synchronize()
                    if st != 0:
                        raise RuntimeError(f"read probe failed ({st})")
                    times.append(e0.elapsed_time(e1))
                best = max(best, nbytes / (float(np.median(times[1:])) * 1e-3) / 1e9)
            res["nontemporal" if nt else "default"] = best
        return res, nbytes

    # operand pair (A fragment, B fragment) of MFMA m of a round, for each issue order of grok_moe_probe_mfma
    ORDERS = {0: [(m >> 2, m & 3) for m in range(16)],
              1: [(m & 3, ((m >> 2) + m) & 3) for m in range(16)],
              2: [(0, 0)] * 16}

    def mfma(self, iters=200000, order=0, zero_a=False):
        """Sustained dense bf16 MFMA (TFLOP/s) on N(0,1) operands (zero_a: the A fragments all zero, so every
        product is zero), issued in `order`; its clock, and a check of the result."""
        import torch
        g = torch.Generator(device="cuda").manual_seed(0)
        ops = torch.randn(8 * 64 * 8, device="cuda", generator=g).to(torch.bfloat16)
        if zero_a:
            ops[:4 * 64 * 8] = 0
        chk = torch.zeros(1024 * 64, dtype=torch.float32, device="cuda")
        clocks = torch.zeros(1024 * 4, dtype=torch.int64, device="cuda")
        s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        args = (ctypes.c_void_p(ops.data_ptr()), ctypes.c_void_p(chk.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                s)
        self.L.grok_moe_probe_mfma(args[0], 1000, order, *args[1:])  # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st = self.L.grok_moe_probe_mfma(args[0], iters, order, *args[1:])
        e1.record()
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"mfma probe failed ({st})")
        ms = e0.elapsed_time(e1)
        flops = 1024.0 * iters * 16 * 32768
        # expected checksum per lane, in float64 from the operands (fragment layouts in grok_moe_probe.h)
        o = ops.float().cpu().numpy().astype(np.float64).reshape(8, 64, 8)
        A = np.zeros((4, 32, 16))
        B = np.zeros((4, 16, 32))
        for f in range(4):
            for lane in range(64):
                A[f, lane & 31, 8 * (lane >> 5):8 * (lane >> 5) + 8] = o[f, lane]
                B[f, 8 * (lane >> 5):8 * (lane >> 5) + 8, lane & 31] = o[4 + f, lane]
        want = np.zeros(64)
        scale = np.zeros(64)
        rows = np.array([[(v & 3) + 8 * (v >> 2) + 4 * (lane >> 5) for v in range(16)] for lane in range(64)])
        for i, j in self.ORDERS[order]:
            C = A[i] @ B[j]
            for lane in range(64):
                vals = C[rows[lane], lane & 31]
                want[lane] += vals.sum()
                scale[lane] += np.abs(vals).sum()
        got = chk.cpu().numpy().reshape(1024, 64).astype(np.float64)
        if zero_a:
            err = float(np.max(np.abs(got)))  # every product is exactly zero
        else:
            err = float(np.max(np.abs(got - iters * want[None, :]) / (iters * scale[None, :])))
        return {"TFLOPs": flops / (ms * 1e-3) / 1e12, "ms": ms, "iters": iters,
                "clock_GHz": self.ghz(clocks.cpu().numpy().view(np.uint64)),
                "checksum_max_err": err, "checksum_ok": bool(err == 0.0 if zero_a else err < 1e-2)}


    def feed(self, copies, iters=50000, images=64):
        """The tile kernels' MFMA stream with its operand fragments read from an LDS ring (copies=0), and with the ring
        fed by direct-to-LDS copies of the same bytes per flop from a source of `images` 32 KB stages that stays in
        L2 (copies=1): TFLOP/s, clock, and a check of the sums.  Operands as in the prefill: A N(0,1), B N(0,0.02)."""
        import torch
        g = torch.Generator(device="cuda").manual_seed(1)
        src = torch.randn(images, 2, 8192, device="cuda", generator=g)
        src[:, 1] *= 0.02
        src = src.to(torch.bfloat16).contiguous()
        chk = torch.zeros(1024 * 64, dtype=torch.float32, device="cuda")
        clocks = torch.zeros(1024 * 4, dtype=torch.int64, device="cuda")
        st_ = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
        call = lambda n: self.L.grok_moe_probe_mfma_feed(ctypes.c_void_p(src.data_ptr()), images * 32768, n, copies,
                                                         ctypes.c_void_p(chk.data_ptr()),
                                                         ctypes.c_void_p(clocks.data_ptr()), st_)
        call(500)  # warm-up
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        st = call(iters)
        e1.record()
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"feed probe failed ({st})")
        ms = e0.elapsed_time(e1)
        want, scale = feed_expected(src.float().cpu().numpy().astype(np.float64), iters, copies)
        got = chk.cpu().numpy().astype(np.float64).reshape(256, 2, 2, 64)
        err = float(np.max(np.abs(got - want[None]) / scale[None]))
        return {"TFLOPs": 1024.0 * iters * 32 * 32768 / (ms * 1e-3) / 1e12, "ms": ms, "iters": iters,
                "clock_GHz": self.ghz(clocks.cpu().numpy().view(np.uint64)), "checksum_max_rel_err": err,
                "checksum_ok": bool(err < 1e-3)}


def feed_expected(src, iters, copies):
    """Per (wm, wn, lane) of grok_moe_probe_mfma_feed: the sum of its accumulators (float64) and the sum of the
    absolute values of the products in them, from the source images (src: [images, 16384] values; stage layout in
    include/grok_moe_probe.h)."""
    images = src.shape[0]
    v = src.reshape(images, 32, 64, 8)  # [image, fragment, lane, 8 values]
    A = np.zeros((images, 2, 2, 4, 32, 16))  # image, wm, ks, i, row, k
    B = np.zeros((images, 2, 2, 4, 16, 32))  # image, wn, ks, j, k, column
    for q in range(2):
        for ks in range(2):
            for i in range(4):
                for h in range(2):
                    A[:, q, ks, i][:, :, 8 * h:8 * h + 8] = v[:, (q * 2 + ks) * 4 + i, 32 * h:32 * h + 32]
                    B[:, q, ks, i][:, 8 * h:8 * h + 8, :] = v[:, 16 + (q * 2 + ks) * 4 + i,
                                                            32 * h:32 * h + 32].transpose(0, 2, 1)
    n_img = images if copies else 4
    C = np.einsum("gmsirk,gnsjkc->gmnsijrc", A[:n_img], B[:n_img])  # every block product of every step half
    uses = np.bincount(np.arange(iters) % n_img, minlength=n_img).astype(np.float64)
    want = np.zeros((2, 2, 64))
    scale = np.zeros((2, 2, 64))
    for h in range(2):
        rows = np.array([(u & 3) + 8 * (u >> 2) + 4 * h for u in range(16)])  # accumulator rows of lanes 32 h ..
        Ch = C[..., rows, :]  # g, wm, wn, ks, i, j, 16 rows, 32 columns
        want[:, :, 32 * h:32 * h + 32] = np.tensordot(uses, Ch.sum(axis=(3, 4, 5, 6)), axes=1)
        scale[:, :, 32 * h:32 * h + 32] = np.tensordot(uses, np.abs(Ch).sum(axis=(3, 4, 5, 6)), axes=1)
    return want, scale


def tile_trace(probe, layer):
    """Where the cycles of the prefill kernels go: the 256-row tiles of each projection (the persistent up-projection,
    the down-projection's 256-row launch) run once more with per-tile timestamps (same kernels, trace points on), on
    the routing of the last timed step.  Per tile: prologue (up to the K loop: tile lookup, activation offsets, first
    copies; for the persistent kernel only a workgroup's first tile has one), K loop, epilogue; the K loop's MFMA density
    (K / 32 steps x 32 MFMAs x 32 cycles); per CU: the gaps between its consecutive tiles and its idle tail before
    the launch ends."""
    import torch
    w, dv = layer.w, layer.dv
    T, d, f, E = w.T, w.d, w.f, w.E
    slots = 2 * T
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    res = {}
    for nmat in (2, 1):
        if nmat == 2:
            a, b0, b1, perm, K, N, out, splits = dv["x"], dv["w1"], dv["wv"], layer.perm, d, f, layer.h, 1
        else:
            a, b0, b1, perm, K, N, out, splits = layer.h, dv["w2"], None, None, f, d, layer.y, layer.S
        NT = N // (256 // nmat)
        gx = ((slots // 256 + E) * NT + 7) // 8 * 8
        nrec = gx * splits
        tr = torch.zeros(nrec * 8, dtype=torch.int64, device="cuda")
        torch.cuda.synchronize()
        st = probe.L.grok_moe_probe_tile_trace(nmat, P(a), P(b0), None if b1 is None else P(b1), P(layer.counts),
                                               P(layer.offsets), None if perm is None else P(perm),
                                               a.numel() * a.element_size(), K, N, E, slots, splits, P(out), P(tr),
                                               nrec, s)
        torch.cuda.synchronize()
        if st != 0:
            raise RuntimeError(f"tile trace failed ({st})")
        r = tr.cpu().numpy().view(np.uint64).reshape(nrec, 8)
        r = r[(r[:, 7] != np.uint64(0xFFFFFFFFFFFFFFFF)) & (((r[:, 7] >> np.uint64(32)) & np.uint64(0xFFF)) != 0)]
        r = r.astype(np.int64)
        cyc = {"prologue": r[:, 2] - r[:, 1], "k_loop": r[:, 3] - r[:, 2], "epilogue": r[:, 4] - r[:, 3],
               "tile": r[:, 4] - r[:, 1]}
        wall = r[:, 6] - r[:, 5]
        ghz = float(cyc["tile"].sum() / wall.sum() * probe.wall_khz * 1e3 / 1e9)
        ticks_per_us = probe.wall_khz / 1e3
        kt = K // splits // 32
        mfma = kt * 32 * 32  # cycles of one wave's MFMAs per tile
        hw, xcc = r[:, 0] & 0xFFFFFFFF, r[:, 0] >> 32
        cu = (xcc & 0xF) * 1024 + ((hw >> 13) & 7) * 64 + ((hw >> 12) & 1) * 16 + ((hw >> 8) & 0xF)
        t0, t1 = r[:, 5].min(), r[:, 6].max()
        span = t1 - t0
        gaps, tails, heads, busy = [], [], [], 0
        for c in np.unique(cu):
            m = cu == c
            st_, en = r[m, 5], r[m, 6]
            o = np.argsort(st_)
            st_, en = st_[o], en[o]
            gaps.extend((st_[1:] - en[:-1]).tolist())
            heads.append(st_[0] - t0)
            tails.append(t1 - en[-1])
            busy += (en - st_).sum()
        ncu = len(np.unique(cu))
        gaps = np.array(gaps, dtype=np.float64)
        res["up" if nmat == 2 else "down"] = {
            "tiles": int(len(r)), "cus": ncu, "span_ms": span / ticks_per_us / 1e3, "clock_GHz": ghz,
            "k_steps": kt, "mfma_cycles_per_tile": mfma,
            "cycles_per_tile_mean": {k: float(v.mean()) for k, v in cyc.items()},
            "cycles_per_tile_p10_p90": {k: [float(np.percentile(v, 10)), float(np.percentile(v, 90))]
                                        for k, v in cyc.items()},
            "k_loop_mfma_density": float(mfma / cyc["k_loop"].mean()),
            "tile_mfma_density": float(mfma / cyc["tile"].mean()),
            "share_of_tile": {k: float(cyc[k].mean() / cyc["tile"].mean()) for k in ("prologue", "k_loop",
                                                                                      "epilogue")},
            "gap_between_tiles_us": {"mean": float(gaps.mean() / ticks_per_us) if len(gaps) else None,
                                     "p90": float(np.percentile(gaps, 90) / ticks_per_us) if len(gaps) else None},
            "cu_busy_frac_of_span": float(busy / (ncu * span)),
            "cu_head_idle_frac": float(np.mean(heads) / span), "cu_tail_idle_frac": float(np.mean(tails) / span),
            "launch_mfma_density": float(len(r) * mfma / (ncu * span * ghz * 1e3 / ticks_per_us)),
        }
        del tr
    return res


def ceilings(probe, buf):
    """Practical ceilings of this GPU: streaming HBM read of a resident weight tensor and sustained MFMA."""
    res = {}
    rd, nbytes = probe.hbm_read(buf)
    res["hbm_read_GBps_default"] = rd["default"]
    res["hbm_read_GBps_nontemporal"] = rd["nontemporal"]
    res["hbm_read_GBps"] = max(rd.values())
    res["hbm_read_bytes"] = nbytes
    m = probe.mfma()
    res.update({"mfma_sustained_TFLOPs": m["TFLOPs"], "mfma_ms": m["ms"], "mfma_iters": m["iters"],
                "mfma_clock_GHz": m["clock_GHz"], "mfma_checksum_max_rel_err": m["checksum_max_err"],
                "mfma_checksum_ok": m["checksum_ok"],
                "mfma_kernel": "1024 waves (one per SIMD), 16 v_mfma_f32_32x32x16_bf16 per round on register operands"})
    res["mfma_frac_of_spec"] = res["mfma_sustained_TFLOPs"] / BF16_PEAK_TFLOPS
    # what the MFMA rate depends on: the operand values (A all zero: nothing toggles in the multipliers) and the
    # issue order (A held for 4 MFMAs as in the tile kernels, both operands changing, or one pair throughout)
    var = {}
    for name, kw in (("zero_a", {"zero_a": True}), ("order_both_change", {"order": 1}),
                     ("order_one_pair", {"order": 2})):
        v = probe.mfma(iters=100000, **kw)
        var[name] = {"TFLOPs": v["TFLOPs"], "clock_GHz": v["clock_GHz"], "checksum_ok": v["checksum_ok"]}
    res["mfma_variants"] = var
    # the tile kernels' K loop alone: fragments from LDS, then also the copies that feed the ring (L2-resident source)
    res["mfma_feed"] = {name: probe.feed(copies=c) for name, c in (("lds_fragments", 0),
                                                                   ("lds_fragments_and_copies", 1))}
    res["hbm_frac_of_spec"] = res["hbm_read_GBps"] / HBM_PEAK_GBS
    return res


# ------------------------------------------------------------------------------------------------ oracle side

def cpu_info():
    """CPU model, logical CPUs this process may run on, their physical cores, and torch's thread count."""
    import torch
    try:
        aff = sorted(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        aff = list(range(os.cpu_count() or 1))
    model, cores, cur = None, set(), {}
    try:
        for line in open("/proc/cpuinfo"):
            if ":" not in line:
                if cur.get("processor") is not None and int(cur["processor"]) in aff:
                    cores.add((cur.get("physical id", "0"), cur.get("core id", cur["processor"])))
                cur = {}
                continue
            k, v = (s.strip() for s in line.split(":", 1))
            cur[k] = v
            if k == "model name" and model is None:
                model = v
        if cur.get("processor") is not None and int(cur["processor"]) in aff:
            cores.add((cur.get("physical id", "0"), cur.get("core id", cur["processor"])))
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": len(aff), "physical_cores": len(cores) or None,
            "threads": torch.get_num_threads()}


def oracle_check(w, inp, layer, oracle, synth, timing=True):
    """Parity of the run's output (layer.out / idx / p / counts after the timed steps) against the oracle, and the
    oracle's time on the same rows."""
    import torch
    from synth.harness import TOL, rel_err, rms_rel_err
    rows = None if w.sampled_rows is None else synth.sampled_rows(w.T, w.sampled_rows)
    n_rows = w.T if rows is None else len(rows)
    kind = "f32" if w.dtype == synth.F32 else "bf16"
    res = {}
    if timing:
        bias = inp.get("router_bias")
        t0 = time.perf_counter()
        oracle.route(oracle.as_f64(inp["x"], kind), oracle.as_f64(inp["router_w"], kind),
                     None if bias is None else torch.from_numpy(np.asarray(bias, np.float64)))
        res["routing_s"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    ref = oracle.forward(inp, w.dtype, rows=rows)
    t_fwd = time.perf_counter() - t0
    rows_t = ref["rows"].numpy()
    out = layer.out.cpu().numpy()[rows_t]
    idx, p, cnt = layer.idx.cpu().numpy(), layer.p.cpu().numpy(), layer.counts.cpu().numpy()
    par = {"rows_checked": n_rows, "routing_tokens": w.T,
           "idx_exact": bool(np.array_equal(idx, ref["idx"].numpy())),
           "counts_exact": bool(np.array_equal(cnt, ref["counts"].numpy())),
           "p_max_rel_err": float(np.max(np.abs(p - ref["p"].numpy()) / ref["p"].numpy())),
           "max_err_over_rms": rel_err(out, ref["out"].numpy()),
           "rms_err_over_rms": rms_rel_err(out, ref["out"].numpy()),
           "tol": TOL[w.dtype], "min_logit_gap_cut": float(ref["min_gap_cut"])}
    if w.dtype != synth.F32:  # against the plain definition, without the bf16 rounding of h
        plain = oracle.forward(inp, w.dtype, rows=rows, round_h=False)["out"].numpy()
        par["vs_unrounded"] = {"max_err_over_rms": rel_err(out, plain), "rms_err_over_rms": rms_rel_err(out, plain)}
    par["pass"] = bool(par["idx_exact"] and par["counts_exact"] and par["p_max_rel_err"] < 1e-6
                       and par["max_err_over_rms"] <= par["tol"])
    res["parity"] = par
    if timing:
        info = cpu_info()
        res["cpu_baseline"] = {
            "value": n_rows / t_fwd, "unit": "tokens/s", "cores": info["threads"], "kind": "oracle",
            "sample": (f"{n_rows} of {w.T} token rows of {w.name} through the float64 oracle (routing on all {w.T} "
                       f"tokens, both selected experts per row), one pass, {t_fwd:.1f} s"),
            "wall_s": t_fwd, "routing_s": res.pop("routing_s"), **info}
        rt = res["cpu_baseline"]["routing_s"]
        if t_fwd > rt:
            res["cpu_baseline"]["expert_rows_tokens_per_s"] = n_rows / (t_fwd - rt)
    return res


def single_thread_baseline(w, inp, oracle):
    import torch
    threads = torch.get_num_threads()
    torch.set_num_threads(1)
    try:
        t0 = time.perf_counter()
        oracle.forward(inp, w.dtype, rows=np.array([0]))
        dt1 = time.perf_counter() - t0
    finally:
        torch.set_num_threads(threads)
    return {"value": 1 / dt1, "unit": "tokens/s", "cores": 1,
            "sample": f"1 token row of {w.name} (routing on all {w.T} tokens), {dt1:.1f} s"}


# ------------------------------------------------------------------------------------------------ one workload

def to_layout(dv, weight_layout):
    """The device weights in the chosen storage: [E, in, out] as drawn, or their transposes [E, out, in] (the same
    values; transposed once on the device, untimed)."""
    if weight_layout != "out_in":
        return dv
    dv = dict(dv)
    for n in ("w1", "wv", "w2"):
        dv[n] = dv[n].transpose(1, 2).contiguous()
    return dv


def measure(gm, w, inp, dv, steps, warmup, a, probe, ceil, oracle, synth, norms=None):
    import torch
    layer = Layer(gm, w, inp, dv, norms, a.weight_layout)
    wall, kms = layer.run_with_kernel_times(steps, warmup)
    ms = wall * 1e3 / steps
    counts = layer.counts.cpu().numpy()
    rl, kernels = roofline(w, layer, kms, ms, a.weight_layout, ceil)
    res = {"workload": w.name + ("_out_in" if a.weight_layout == "out_in" else "") + ("_block" if norms else ""),
           "T": w.T, "d_model": w.d, "d_ff": w.f, "experts": w.E, "top_k": 2,
           "dtype": {0: "f32", 1: "bf16", 2: "bf16 x int8-weight"}[w.dtype],
           "value": w.T / (ms / 1e3), "unit": "tokens/s", "ms_per_step": ms, "steps": steps, "warmup": warmup,
           "step_ms": layer.step_stats, "roofline": rl, "kernels": kernels,
           "routing": {"counts": counts.tolist(), "experts_hit": n_hit(counts)}, "down_splits": layer.S}
    # the whole-layer entry point, and a check that it reproduces the timed steps bit for bit
    out_e, idx_e, p_e, cnt_e = layer.forward_entry()
    torch.cuda.synchronize()
    res["entry_point_equal_to_steps"] = bool(torch.equal(out_e, layer.out) and torch.equal(idx_e, layer.idx)
                                             and torch.equal(cnt_e, layer.counts))
    del out_e, idx_e, p_e, cnt_e
    res["entry_point_ms_per_step"] = layer.time_entry_point(max(3, min(steps, 20)))
    if probe is not None:
        nclk = max(3, int(np.ceil(40.0 / max(ms, 1e-3))))  # extra untimed steps, about 40 ms of work
        res["clock_GHz"] = probe.clock_during(lambda: [layer.step() for _ in range(nclk)], nclk * ms)
    log(f"{res['workload']}: {ms:.3f} ms/step, {res['value']:.1f} tokens/s, up {kms[0]:.3f} ms, down "
        f"{kms[1]:.3f} ms, {rl['unit']} {rl['achieved']:.0f} ({100 * rl['frac']:.1f}% of peak), clock "
        f"{res.get('clock_GHz')}")
    if oracle is not None:
        if norms is None:
            res.update(oracle_check(w, inp, layer, oracle, synth))
            par = res["parity"]
            log(f"{res['workload']}: parity {'ok' if par['pass'] else 'FAILED'}: idx {par['idx_exact']}, counts "
                f"{par['counts_exact']}, max err / rms {par['max_err_over_rms']:.2e} over {par['rows_checked']} rows"
                + (f", unrounded {par['vs_unrounded']['max_err_over_rms']:.2e}" if "vs_unrounded" in par else ""))
        else:
            res["parity"] = None  # the block form's parity is a GPU test; not repeated here
    return res, layer


# ------------------------------------------------------------------------------------------------ context

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


# ------------------------------------------------------------------------------------------------ main

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
    from synth.harness import dev_inputs

    gm.lib()
    torch.cuda.set_device(0)
    oracle = None
    if not a.no_parity:
        import oracle  # noqa: F811  (the CPU check and baseline only; never on the timed path)
    probe = Probe(gm)

    w = synth.WORKLOADS[a.workload]
    if a.tokens:
        w = dataclasses.replace(w, T=a.tokens, name=f"{w.name}_T{a.tokens}",
                                sampled_rows=w.sampled_rows or (256 if a.tokens > 256 else None))
    if a.d_ff:
        w = dataclasses.replace(w, f=a.d_ff, name=f"{w.name}_f{a.d_ff}")
    log(f"workload {w.name}: drawing weights")
    t0 = time.perf_counter()
    wts = {w.dtype: synth.make_weights(w)}
    inp = synth.make_inputs(w, weights=wts[w.dtype])  # (host copies stay for the oracle)
    dv = to_layout(dev_inputs(inp, w.dtype), a.weight_layout)
    log(f"inputs resident ({time.perf_counter() - t0:.1f} s)")

    if a.copy_probe_mib:
        src = torch.empty(a.copy_probe_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ceil = None
    if not a.no_ceilings and w.dtype != synth.F32 and dv["w1"].numel() * dv["w1"].element_size() >= (1 << 30):
        log("ceilings: HBM read and MFMA probes")
        ceil = ceilings(probe, dv["w1"])
        log(f"ceilings: read {ceil['hbm_read_GBps']:.0f} GB/s, MFMA {ceil['mfma_sustained_TFLOPs']:.0f} TFLOP/s at "
            f"{ceil['mfma_clock_GHz']:.2f} GHz (checksum {'ok' if ceil['mfma_checksum_ok'] else 'WRONG'})")

    norms = None
    if a.block:
        ns = synth.make_norm_scales(w)
        if w.dtype == synth.F32:
            conv = lambda v: torch.from_numpy(v).cuda()
        else:
            conv = lambda v: torch.from_numpy(v.view(np.int16)).view(torch.bfloat16).cuda()
        norms = (conv(ns["pre_scale"]), conv(ns["post_scale"]), ns["eps"])
    head, hlayer = measure(gm, w, inp, dv, a.steps, a.warmup, a, probe, ceil, oracle, synth, norms)
    res = {"metric": METRIC, "value": head["value"], "unit": "tokens/s", "n_gpus": 1, "steps": a.steps,
           "warmup": a.warmup, "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": {0: "f32", 1: "bf16", 2: "bf16 x int8-weight"}[w.dtype],
           "data": "synthetic",
           "config": {"workload": head["workload"], "T": w.T, "d_model": w.d, "d_ff": w.f, "experts": w.E,
                      "top_k": 2, "experts_hit": head["routing"]["experts_hit"], "down_splits": head["down_splits"],
                      "rmsnorm_residual": bool(a.block), "weight_layout": a.weight_layout},
           "roofline": head["roofline"]}
    if "cpu_baseline" in head:
        res["cpu_baseline"] = head.pop("cpu_baseline")
        if not a.no_cpu_baseline:
            res["cpu_baseline"]["single_thread"] = single_thread_baseline(w, inp, oracle)
    for k in ("kernels", "step_ms", "routing", "parity", "clock_GHz", "entry_point_ms_per_step",
              "entry_point_equal_to_steps"):
        if k in head:
            res[k] = head[k]
    if ceil is not None:
        res["ceilings"] = ceil
    if a.trace and w.dtype == synth.BF16 and a.weight_layout == "in_out" and not stream_path(w) and not a.block:
        res["tile_trace"] = tile_trace(probe, hlayer)
        for k, v in res["tile_trace"].items():
            log(f"trace {k}: {v['tiles']} tiles, clock {v['clock_GHz']:.2f} GHz, cycles/tile "
                f"{v['cycles_per_tile_mean']['tile']:.0f} (prologue {v['cycles_per_tile_mean']['prologue']:.0f}, "
                f"loop {v['cycles_per_tile_mean']['k_loop']:.0f}, epilogue {v['cycles_per_tile_mean']['epilogue']:.0f});"
                f" loop MFMA density {v['k_loop_mfma_density']:.3f}, tile {v['tile_mfma_density']:.3f}, launch "
                f"{v['launch_mfma_density']:.3f}; gap {v['gap_between_tiles_us']['mean']:.2f} us; busy "
                f"{v['cu_busy_frac_of_span']:.3f}")
    del hlayer
    torch.cuda.empty_cache()

    names = [] if a.configs == "none" else (list(ALL_CONFIGS) if a.configs == "all" else a.configs.split(","))
    names = [n for n in names if n != w.name]
    if a.tokens or a.d_ff or a.block:
        names = []  # variants of the headline workload stand alone
    res["configs"] = {}
    for name in names:
        cw = synth.WORKLOADS[name]
        log(f"config {name}")
        share = cw.dtype == w.dtype and (cw.d, cw.f, cw.E, cw.groups_up, cw.groups_down, cw.scale_experts) == \
            (w.d, w.f, w.E, w.groups_up, w.groups_down, w.scale_experts)
        if share:  # the same weights (decode, prefill and skewed routing), already resident
            cinp = synth.make_inputs(cw, weights=wts[w.dtype])
            cdv = dict(dv)
            part = dev_inputs({**cinp, "w1": None, "wv": None, "w2": None, "s1": None, "sv": None, "s2": None},
                              cw.dtype)
            cdv["x"], cdv["router_w"], cdv["router_bias"] = part["x"], part["router_w"], part["router_bias"]
        else:
            cinp = synth.make_inputs(cw)
            cdv = to_layout(dev_inputs(cinp, cw.dtype), a.weight_layout)
        steps = a.config_steps or CONFIG_STEPS.get(name, 10)
        cres, clayer = measure(gm, cw, cinp, cdv, steps, 2, a, probe, ceil, oracle, synth)
        res["configs"][name] = cres
        del clayer, cdv
        torch.cuda.empty_cache()
    if not res["configs"]:
        del res["configs"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
