"""The C ABI library without a GPU: it loads, exports every entry point its header declares, and rejects bad
arguments on the host before touching the device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "grok_moe.h")


@pytest.fixture(scope="module")
def L():
    import mixture_experts_transformer_gemv_amd as gm
    if not os.path.exists(gm.LIB_PATH):
        from mixture_experts_transformer_gemv_amd import build
        build.build()
    return gm.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(grok_moe_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("grok_moe_forward", "grok_moe_workspace_size", "grok_moe_strerror", "grok_moe_route", "grok_moe_bin",
              "grok_moe_expert_up", "grok_moe_expert_down", "grok_moe_combine", "grok_moe_down_splits"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for n in declared_functions():
        assert hasattr(L, n), n


def test_strerror(L):
    import mixture_experts_transformer_gemv_amd as gm
    assert gm.strerror(0) == "ok"
    for s in (-1, -2, -3, -4, 7):
        assert gm.strerror(s)


def test_workspace_size_and_splits(L):
    import mixture_experts_transformer_gemv_amd as gm
    assert gm.workspace_size(0, 6144, 32768) == 0
    assert gm.workspace_size(8, 6144, 32768, 8, 3) == 0  # k != 2
    assert gm.workspace_size(8, 6100, 32768) == 0        # d not a multiple of 256
    ws_dec = gm.workspace_size(8, 6144, 32768)
    assert ws_dec >= 16 * 32768 * 2 + 16 * 6144 * 4 * gm.down_splits(8, 6144, 32768)
    # streaming batches: 5 chunks, or 2 for bf16 16-row token tiles with at least as many tokens as experts
    assert gm.down_splits(8, 6144, 32768) == 2 and gm.down_splits(16, 6144, 32768) == 2
    assert gm.down_splits(4, 6144, 32768) == 5 and gm.down_splits(17, 6144, 32768) == 5
    assert gm.down_splits(8, 6144, 32768, 16) == 5 and gm.down_splits(16, 6144, 32768, 16) == 2
    assert gm.down_splits(8, 6144, 32768, 8, 2, gm.W8) == 5
    assert gm.down_splits(8192, 6144, 32768) == 2   # LDS-tiled bf16 path splits K in two
    assert gm.down_splits(8192, 6144, 32768, 8, 2, gm.W8) == 1
    # the streaming kernels take bf16 batches up to 96 tokens and int8 batches up to 128
    assert gm.down_splits(96, 6144, 32768) == 5 and gm.down_splits(97, 6144, 32768) == 2
    assert gm.down_splits(128, 6144, 32768, 8, 2, gm.W8) == 5 and gm.down_splits(129, 6144, 32768, 8, 2, gm.W8) == 1
    # streaming chunks: at least 2048 rows each, at most 5, boundaries on multiples of 128 rows
    assert [gm.down_splits(4, 6144, f) for f in (1024, 4096, 6144, 6400, 8192, 16384, 6208)] == [1, 2, 3, 3, 4, 5, 1]
    assert [gm.down_splits(8, 6144, f) for f in (1024, 4096, 6144, 6400, 8192, 16384, 6208)] == [1, 2, 2, 2, 2, 2, 1]
    assert gm.down_splits(64, 128, 512, 8, 2, gm.F32) == 4   # small fp32 batch: K split in parts of 128
    assert gm.down_splits(300, 128, 512, 8, 2, gm.F32) == 1
    ws_pre = gm.workspace_size(8192, 6144, 32768)
    assert ws_pre >= 16384 * 32768 * 2 + 16384 * 6144 * 4
    assert gm.workspace_size(64, 128, 512, 8, 2, gm.F32) >= 128 * 512 * 4 + 128 * 128 * 4


def test_long_batches_run_in_passes(L):
    """bf16 at d = 6144, f = 32768 runs at most 16383 tokens per pass (32-bit offsets into x and h); a longer
    batch is split into near-equal passes, and the workspace is that of the larger pass."""
    import mixture_experts_transformer_gemv_amd as gm
    d, f = 6144, 32768
    assert gm.workspace_size(16383, d, f) > gm.workspace_size(16382, d, f)      # one pass
    assert gm.workspace_size(16384, d, f) == gm.workspace_size(8192, d, f)      # two passes of 8192
    assert gm.workspace_size(16385, d, f) == gm.workspace_size(8193, d, f)      # 8193 + 8192
    assert gm.workspace_size(50000, d, f) == gm.workspace_size(12500, d, f)     # four passes
    assert gm.block_workspace_size(20000, d, f) == gm.block_workspace_size(10000, d, f)
    assert gm.down_splits(20000, d, f) == 2
    # int8 layers run their tiled kernels on the same 32-bit offsets into x and h: the same passes as bf16
    assert gm.workspace_size(16383, d, f, 8, 2, gm.W8) > gm.workspace_size(16382, d, f, 8, 2, gm.W8)
    assert gm.workspace_size(16384, d, f, 8, 2, gm.W8) == gm.workspace_size(8192, d, f, 8, 2, gm.W8)
    assert gm.workspace_size(20000, d, f, 8, 2, gm.W8) == gm.workspace_size(10000, d, f, 8, 2, gm.W8)
    assert gm.down_splits(20000, d, f, 8, 2, gm.W8) == 1
    # the fp32 layer addresses with 64-bit offsets: one pass
    assert gm.workspace_size(20000, 1024, 1024, 8, 2, gm.F32) > gm.workspace_size(10000, 1024, 1024, 8, 2, gm.F32)
    # the limit comes from h [2 T, f] (and from x [T, d] when d is large)
    assert gm.workspace_size(2047, 256, 1 << 18) > gm.workspace_size(2046, 256, 1 << 18)  # P = 2047: one pass
    assert gm.workspace_size(2048, 256, 1 << 18) == gm.workspace_size(1024, 256, 1 << 18)
    assert gm.workspace_size(2100, 256, 1 << 18) == gm.workspace_size(1050, 256, 1 << 18)
    assert gm.workspace_size(1100, 1 << 20, 256) == gm.workspace_size(550, 1 << 20, 256)  # P = 1023
    # one expert matrix must stay below 2^32 bytes
    assert gm.workspace_size(8, 1 << 20, 1 << 11) == 0
    # the expert steps take one pass at most (rejected on the host, before any pointer is read)
    fake = ctypes.c_void_p(0x100000)
    for dt in (1, 2):  # bf16, int8
        sc = None if dt == 1 else fake
        assert L.grok_moe_expert_up(fake, fake, fake, sc, sc, 0, 8, 1, fake, fake, fake, 16384, d, f, 8, 2, dt, fake,
                                    None) == -2
        assert L.grok_moe_expert_up(fake, fake, fake, sc, sc, 0, 8, 1, fake, fake, None, 16383, d, f, 8, 2, dt, fake,
                                    None) == -1
        assert L.grok_moe_expert_down(fake, fake, sc, 0, 8, 1, fake, fake, 16384, d, f, 8, 2, dt, 1 if dt == 2 else 2,
                                      fake, None) == -2


def _fwd(L, **kw):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first
    a = dict(x=fake, router_w=fake, w1=fake, wv=fake, w2=fake, s1=None, sv=None, s2=None, T=8, d=256, f=512, E=8,
             k=2, dtype=1, out=fake, bias=None, idx=None, p=None, cnt=None, ws=ctypes.c_void_p(0x200000),
             ws_bytes=0, stream=None)
    a.update(kw)
    return L.grok_moe_forward(a["x"], a["router_w"], a["w1"], a["wv"], a["w2"], a["s1"], a["sv"], a["s2"], a["T"],
                              a["d"], a["f"], a["E"], a["k"], a["dtype"], a["out"], a["bias"], a["idx"], a["p"],
                              a["cnt"], a["ws"], a["ws_bytes"], a["stream"])


def test_forward_rejects_bad_arguments_on_host(L):
    assert _fwd(L, dtype=5) == -1
    assert _fwd(L, T=-1) == -1
    assert _fwd(L, k=3) == -2
    assert _fwd(L, E=1) == -2
    assert _fwd(L, E=65) == -2
    assert _fwd(L, d=300) == -2
    assert _fwd(L, f=320) == -2                    # bf16 needs multiples of 256
    assert _fwd(L, x=None) == -1
    assert _fwd(L, out=ctypes.c_void_p(0x100004)) == -1   # misaligned
    assert _fwd(L, s1=ctypes.c_void_p(0x100000)) == -1    # scales given for a bf16 layer
    assert _fwd(L, dtype=2) == -1                           # int8 layer without scales
    assert _fwd(L, ws=None) == -1
    assert _fwd(L, ws=ctypes.c_void_p(0x200010)) == -1      # workspace not 256-byte aligned
    assert _fwd(L, ws_bytes=1024) == -3                     # too small
    assert _fwd(L, T=0) == 0                                # nothing to do
    assert _fwd(L, T=0, x=None) == 0


def test_step_entry_points_reject_bad_arguments_on_host(L):
    fake = ctypes.c_void_p(0x100000)
    assert L.grok_moe_route(None, fake, None, 8, 256, 8, 2, 1, fake, fake, None) == -1
    assert L.grok_moe_route(fake, fake, None, 8, 256, 8, 3, 1, fake, fake, None) == -2
    assert L.grok_moe_bin(fake, -1, 8, 2, fake, fake, fake, fake, None) == -1
    assert L.grok_moe_bin(fake, 8, 99, 2, fake, fake, fake, fake, None) == -2
    assert L.grok_moe_expert_up(fake, fake, fake, None, None, 0, 8, 1, fake, fake, None, 8, 256, 512, 8, 2, 1, fake,
                                None) == -1
    assert L.grok_moe_expert_up(fake, fake, fake, None, None, 2, 8, 1, fake, fake, fake, 8, 256, 512, 8, 2, 1, fake,
                                None) == -1  # unknown weight layout
    S = L.grok_moe_down_splits(8, 256, 512, 8, 2, 1)
    assert L.grok_moe_expert_down(fake, fake, None, 0, 8, 1, fake, fake, 8, 256, 512, 8, 2, 1, S + 1, fake,
                                  None) == -1
    assert L.grok_moe_block_forward(fake, None, fake, 1e-5, fake, fake, fake, fake, None, None, None, 0, 8, 1, 1, 8,
                                    256, 512, 8, 2, 1, fake, None, None, None, None, ctypes.c_void_p(0x200000),
                                    1 << 30, None) == -1  # no pre-norm scale
    assert L.grok_moe_combine(fake, 0, fake, fake, 8, 256, 2, fake, None) == -1


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    import mixture_experts_transformer_gemv_amd as gm
    monkeypatch.setattr(gm, "_lib", None)
    monkeypatch.setattr(gm, "LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(gm.GrokMoeError):
        gm.lib()


def _fwd_g(L, se=8, g1=2, g2=4, layout=0, dtype=2, **kw):
    fake = ctypes.c_void_p(0x100000)  # never dereferenced: every call below fails validation first
    a = dict(T=8, d=512, f=1024, E=8, k=2, ws_bytes=0)
    a.update(kw)
    sc = fake if dtype == 2 else None
    return L.grok_moe_forward_ex(fake, fake, fake, fake, fake, sc, sc, sc, layout, se, g1, g2, a["T"], a["d"],
                                 a["f"], a["E"], a["k"], dtype, fake, None, None, None, None,
                                 ctypes.c_void_p(0x200000), a["ws_bytes"], None)


def test_grouped_scale_layouts_rejected_on_host(L):
    assert _fwd_g(L) == -3                    # valid layout: only the (zero-byte) workspace is short
    assert _fwd_g(L, se=1) == -3              # shared scales
    assert _fwd_g(L, se=3) == -1              # scale_experts neither 1 nor E
    assert _fwd_g(L, g1=0) == -1
    assert _fwd_g(L, g2=-2) == -1
    assert _fwd_g(L, g1=3) == -2              # does not divide d
    assert _fwd_g(L, g1=16) == -2             # d / 16 = 32 rows: not a multiple of 64
    assert _fwd_g(L, g2=32) == -2             # f / 32 = 32 rows
    assert _fwd_g(L, g1=8, g2=16) == -3       # 64-row groups are accepted
    assert _fwd_g(L, k=3) == -2
    assert _fwd_g(L, T=0) == 0
    assert _fwd_g(L, layout=1) == -3          # [out, in] weights
    assert _fwd_g(L, layout=2) == -1          # unknown layout
    assert _fwd_g(L, se=3, g1=3, dtype=1) == -3   # scale layout ignored for bf16
    fake = ctypes.c_void_p(0x100000)
    assert L.grok_moe_expert_up(fake, fake, fake, fake, fake, 0, 8, 3, fake, fake, fake, 8, 512, 1024, 8, 2, 2,
                                fake, None) == -2
    assert L.grok_moe_expert_up(fake, fake, fake, None, fake, 0, 8, 2, fake, fake, fake, 8, 512, 1024, 8, 2, 2,
                                fake, None) == -1
    S = L.grok_moe_down_splits(8, 512, 1024, 8, 2, 2)
    assert L.grok_moe_expert_down(fake, fake, fake, 0, 2, 4, fake, fake, 8, 512, 1024, 8, 2, 2, S, fake,
                                  None) == -1
    assert L.grok_moe_expert_down(fake, fake, fake, 0, 8, 4, fake, fake, 8, 512, 1024, 8, 2, 2, S + 1, fake,
                                  None) == -1


def test_export_count(L):
    """The boundary stays small: the declared entry points and nothing else."""
    import subprocess
    import mixture_experts_transformer_gemv_amd as gm
    r = subprocess.run(["nm", "-D", "--defined-only", gm.LIB_PATH], capture_output=True, text=True)
    if r.returncode != 0:
        pytest.skip("nm not available")
    exported = sorted({ln.split()[-1] for ln in r.stdout.splitlines() if " T grok_moe" in ln})
    assert exported == declared_functions()
    assert len(exported) <= 16


def test_probe_library_exports_its_header():
    """The measurement probes (include/grok_moe_probe.h) load and export every declared function; argument errors
    are caught on the host."""
    import mixture_experts_transformer_gemv_amd as gm
    from mixture_experts_transformer_gemv_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    P = ctypes.CDLL(build.PROBE_LIB)
    text = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "grok_moe_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(grok_moe_probe_[a-z_0-9]+)\s*\(", text)))
    assert len(names) == 6
    for n in names:
        assert hasattr(P, n), n
    f = P.grok_moe_probe_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert f(ctypes.c_void_p(0x100008), 64, 4, 0, ctypes.c_void_p(0x200000), None) == -1  # misaligned
    assert f(ctypes.c_void_p(0x100000), 65, 4, 0, ctypes.c_void_p(0x200000), None) == -1  # not a multiple of 16
    g = P.grok_moe_probe_clock
    g.argtypes = [ctypes.c_int, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
    assert g(0, 100, ctypes.c_void_p(0x200000), None) == -1
    m = P.grok_moe_probe_mfma
    m.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    ok = (ctypes.c_void_p(0x100000), 10)
    assert m(*ok, 3, ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), None) == -1  # no such issue order
    assert m(*ok, -1, ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), None) == -1
    assert m(ctypes.c_void_p(0x100000), 0, 0, ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), None) == -1
    fd = P.grok_moe_probe_mfma_feed
    fd.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                   ctypes.c_void_p]
    out = (ctypes.c_void_p(0x200000), ctypes.c_void_p(0x300000), None)
    assert fd(ctypes.c_void_p(0x100000), 3 * 32768, 10, 1, *out) == -1  # fewer than 4 stage images
    assert fd(ctypes.c_void_p(0x100000), 4 * 32768 + 16, 10, 1, *out) == -1  # not whole images
    assert fd(ctypes.c_void_p(0x100000), 4 * 32768, 10, 2, *out) == -1  # copies is 0 or 1
    assert fd(ctypes.c_void_p(0x100008), 4 * 32768, 10, 0, *out) == -1  # misaligned
    assert fd(ctypes.c_void_p(0x100000), 4 * 32768, (1 << 30) + 1, 0, *out) == -1  # step index would overflow
    assert gm.LIB_PATH != build.PROBE_LIB


def test_noalloc_rejects_on_host(L):
    """grok_moe_forward_noalloc: shape errors and batches beyond the static scratch array are rejected before
    anything else (no device is touched)."""
    import mixture_experts_transformer_gemv_amd as gm
    fake = ctypes.c_void_p(0x100000)
    args = lambda T, d, f, k=2, dt=1: (fake, fake, fake, fake, fake, None, None, None, T, d, f, 8, k, dt, fake, None,
                                       None, None, None, None)
    assert L.grok_moe_forward_noalloc(*args(8, 256, 512, k=3)) == -2
    assert L.grok_moe_forward_noalloc(*args(300, 256, 65536)) == -5
    assert L.grok_moe_forward_noalloc(*args(0, 256, 512)) == 0
    assert gm.workspace_size(292, 6144, 32768) <= gm.SCRATCH_BYTES < gm.workspace_size(293, 6144, 32768)
    assert "scratch" in gm.strerror(-5)
