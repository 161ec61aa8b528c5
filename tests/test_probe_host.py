"""The host-side expectation of the K-loop feed probe (bench.feed_expected) against a step-by-step evaluation of
what include/grok_moe_probe.h says the probe computes: per step the ring image, per half step the 16 MFMA block
products of the wave's A and B fragments, each lane summing the accumulator elements it holds.  CPU only."""
import numpy as np
import pytest


def emulate(src, iters, copies):
    images = src.shape[0]
    out = np.zeros((2, 2, 64))
    for it in range(iters):
        stage = src[it % (images if copies else 4)].reshape(32, 64, 8)  # 32 fragments of 64 lanes x 8 values
        for wm in range(2):
            for wn in range(2):
                acc = np.zeros((4, 4, 32, 32))
                for ks in range(2):
                    for i in range(4):
                        a = np.zeros((32, 16))
                        for lane in range(64):
                            a[lane & 31, 8 * (lane >> 5):8 * (lane >> 5) + 8] = stage[(wm * 2 + ks) * 4 + i, lane]
                        for j in range(4):
                            b = np.zeros((16, 32))
                            for lane in range(64):
                                b[8 * (lane >> 5):8 * (lane >> 5) + 8, lane & 31] = stage[16 + (wn * 2 + ks) * 4 + j, lane]
                            acc[i, j] += a @ b
                for lane in range(64):
                    rows = [(v & 3) + 8 * (v >> 2) + 4 * (lane >> 5) for v in range(16)]
                    out[wm, wn, lane] += acc[:, :, rows, lane & 31].sum()
    return out


@pytest.mark.parametrize("images,iters,copies", [(4, 3, 1), (5, 7, 1), (6, 5, 0)])
def test_feed_expected_matches_step_by_step(images, iters, copies):
    import bench
    src = np.random.default_rng(images * 10 + iters).standard_normal((images, 16384))
    want, scale = bench.feed_expected(src, iters, copies)
    got = emulate(src, iters, copies)
    assert np.max(np.abs(got - want)) <= 1e-9 * np.max(scale)
    assert np.all(scale > 0)
