"""Seeded synthetic inputs: reproducible, subset-consistent, right shapes and
distributions (CPU)."""
import numpy as np

import synth


def test_workload_shapes_and_flops():
    g3 = synth.gemms(3)
    assert len(g3) == 8
    assert sum(g.flops for g in g3) == 1_159_641_169_920
    assert all(g.M == 552_960 for g in g3)
    assert [(g.N, g.K) for g in g3] == [(768, 256), (256, 768), (256, 256), (256, 256),
                                        (512, 256), (256, 512), (256, 512), (512, 256)]
    assert [(g.trans_a, g.trans_b) for g in g3] == [(False, False), (False, True)] * 4
    assert sum(g.flops for g in synth.gemms(4)) == 309_237_645_312
    assert synth.gemms(0)[0].flops == 2 * 256**3


def test_reproducible_and_row_subsets():
    g = synth.gemms(2)[1]
    full = synth.make_a(g)
    assert full.shape == (6144, 768) and full.dtype == np.float32
    assert np.array_equal(full, synth.make_a(g))
    idx = synth.sample_rows(g.M, 64, 5)
    assert np.array_equal(synth.make_a(g, rows=idx), full[idx])
    assert np.array_equal(synth.make_a(g, rows=(4000, 4100)), full[4000:4100])
    assert abs(float(full.mean())) < 0.01 and abs(float(full.std()) - 1) < 0.01
    w = synth.make_b(g)
    assert w.shape == (256, 768)
    assert abs(float(w.std()) * 16 - 1) < 0.02


def test_config0_and_stress():
    a, b = synth.make_a(synth.gemms(0)[0]), synth.make_b(synth.gemms(0)[0])
    assert a.shape == b.shape == (256, 256) and np.abs(a).max() < 1
    s = synth.make_a(synth.gemms(1)[0])
    n = s.size
    assert abs((s == 0).sum() / n - 0.01) < 0.001
    big = np.abs(s) > 2.0**40
    assert abs(big.sum() / n - 0.001 * 0.99) < 0.0002
    mags = np.abs(s[(s != 0) & ~big])
    assert mags.min() >= 2.0**-30 * 0.999 and mags.max() <= 2.0**31
    assert np.all(np.isfinite(s))
