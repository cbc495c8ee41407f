"""The seeded generator: determinism, structure and distribution of the synthetic inputs."""
import numpy as np

import synth


def test_same_name_same_bits():
    a = synth.tensor("t/a", 33, 48, 1.0, synth.BF16)
    b = synth.tensor("t/a", 33, 48, 1.0, synth.BF16)
    c = synth.tensor("t/b", 33, 48, 1.0, synth.BF16)
    assert a.dtype == np.uint16
    np.testing.assert_array_equal(a, b)
    assert np.mean(a == c) < 0.05


def test_counter_based_rows_independent_of_shape():
    a = synth.tensor("t/c", 10, 64, 1.0, synth.F32)
    b = synth.tensor("t/c", 20, 64, 1.0, synth.F32)
    np.testing.assert_array_equal(a, b[:10])


def test_normal_moments():
    x = synth.tensor("t/m", 512, 512, 2.0, synth.F32).astype(np.float64)
    assert abs(x.mean()) < 0.02
    assert abs(x.std() - 2.0) < 0.02
    assert abs(np.mean(np.abs(x) < 2.0) - 0.6827) < 0.005


def test_bf16_is_rounded_fp32():
    f = synth.tensor("t/r", 64, 64, 1.0, synth.F32)
    h = synth.widen(synth.tensor("t/r", 64, 64, 1.0, synth.BF16))
    # nearest bf16: error at most half a bf16 ulp (2^-8 relative)
    assert np.all(np.abs(h - f) <= np.abs(f) * 2.0 ** -8 + 1e-30)
    assert np.all((h.view(np.uint32) & 0xFFFF) == 0)


def test_outlier_channels_and_row_scale():
    c = synth.cases("opt67b")[0]
    ch = c.x_channels()
    assert len(ch) == 41 and len(set(ch.tolist())) == 41
    np.testing.assert_array_equal(ch, c.x_channels())
    x = synth.widen(c.x_batch(0, T=256))
    m = np.abs(x).max(0)
    assert np.min(m[ch]) > 60 * 1.0 and np.median(np.delete(m, ch)) < 5
    # same channels in every calibration batch
    x1 = synth.widen(c.x_batch(1, T=256))
    assert np.min(np.abs(x1).max(0)[ch]) > 60
    w = synth.widen(synth.weight("t/w", 400, 256, synth.BF16, 0.02, 0.1, 1.0))
    rs = w.std(1) / 0.02
    assert rs.min() > 0.08 and rs.max() < 1.15


def test_tiny_fixed_outliers():
    c = synth.cases("tiny")[0]
    assert c.x_channels().tolist() == [3, 41]
    x = c.x_batch(0)
    assert x.dtype == np.float32 and x.shape == (16, 64)
    np.testing.assert_array_equal(x, c.x_batch(c.eval_index()))


def test_heavy_tail_fraction():
    c = synth.cases("ssz_scale")[0]
    assert (c.N, c.K) == (12288, 4096) and len(synth.cases("ssz_scale")) == 128
    u = synth.uniform_stream(synth.seed_of("x/tail"), 1_000_000)
    assert abs(np.mean(u < 0.001) - 0.001) < 0.0002
