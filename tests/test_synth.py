"""The seeded input generator: determinism, slices, moments, tails, outliers."""
import numpy as np
import pytest
from scipy import stats

import oracle
import synth
from synth import configs


def test_same_seed_same_bytes_and_thread_count_independent():
    cfg = configs.SINGLE
    a = synth.generate(cfg, 0, count=1 << 20, threads=1)
    b = synth.generate(cfg, 0, count=1 << 20, threads=4)
    assert np.array_equal(a, b)


def test_slices_regenerate_alone():
    cfg = configs.S14B
    full = synth.generate(cfg, 4, count=4096 * 40)
    part = synth.generate(cfg, 4, first=4096 * 13, count=4096 * 5 + 17)
    assert np.array_equal(part, full[4096 * 13: 4096 * 18 + 17])
    with pytest.raises(ValueError):
        synth.generate(cfg, 4, first=100, count=10)


def test_layers_differ():
    cfg = configs.TOY
    assert not np.array_equal(synth.generate(cfg, 0), synth.generate(cfg, 1))


def test_normal_moments():
    cfg = configs.S14B
    x = oracle.from16(synth.generate(cfg, 0, count=1 << 22), 0).astype(np.float64)
    pos = synth.outlier_positions(cfg, 0)
    mask = np.ones(x.size, bool)
    mask[pos[pos < x.size]] = False
    y = x[mask]
    se = 0.02 / np.sqrt(y.size)
    assert abs(y.mean()) < 5 * se
    assert abs(y.std() - 0.02) < 0.02 * 5 / np.sqrt(2 * y.size) + 0.02 * 2**-8
    # Kolmogorov-Smirnov against N(0, 0.02) on a subsample
    ks = stats.kstest(y[::16] / 0.02, "norm")
    assert ks.statistic < 0.005


def test_student_t4_tail_quantiles():
    cfg = configs.S7B
    x = oracle.from16(synth.generate(cfg, 0, count=1 << 22), 0).astype(np.float64)
    z = x / (0.02 / np.sqrt(2.0))
    for q in (0.001, 0.01, 0.1, 0.5, 0.9, 0.99, 0.999):
        emp = np.quantile(z, q)
        ref = stats.t.ppf(q, 4)
        assert abs(emp - ref) < 0.03 * max(1.0, abs(ref))


def test_outliers_count_distinct_and_scaled():
    cfg = configs.SINGLE
    pos = synth.outlier_positions(cfg, 0)
    assert pos.size == round(0.001 * cfg.n(0)) == 16777
    assert np.unique(pos).size == pos.size
    assert pos.min() >= 0 and pos.max() < cfg.n(0)
    x = oracle.from16(synth.generate(cfg, 0), 0)
    assert np.median(np.abs(x[pos])) > 5 * np.median(np.abs(x))
    c5 = configs.S14B
    assert synth.outlier_positions(c5, 0).size == 13107
    assert synth.outlier_positions(c5, 4).size == 35389


def test_per_matrix_sigma_range():
    cfg = configs.S1P4B
    sig = [synth.layer_sigma(cfg, i) for i in range(cfg.n_layers)]
    assert all(0.01 <= s < 0.04 for s in sig)
    assert len(set(sig)) == cfg.n_layers
    x = oracle.from16(synth.generate(cfg, 3, count=1 << 20), 0).astype(np.float64)
    assert abs(x.std() / sig[3] - 1) < 0.01


def test_fp16_output_is_truncated_not_rounded():
    cfg = configs.TOY
    w = synth.generate(cfg, 0)
    x = oracle.from16(w, 1)
    assert np.all(np.isfinite(x))
    assert 0.019 < x.std() < 0.021


def test_config_shapes():
    assert configs.TOY.total == 1_581_056 and configs.TOY.n_layers == 14
    assert configs.SINGLE.total == 16_777_216
    assert configs.S1P4B.total == 1_207_959_552 and configs.S1P4B.n_layers == 96
    assert configs.S7B.total == 6_476_005_376 and configs.S7B.n_layers == 224
    assert configs.S14B.total == 12_687_769_600 and configs.S14B.n_layers == 280
