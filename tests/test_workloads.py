"""The seeded generator: deterministic bytes, chunk-independent, recipe features present."""
import numpy as np

import workloads


def test_deterministic_and_row_ranges():
    cfg = workloads.config(1)
    full = workloads.draw_tensor(cfg, "X", rows=(0, 1024))
    again = workloads.draw_tensor(cfg, "X", rows=(0, 1024))
    np.testing.assert_array_equal(full, again)
    part = workloads.draw_tensor(cfg, "X", rows=(512, 1024))
    np.testing.assert_array_equal(full[512:], part)


def test_zero_blocks_and_outliers_small_config():
    cfg = workloads.config(0)
    a = workloads.draw_tensor(cfg, "A")
    b = workloads.draw_tensor(cfg, "B")
    assert a.shape == (256, 512) and b.shape == (512, 256)
    assert not (a[7, 96:128] & 0x7FFF).any()
    assert not (b[288:320, 200] & 0x7FFF).any()
    af = workloads.bf16_bits_to_f32(a)
    frac = np.mean(np.abs(af) > 6.0)  # |N(0,1)| > 6 is ~2e-9; the 1% x30 outliers exceed it often
    assert 0.003 < frac < 0.02


def test_outlier_channels():
    cfg = workloads.config(1)
    x = workloads.bf16_bits_to_f32(workloads.draw_tensor(cfg, "X", rows=(0, 256)))
    col_rms = np.sqrt((x.astype(np.float64) ** 2).mean(axis=0))
    assert int(np.sum(col_rms > 20)) == 4  # round(0.001 * 4096) channels scaled x50


def test_distinct_tensors_and_configs():
    a = workloads.draw_tensor(workloads.config(1), "X", rows=(0, 256))
    b = workloads.draw_tensor(workloads.config(2), "X", rows=(0, 256))
    assert not np.array_equal(a, b)


def test_config_shapes_consistent():
    for cfg in workloads.CONFIGS:
        for g in cfg.gemms:
            qa, qb = cfg.quant(g.a), cfg.quant(g.b)
            ta, tb = cfg.tensor(qa.tensor), cfg.tensor(qb.tensor)
            a_rows, a_k = (ta.rows, ta.cols) if qa.kind == "row" else (ta.cols, ta.rows)
            b_rows, b_k = (tb.rows, tb.cols) if qb.kind == "row" else (tb.cols, tb.rows)
            assert (a_rows, b_rows, a_k, b_k) == (g.M, g.N, g.K, g.K), (cfg.name, g.name)
