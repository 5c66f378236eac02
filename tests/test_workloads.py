"""The seeded input generator: determinism, shapes, outlier columns, MoE counts."""

import numpy as np

import workloads
from oracle.formats import bf16_to_float64


def test_deterministic_and_seed_separated():
    a = workloads.normal_bf16(2, 0, (64, 128), 1.0, 0.01)
    b = workloads.normal_bf16(2, 0, (64, 128), 1.0, 0.01)
    c = workloads.normal_bf16(2, 1, (64, 128), 1.0, 0.01)
    assert a.dtype == np.uint16 and a.shape == (64, 128)
    assert np.array_equal(a, b) and not np.array_equal(a, c)


def test_sigma_and_outliers():
    x = bf16_to_float64(workloads.normal_bf16(9, 9, (2048, 1000), 0.02, 0.01))
    col_std = x.std(axis=0)
    big = col_std > 0.1
    assert big.sum() == 10  # round(1% of 1000) columns x20
    assert abs(np.median(col_std) - 0.02) < 0.002
    assert np.allclose(col_std[big], 0.4, rtol=0.15)


def test_moe_counts():
    c = workloads.moe_counts()
    assert c.shape == (32,) and c.sum() == 16384 and c.dtype == np.int32
    assert np.any(c % 256 != 0)
    assert np.array_equal(c, workloads.moe_counts())


def test_config_shapes():
    w = workloads.hybrid_backward()
    dgrad, wgrad = w.gemms
    assert (dgrad.M, dgrad.N, dgrad.K) == (4096, 4096, 14336)
    assert (wgrad.M, wgrad.N, wgrad.K) == (14336, 4096, 4096)
    assert dgrad.a_src.shape == (4096, 14336) and dgrad.b_src.shape == (14336, 4096)
    d = workloads.decoder_forward()
    assert [(g.M, g.N, g.K) for g in d.gemms] == [(4096, 3072, 1024), (4096, 4096, 1024), (4096, 1024, 4096)]
    for name, fn in workloads.ALL.items():
        assert fn().name
