"""The seeded generators: deterministic, right shapes, right structure."""
import numpy as np

import workloads


def test_deterministic_and_distinct():
    a = workloads.head("small", "q", 0, 3)
    b = workloads.head("small", "q", 0, 3)
    c = workloads.head("small", "k", 0, 3)
    np.testing.assert_array_equal(a, b)
    assert not np.array_equal(a, c)
    q, k, v = workloads.qkv("tiny")
    assert q.shape == (1, 1, 256, 64) and q.dtype == np.uint16
    np.testing.assert_array_equal(q[0, 0], workloads.head("tiny", "q", 0, 0))


def test_small_outliers_shared_by_q_and_k():
    q = workloads.bf16_to_f32(workloads.head("small", "q", 0, 2))
    k = workloads.bf16_to_f32(workloads.head("small", "k", 0, 2))
    ch = workloads.outlier_channels("small", 1, 0, 2, 128)
    for x in (q, k):
        rms = np.sqrt(np.mean(x.astype(np.float64) ** 2, axis=0))
        assert set(np.argsort(rms)[-4:].tolist()) == set(ch.tolist())


def test_hunyuan_heavy_tokens():
    idx = workloads.heavy_tokens("hunyuan", 3, 65536)
    assert idx.size == 655 and np.unique(idx).size == 655


def test_sweep_range_and_sign():
    x = workloads.bf16_to_f32(workloads.sweep(16)).astype(np.float64)
    assert x.size == 65536
    a = np.abs(x)
    assert a.min() >= 2.0 ** -20.5 and a.max() <= 2.0 ** 10.5
    assert 0.45 < np.mean(x < 0) < 0.55


def test_f32_to_bf16_rne():
    f = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    assert workloads.f32_to_bf16(f).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xBF80, 0x3F81]


def test_sample_rows():
    r = workloads.sample_rows(40, 32760, 512)
    assert r[0] == 0 and r[-1] == 40 * 32760 - 1 and np.all(np.diff(r) > 0)
    np.testing.assert_array_equal(r, workloads.sample_rows(40, 32760, 512))
