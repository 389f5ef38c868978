"""Pins of the oracle's MXFP4 GEMM, Y = X_q W_q^T (host only).

The oracle composes its quantizer (pinned in test_oracle_quant.py), its
dequantizer and a library matmul.  These tests fix the composition, the part
a plausible mistake would break (blocking along the wrong axis, a transposed
operand, a scale applied to the wrong block, nibble order):
  - brute force on tiny shapes: every output summed from the raw code and
    scale bytes in exact rational arithmetic;
  - W = identity (N = K): Y is exactly the dequantized X;
  - power-of-two equivariance: scaling X by 2^k shifts every block exponent
    by k and leaves the codes alone, so Y scales by exactly 2^k;
  - without quantization the oracle is the plain product of the bf16 inputs.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4),
        Fraction(6)]


def _rand(seed, shape, scale=1.0):
    g = np.random.default_rng(seed)
    return workloads.f32_to_bf16((g.standard_normal(shape) * scale).astype(np.float32))


def _exact_row_values(codes, scales, K):
    """Exact values of one quantized row from its bytes: element 2i in the low
    nibble of byte i, bit 3 the sign, block b scaled by 2^(scale[b] - 127)."""
    vals = []
    for kk in range(K):
        byte = int(codes[kk // 2])
        nib = byte & 0xF if kk % 2 == 0 else byte >> 4
        mag = E2M1[nib & 7] * Fraction(2) ** (int(scales[kk // 32]) - 127)
        vals.append(-mag if nib & 8 else mag)
    return vals


@pytest.mark.parametrize("mode", [oracle.MODE_OCP, oracle.MODE_UOS])
@pytest.mark.parametrize("M,N,K", [(3, 5, 64), (2, 4, 128), (4, 3, 96)])
def test_brute_force_from_bytes(mode, M, N, K):
    x = _rand(M * 100 + K, (M, K), 3.0)
    w = _rand(N * 100 + K + 1, (N, K), 0.5)
    r = oracle.gemm_rows(x, w, M, N, K, mode)
    xc, xs = oracle.quantize_bf16(x, 1, M, K, 1, mode)
    wc, ws = oracle.quantize_bf16(w, 1, N, K, 1, mode)
    cb, sb = K // 2, K // 32
    xv = [_exact_row_values(xc[i * cb:(i + 1) * cb], xs[i * sb:(i + 1) * sb], K) for i in range(M)]
    wv = [_exact_row_values(wc[j * cb:(j + 1) * cb], ws[j * sb:(j + 1) * sb], K) for j in range(N)]
    for i in range(M):
        for j in range(N):
            exact = sum(a * b for a, b in zip(xv[i], wv[j]))
            assert r["out"][i, j] == float(exact)
            assert r["absdot"][i, j] == float(sum(abs(a * b) for a, b in zip(xv[i], wv[j])))


@pytest.mark.parametrize("mode", [oracle.MODE_OCP, oracle.MODE_UOS])
def test_identity_weight_returns_quantized_x(mode):
    K = 256
    x = _rand(7, (9, K), 2.0)
    w = workloads.f32_to_bf16(np.eye(K, dtype=np.float32))
    r = oracle.gemm_rows(x, w, 9, K, K, mode)
    xc, xs = oracle.quantize_bf16(x, 1, 9, K, 1, mode)
    # the identity's rows quantize exactly (one 1.0 per block, or a zero block)
    assert np.array_equal(r["out"], oracle.dequantize(xc, xs, 9, K))


@pytest.mark.parametrize("mode", [oracle.MODE_OCP, oracle.MODE_UOS])
@pytest.mark.parametrize("k", [-3, 5])
def test_power_of_two_equivariance(mode, k):
    M, N, K = 6, 10, 384
    x = _rand(11, (M, K))
    w = _rand(12, (N, K))
    x2 = workloads.f32_to_bf16(workloads.bf16_to_f32(x) * np.float32(2.0 ** k))
    r1 = oracle.gemm_rows(x, w, M, N, K, mode)
    r2 = oracle.gemm_rows(x2, w, M, N, K, mode)
    assert np.array_equal(r2["out"], r1["out"] * 2.0 ** k)


def test_identity_quantizer_is_plain_product():
    M, N, K = 5, 7, 64
    x, w = _rand(3, (M, K)), _rand(4, (N, K))
    r = oracle.gemm_rows(x, w, M, N, K, oracle.MODE_NONE)
    xf = oracle.bf16_to_f64(x).reshape(M, K)
    wf = oracle.bf16_to_f64(w).reshape(N, K)
    expect = np.array([[sum(float(a) * float(b) for a, b in zip(xf[i], wf[j])) for j in range(N)]
                       for i in range(M)])
    assert np.allclose(r["out"], expect, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    M, N, K = 40, 12, 128
    x, w = _rand(5, (M, K)), _rand(6, (N, K))
    full = oracle.gemm_rows(x, w, M, N, K, oracle.MODE_UOS)
    rows = np.array([0, 7, 39])
    sub = oracle.gemm_rows(x, w, M, N, K, oracle.MODE_UOS, rows)
    assert np.array_equal(sub["out"], full["out"][rows])
