"""Pins of the oracle over a varlen batch (sequences of different lengths
packed along one token axis; host only).

``oracle.attn_varlen_rows`` applies the pinned single-sequence oracle to each
sequence's slice.  These tests fix what the packing could get wrong, against
forms that do not go through that slicing:
  - one sequence over all tokens equals the head-major single-sequence oracle;
  - a sequence's outputs do not depend on other sequences' tokens;
  - a one-token sequence gives p = 1 exactly, so O is that token's V row
    quantized as a block of one value (the rest of the block is padding),
    built here from the pinned scalar encoder;
  - Q = 0 makes every exponential 1, so O is the mean of V quantized in
    32-token blocks counted from the sequence's own first token (not from
    token 0 of the batch), again built from the scalar encoder.
"""
import numpy as np
import pytest

import oracle
import workloads

MODES = [oracle.MODE_OCP, oracle.MODE_UOS]


def _packed(lengths, H, d, seed, scale=1.0):
    q, k, v, cu = workloads.varlen_qkv(lengths, H, d, seed=seed, dist="tiny")
    if scale != 1.0:
        q, k, v = (workloads.f32_to_bf16(workloads.bf16_to_f32(x) * np.float32(scale)) for x in (q, k, v))
    return q, k, v, cu


def _rows_all(cu, H):
    return np.array([(t, h) for t in range(int(cu[-1])) for h in range(H)], np.int64)


def _quantized_block_values(x, mode):
    """Dequantized values of one block (up to 32 values, zero-padded) from
    the scalar encoder and exponent rule."""
    amax = float(np.max(np.abs(x))) if x.size else 0.0
    e = oracle.block_exponent(amax, mode)
    return np.array([oracle.e2m1_value(oracle.e2m1_encode(float(xi) / 2.0 ** e), e) for xi in x])


@pytest.mark.parametrize("mode", MODES)
def test_single_sequence_equals_dense(mode):
    H, d, N = 2, 64, 150
    q, k, v, cu = _packed([N], H, d, seed=3)
    rows = _rows_all(cu, H)
    r = oracle.attn_varlen_rows(q, k, v, cu, H, d, mode, True, 128, 0.125, rows)
    hm = lambda x: np.ascontiguousarray(x.transpose(1, 0, 2))  # [H][T][d]
    dense = oracle.attn_rows(hm(q), hm(k), hm(v), H, N, d, mode, True, 128, 0.125,
                             rows[:, 1] * N + rows[:, 0])
    assert np.array_equal(r["out"], dense["out"])
    assert np.array_equal(r["l"], dense["l"])


@pytest.mark.parametrize("mode", MODES)
def test_sequences_do_not_interact(mode):
    H, d = 2, 64
    lengths = [40, 97, 5]
    q, k, v, cu = _packed(lengths, H, d, seed=4)
    rows = _rows_all(cu, H)
    r1 = oracle.attn_varlen_rows(q, k, v, cu, H, d, mode, True, 128, 0.125, rows)
    k2, v2 = k.copy(), v.copy()
    k2[cu[1]:cu[2]] ^= 0x0140  # new keys and values in sequence 1 only
    v2[cu[1]:cu[2]] ^= 0x0140
    r2 = oracle.attn_varlen_rows(q, k2, v2, cu, H, d, mode, True, 128, 0.125, rows)
    seq = np.searchsorted(cu, rows[:, 0], side="right") - 1
    same = seq != 1
    assert np.array_equal(r1["out"][same], r2["out"][same])
    assert not np.array_equal(r1["out"][~same], r2["out"][~same])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("pnq", [False, True])
def test_one_token_sequence_closed_form(mode, pnq):
    H, d = 3, 64
    q, k, v, cu = _packed([37, 1, 20], H, d, seed=5, scale=4.0)
    t = int(cu[1])
    rows = np.array([(t, h) for h in range(H)])
    r = oracle.attn_varlen_rows(q, k, v, cu, H, d, mode, pnq, 128, 0.0884, rows)
    vv = oracle.bf16_to_f64(v[t])  # [H][d]
    expect = np.array([[_quantized_block_values(vv[h, c:c + 1], mode)[0] for c in range(d)] for h in range(H)])
    assert np.array_equal(r["out"], expect)
    assert np.all(r["l"] == 1.0)


@pytest.mark.parametrize("mode", MODES)
def test_q_zero_blocks_start_at_sequence_start(mode):
    H, d = 1, 64
    lengths = [5, 70, 33]  # sequence 1 starts at token 5, sequence 2 at 75
    q, k, v, cu = _packed(lengths, H, d, seed=6, scale=3.0)
    q[:] = 0
    rows = np.array([(int(cu[s]), 0) for s in range(3)])
    r = oracle.attn_varlen_rows(q, k, v, cu, H, d, mode, True, 128, 0.125, rows)
    for s in range(3):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        x = oracle.bf16_to_f64(v[t0:t1, 0])  # [N][d]
        deq = np.concatenate([np.stack([_quantized_block_values(x[b:b + 32, c], mode) for c in range(d)], axis=1)
                              for b in range(0, t1 - t0, 32)])
        np.testing.assert_allclose(r["out"][s], deq.sum(axis=0) / (t1 - t0), rtol=1e-15, atol=0)
        assert r["l"][s] == t1 - t0
    # blocking from token 0 of the batch instead would change sequence 1's V
    x = oracle.bf16_to_f64(v[:, 0])
    wrong = np.concatenate([np.stack([_quantized_block_values(x[b:b + 32, c], mode) for c in range(d)], axis=1)
                            for b in range(0, int(cu[-1]), 32)])[5:75].mean(axis=0)
    assert not np.allclose(r["out"][1], wrong, rtol=1e-12, atol=0)
