"""Pins of the oracle's MXFP4 quantizer (host only).

Each test checks the oracle against something that does not come from the
oracle: hand-worked blocks, the closed-form E2M1 decision intervals, the
interval invariants of the two scale rules, a brute-force search over block
scales (which must land on the UOS boundary Qmax = 7.25 that the MXAttention
abstract states), and layout identities.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_blocks.json")
MODES = {"ocp": oracle.MODE_OCP, "uos": oracle.MODE_UOS}


def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["blocks"]


@pytest.mark.parametrize("blk", _golden(), ids=lambda b: b["name"])
def test_worked_blocks(blk):
    bits = np.zeros(32, np.uint16)
    inp = [int(h, 16) for h in blk["input_hex"]]
    bits[: len(inp)] = inp
    # the hex patterns are the stated values
    np.testing.assert_array_equal(workloads.bf16_to_f32(bits[: len(inp)]).astype(np.float64),
                                  np.array(blk["input_values"]))
    codes, scales = oracle.quantize_bf16(bits, 1, 1, 32, 1, MODES[blk["mode"]])
    assert scales.tolist() == [blk["scale"]]
    expect_bytes = np.zeros(16, np.uint8)
    for i, h in enumerate(blk["bytes"]):
        expect_bytes[i] = int(h, 16)
    np.testing.assert_array_equal(codes, expect_bytes)
    unpacked = [(codes[i // 2] >> (4 * (i % 2))) & 15 for i in range(len(blk["codes"]))]
    assert unpacked == blk["codes"]
    deq = oracle.dequantize(codes, scales, 1, 32)[0]
    if "deq" in blk:
        got = deq[: len(blk["deq"])]
        np.testing.assert_array_equal(got, np.array(blk["deq"]))
        np.testing.assert_array_equal(np.signbit(got), np.signbit(np.array(blk["deq"])))
    if "sse" in blk:
        x = np.array(blk["input_values"] + [0.0] * (32 - len(inp)))
        assert float(np.sum((x - deq) ** 2)) == blk["sse"]


def _closed_form_e2m1(y):
    """E2M1 decision intervals with ties to the even code, saturating at 6."""
    a = np.abs(y)
    code = np.select(
        [a <= 0.25, a < 0.75, a <= 1.25, a < 1.75, a <= 2.5, a < 3.5, a <= 5.0],
        [0, 1, 2, 3, 4, 5, 6], default=7).astype(np.uint8)
    return code | (np.signbit(y).astype(np.uint8) << 3)


def test_e2m1_encoder_exhaustive_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]  # finite patterns only
    x = workloads.bf16_to_f32(bits).astype(np.float64)
    for e in (-127, -126, -120, -10, -3, -2, -1, 0, 1, 2, 3, 10, 100, 125, 127):
        y = np.ldexp(x, -e)
        y = y[np.isfinite(y)]
        np.testing.assert_array_equal(oracle.e2m1_encode_array(y), _closed_form_e2m1(y), err_msg=f"e={e}")


def test_e2m1_encoder_ties_and_neighbours():
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for t in ties:
        for y in (t, np.nextafter(t, 0), np.nextafter(t, 10)):
            for s in (1.0, -1.0):
                assert oracle.e2m1_encode_array([s * y])[0] == _closed_form_e2m1(np.array([s * y]))[0]
    assert oracle.e2m1_encode(1e30) == 7 and oracle.e2m1_encode(-1e30) == 15
    assert oracle.e2m1_encode(-0.0) == 8 and oracle.e2m1_encode(0.0) == 0


def test_value_table():
    mags = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    for c in range(16):
        v = oracle.e2m1_value(c, 0)
        assert abs(v) == mags[c & 7] and (np.signbit(v) == bool(c & 8))
        assert oracle.e2m1_value(c, 5) == v * 32


def test_scale_rule_interval_invariants():
    g = np.random.default_rng(123)
    amax = np.exp2(g.uniform(-120, 120, 200000))
    amax = np.concatenate([amax, np.exp2(np.arange(-120, 121, dtype=np.float64)),
                           7.25 * np.exp2(np.arange(-110, 110, dtype=np.float64)),
                           3.625 * np.exp2(np.arange(-110, 110, dtype=np.float64))])
    eo = oracle.block_exponent_array(amax, oracle.MODE_OCP).astype(np.float64)
    eu = oracle.block_exponent_array(amax, oracle.MODE_UOS).astype(np.float64)
    ro = amax / np.exp2(eo)
    ru = amax / np.exp2(eu)
    assert np.all((ro >= 4) & (ro < 8))
    assert np.all((ru > 3.625) & (ru <= 7.25))
    mant = amax / np.exp2(np.floor(np.log2(amax)))
    np.testing.assert_array_equal(eu - eo, (mant > 1.8125).astype(np.float64))
    # share of blocks whose exponent differs, for log-uniform amax: 1 - log2(1.8125)
    share = np.mean(eu[:200000] != eo[:200000])
    assert abs(share - (1 - np.log2(1.8125))) < 0.005


def test_scale_rule_clamps():
    for mode in (oracle.MODE_OCP, oracle.MODE_UOS):
        assert oracle.block_exponent(0.0, mode) == -127
        assert oracle.block_exponent(2.0 ** -140, mode) == -127
        assert oracle.block_exponent(float(np.finfo(np.float64).max), mode) == 127
        assert oracle.block_exponent(2.0 ** -124, mode) == -126


def _mse_sweep(blocks):
    """Brute force over block exponents: SSE of each block at every candidate
    exponent around floor(log2 amax), then the total SSE of the rule
    'smallest e with amax <= Qmax 2^e' for each Qmax on a 1/32 grid."""
    amax = np.max(np.abs(blocks), axis=1)
    E = np.floor(np.log2(amax)).astype(int)
    sse = np.empty((blocks.shape[0], 5))
    for e_val in np.unique(E):
        sel = E == e_val
        sse[sel] = oracle.block_sse_batch(blocks[sel], int(e_val) - 3, 5)  # e = E-3 .. E+1
    grid = np.arange(6.0, 8.0 + 1e-9, 1.0 / 32)
    tot = []
    for qmax in grid:
        # smallest e (relative to E) with amax <= qmax 2^e
        rel = np.full(amax.shape, 1)
        for r in (0, -1, -2, -3):
            ok = amax <= qmax * np.exp2(E + r)
            rel = np.where(ok, r, rel)
        tot.append(np.sum(sse[np.arange(len(amax)), rel + 3]))
    tot = np.array(tot)
    best_per_block = np.sum(np.min(sse, axis=1))
    return grid, tot, best_per_block, sse, E


def test_uos_boundary_is_brute_force_mse_optimum():
    """The MXAttention abstract claims Qmax = 7.25 is an optimal, distribution-
    independent scaling boundary.  Brute-force the boundary on Gaussian blocks
    whose amax is spread uniformly over the octave and check that 7.25 is the
    argmin of the total MSE (within the flat optimum) and that the oracle's
    UOS rule picks exactly the exponents of Qmax = 7.25."""
    g = np.random.default_rng(2024)
    nblk = 200000
    blocks = g.standard_normal((nblk, 32)) * np.exp2(g.uniform(0, 1, (nblk, 1)))
    grid, tot, best, sse, E = _mse_sweep(blocks)
    argmin = grid[np.argmin(tot)]
    i725 = int(np.argmin(np.abs(grid - 7.25)))
    assert 7.125 <= argmin <= 7.375, argmin
    assert tot[i725] <= 1.005 * tot.min()
    # the oracle's UOS rule equals the Qmax = 7.25 rule block by block
    amax = np.max(np.abs(blocks), axis=1)
    eu = oracle.block_exponent_array(amax, oracle.MODE_UOS)
    eo = oracle.block_exponent_array(amax, oracle.MODE_OCP)
    sse_uos = np.sum(sse[np.arange(nblk), eu - E + 3])
    sse_ocp = np.sum(sse[np.arange(nblk), eo - E + 3])
    assert sse_uos == pytest.approx(tot[i725], rel=1e-12)
    # OCP corresponds to Qmax = 8 with the top end open; UOS must beat it
    assert sse_uos < 0.96 * sse_ocp
    # and UOS is within 0.5% of the per-block brute-force optimum
    assert sse_uos <= 1.005 * best


def _workload_blocks(name, axis):
    if name == "sweep":
        x = workloads.bf16_to_f32(workloads.sweep(18)).astype(np.float64).reshape(-1, 1024)
        return x.reshape(-1, 32)
    cfg = workloads.CONFIGS[name]
    x = workloads.bf16_to_f32(workloads.head(name, "k", 0, 0, N=min(cfg["N"], 4096))).astype(np.float64)
    if axis == 0:
        x = x.T.copy()
    return x.reshape(-1, 32)


@pytest.mark.parametrize("name,axis", [("tiny", 1), ("small", 1), ("wan", 1), ("wan", 0),
                                       ("hunyuan", 1), ("hunyuan", 0), ("sweep", 1)])
def test_uos_beats_ocp_on_every_workload(name, axis):
    blocks = _workload_blocks(name, axis)
    tot = {}
    for mode in (oracle.MODE_OCP, oracle.MODE_UOS):
        codes, scales = oracle.quantize_f64(blocks.reshape(-1), mode)
        deq = oracle.dequantize(codes, scales, 1, blocks.size)[0]
        # relative error per block, so tiny and huge blocks weigh alike
        err = np.sum((blocks.reshape(-1) - deq).reshape(blocks.shape) ** 2, axis=1)
        nrm = np.sum(blocks ** 2, axis=1)
        tot[mode] = np.mean(err[nrm > 0] / nrm[nrm > 0])
    assert tot[oracle.MODE_UOS] < tot[oracle.MODE_OCP]


def test_axis0_is_axis1_of_transpose():
    g = np.random.default_rng(5)
    batch, rows, cols = 3, 75, 40  # ragged along both axes
    x = workloads.f32_to_bf16(g.standard_normal((batch, rows, cols)).astype(np.float32) *
                              np.exp2(g.integers(-8, 8, (batch, 1, cols))).astype(np.float32))
    for mode in (oracle.MODE_OCP, oracle.MODE_UOS):
        c0, s0 = oracle.quantize_bf16(x, batch, rows, cols, 0, mode)
        c1, s1 = oracle.quantize_bf16(np.ascontiguousarray(np.swapaxes(x, 1, 2)), batch, cols, rows, 1, mode)
        np.testing.assert_array_equal(c0, c1)
        np.testing.assert_array_equal(s0, s1)


def test_layout_and_padding_axis0():
    rows, cols = 40, 2
    x = np.zeros((rows, cols), np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 2.0
    c, s = oracle.quantize_bf16(workloads.f32_to_bf16(x), 1, rows, cols, 0, oracle.MODE_UOS)
    c = c.reshape(cols, 2, 16)
    s = s.reshape(cols, 2)
    assert s.tolist() == [[125, 125], [126, 126]]
    assert np.all(c[:, 0, :] == 0x66)
    assert np.all(c[:, 1, :4] == 0x66) and np.all(c[:, 1, 4:] == 0)


def test_dequantize_reproduces_grid_values():
    g = np.random.default_rng(9)
    mags = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    for mode in (oracle.MODE_OCP, oracle.MODE_UOS):
        for _ in range(50):
            e = int(g.integers(-20, 20))
            v = mags[g.integers(0, 8, 32)] * np.where(g.random(32) < 0.5, -1, 1)
            v[0] = 6.0 if mode == oracle.MODE_OCP else 4.0  # the block's amax fixes e
            v[1:] = np.clip(v[1:], -4.0 if mode == oracle.MODE_UOS else -6, 4.0 if mode == oracle.MODE_UOS else 6)
            x = np.ldexp(v, e)
            codes, scales = oracle.quantize_f64(x, mode)
            assert int(scales[0]) - 127 == e
            np.testing.assert_array_equal(oracle.dequantize(codes, scales, 1, 32)[0], x)


def test_bf16_rounding_two_ways():
    g = np.random.default_rng(11)
    f = (g.standard_normal(100000) * np.exp2(g.integers(-130, 120, 100000))).astype(np.float32)
    # exact ties: 8 significant bits plus a half
    ties = (np.float32(1.0) + np.float32(2.0 ** -8) * np.arange(1, 400, 2).astype(np.float32)).astype(np.float32)
    f = np.concatenate([f, ties, -ties]).astype(np.float32)
    np.testing.assert_array_equal(oracle.f64_to_bf16(f.astype(np.float64)), workloads.f32_to_bf16(f))


def read_mxq1(path):
    """Parse an "MXQ1" dump: 256-byte JSON header, code bytes, scale bytes."""
    with open(path, "rb") as f:
        raw = f.read()
    assert raw[255:256] == b"\n"
    hdr = json.loads(raw[:256].decode("ascii").strip())
    nb = (hdr["L"] + 31) // 32
    ncode = hdr["batch"] * hdr["nvec"] * nb * 16
    nscale = hdr["batch"] * hdr["nvec"] * nb
    assert len(raw) == 256 + ncode + nscale
    codes = np.frombuffer(raw[256:256 + ncode], np.uint8)
    scales = np.frombuffer(raw[256 + ncode:], np.uint8)
    return hdr, codes, scales


def test_oracle_dump_format(tmp_path):
    g = np.random.default_rng(0)
    x = workloads.f32_to_bf16(g.standard_normal((2, 70, 96)).astype(np.float32))
    c, s = oracle.quantize_bf16(x, 2, 70, 96, 0, oracle.MODE_UOS)
    p = str(tmp_path / "v.mxq")
    oracle.dump(p, c, s, 2, 96, 70, 0, oracle.MODE_UOS)
    hdr, c2, s2 = read_mxq1(p)
    assert hdr == {"magic": "MXQ1", "version": 1, "mode": "uos", "axis": 0, "batch": 2, "nvec": 96,
                   "L": 70, "block": 32, "elem": "e2m1", "scale": "e8m0", "nibble": "lo-first"}
    np.testing.assert_array_equal(c2, c)
    np.testing.assert_array_equal(s2, s)
    with pytest.raises(OSError):
        oracle.dump(str(tmp_path / "no" / "such" / "dir.mxq"), c, s, 2, 96, 70, 0, oracle.MODE_UOS)
