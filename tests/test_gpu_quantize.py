"""GPU parity of mxq_quantize against the oracle: bit-exact codes and scales."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import HAVE_GPU, to_gpu_bf16, to_np_u8

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import mxfp4_quantized_attention_amd as mx

MODES = [(oracle.MODE_OCP, "ocp"), (oracle.MODE_UOS, "uos")]


def gpu_quant(bits3, axis, mode):
    x = to_gpu_bf16(bits3)
    c, s = mx.quantize(x, mode=mode, axis=axis)
    return to_np_u8(c).reshape(-1), to_np_u8(s).reshape(-1)


def check(bits3, axis, omode, gmode, what=""):
    batch, rows, cols = bits3.shape
    c, s = gpu_quant(bits3, axis, gmode)
    ec, es = oracle.quantize_bf16(bits3, batch, rows, cols, axis, omode)
    bad_s = np.flatnonzero(s != es)
    bad_c = np.flatnonzero(c != ec)
    assert bad_s.size == 0, f"{what}: {bad_s.size} scale bytes differ, first {bad_s[:5]}"
    assert bad_c.size == 0, f"{what}: {bad_c.size} code bytes differ, first {bad_c[:5]}"


def exhaustive_blocks(seed=0):
    """Blocks [A, x1..x31] where A = +-7 * 2^e fixes the block exponent e (for
    both rules) and the x run over every finite bf16 pattern with |x| <= |A|,
    for every e in [-127, 125]."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[(bits & 0x7F80) != 0x7F80]
    mags = np.abs(workloads.bf16_to_f32(bits).astype(np.float64))
    g = np.random.default_rng(seed)
    out = []
    for e in range(-127, 126):
        A = 7.0 * 2.0 ** e
        sel = g.permutation(bits[mags <= A])
        pad = (-sel.size) % 31
        sel = np.concatenate([sel, sel[:pad]]).reshape(-1, 31)
        a = workloads.f32_to_bf16(np.array([A if e % 2 else -A], np.float32))[0]
        out.append(np.concatenate([np.full((sel.shape[0], 1), a, np.uint16), sel], axis=1))
    return np.concatenate(out)


@pytest.fixture(scope="module")
def exhaustive():
    return exhaustive_blocks()


@pytest.mark.parametrize("omode,gmode", MODES)
def test_exhaustive_bf16_every_exponent_axis1(exhaustive, omode, gmode):
    blk = exhaustive
    check(blk.reshape(1, blk.shape[0], 32), 1, omode, gmode, "exhaustive axis 1")


@pytest.mark.parametrize("omode,gmode", MODES)
def test_exhaustive_bf16_every_exponent_axis0(exhaustive, omode, gmode):
    blk = exhaustive[: (exhaustive.shape[0] // 64) * 64]
    R = blk.shape[0] // 64
    x = blk.reshape(R, 64, 32).transpose(0, 2, 1).reshape(1, 32 * R, 64)
    check(np.ascontiguousarray(x), 0, omode, gmode, "exhaustive axis 0")


@pytest.mark.parametrize("omode,gmode", MODES)
@pytest.mark.parametrize("name,heads", [("tiny", 1), ("small", 8), ("wan", 2), ("hunyuan", 2)])
def test_workloads_both_axes(name, heads, omode, gmode):
    cfg = workloads.CONFIGS[name]
    for t in ("q", "v"):
        x = np.stack([workloads.head(name, t, 0, h) for h in range(heads)])
        check(x, 1, omode, gmode, f"{name} {t} axis 1")
        check(x, 0, omode, gmode, f"{name} {t} axis 0")


@pytest.mark.parametrize("shape", [(2, 75, 100), (1, 32760, 128), (3, 33, 37), (1, 1, 1), (2, 300, 8),
                                   (1, 257, 65), (4, 31, 96)])
@pytest.mark.parametrize("omode,gmode", MODES)
def test_ragged_shapes(shape, omode, gmode):
    g = np.random.default_rng(sum(shape))
    x = workloads.f32_to_bf16((g.standard_normal(shape) * np.exp2(g.uniform(-30, 30, shape))).astype(np.float32))
    check(x, 1, omode, gmode, f"{shape} axis 1")
    check(x, 0, omode, gmode, f"{shape} axis 0")


@pytest.mark.parametrize("shape", [(3, 1000, 700), (1, 2049, 1030), (2, 300, 257), (1, 64, 4096)])
@pytest.mark.parametrize("omode,gmode", MODES)
def test_axis0_wide_ragged(shape, omode, gmode):
    """Blocks along rows for inputs wider than one 64-column tile: every
    column tile (the ragged last one too) and every row tile, bit for bit."""
    g = np.random.default_rng(sum(shape) + 7)
    x = workloads.f32_to_bf16((g.standard_normal(shape) * np.exp2(g.uniform(-20, 20, shape))).astype(np.float32))
    check(x, 0, omode, gmode, f"{shape} axis 0")


def test_sweep_axis0_sampled():
    """The sweep's row-axis case, 2^28 values viewed [2^18, 1024] with blocks
    along rows (the configuration the bench times), on 8192 seeded sampled
    (column, block) pairs per mode, every column tile represented."""
    R, C = 1 << 18, 1024
    x = workloads.sweep(28).reshape(R, C)
    xg = to_gpu_bf16(x.reshape(1, R, C))
    g = np.random.default_rng(2028)
    nb = R // 32
    cols = np.concatenate([np.arange(C), g.integers(0, C, 8192 - C)])
    blks = np.concatenate([g.integers(0, nb, C - 2), [0, nb - 1], g.integers(0, nb, 8192 - C)])
    sub = np.stack([x[32 * b: 32 * b + 32, c] for c, b in zip(cols, blks)])
    flat = torch_index(cols.astype(np.int64) * nb + blks)
    for omode, gmode in MODES:
        c, s = mx.quantize(xg, mode=gmode, axis=0)
        cg = c.view(-1, 16)[flat].cpu().numpy().reshape(-1)
        sg = s.view(-1)[flat].cpu().numpy()
        ec, es = oracle.quantize_bf16(sub, 1, sub.shape[0], 32, 1, omode)
        np.testing.assert_array_equal(sg, es)
        np.testing.assert_array_equal(cg, ec)
        del c, s


@pytest.mark.parametrize("p", [20, 22, 24])
@pytest.mark.parametrize("omode,gmode", MODES)
def test_sweep_full(p, omode, gmode):
    x = workloads.sweep(p)
    check(x.reshape(1, -1, 1024), 1, omode, gmode, f"sweep 2^{p}")


@pytest.mark.parametrize("p", [28, 30])
def test_sweep_large_sampled(p):
    """Full-size sweep tensors (the roofline sizes), checked on 8192 seeded
    sampled blocks per mode."""
    x = workloads.sweep(p)
    xg = to_gpu_bf16(x.reshape(1, -1, 1024))
    g = np.random.default_rng(p)
    nblk = x.size // 32
    idx = np.sort(g.choice(nblk, 8192, replace=False))
    for omode, gmode in MODES:
        c, s = mx.quantize(xg, mode=gmode, axis=1)
        c = c.view(-1, 16)[torch_index(idx)].cpu().numpy().reshape(-1)
        s = s.view(-1)[torch_index(idx)].cpu().numpy()
        sub = x.reshape(-1, 32)[idx]
        ec, es = oracle.quantize_bf16(sub, 1, idx.size, 32, 1, omode)
        np.testing.assert_array_equal(s, es)
        np.testing.assert_array_equal(c, ec)
        del c, s


def torch_index(idx):
    import torch
    return torch.from_numpy(idx).to("cuda:0")


def test_empty_is_noop():
    import torch
    x = torch.empty((0, 5, 32), dtype=torch.bfloat16, device="cuda:0")
    c, s = mx.quantize(x, mode="uos", axis=1)
    assert c.numel() == 0 and s.numel() == 0


def test_dump_matches_oracle_dump(tmp_path):
    from test_oracle_quant import read_mxq1
    x = np.stack([workloads.head("small", "v", 0, h) for h in range(2)])
    for axis in (0, 1):
        for omode, gmode in MODES:
            c, s = mx.quantize(to_gpu_bf16(x), mode=gmode, axis=axis)
            nvec, L = (4096, 128) if axis == 1 else (128, 4096)
            p1, p2 = str(tmp_path / "gpu.mxq"), str(tmp_path / "orc.mxq")
            mx.dump(p1, c, s, 2, nvec, L, axis, gmode)
            ec, es = oracle.quantize_bf16(x, 2, 4096, 128, axis, omode)
            oracle.dump(p2, ec, es, 2, nvec, L, axis, omode)
            assert open(p1, "rb").read() == open(p2, "rb").read()
            hdr, _, _ = read_mxq1(p1)
            assert hdr["axis"] == axis and hdr["mode"] == gmode
