"""GPU parity of the MXFP4 GEMM (mxgemm_quantized, mxgemm) against the oracle.

Acceptance: the GPU's bf16 Y against the oracle's exact Y = X_q W_q^T, per
element |diff| <= g |X_q| |W_q|^T + one bf16 ulp of (|Y| + that term), with
g = (K/128 + 16) 2^-24.  Every product of two dequantized MXFP4 values is
exact; the MFMA sums them in fp32, and each of the K/128 accumulations of a
128-deep MFMA into the fp32 result rounds once, plus a few roundings inside
one MFMA: g bounds that, and the ulp term the final rounding to bf16.  A
wrong code, scale or index moves an output by a large fraction of
|X_q| |W_q|^T and fails by orders of magnitude.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import HAVE_GPU, bf16_ulp, to_np_u16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx

MODES = [(oracle.MODE_UOS, "uos"), (oracle.MODE_OCP, "ocp")]


def up(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def compare_gemm(got_bits, ref, K, what=""):
    g = (K / 128 + 16) * 2.0 ** -24
    y = oracle.bf16_to_f64(got_bits).reshape(ref["out"].shape)
    err = g * ref["absdot"]
    tol = err + bf16_ulp(np.abs(ref["out"]) + err)
    diff = np.abs(y - ref["out"])
    info = dict(max_abs=float(diff.max()), worst_over_tol=float((diff / tol).max()),
                rel_l2=float(np.linalg.norm(y - ref["out"]) / max(np.linalg.norm(ref["out"]), 1e-300)))
    print(what, info)
    assert np.all(diff <= tol), f"{what}: {info}"
    return info


def run_gemm(x, w, M, N, K, gmode):
    xg, wg = up(x), up(w)
    xc, xs = mx.quantize(xg.view(1, M, K), mode=gmode, axis=1)
    wc, ws = mx.quantize(wg.view(1, N, K), mode=gmode, axis=1)
    y = mx.gemm_quantized(xc, xs, wc, ws, M, N, K)
    torch.cuda.synchronize()
    return y, (xg, wc, ws)


@pytest.mark.parametrize("omode,gmode", MODES)
@pytest.mark.parametrize("M,N,K", [(256, 256, 256), (300, 260, 384), (1, 4, 128), (513, 768, 640),
                                   (1000, 1000, 1024), (64, 520, 2048), (700, 300, 128), (70, 264, 20480)])
def test_gemm_full(omode, gmode, M, N, K):
    x, w = workloads.gemm_inputs(M=M, N=N, K=K, seed=M + N + K)
    y, _ = run_gemm(x, w, M, N, K, gmode)
    ref = oracle.gemm_rows(x, w, M, N, K, omode)
    compare_gemm(to_np_u16(y), ref, K, what=f"gemm {M}x{N}x{K} {gmode}")


@pytest.mark.parametrize("omode,gmode", MODES)
def test_gemm_dit_shape_sampled_rows(omode, gmode):
    """The Wan-style FFN up-projection (M=32760 tokens, K=5120, N=13824) on 64
    seeded rows (every row of Y depends only on its row of X)."""
    cfg = workloads.GEMM_CONFIGS["gemm"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    x, w = workloads.gemm_inputs("gemm")
    y, _ = run_gemm(x, w, M, N, K, gmode)
    rows = np.sort(np.random.default_rng(3).choice(M, 64, replace=False))
    rows[-1] = M - 1
    ref = oracle.gemm_rows(x, w, M, N, K, omode, rows)
    compare_gemm(to_np_u16(y)[rows], ref, K, what=f"gemm dit {gmode} (64 rows)")


@pytest.mark.parametrize("K", [384, 512, 640])
def test_gemm_several_tiles_per_workgroup(K):
    """17 x 17 tiles of 256 x 256 over a grid of one workgroup per CU, so some
    workgroups take a second tile: with an even number of 256-deep K steps
    (K = 384 with a half last step, K = 512) the second tile's first fills are
    issued before the first tile's epilogue; K = 640 (odd) takes the plain
    path.  256 seeded rows, the last M tile included."""
    M, N = 4113, 4196
    x, w = workloads.gemm_inputs(M=M, N=N, K=K, seed=K)
    y, _ = run_gemm(x, w, M, N, K, "uos")
    rows = np.sort(np.concatenate([np.random.default_rng(K).choice(M - 17, 240, replace=False),
                                   np.arange(M - 16, M)]))
    ref = oracle.gemm_rows(x, w, M, N, K, oracle.MODE_UOS, rows)
    compare_gemm(to_np_u16(y)[rows], ref, K, what=f"gemm {M}x{N}x{K} (256 rows)")


@pytest.mark.parametrize("gmode", ["uos", "ocp"])
def test_gemm_bf16_entry_equals_quantized_entry(gmode):
    M, N, K = 777, 512, 1280
    x, w = workloads.gemm_inputs(M=M, N=N, K=K, seed=1)
    y1, (xg, wc, ws) = run_gemm(x, w, M, N, K, gmode)
    y2 = mx.gemm(xg, wc, ws, N, mode=gmode)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


def test_gemm_zero_and_extreme_blocks():
    """A zero X row gives a zero Y row; X blocks at the ends of the exponent
    range still match the oracle."""
    M, N, K = 64, 64, 256
    x, w = workloads.gemm_inputs(M=M, N=N, K=K, seed=2)
    x[0] = 0
    x[1, :32] = workloads.f32_to_bf16(np.full(32, 3e-38, np.float32))
    x[2, :32] = workloads.f32_to_bf16(np.full(32, 1e30, np.float32))
    y, _ = run_gemm(x, w, M, N, K, "uos")
    got = to_np_u16(y)
    assert np.all(oracle.bf16_to_f64(got[0]) == 0.0)
    compare_gemm(got, oracle.gemm_rows(x, w, M, N, K, oracle.MODE_UOS), K, what="gemm extremes")
