"""Shared helpers for the GPU parity tests (device transfer, bf16 comparison)."""
import numpy as np
import pytest

import oracle
import workloads

try:
    import torch
    HAVE_GPU = torch.cuda.is_available()
except Exception:  # pragma: no cover
    torch = None
    HAVE_GPU = False

needs_gpu = pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")


def to_gpu_bf16(bits):
    a = np.ascontiguousarray(bits, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16)).to("cuda:0").view(torch.bfloat16)


def to_np_u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def to_np_u8(t):
    return t.contiguous().cpu().numpy()


def bf16_ulp(x):
    """Spacing of the bf16 grid at |x| (2^-133 below the normal range)."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126)
    return np.where(a > 0, np.exp2(e - 7), 2.0 ** -133)


def compare_attention(gpu_bits, ref, near_tie=None, atol=2e-3, rel_l2_max=1e-3, what=""):
    """Acceptance for the bf16 attention output against the oracle.

    The oracle's fp64 output is rounded to bf16 (round to nearest even) and
    compared with the GPU's bf16 output: relative L2 <= rel_l2_max over all
    checked elements, and per element |diff| <= max(atol, one bf16 ulp of the
    reference).  Rows the oracle flags as holding a quantization decision
    that the fp32 definition of the exponentials does not settle (within
    2^-22 (4 + |t| + |m|) of a tie) may differ beyond the per-element bound
    (either rounding is correct there); they still count in the relative L2,
    and at most 1% of the rows (plus one) may exceed the per-element bound."""
    g = oracle.bf16_to_f64(gpu_bits).reshape(ref["out"].shape)
    r = oracle.bf16_to_f64(ref["out_bf16"]).reshape(ref["out"].shape)
    diff = np.abs(g - r)
    tol = np.maximum(atol, bf16_ulp(r))
    bad_rows = np.where(np.any(diff > tol, axis=1))[0]
    flagged = ref["near_tie"] if near_tie is None else near_tie
    unexplained = [int(i) for i in bad_rows if not flagged[i]]
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    info = dict(max_abs=float(diff.max()), rel_l2=rel, bad_rows=len(bad_rows),
                flagged_rows=int(np.sum(flagged)), unexplained=unexplained[:10])
    print(what, info)
    assert not unexplained, f"{what}: rows beyond tolerance that the oracle did not flag: {info}"
    n = len(flagged)
    assert len(bad_rows) <= 1 + n // 100, f"{what}: too many rows beyond tolerance: {info}"
    assert rel <= rel_l2_max, f"{what}: relative L2 {rel} > {rel_l2_max}"
    return info
