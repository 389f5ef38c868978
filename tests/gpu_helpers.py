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


def attention_tolerance(ref, atol=2e-3):
    """Per-element bound for the GPU's bf16 output against the oracle's
    bf16-rounded output: max(atol, one bf16 ulp of the reference), plus, on
    rows with decisions the fp32 definition of the exponentials does not
    settle (within 2^-22 (4 + |t| + |m|) of a tie, where either rounding is
    correct), the oracle's budget for those decisions going the other way
    and one more ulp for rounding the moved value."""
    r = oracle.bf16_to_f64(ref["out_bf16"]).reshape(ref["out"].shape)
    tol = np.maximum(atol, bf16_ulp(r))
    budget = ref.get("budget")
    if budget is not None:
        tol = tol + np.where(budget > 0, budget + bf16_ulp(np.abs(r) + budget), 0.0)
    return r, tol


def compare_attention(gpu_bits, ref, atol=2e-3, rel_l2_max=1e-3, what="", max_budget_rows=None):
    """Acceptance for the bf16 attention output against the oracle: every
    element within attention_tolerance, and relative L2 <= rel_l2_max over all
    checked elements.  max_budget_rows: at most this many rows may have an
    element beyond the base bound max(atol, 1 bf16 ulp), i.e. lean on the flip
    budget of their near-tie decisions (0: none may)."""
    r, tol = attention_tolerance(ref, atol)
    g = oracle.bf16_to_f64(gpu_bits).reshape(r.shape)
    diff = np.abs(g - r)
    base = np.maximum(atol, bf16_ulp(r))
    bad = np.any(diff > tol, axis=1)
    rel = float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))
    info = dict(max_abs=float(diff.max()), rel_l2=rel, worst_over_tol=float((diff / tol).max()),
                flagged_rows=int(np.sum(ref["near_tie"])),
                rows_using_budget=int(np.sum(np.any(diff > base, axis=1))),
                bad_rows=[int(i) for i in np.where(bad)[0][:10]])
    print(what, info)
    assert not bad.any(), f"{what}: elements beyond tolerance: {info}"
    assert rel <= rel_l2_max, f"{what}: relative L2 {rel} > {rel_l2_max}"
    if max_budget_rows is not None:
        assert info["rows_using_budget"] <= max_budget_rows, f"{what}: rows needing their flip budget: {info}"
    return info
