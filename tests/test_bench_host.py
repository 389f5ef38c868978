"""bench.py's host-side pieces that need no GPU: the oracle baseline on a
configuration small enough to time in full, and the argument clamping that
keeps its sample inside the workload."""
import numpy as np

import bench
import oracle
import workloads


def _oracle_out(q, k, v, mode, pnq):
    B, H, N, d = q.shape
    rows = np.arange(B * H * N)
    ref = oracle.attn_rows(q.reshape(B * H, N, d), k.reshape(B * H, N, d), v.reshape(B * H, N, d), B * H, N, d,
                           mode, pnq, 128, 1.0 / np.sqrt(d), rows, want_budget=False)
    return ref["out_bf16"].reshape(B, H, N, d)


def test_cpu_baseline_tiny_in_full_agrees_with_itself():
    q, k, v = workloads.qkv("tiny")
    B, H, N, d = q.shape
    out = _oracle_out(q, k, v, oracle.MODE_UOS, 1)
    res = bench.cpu_baseline(q, k, v, "tiny", oracle.MODE_UOS, 1, 128, out, heads=B * H, rows_per_head=N)
    assert res["kind"] == "oracle" and res["cores"] >= 1
    assert res["vs_gpu_on_sample"]["rel_l2"] == 0.0
    assert res["vs_gpu_on_sample"]["max_diff_over_bound_unflagged_rows"] == 0.0
    assert res["extrapolated_full_workload_seconds"] == res["seconds"]  # the sample is the workload
    assert f"{B * H * N} seeded query rows" in res["sample"]


def test_cpu_baseline_clamps_the_default_sample_to_the_workload():
    # the defaults (8 heads, 3072 rows each) exceed tiny's 1 head of 256 tokens
    q, k, v = workloads.qkv("tiny")
    out = _oracle_out(q, k, v, oracle.MODE_OCP, 0)
    res = bench.cpu_baseline(q, k, v, "tiny", oracle.MODE_OCP, 0, 128, out)
    assert "K/V quantization of 1 heads + 256 seeded query rows" in res["sample"]
    assert res["vs_gpu_on_sample"]["rel_l2"] == 0.0


def test_valu_ceiling_is_the_stated_arithmetic():
    # 1024 SIMDs x 64 lanes / (7.05 slots x 1.13 ns) score elements per second,
    # 4 d FLOP each
    assert abs(bench.valu_ceiling_tflops(128) - 4.0 * 128 * 1024 * 64 / (7.05 * 1.13e-9) / 1e12) < 1e-6
    assert abs(bench.valu_ceiling_tflops(64) * 2 - bench.valu_ceiling_tflops(128)) < 1e-6
