"""bench.py's host-side pieces that need no GPU: the oracle baseline on a
configuration small enough to time in full, and the argument clamping that
keeps its sample inside the workload, the vector-unit ceiling read from the
committed probe summary, and the rule that a failed in-run check invalidates
the line."""
import json

import numpy as np
import pytest

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


def test_valu_ceiling_from_the_committed_probe():
    """The ceiling is priced from profiles/attn_valu_probe.json, taken on the
    current probe kernel, and is independent arithmetic on its figures: one
    fma, one exp, half a cvt and half a max3 per score at the probe's cycle
    costs, 1024 SIMDs, 4 d FLOP per score."""
    probe = bench.measured_probe()
    assert probe is not None, "the committed probe summary does not match probe.hip"
    ns = probe["ns_per_wave_instruction"]
    ghz = 2.0
    c = bench.valu_ceilings(128, probe, ghz)
    per_score_ns = (ns["fma"] + ns["exp"] + ns["cvt"] / 2 + ns["max3"] / 2) / 64 * probe["clock_ghz"] / ghz
    assert abs(c["ceiling"] - 4 * 128 * 1024 / per_score_ns * 1e9 / 1e12) < 1e-6 * c["ceiling"]
    assert c["ceiling_mfma_serialized"] < c["ceiling"]
    # the core work alone leaves the 50% target (5050 TFLOP/s) out of reach at
    # any plausible shader clock
    assert bench.valu_ceilings(128, probe, 2.4)["ceiling"] < 0.5 * bench.PEAK_FP4_TFLOPS
    assert abs(bench.valu_ceilings(64, probe, ghz)["ceiling"] * 2 - c["ceiling"]) < 1e-6 * c["ceiling"]


def test_emit_marks_a_failed_check_and_exits(capsys):
    """A bench line whose in-run check failed says so and ends the run with
    status 3; one whose checks held is marked valid."""
    bench.emit({"metric": "m", "value": 1.0}, {"a": True, "b": True})
    line = json.loads(capsys.readouterr().out.strip())
    assert line["valid"] is True and line["checks"] == {"a": True, "b": True}
    with pytest.raises(SystemExit) as e:
        bench.emit({"metric": "m", "value": 1.0}, {"a": True, "b": False})
    assert e.value.code == 3
    line = json.loads(capsys.readouterr().out.strip())
    assert line["valid"] is False and line["checks"]["b"] is False


def test_oracle_sample_agreement_rule():
    ok = {"max_diff_over_bound_unflagged_rows": 0.9, "rel_l2": 2e-4}
    assert bench.oracle_sample_ok(ok)
    assert not bench.oracle_sample_ok(dict(ok, max_diff_over_bound_unflagged_rows=1.01))
    assert not bench.oracle_sample_ok(dict(ok, rel_l2=2e-3))


def test_bench_refuses_more_than_one_gpu():
    """Only one GPU is measured: --gpus 2 exits with status 2 and says so,
    before anything touches a GPU."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=root, capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr
