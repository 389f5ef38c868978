"""The oracle's C source under AddressSanitizer and UBSan.

The same mxoracle.c is built a second time with -fsanitize=address,undefined
(every report fatal) into a scratch directory, and a subprocess runs the
oracle's pins against that build: the hand-worked blocks, the encoder and
scale-rule pins, the closed forms of the attention recurrence, the PNQ and
Q = 0 invariants, the varlen composition and the GEMM pins.  An out-of-bounds
access, use after free or undefined operation anywhere on those paths ends the
subprocess with a sanitizer report, which fails this test.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PINS = [
    "tests/test_oracle_quant.py::test_worked_blocks",
    "tests/test_oracle_quant.py::test_e2m1_encoder_ties_and_neighbours",
    "tests/test_oracle_quant.py::test_scale_rule_clamps",
    "tests/test_oracle_quant.py::test_layout_and_padding_axis0",
    "tests/test_oracle_quant.py::test_axis0_is_axis1_of_transpose",
    "tests/test_oracle_quant.py::test_oracle_dump_format",
    "tests/test_oracle_attn.py::test_recurrence_equals_closed_form",
    "tests/test_oracle_attn.py::test_identity_quantizer_is_textbook_attention",
    "tests/test_oracle_attn.py::test_pnq_v_ones_gives_exact_ones",
    "tests/test_oracle_attn.py::test_q_zero_closed_form",
    "tests/test_oracle_attn.py::test_bad_arguments_rejected",
    "tests/test_oracle_attn.py::test_tie_case_is_flagged_with_a_budget",
    "tests/test_oracle_varlen.py",
    "tests/test_oracle_gemm.py::test_brute_force_from_bytes",
    "tests/test_oracle_gemm.py::test_row_subset_matches_full",
]


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_pins_under_asan_and_ubsan(tmp_path):
    asan, ubsan = _runtime("libasan.so"), _runtime("libubsan.so")
    if asan is None or ubsan is None:
        pytest.skip("gcc sanitizer runtimes not installed")
    lib = oracle.build(force=True, out=str(tmp_path / "libmxoracle_asan.so"), sanitize=True)
    env = dict(os.environ)
    # The uninstrumented interpreter loads the instrumented library, so the
    # sanitizer runtimes are preloaded ahead of anything already listed.
    env["LD_PRELOAD"] = ":".join(p for p in (asan, ubsan, env.get("LD_PRELOAD", "")) if p)
    env["ASAN_OPTIONS"] = "detect_leaks=0:verify_asan_link_order=0:abort_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    env["MXORACLE_LIB"] = lib
    env["OMP_NUM_THREADS"] = "4"
    cmd = [sys.executable, "-m", "pytest", "-q", "-s", "-x", "-p", "no:cacheprovider", "-m", "not gpu", *PINS]
    r = subprocess.run(cmd, cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in out, out[-2000:]
