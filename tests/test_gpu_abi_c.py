"""The C ABI from C: tests/abi_demo.c, built by the package build next to the
library, allocates with the HIP runtime and calls libmxattn.so directly (no
Python, no torch).  It checks that mxattn_fwd equals mxq_quantize followed by
mxattn_fwd_quantized bit for bit, that rejected calls return their documented
status, and that mxq_dump writes the documented file size."""
import os
import subprocess

import pytest

from gpu_helpers import HAVE_GPU

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DEMO = os.path.join(ROOT, "mxfp4_quantized_attention_amd", "_build", "abi_demo")


def test_c_consumer(tmp_path):
    assert os.path.exists(DEMO), "abi_demo is built by __graft_entry__.build()"
    r = subprocess.run([DEMO, str(tmp_path / "v.mxq")], capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert r.stdout.startswith("abi_demo ok")
