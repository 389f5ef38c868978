import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # a sanitizer build of the same sources, loaded in place of the in-tree
    # library by the host-only ABI tests that test_abi_sanitized.py runs
    alt = os.environ.get("MXATTN_TEST_LIB")
    if alt:
        import mxfp4_quantized_attention_amd as mx
        mx.LIB_PATH = alt
