"""mxattn_fwd_noalloc, the entry point that allocates nothing, against
mxattn_fwd: bit-identical outputs on two calls in a row (the second smaller,
so it runs on what the first left in the library's array), plus the size
limit and the argument errors it shares with mxattn_fwd.  Calls go through
the C ABI."""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_helpers import HAVE_GPU, to_gpu_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx


def _inputs(B, H, N, d, seed):
    g = np.random.default_rng(seed)
    return [to_gpu_bf16(workloads.f32_to_bf16((g.standard_normal((B, H, N, d)) * 2).astype(np.float32)))
            for _ in range(3)]


def _noalloc(q, k, v, mode, pnq):
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    st = mx.lib().mxattn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, mode, pnq, 0.0,
                                     o.data_ptr(), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, mx.status_string(st)
    return o


@pytest.mark.parametrize("mode,pnq", [(1, 1), (0, 0)])
def test_two_calls_match_mxattn_fwd(mode, pnq):
    gmode = "uos" if mode == 1 else "ocp"
    first = _inputs(1, 8, 4096, 128, seed=11)
    second = _inputs(2, 3, 1000, 64, seed=12)   # smaller: runs over the first call's leftovers
    o1 = _noalloc(*first, mode, pnq)
    o2 = _noalloc(*second, mode, pnq)
    r1 = mx.fwd(*first, mode=gmode, pnq=bool(pnq))
    r2 = mx.fwd(*second, mode=gmode, pnq=bool(pnq))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), r1.view(torch.int16))
    assert torch.equal(o2.view(torch.int16), r2.view(torch.int16))
    # the binding's wrapper goes through the same entry point
    o3 = mx.fwd_noalloc(*second, mode=gmode, pnq=bool(pnq))
    torch.cuda.synchronize()
    assert torch.equal(o3.view(torch.int16), r2.view(torch.int16))


def test_wan_shape_fits_and_matches():
    """The Wan video DiT shape (B=1, H=40, N=32760, d=128) fits the array."""
    B, H, N, d = 1, 40, 32760, 128
    assert mx.workspace_bytes(B, H, N, d) <= mx.noalloc_max_bytes()
    q, k, v = _inputs(B, H, N, d, seed=13)
    o = _noalloc(q, k, v, 1, 1)
    r = mx.fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.view(torch.int16), r.view(torch.int16))


def test_size_limit_and_errors():
    L = mx.lib()
    A = 1 << 20  # never dereferenced: every call below is rejected on the host
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    cap = mx.noalloc_max_bytes()
    assert cap == 256 << 20
    # B*H*N*d past what the array holds: MXQ_ERR_WORKSPACE, nothing enqueued
    N = 65536
    H = 1
    while mx.workspace_bytes(1, H, N, 128) <= cap:
        H *= 2
    assert L.mxattn_fwd_noalloc(A, A, A, 1, H, N, 128, 1, 1, 0.0, A, s) == -3
    assert L.mxattn_fwd_noalloc(A, A, A, 1, 1, 0, 128, 1, 1, 0.0, A, s) == -1    # N < 1
    assert L.mxattn_fwd_noalloc(A, A, A, 1, 1, 64, 96, 1, 1, 0.0, A, s) == -2    # d
    assert L.mxattn_fwd_noalloc(None, A, A, 1, 1, 64, 128, 1, 1, 0.0, A, s) == -1
    assert L.mxattn_fwd_noalloc(A, A, A, 1, 1, 64, 128, 7, 1, 0.0, A, s) == -1   # mode
    assert L.mxattn_fwd_noalloc(A, A, A, 1, H, N, 128, 7, 1, 0.0, A, s) == -1    # mode before size
