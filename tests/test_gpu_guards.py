"""Guard bytes around every buffer the kernels write.

Each output (O, the workspace, codes and scales, the GEMM's Y and the QKV
projection's five outputs) sits inside a larger allocation whose head and
tail (4 KiB each) are filled with a fixed pattern before the call; after the
call the pattern must be intact, so no kernel writes past either end of what
the header says it owns.  The workspace is given exactly the size the
library asks for.  Shapes cover ragged N (1, 33, 32760, 262143), varlen
batches with empty sequences and with 1000 short sequences (and tokens
outside every sequence, which must keep the pattern too), strided BNHD views,
the QKV-projection epilogue and the GEMM.  The calls go straight through the
C ABI with pointers into the guarded allocations.
"""
import ctypes

import numpy as np
import pytest

import workloads
from gpu_helpers import HAVE_GPU, to_gpu_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx

GUARD = 4096
PATTERN = 0xA5


class Guarded:
    """nbytes of device memory (16-byte aligned) between two guard zones."""

    def __init__(self, nbytes):
        self.n = int(nbytes)
        self.buf = torch.full((GUARD + self.n + GUARD,), PATTERN, dtype=torch.uint8, device="cuda:0")
        self.body = self.buf[GUARD:GUARD + self.n]

    @property
    def ptr(self):
        return self.body.data_ptr()

    def as_bf16(self, *shape):
        return self.body.view(torch.bfloat16).view(*shape)

    def check(self, what):
        torch.cuda.synchronize()
        head = self.buf[:GUARD].cpu().numpy()
        tail = self.buf[GUARD + self.n:].cpu().numpy()
        assert np.all(head == PATTERN), f"{what}: {np.count_nonzero(head != PATTERN)} guard bytes before it changed"
        assert np.all(tail == PATTERN), f"{what}: {np.count_nonzero(tail != PATTERN)} guard bytes after it changed"


def stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def rand_bits(shape, seed, scale=1.5):
    g = np.random.default_rng(seed)
    return workloads.f32_to_bf16((g.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("N,d", [(1, 128), (33, 64), (32760, 128), (262143, 64)])
def test_fwd_output_and_workspace(N, d):
    B, H = 1, 2 if N < 100000 else 1
    q, k, v = (to_gpu_bf16(rand_bits((B, H, N, d), seed=N + i)) for i in range(3))
    o = Guarded(B * H * N * d * 2)
    ws = Guarded(mx.workspace_bytes(B, H, N, d))
    st = mx.lib().mxattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, 1, 1, 0.0, o.ptr, ws.ptr, ws.n,
                             stream())
    assert st == 0, mx.status_string(st)
    o.check(f"O N={N}")
    ws.check(f"workspace N={N}")
    ref = mx.fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o.as_bf16(B, H, N, d).view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("shape", [(3, 1000, 700), (1, 33, 128), (2, 257, 65), (1, 32760, 128)])
@pytest.mark.parametrize("axis", [0, 1])
def test_quantize_codes_and_scales(shape, axis):
    batch, rows, cols = shape
    x = to_gpu_bf16(rand_bits(shape, seed=rows * cols, scale=30.0))
    nvec, L = (rows, cols) if axis == 1 else (cols, rows)
    nb = (L + 31) // 32
    c, s = Guarded(batch * nvec * nb * 16), Guarded(batch * nvec * nb)
    st = mx.lib().mxq_quantize(x.data_ptr(), batch, rows, cols, axis, 1, c.ptr, s.ptr, stream())
    assert st == 0, mx.status_string(st)
    c.check(f"codes {shape} axis {axis}")
    s.check(f"scales {shape} axis {axis}")
    rc, rs = mx.quantize(x, mode="uos", axis=axis)
    torch.cuda.synchronize()
    assert torch.equal(c.body, rc.view(-1)) and torch.equal(s.body, rs.view(-1))


@pytest.mark.parametrize("lengths", [[0, 5, 0, 200, 0], [1 + (i * 37) % 50 for i in range(1000)]],
                         ids=["empties", "1000-short"])
def test_varlen_output_workspace_and_untouched_tokens(lengths):
    H, d = 2, 64
    q, k, v, cu = workloads.varlen_qkv(lengths, H, d, seed=len(lengths))
    T = q.shape[0]
    pad = 7  # tokens after the last sequence: outside every sequence
    Tp = T + pad
    qg, kg, vg = (to_gpu_bf16(np.concatenate([x, np.zeros((pad, H, d), np.uint16)])) for x in (q, k, v))
    cug = torch.from_numpy(cu.astype(np.int32)).to("cuda:0")
    o = Guarded(Tp * H * d * 2)
    ws = Guarded(mx.varlen_workspace_bytes(len(lengths), Tp, H, d))
    st = mx.lib().mxattn_fwd_varlen(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.ptr, cug.data_ptr(),
                                    len(lengths), Tp, H, d, None, 1, 1, 0.0, ws.ptr, ws.n, stream())
    assert st == 0, mx.status_string(st)
    o.check("varlen O")
    ws.check("varlen workspace")
    rows = o.body.view(Tp, H * d * 2).cpu().numpy()
    assert np.all(rows[T:] == PATTERN), "tokens outside every sequence were written"
    ref = mx.fwd_varlen(qg, kg, vg, cug)
    torch.cuda.synchronize()
    assert torch.equal(o.as_bf16(Tp, H, d)[:T].view(torch.int16), ref[:T].view(torch.int16))


def test_strided_bnhd_output():
    B, H, N, d = 2, 3, 1000, 128
    q, k, v = (to_gpu_bf16(rand_bits((B, N, H, d), seed=40 + i)).transpose(1, 2) for i in range(3))
    o = Guarded(B * N * H * d * 2)
    ov = o.as_bf16(B, N, H, d).transpose(1, 2)
    ws = Guarded(mx.workspace_bytes(B, H, N, d))
    s3 = lambda t: (ctypes.c_int64 * 3)(*t.stride()[:3])
    st = mx.lib().mxattn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), ov.data_ptr(), B, H, N, d, s3(q),
                                     s3(k), s3(v), s3(ov), 1, 1, 0.0, ws.ptr, ws.n, stream())
    assert st == 0, mx.status_string(st)
    o.check("strided O")
    ws.check("strided workspace")
    ref = mx.fwd(q.contiguous(), k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    assert torch.equal(ov.contiguous().view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("T,C,H,d", [(300, 256, 3, 64), (513, 640, 4, 128), (33, 256, 8, 64)])
def test_qkv_projection_outputs(T, C, H, d):
    x, w = workloads.gemm_inputs(M=T, N=3 * H * d, K=C, seed=T + C)
    xg, wg = to_gpu_bf16(x), to_gpu_bf16(w)
    xc, xs = mx.quantize(xg.view(1, T, C), axis=1)
    wc, wsc = mx.quantize(wg.view(1, 3 * H * d, C), axis=1)
    nbm = (T + 31) // 32
    outs = [Guarded(H * T * d * 2), Guarded(H * T * d // 2), Guarded(H * T * d // 32), Guarded(H * d * nbm * 16),
            Guarded(H * d * nbm)]
    st = mx.lib().mxqkv_proj_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), wsc.data_ptr(), T, C, H, d, 1,
                                       *(g.ptr for g in outs), stream())
    assert st == 0, mx.status_string(st)
    for g, name in zip(outs, ("q", "kc", "ks", "vc", "vs")):
        g.check(f"QKV {name} {(T, C, H, d)}")
    ref = mx.qkv_proj_quantized(xc, xs, wc, wsc, T, C, H, d)
    torch.cuda.synchronize()
    for g, r in zip(outs, ref):
        assert torch.equal(g.body, r.contiguous().view(-1).view(torch.uint8))


@pytest.mark.parametrize("M,N,K", [(1, 4, 128), (300, 260, 384), (1000, 516, 256)])
def test_gemm_output(M, N, K):
    x, w = workloads.gemm_inputs(M=M, N=N, K=K, seed=M + N)
    xc, xs = mx.quantize(to_gpu_bf16(x).view(1, M, K), axis=1)
    wc, wsc = mx.quantize(to_gpu_bf16(w).view(1, N, K), axis=1)
    y = Guarded(M * N * 2)
    st = mx.lib().mxgemm_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), wsc.data_ptr(), M, N, K, y.ptr,
                                   stream())
    assert st == 0, mx.status_string(st)
    y.check(f"GEMM Y {(M, N, K)}")
    ref = mx.gemm_quantized(xc, xs, wc, wsc, M, N, K)
    torch.cuda.synchronize()
    assert torch.equal(y.as_bf16(M, N).view(torch.int16), ref.view(torch.int16))


def test_binding_rejects_bad_outputs_on_gpu():
    """The binding's own checks with real device tensors: wrong output shape,
    dtype or device, a short quantized operand, and mxq_dump with codes on
    the device and scales on the host."""
    B, H, N, d = 1, 2, 64, 128
    q, k, v = (to_gpu_bf16(rand_bits((B, H, N, d), seed=i)) for i in range(3))
    with pytest.raises(ValueError, match="shape"):
        mx.fwd(q, k, v, out=torch.empty((B, H, N - 1, d), dtype=torch.bfloat16, device="cuda:0"))
    with pytest.raises(TypeError, match="bfloat16"):
        mx.fwd(q, k, v, out=torch.empty((B, H, N, d), dtype=torch.float16, device="cuda:0"))
    with pytest.raises(TypeError, match="CUDA"):
        mx.fwd(q, k, v, out=torch.empty((B, H, N, d), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="contiguous"):
        mx.fwd(q, k, v, out=torch.empty((B, N, H, d), dtype=torch.bfloat16, device="cuda:0").transpose(1, 2))
    kc, ks = mx.quantize(k.view(B * H, N, d), axis=1)
    vc, vs = mx.quantize(v.view(B * H, N, d), axis=0)
    with pytest.raises(ValueError, match="needs"):
        mx.fwd_kv_quantized(q, kc.view(-1)[:-1], ks, vc, vs)
    with pytest.raises(TypeError, match="CUDA"):
        mx.fwd_kv_quantized(q, kc.cpu(), ks, vc, vs)
    with pytest.raises(ValueError, match="same memory"):
        mx.dump("/tmp/never-written.mxq", kc, ks.cpu(), B * H, N, d, 1)
    torch.cuda.synchronize()
    host_scales = ks.cpu().numpy()
    st = mx.lib().mxq_dump(b"/tmp/never-written.mxq", kc.data_ptr(), host_scales.ctypes.data, B * H, N, d, 1, 1,
                           None)
    assert st == -1  # MXQ_ERR_INVALID_ARG: one device and one host pointer
