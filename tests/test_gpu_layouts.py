"""Strided layouts: mxattn_fwd_strided, mxq_quantize_strided and the torch
custom operator must give exactly what the dense entry points give on dense
copies (the kernels read the same values; only the addressing differs)."""
import numpy as np
import pytest

import workloads
from gpu_helpers import HAVE_GPU

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx


def rand_bf16(shape, seed, scale=1.5):
    g = np.random.default_rng(seed)
    bits = workloads.f32_to_bf16((g.standard_normal(shape) * scale).astype(np.float32))
    return torch.from_numpy(bits.view(np.int16)).to("cuda:0").view(torch.bfloat16)


def same_bits(a, b):
    return torch.equal(a.contiguous().view(torch.int16), b.contiguous().view(torch.int16))


SHAPES = [(2, 3, 1000, 128), (1, 4, 513, 64), (1, 1, 1, 128), (3, 2, 256, 64)]


@pytest.mark.parametrize("B,H,N,d", SHAPES)
@pytest.mark.parametrize("mode,pnq", [("uos", True), ("ocp", False)])
def test_bnhd_equals_dense(B, H, N, d, mode, pnq):
    q, k, v = (rand_bf16((B, N, H, d), seed=i + N) .transpose(1, 2) for i in range(3))
    o = mx.fwd_strided(q, k, v, mode=mode, pnq=pnq)
    assert o.stride() == q.stride()  # O in the caller's BNHD layout
    ref = mx.fwd(q.contiguous(), k.contiguous(), v.contiguous(), mode=mode, pnq=pnq)
    torch.cuda.synchronize()
    assert same_bits(o, ref)


@pytest.mark.parametrize("B,H,N,d,mode,pnq", [(2, 3, 1000, 128, "uos", True), (1, 4, 513, 64, "ocp", False),
                                              (1, 2, 4096, 128, "uos", True)])
def test_bnhd_against_oracle(B, H, N, d, mode, pnq):
    """mxattn_fwd_strided on [B, N, H, d] tensors compared with the oracle
    directly (not only with the dense entry point)."""
    import oracle
    from gpu_helpers import compare_attention, to_np_u16
    g = np.random.default_rng(B * 100 + H * 10 + N + d)
    bnhd = [workloads.f32_to_bf16((g.standard_normal((B, N, H, d)) * 1.5).astype(np.float32)) for _ in range(3)]
    q, k, v = (torch.from_numpy(x.view(np.int16)).to("cuda:0").view(torch.bfloat16).transpose(1, 2) for x in bnhd)
    o = mx.fwd_strided(q, k, v, mode=mode, pnq=pnq)
    torch.cuda.synchronize()
    got = to_np_u16(o).reshape(B * H * N, d)  # .contiguous() gives [B][H][N][d] order
    bhnd = [np.ascontiguousarray(x.transpose(0, 2, 1, 3)) for x in bnhd]
    omode = oracle.MODE_UOS if mode == "uos" else oracle.MODE_OCP
    rows = np.arange(B * H * N) if B * H * N <= 8192 else workloads.sample_rows(B * H, N, 1024)
    ref = oracle.attn_rows(*bhnd, B * H, N, d, omode, pnq, mx.kv_tile(d), 1 / np.sqrt(d), rows)
    compare_attention(got[rows], ref, what=f"BNHD {(B, N, H, d)} {mode} pnq={pnq}")


@pytest.mark.parametrize("B,H,N,d", SHAPES[:2])
def test_packed_qkv_slices(B, H, N, d):
    qkv = rand_bf16((B, N, 3, H, d), seed=5)
    q, k, v = (qkv[:, :, i].transpose(1, 2) for i in range(3))
    o = mx.fwd_strided(q, k, v)
    ref = mx.fwd(q.contiguous(), k.contiguous(), v.contiguous())
    torch.cuda.synchronize()
    assert same_bits(o, ref)


@pytest.mark.parametrize("B,H,N,d", SHAPES)
@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("mode", ["uos", "ocp"])
def test_quantize_strided_equals_dense(B, H, N, d, axis, mode):
    x = rand_bf16((B, N, H, d), seed=7 + N, scale=20.0).transpose(1, 2)
    c1, s1 = mx.quantize_strided(x, mode=mode, axis=axis)
    c2, s2 = mx.quantize(x.contiguous().view(B * H, N, d), mode=mode, axis=axis)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2.view(-1)) and torch.equal(s1, s2.view(-1))


def test_custom_op_matches_binding():
    import mxfp4_quantized_attention_amd.torch_ops  # noqa: F401  registers the operator
    q, k, v = (rand_bf16((2, 300, 4, 128), seed=i).transpose(1, 2) for i in range(3))
    o1 = torch.ops.mxfp4_attn.attention(q, k, v, "uos", True, 0.0)
    o2 = mx.fwd_strided(q, k, v)
    torch.cuda.synchronize()
    assert o1.shape == q.shape and o1.stride() == q.stride()
    assert same_bits(o1, o2)


def test_custom_op_fake_and_compile():
    """The operator's fake implementation agrees with the real one (shape,
    dtype, strides) under torch.library.opcheck, and a torch.compile'd caller
    (aot_eager: graph capture, no code generation) returns the same bits."""
    import mxfp4_quantized_attention_amd.torch_ops  # noqa: F401
    q, k, v = (rand_bf16((1, 130, 2, 64), seed=20 + i).transpose(1, 2) for i in range(3))
    torch.library.opcheck(torch.ops.mxfp4_attn.attention.default, (q, k, v, "uos", True, 0.0),
                          test_utils=("test_schema", "test_faketensor"))

    def f(q, k, v):
        return torch.ops.mxfp4_attn.attention(q, k, v, "ocp", False, 0.0) * 1.0

    o1 = torch.compile(f, backend="aot_eager", fullgraph=True)(q, k, v)
    o2 = mx.fwd_strided(q, k, v, mode="ocp", pnq=False)
    torch.cuda.synchronize()
    assert o1.shape == q.shape and same_bits(o1, o2)
