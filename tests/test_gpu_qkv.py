"""GPU parity of the QKV projection with the attention operand epilogue
(mxqkv_proj_quantized, mxqkv_proj).

The fused kernel must equal the unfused path bit for bit: mxgemm_quantized
to bf16 Y = [Q | K | V], then Q rearranged to [H][T][d], K quantized along d
and V along T with mxq_quantize_strided (which the quantizer tests pin
against the oracle bit for bit, and which a direct oracle check repeats here
on a small shape).  Shapes cover tiles that lie wholly inside Q, K or V
(H*d a multiple of 256, written as whole tiles) and tiles that straddle the
Q/K/V boundaries (written cell by cell), ragged T (partial last V block and partial
last tile), both head dims and both scale rules, and the Wan attention block
(T = 32760, C = 5120, H = 40, d = 128).  End to end, projection plus
mxattn_fwd_kv_quantized equals mxattn_fwd on the bf16 Q, K, V of the unfused
projection.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import HAVE_GPU, to_np_u8, to_np_u16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx

# H*d = 256 or 512 give tiles that lie wholly inside Q, K or V (the whole-tile
# writers); 192 and 320 give tiles that straddle two regions (the cell walk)
SHAPES = [(300, 256, 3, 64), (1000, 512, 2, 128), (257, 128, 5, 64), (64, 384, 1, 128), (513, 640, 4, 128),
          (260, 384, 4, 64), (33, 256, 8, 64)]


def up(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda:0").view(torch.bfloat16)


def _project(T, C, H, d, mode, seed):
    x, w = workloads.gemm_inputs(M=T, N=3 * H * d, K=C, seed=seed)
    xg, wg = up(x), up(w)
    xc, xs = mx.quantize(xg.view(1, T, C), mode=mode, axis=1)
    wc, ws = mx.quantize(wg.view(1, 3 * H * d, C), mode=mode, axis=1)
    return xg, xc, xs, wc, ws


def _unfused(xc, xs, wc, ws, T, C, H, d, mode):
    y = mx.gemm_quantized(xc, xs, wc, ws, T, 3 * H * d, C)  # [T][3 H d] bf16
    HD = H * d
    q = y[:, :HD].reshape(T, H, d).permute(1, 0, 2).contiguous().unsqueeze(0)
    kview = y[:, HD:2 * HD].unflatten(1, (H, d)).permute(1, 0, 2).unsqueeze(0)  # [1, H, T, d] strided
    vview = y[:, 2 * HD:].unflatten(1, (H, d)).permute(1, 0, 2).unsqueeze(0)
    kc, ks = mx.quantize_strided(kview, mode=mode, axis=1)
    vc, vs = mx.quantize_strided(vview, mode=mode, axis=0)
    return y, q, kc, ks, vc, vs


def _same(a, b, what):
    a, b = a.contiguous().view(-1), b.contiguous().view(-1)
    if a.dtype == torch.bfloat16:
        a, b = a.view(torch.int16), b.view(torch.int16)
    if not torch.equal(a, b):
        bad = torch.nonzero(a != b).view(-1)[:8].tolist()
        raise AssertionError(f"{what}: {int((a != b).sum())} of {a.numel()} differ, first at {bad}")


@pytest.mark.parametrize("mode", ["uos", "ocp"])
@pytest.mark.parametrize("T,C,H,d", SHAPES)
def test_fused_equals_unfused(T, C, H, d, mode):
    _, xc, xs, wc, ws = _project(T, C, H, d, mode, seed=T + C + H)
    fused = mx.qkv_proj_quantized(xc, xs, wc, ws, T, C, H, d, mode=mode)
    _, *ref = _unfused(xc, xs, wc, ws, T, C, H, d, mode)
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "kc", "ks", "vc", "vs"), fused, ref):
        _same(a, b, f"{name} T={T} C={C} H={H} d={d} {mode}")


@pytest.mark.parametrize("mode,omode", [("uos", oracle.MODE_UOS), ("ocp", oracle.MODE_OCP)])
@pytest.mark.parametrize("T,C,H,d", [(300, 256, 3, 64), (260, 384, 4, 64)])
def test_fused_codes_match_oracle_quantizer(mode, omode, T, C, H, d):
    _, xc, xs, wc, ws = _project(T, C, H, d, mode, seed=5)
    q, kc, ks, vc, vs = mx.qkv_proj_quantized(xc, xs, wc, ws, T, C, H, d, mode=mode)
    y = mx.gemm_quantized(xc, xs, wc, ws, T, 3 * H * d, C)
    torch.cuda.synchronize()
    yb = to_np_u16(y).reshape(T, 3, H, d)
    kb = np.ascontiguousarray(yb[:, 1].transpose(1, 0, 2))  # [H][T][d]
    vb = np.ascontiguousarray(yb[:, 2].transpose(1, 0, 2))
    okc, oks = oracle.quantize_bf16(kb, H, T, d, 1, omode)
    ovc, ovs = oracle.quantize_bf16(vb, H, T, d, 0, omode)
    assert np.array_equal(to_np_u8(kc), okc) and np.array_equal(to_np_u8(ks), oks)
    assert np.array_equal(to_np_u8(vc), ovc) and np.array_equal(to_np_u8(vs), ovs)
    assert np.array_equal(to_np_u16(q).reshape(H, T, d), np.ascontiguousarray(yb[:, 0].transpose(1, 0, 2)))


def test_bf16_entry_equals_quantized_entry():
    T, C, H, d = 777, 384, 2, 128
    xg, xc, xs, wc, ws = _project(T, C, H, d, "uos", seed=9)
    a = mx.qkv_proj(xg, wc, ws, H, d, mode="uos")
    b = mx.qkv_proj_quantized(xc, xs, wc, ws, T, C, H, d, mode="uos")
    torch.cuda.synchronize()
    for name, u, v in zip(("q", "kc", "ks", "vc", "vs"), a, b):
        _same(u, v, name)


@pytest.mark.parametrize("T,C,H,d", [(1000, 512, 2, 128), (300, 256, 3, 64)])
def test_projection_then_attention_equals_mxattn_fwd(T, C, H, d):
    _, xc, xs, wc, ws = _project(T, C, H, d, "uos", seed=3)
    q, kc, ks, vc, vs = mx.qkv_proj_quantized(xc, xs, wc, ws, T, C, H, d, mode="uos")
    o1 = mx.fwd_kv_quantized(q, kc, ks, vc, vs, mode="uos", pnq=True)
    y = mx.gemm_quantized(xc, xs, wc, ws, T, 3 * H * d, C)
    qkv = [y[:, i * H * d:(i + 1) * H * d].reshape(T, H, d).permute(1, 0, 2).contiguous().unsqueeze(0)
           for i in range(3)]
    o2 = mx.fwd(*qkv, mode="uos", pnq=True)
    torch.cuda.synchronize()
    _same(o1, o2, "attention after the fused projection")


def test_wan_block_shape():
    """The Wan attention block: X [32760][5120], W_qkv [15360][5120]."""
    T, C, H, d = 32760, 5120, 40, 128
    _, xc, xs, wc, ws = _project(T, C, H, d, "uos", seed=21)
    fused = mx.qkv_proj_quantized(xc, xs, wc, ws, T, C, H, d, mode="uos")
    _, *ref = _unfused(xc, xs, wc, ws, T, C, H, d, "uos")
    torch.cuda.synchronize()
    for name, a, b in zip(("q", "kc", "ks", "vc", "vs"), fused, ref):
        _same(a, b, f"{name} wan block")
