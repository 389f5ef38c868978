"""The Python binding rejects tensors that the C ABI cannot check.

The C ABI receives raw pointers, so a host tensor or an undersized output
would reach the kernels as a bad address.  Every binding entry point must
raise before it touches the library.  These tests use CPU tensors (no GPU, no
kernel launch) and replace the loaded library with an object that fails the
test if any C function is looked up, which proves that no call reached the
ABI.
"""
import pytest
import torch

import mxfp4_quantized_attention_amd as mx


class _NoCalls:
    def __getattr__(self, name):
        raise AssertionError(f"the binding reached the C ABI ({name}) with invalid tensors")


@pytest.fixture
def no_abi(monkeypatch):
    monkeypatch.setattr(mx, "_lib", _NoCalls())


def bf16(*shape):
    return torch.zeros(shape, dtype=torch.bfloat16)


def u8(n):
    return torch.zeros(n, dtype=torch.uint8)


B, H, N, d = 1, 2, 64, 128
NBN = (N + 31) // 32


def kv_quantized():
    return u8(B * H * N * d // 2), u8(B * H * N * d // 32), u8(B * H * d * NBN * 16), u8(B * H * d * NBN)


CALLS = {
    "quantize": lambda: mx.quantize(bf16(4, 64), axis=1),
    "fwd": lambda: mx.fwd(bf16(B, H, N, d), bf16(B, H, N, d), bf16(B, H, N, d)),
    "fwd_quantized": lambda: mx.fwd_quantized(u8(B * H * N * d // 2), u8(B * H * N * d // 32), *kv_quantized(),
                                              B, H, N, d),
    "fwd_kv_quantized": lambda: mx.fwd_kv_quantized(bf16(B, H, N, d), *kv_quantized()),
    "fwd_strided": lambda: mx.fwd_strided(*(bf16(B, N, H, d).transpose(1, 2) for _ in range(3))),
    "fwd_varlen": lambda: mx.fwd_varlen(bf16(N, H, d), bf16(N, H, d), bf16(N, H, d),
                                        torch.tensor([0, N], dtype=torch.int32)),
    "quantize_strided": lambda: mx.quantize_strided(bf16(B, N, H, d).transpose(1, 2)),
    "gemm_quantized": lambda: mx.gemm_quantized(u8(64 * 64), u8(64 * 4), u8(32 * 64), u8(32 * 4), 64, 32, 128),
    "gemm": lambda: mx.gemm(bf16(64, 128), u8(32 * 64), u8(32 * 4), 32),
    "qkv_proj_quantized": lambda: mx.qkv_proj_quantized(u8(64 * 64), u8(64 * 4), u8(3 * H * d * 64),
                                                        u8(3 * H * d * 4), 64, 128, H, d),
    "qkv_proj": lambda: mx.qkv_proj(bf16(64, 128), u8(3 * H * d * 64), u8(3 * H * d * 4), H, d),
}


@pytest.mark.parametrize("name", sorted(CALLS))
def test_host_tensors_never_reach_the_abi(name, no_abi):
    with pytest.raises(TypeError, match="CUDA"):
        CALLS[name]()


def test_dump_rejects_mixed_or_short_buffers(no_abi, tmp_path):
    path = str(tmp_path / "x.mxq")
    with pytest.raises(ValueError, match="needs"):
        mx.dump(path, u8(15), u8(1), 1, 1, 32, 1)       # one 32-block needs 16 code bytes
    with pytest.raises(ValueError, match="needs"):
        mx.dump(path, u8(32), u8(1), 1, 1, 64, 1)       # two blocks need 2 scale bytes
    with pytest.raises(TypeError):
        mx.dump(path, u8(16).to(torch.int16), u8(1), 1, 1, 32, 1)


def test_quantize_rejects_bad_axis(no_abi):
    with pytest.raises(TypeError):   # host tensor is caught first
        mx.quantize(bf16(4, 64), axis=2)


def test_check_helpers_on_host_tensors():
    """The shape/dtype/size checks themselves (exercised on the GPU by the
    parity tests) reject what they must."""
    with pytest.raises(ValueError, match="needs"):
        mx._u8_operand(u8(10), "kc", 11)
    with pytest.raises(TypeError, match="uint8"):
        mx._u8_operand(bf16(10), "kc", 1)
    with pytest.raises(ValueError, match="contiguous"):
        mx._u8_operand(torch.zeros(4, 4, dtype=torch.uint8).t(), "kc", 1)
    with pytest.raises(TypeError, match="CUDA"):
        mx._check_out(bf16(2, 2), (2, 2), torch.device("cpu"))
    with pytest.raises(TypeError, match="CUDA"):
        mx._on_one_gpu(((bf16(2), "q"),))
