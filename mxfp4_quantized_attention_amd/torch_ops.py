"""A torch custom operator around the C ABI, for use inside model code.

    import mxfp4_quantized_attention_amd.torch_ops
    o = torch.ops.mxfp4_attn.attention(q, k, v, "uos", True, 0.0)

q, k, v: bf16 [B, H, N, d]-shaped CUDA tensors with any strides and
contiguous d (a [B, N, H, d] tensor through .transpose(1, 2) works as it is).
The operator only marshals arguments to mxattn_fwd_strided; every step runs
in the HIP library.  The fake (meta) implementation gives torch.compile the
output's shape, dtype and strides without running anything.
"""
from __future__ import annotations

import torch

from . import fwd_strided


@torch.library.custom_op("mxfp4_attn::attention", mutates_args=(), device_types="cuda")
def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, mode: str = "uos", pnq: bool = True,
              softmax_scale: float = 0.0) -> torch.Tensor:
    return fwd_strided(q, k, v, mode=mode, pnq=pnq, softmax_scale=softmax_scale)


@attention.register_fake
def _attention_fake(q, k, v, mode="uos", pnq=True, softmax_scale=0.0):
    out = torch.empty_like(q)
    return out if out.stride(3) == 1 else torch.empty(q.shape, dtype=q.dtype, device=q.device)
