"""The library under HIP graph capture.

Every entry point only enqueues kernels on the caller's stream (no
allocation, no synchronization, no memset), so a whole step can be captured
once and replayed.  The test captures mxattn_fwd (K and V quantization plus
the fused kernel) and the varlen call on a torch CUDA graph, changes the
inputs in place between replays with eager work and synchronizations in
between, and checks every replay against an eager call on the same inputs,
bit for bit.
"""
import numpy as np
import pytest

import workloads
from gpu_helpers import HAVE_GPU, to_gpu_bf16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx


def test_fwd_replays_match_eager():
    B, H, N, d = 1, 4, 1000, 128
    q, k, v = workloads.qkv("tiny", seed=3, B=B, H=H, N=N, d=d)
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    ws = torch.empty(mx.workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(qg)
    mx.fwd(qg, kg, vg, workspace=ws, out=out)  # warm-up outside the capture
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            mx.fwd(qg, kg, vg, workspace=ws, out=out)
    torch.cuda.synchronize()
    g = np.random.default_rng(0)
    for rep in range(4):
        # new inputs in place, eager work and a synchronization between replays
        for t in (qg, kg, vg):
            t.copy_(torch.from_numpy(g.standard_normal(t.shape).astype(np.float32)).to(t.device).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = mx.fwd(qg, kg, vg)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"


def test_varlen_replays_match_eager():
    H, d = 3, 64
    lengths = [100, 0, 257, 31]
    q, k, v, cu = workloads.varlen_qkv(lengths, H, d, seed=4, dist="tiny")
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    cug = torch.from_numpy(cu).to("cuda:0")
    T = int(cu[-1])
    ws = torch.empty(mx.varlen_workspace_bytes(len(lengths), T, H, d), dtype=torch.uint8, device="cuda:0")
    out = torch.empty_like(qg)
    mx.fwd_varlen(qg, kg, vg, cug, workspace=ws, out=out)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            mx.fwd_varlen(qg, kg, vg, cug, workspace=ws, out=out)
    torch.cuda.synchronize()
    g = np.random.default_rng(1)
    for rep in range(4):
        for t in (qg, kg, vg):
            t.copy_(torch.from_numpy(g.standard_normal(t.shape).astype(np.float32)).to(t.device).to(torch.bfloat16))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager = mx.fwd_varlen(qg, kg, vg, cug)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
