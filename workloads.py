"""Seeded synthetic inputs for the MXFP4 attention path.

This module holds no arithmetic of the method: only seeded random draws and
the rounding of the drawn fp32 values to bf16 (the input format).  Both the
GPU tests/benchmark and the CPU oracle take their inputs from here.

Workloads (shapes and value structure stand in for the video diffusion
models the MXAttention abstract evaluates on, Wan2.2 and HunyuanVideo; no
weights, prompts or videos from those models are used or needed):

  tiny     B=1, H=1,  N=256,   d=64   Q, K, V ~ N(0, 1)
  small    B=1, H=8,  N=4096,  d=128  Q, K ~ N(0, 1) with 4 outlier channels per
                                      head (the same 4 for Q and K) scaled x20;
                                      V ~ N(0, 1)
  wan      B=1, H=40, N=32760, d=128  Student-t(4) per element times a
                                      LogNormal(0, 1) scale drawn per
                                      (tensor, head, channel); N = 21 x 1560
  hunyuan  B=1, H=24, N=65536, d=128  N(0, 1) with one set of floor(0.01 N)
                                      token indices, shared by Q, K, V and all
                                      heads, scaled x10
  sweep    2^p elements, x = s * 2^U, U ~ Uniform(-20, 10), s = +-1
  gemm     X [32760][5120] (Wan-style tokens x hidden: Student-t(4) times a
           LogNormal(0, 1) scale per channel), W [13824][5120] (an FFN
           up-projection) ~ N(0, 0.02^2); both bf16
  wan_varlen a varlen batch of four Wan-style videos of 21, 13, 5 and 1
           latent frames (1560 tokens each: N = 32760, 20280, 7800, 1560,
           T = 62400 packed tokens), H=40, d=128, the Wan value distribution
           per (sequence, head)
  tie_case structured Q/K (and a chosen softmax scale) that put one
           exponential in eight on an E2M1 rounding tie; V ~ N(0, 1)

Every head of every tensor has its own seed stream, so a single head can be
regenerated without drawing the rest (the oracle checks sampled rows of the
large workloads head by head).
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor
import os

import numpy as np

CONFIGS = {
    "tiny": dict(B=1, H=1, N=256, d=64, seed=0),
    "small": dict(B=1, H=8, N=4096, d=128, seed=1),
    "wan": dict(B=1, H=40, N=32760, d=128, seed=2),
    "hunyuan": dict(B=1, H=24, N=65536, d=128, seed=3),
}
_CFG_ID = {"tiny": 0, "small": 1, "wan": 2, "hunyuan": 3, "custom": 4}
_TENSOR_ID = {"q": 0, "k": 1, "v": 2}


def f32_to_bf16(x) -> np.ndarray:
    """Round fp32 values to bf16 bit patterns (round-to-nearest-even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits) -> np.ndarray:
    return (np.ascontiguousarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _rng(*key) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(x) for x in key]))


def outlier_channels(name: str, seed: int, b: int, h: int, d: int) -> np.ndarray:
    """The 4 outlier channels of head (b, h) for the 'small' workload."""
    return _rng(seed, _CFG_ID[name], 10, b, h).choice(d, size=4, replace=False)


def heavy_tokens(name: str, seed: int, N: int) -> np.ndarray:
    """The shared heavy-token indices of the 'hunyuan' workload."""
    return np.sort(_rng(seed, _CFG_ID[name], 11).choice(N, size=(N // 100), replace=False))


def head(name: str, tensor: str, b: int, h: int, seed: int | None = None, N: int | None = None,
         d: int | None = None) -> np.ndarray:
    """One head of Q, K or V as bf16 bit patterns, shape [N, d]."""
    cfg = CONFIGS.get(name, {})
    seed = cfg["seed"] if seed is None else seed
    N = cfg["N"] if N is None else N
    d = cfg["d"] if d is None else d
    dist = name if name in CONFIGS else "tiny"
    g = _rng(seed, _CFG_ID.get(name, 4), _TENSOR_ID[tensor], b, h, N, d)
    if dist in ("tiny",):
        x = g.standard_normal((N, d), dtype=np.float32)
    elif dist == "small":
        x = g.standard_normal((N, d), dtype=np.float32)
        if tensor in ("q", "k"):
            x[:, outlier_channels(name, seed, b, h, d)] *= 20.0
    elif dist == "wan":
        chan = np.exp(g.standard_normal(d)).astype(np.float32)
        x = g.standard_t(4.0, size=(N, d)).astype(np.float32) * chan[None, :]
    elif dist == "hunyuan":
        x = g.standard_normal((N, d), dtype=np.float32)
        x[heavy_tokens(name, seed, N), :] *= 10.0
    else:
        raise ValueError(name)
    return f32_to_bf16(x)


def qkv(name: str, seed: int | None = None, B: int | None = None, H: int | None = None,
        N: int | None = None, d: int | None = None, threads: int | None = None):
    """Q, K, V as bf16 bit patterns, each [B, H, N, d] (uint16)."""
    cfg = CONFIGS.get(name, {})
    B = cfg["B"] if B is None else B
    H = cfg["H"] if H is None else H
    N = cfg["N"] if N is None else N
    d = cfg["d"] if d is None else d
    out = {t: np.empty((B, H, N, d), np.uint16) for t in ("q", "k", "v")}
    jobs = [(t, b, h) for t in ("q", "k", "v") for b in range(B) for h in range(H)]

    def fill(job):
        t, b, h = job
        out[t][b, h] = head(name, t, b, h, seed=seed, N=N, d=d)

    nt = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(fill, jobs))
    return out["q"], out["k"], out["v"]


def sweep(p: int, seed: int = 4, chunk_log2: int = 24) -> np.ndarray:
    """2^p bf16 values, log-uniform magnitudes over 2^-20..2^10, random sign."""
    n = 1 << p
    out = np.empty(n, np.uint16)
    csz = min(n, 1 << chunk_log2)

    def fill(ci):
        g = _rng(seed, 5, p, ci)
        u = g.random(csz, dtype=np.float32) * 30.0 - 20.0
        s = np.where(g.random(csz, dtype=np.float32) < 0.5, -1.0, 1.0).astype(np.float32)
        out[ci * csz:(ci + 1) * csz] = f32_to_bf16(s * np.exp2(u))

    with ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        list(ex.map(fill, range(n // csz)))
    return out


def sample_rows(BH: int, N: int, count: int = 512, seed: int = 7) -> np.ndarray:
    """Seeded flat query-row indices in [0, BH*N), sorted, without repeats.

    Always includes the first and last query row so the ragged query tail is
    covered."""
    g = _rng(seed, 6, BH, N)
    count = min(count, BH * N)
    rows = set(g.choice(BH * N, size=count, replace=False).tolist())
    rows |= {0, BH * N - 1}
    return np.array(sorted(rows), dtype=np.int64)


def tie_case(N: int = 256, d: int = 64, seed: int = 9):
    """Inputs with one exponential in eight on an E2M1 tie.  Every query is
    the unit vector e_0; key j has 1.0 in channel 0 when j % 64 == 0, 0.5
    when j % 8 == 4, and 0 otherwise, so s is 1, 0.5 or 0 (exact in MXFP4).
    With softmax scale -2 ln(0.3125), the keys with s = 0.5 get
    p = exp(-0.5 * scale) = 0.3125 up to the fp32 roundings: in a block that
    holds a maximal key (amax 1, e = -2) that is y = 1.25, the tie between 1
    and 1.5; in a block without one (amax 0.3125, e = -4) it is y = 5, the tie
    between 4 and 6.  The keys with s = 0 get p = 0.3125^2, y = 0.39 or 1.56,
    well away from any tie."""
    q = np.zeros((N, d), np.float32)
    q[:, 0] = 1.0
    k = np.zeros((N, d), np.float32)
    j = np.arange(N)
    k[:, 0] = np.where(j % 64 == 0, 1.0, np.where(j % 8 == 4, 0.5, 0.0))
    v = np.random.default_rng(seed).standard_normal((N, d)).astype(np.float32)
    scale = float(-2.0 * np.log(0.3125))
    return f32_to_bf16(q), f32_to_bf16(k), f32_to_bf16(v), scale


VARLEN_CONFIGS = {
    "wan_varlen": dict(lengths=(32760, 20280, 7800, 1560), H=40, d=128, seed=6, dist="wan"),
}


def varlen_qkv(lengths, H: int, d: int, seed: int, dist: str = "wan", threads: int | None = None):
    """Q, K, V of a varlen batch as bf16 bit patterns packed [T][H][d], plus
    cu_seqlens (int32, len(lengths) + 1).  Sequence s, head h draws like head
    (b = s, h) of the named distribution at N = lengths[s]."""
    lengths = [int(n) for n in lengths]
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    T = int(cu[-1])
    out = {t: np.empty((T, H, d), np.uint16) for t in ("q", "k", "v")}
    jobs = [(t, s, h) for t in ("q", "k", "v") for s in range(len(lengths)) for h in range(H) if lengths[s] > 0]

    def fill(job):
        t, s, h = job
        out[t][cu[s]:cu[s + 1], h] = head(dist, t, s, h, seed=seed, N=lengths[s], d=d)

    nt = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(fill, jobs))
    return out["q"], out["k"], out["v"], cu


GEMM_CONFIGS = {
    "gemm": dict(M=32760, N=13824, K=5120, seed=5),
}


def gemm_inputs(name: str = "gemm", M: int | None = None, N: int | None = None, K: int | None = None,
                seed: int | None = None, threads: int | None = None):
    """X [M][K] and W [N][K] as bf16 bit patterns.  X rows are tokens with a
    per-channel LogNormal(0, 1) scale on Student-t(4) entries; W ~ N(0, 0.02^2).
    Rows are drawn in chunks with their own seed streams, so any row range
    can be regenerated alone."""
    cfg = GEMM_CONFIGS.get(name, {})
    M = cfg["M"] if M is None else M
    N = cfg["N"] if N is None else N
    K = cfg["K"] if K is None else K
    seed = cfg.get("seed", 5) if seed is None else seed
    chan = np.exp(_rng(seed, 20, K).standard_normal(K)).astype(np.float32)
    x = np.empty((M, K), np.uint16)
    w = np.empty((N, K), np.uint16)
    rows = 1024

    def fill_x(ci):
        g = _rng(seed, 21, M, K, ci)
        r0, r1 = ci * rows, min(M, (ci + 1) * rows)
        x[r0:r1] = f32_to_bf16(g.standard_t(4.0, size=(r1 - r0, K)).astype(np.float32) * chan[None, :])

    def fill_w(ci):
        g = _rng(seed, 22, N, K, ci)
        r0, r1 = ci * rows, min(N, (ci + 1) * rows)
        w[r0:r1] = f32_to_bf16(g.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(0.02))

    nt = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=nt) as ex:
        list(ex.map(fill_x, range((M + rows - 1) // rows)))
        list(ex.map(fill_w, range((N + rows - 1) // rows)))
    return x, w
