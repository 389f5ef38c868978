"""CPU oracle for MXFP4 attention with UOS and PNQ -- TEST INFRASTRUCTURE.

This package wraps ``mxoracle.c``, a plain and slow C implementation of
what the MXAttention path computes (MXAttention: Data-Free Optimal Scaling
and Pre-Normalization Quantization for MXFP4 Attention, abstract).  Only the
test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import it.  It shares no code with the HIP library and never
imports it; the HIP library never calls it.

All arrays cross the boundary as numpy arrays: bf16 tensors as ``uint16``
bit patterns, codes and scales as ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

MODE_OCP = 0
MODE_UOS = 1
MODE_NONE = 2  # identity quantizer, pins only

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mxoracle.c")
_LIB = os.path.join(_HERE, "libmxoracle.so")
# An alternative build of the same source (the sanitizer test points this at
# an AddressSanitizer/UBSan build); the default is the library build() makes.
_LIB_OVERRIDE = os.environ.get("MXORACLE_LIB")
_lib = None


GCC_FLAGS = ["-std=c99", "-D_GNU_SOURCE", "-fopenmp", "-ffp-contract=off", "-Wall", "-shared", "-fPIC"]
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(force: bool = True, out: str | None = None, sanitize: bool = False) -> str:
    """Compile the oracle with gcc (strict IEEE: no fast-math, no FMA
    contraction).  sanitize=True builds the same source with AddressSanitizer
    and UBSan (every report fatal) into `out` instead, for the sanitizer test."""
    target = out or _LIB
    if force or not os.path.exists(target):
        tmp = target + ".tmp%d" % os.getpid()
        opt = SANITIZE_FLAGS if sanitize else ["-O2"]
        cmd = ["gcc", *opt, *GCC_FLAGS, _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, target)
    return target


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if _LIB_OVERRIDE:
        lib = ctypes.CDLL(_LIB_OVERRIDE)
    else:
        if not os.path.exists(_LIB):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
    P = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int
    lib.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
    lib.orc_bf16_to_double.restype = ctypes.c_double
    lib.orc_double_to_bf16.argtypes = [ctypes.c_double]
    lib.orc_double_to_bf16.restype = ctypes.c_uint16
    lib.orc_double_to_bf16_array.argtypes = [P, i64, P]
    lib.orc_double_to_bf16_array.restype = None
    lib.orc_e2m1_encode.argtypes = [ctypes.c_double]
    lib.orc_e2m1_encode.restype = i32
    lib.orc_e2m1_value.argtypes = [i32, i32]
    lib.orc_e2m1_value.restype = ctypes.c_double
    lib.orc_block_exponent.argtypes = [ctypes.c_double, i32]
    lib.orc_block_exponent.restype = i32
    lib.orc_e2m1_encode_array.argtypes = [P, i64, P]
    lib.orc_e2m1_encode_array.restype = None
    lib.orc_block_exponent_array.argtypes = [P, i64, i32, P]
    lib.orc_block_exponent_array.restype = None
    lib.orc_quantize_bf16.argtypes = [P, i64, i64, i64, i32, i32, P, P]
    lib.orc_quantize_bf16.restype = i32
    lib.orc_quantize_f64.argtypes = [P, i64, i32, P, P]
    lib.orc_quantize_f64.restype = i32
    lib.orc_dequantize.argtypes = [P, P, i64, i64, P]
    lib.orc_dequantize.restype = None
    lib.orc_block_sse.argtypes = [P, i64, i32]
    lib.orc_block_sse.restype = ctypes.c_double
    lib.orc_block_sse_batch.argtypes = [P, i64, i64, i32, i32, P]
    lib.orc_block_sse_batch.restype = None
    lib.orc_attn_rows.argtypes = [P, P, P, i64, i64, i64, i32, i32, i64, ctypes.c_double,
                                  P, i64, P, P, P, P, P]
    lib.orc_attn_rows.restype = i32
    lib.orc_dump.argtypes = [ctypes.c_char_p, P, P, i64, i64, i64, i32, i32]
    lib.orc_dump.restype = i32
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = i32
    lib.orc_set_num_threads.argtypes = [i32]
    lib.orc_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray | None):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    """OpenMP threads the oracle's row loop runs on."""
    return int(_load().orc_num_threads())


def set_num_threads(n: int) -> None:
    """OpenMP threads for later calls (for timing the oracle on fewer cores)."""
    _load().orc_set_num_threads(int(n))


def bf16_to_f64(bits) -> np.ndarray:
    b = _c(bits, np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(x) -> np.ndarray:
    """Round fp64 values to bf16 bit patterns, round-to-nearest-even."""
    x = _c(x, np.float64)
    out = np.empty(x.shape, np.uint16)
    _load().orc_double_to_bf16_array(_ptr(x), x.size, _ptr(out))
    return out


def e2m1_encode(y: float) -> int:
    return int(_load().orc_e2m1_encode(float(y)))


def e2m1_value(code: int, e: int) -> float:
    return float(_load().orc_e2m1_value(int(code), int(e)))


def block_exponent(amax: float, mode: int) -> int:
    return int(_load().orc_block_exponent(float(amax), int(mode)))


def e2m1_encode_array(y) -> np.ndarray:
    y = _c(y, np.float64).reshape(-1)
    out = np.empty(y.size, np.uint8)
    _load().orc_e2m1_encode_array(_ptr(y), y.size, _ptr(out))
    return out


def block_exponent_array(amax, mode: int) -> np.ndarray:
    a = _c(amax, np.float64).reshape(-1)
    out = np.empty(a.size, np.int32)
    _load().orc_block_exponent_array(_ptr(a), a.size, int(mode), _ptr(out))
    return out


def n_blocks(L: int) -> int:
    return (L + 31) // 32


def quantize_bf16(x_bits, batch: int, rows: int, cols: int, axis: int, mode: int):
    """Canonical MXFP4 quantization of a bf16 tensor [batch][rows][cols].

    Returns (codes, scales) as flat uint8 arrays in the canonical layout:
    axis 1 -> codes [batch][rows][nb*16], axis 0 -> codes [batch][cols][nb*16].
    """
    x = _c(x_bits, np.uint16).reshape(-1)
    assert x.size == batch * rows * cols
    nvec, L = (rows, cols) if axis == 1 else (cols, rows)
    nb = n_blocks(L)
    codes = np.zeros(batch * nvec * nb * 16, np.uint8)
    scales = np.zeros(batch * nvec * nb, np.uint8)
    rc = _load().orc_quantize_bf16(_ptr(x), batch, rows, cols, axis, mode, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    return codes, scales


def quantize_f64(x, mode: int):
    x = _c(x, np.float64).reshape(-1)
    nb = n_blocks(x.size)
    codes = np.zeros(nb * 16, np.uint8)
    scales = np.zeros(nb, np.uint8)
    rc = _load().orc_quantize_f64(_ptr(x), x.size, mode, _ptr(codes), _ptr(scales))
    if rc != 0:
        raise ValueError("oracle quantize rejected its arguments")
    return codes, scales


def dequantize(codes, scales, nvec: int, L: int) -> np.ndarray:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    assert codes.size == nvec * n_blocks(L) * 16 and scales.size == nvec * n_blocks(L)
    out = np.empty(nvec * L, np.float64)
    _load().orc_dequantize(_ptr(codes), _ptr(scales), nvec, L, _ptr(out))
    return out.reshape(nvec, L)


def block_sse(x, e: int) -> float:
    x = _c(x, np.float64).reshape(-1)
    return float(_load().orc_block_sse(_ptr(x), x.size, int(e)))


def block_sse_batch(blocks, e0: int, ne: int) -> np.ndarray:
    """blocks: [nblk, n] fp64 -> sse [nblk, ne] at exponents e0..e0+ne-1."""
    blocks = _c(blocks, np.float64)
    nblk, n = blocks.shape
    sse = np.empty((nblk, ne), np.float64)
    _load().orc_block_sse_batch(_ptr(blocks), nblk, n, int(e0), int(ne), _ptr(sse))
    return sse


def attn_rows(q, k, v, BH: int, N: int, d: int, mode: int, pnq: bool, Bc: int,
              softmax_scale: float, rows, want_weights: bool = False, want_budget: bool = True):
    """Oracle attention for the query rows ``rows`` (flat indices into [BH*N]).

    q, k, v: bf16 bit patterns, [BH][N][d].  Returns a dict with
    ``out`` [nrows, d] fp64, ``out_bf16`` [nrows, d] uint16, ``l`` [nrows],
    ``near_tie`` [nrows] bool, ``budget`` [nrows, d] (the bound on |dO| when
    every flagged decision of the row goes the other way; see orc_attn_rows)
    and, if asked, ``weights`` [nrows, N].
    """
    q = _c(q, np.uint16).reshape(-1)
    k = _c(k, np.uint16).reshape(-1)
    v = _c(v, np.uint16).reshape(-1)
    assert q.size == BH * N * d and k.size == q.size and v.size == q.size
    rows = _c(rows, np.int64).reshape(-1)
    nr = rows.size
    out = np.empty((nr, d), np.float64)
    lsum = np.empty(nr, np.float64)
    flags = np.zeros(nr, np.int32)
    weights = np.empty((nr, N), np.float64) if want_weights else None
    budget = np.zeros((nr, d), np.float64) if want_budget else None
    rc = _load().orc_attn_rows(_ptr(q), _ptr(k), _ptr(v), BH, N, d, int(mode), int(bool(pnq)),
                               int(Bc), float(softmax_scale), _ptr(rows), nr, _ptr(out),
                               _ptr(lsum), _ptr(flags), _ptr(weights), _ptr(budget))
    if rc != 0:
        raise ValueError("oracle attention rejected its arguments")
    res = {"out": out, "out_bf16": f64_to_bf16(out), "l": lsum, "near_tie": flags != 0}
    if want_weights:
        res["weights"] = weights
    if want_budget:
        res["budget"] = budget
    return res


def attn_varlen_rows(q, k, v, cu_seqlens, H: int, d: int, mode: int, pnq: bool, Bc: int,
                     softmax_scale: float, rows, want_budget: bool = True):
    """Oracle attention over a varlen batch: q, k, v are bf16 bit patterns
    [T][H][d] (tokens packed along one axis) and sequence s holds tokens
    [cu_seqlens[s], cu_seqlens[s+1]).  Every sequence is its own attention
    problem: a query attends to the keys of its own sequence only, with key
    tiles and 32-key blocks counted from the sequence's first token, which is
    ``attn_rows`` on that sequence's slice.  ``rows`` are (token, head)
    pairs [nrows][2]; each token must lie in some sequence.  Returns the
    ``attn_rows`` dict fields for the rows in the order given."""
    q = _c(q, np.uint16)
    k = _c(k, np.uint16)
    v = _c(v, np.uint16)
    T = q.size // (H * d)
    q, k, v = (a.reshape(T, H, d) for a in (q, k, v))
    cu = np.asarray(cu_seqlens, np.int64)
    rows = np.asarray(rows, np.int64).reshape(-1, 2)
    nr = rows.shape[0]
    out = np.empty((nr, d), np.float64)
    lsum = np.empty(nr, np.float64)
    tie = np.zeros(nr, bool)
    budget = np.zeros((nr, d), np.float64)
    seq = np.searchsorted(cu, rows[:, 0], side="right") - 1
    for s in np.unique(seq):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        assert 0 <= s < cu.size - 1 and t0 < t1
        for h in np.unique(rows[seq == s, 1]):
            sel = np.nonzero((seq == s) & (rows[:, 1] == h))[0]
            part = attn_rows(q[t0:t1, h], k[t0:t1, h], v[t0:t1, h], 1, t1 - t0, d, mode, pnq, Bc,
                             softmax_scale, rows[sel, 0] - t0, want_budget=want_budget)
            out[sel] = part["out"]
            lsum[sel] = part["l"]
            tie[sel] = part["near_tie"]
            if want_budget:
                budget[sel] = part["budget"]
    res = {"out": out, "out_bf16": f64_to_bf16(out), "l": lsum, "near_tie": tie}
    if want_budget:
        res["budget"] = budget
    return res


def gemm_rows(x, w, M: int, N: int, K: int, mode: int, rows=None):
    """Oracle MXFP4 GEMM: Y = X_q W_q^T for the rows ``rows`` of X (all rows if
    None).  x: bf16 bits [M][K], w: bf16 bits [N][K]; both are quantized
    along K with ``mode`` by this oracle's quantizer (MODE_NONE: used as they
    are), dequantized, and multiplied in fp64 (a library matmul; the products
    of dequantized MXFP4 values are exact and fp64 sums of K of them lose
    nothing the acceptance can see).  Returns ``out`` [nr, N] fp64,
    ``out_bf16`` (round to nearest even) and ``absdot`` [nr, N] = |X_q| |W_q|^T,
    the scale of the fp32 accumulation error a GPU may add."""
    x = _c(x, np.uint16).reshape(M, K)
    w = _c(w, np.uint16).reshape(N, K)
    rows = np.arange(M, dtype=np.int64) if rows is None else _c(rows, np.int64).reshape(-1)
    xr = np.ascontiguousarray(x[rows])
    if mode == MODE_NONE:
        xd = bf16_to_f64(xr).reshape(rows.size, K)
        wd = bf16_to_f64(w).reshape(N, K)
    else:
        xcod, xsc = quantize_bf16(xr, 1, rows.size, K, 1, mode)
        wcod, wsc = quantize_bf16(w, 1, N, K, 1, mode)
        xd = dequantize(xcod, xsc, rows.size, K)
        wd = dequantize(wcod, wsc, N, K)
    out = xd @ wd.T
    absdot = np.abs(xd) @ np.abs(wd).T
    return {"out": out, "out_bf16": f64_to_bf16(out), "absdot": absdot}


def dump(path: str, codes, scales, batch: int, nvec: int, L: int, axis: int, mode: int) -> None:
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint8)
    rc = _load().orc_dump(path.encode(), _ptr(codes), _ptr(scales), batch, nvec, L, axis, mode)
    if rc != 0:
        raise OSError("oracle dump failed: %s" % path)
