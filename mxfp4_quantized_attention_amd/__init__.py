"""MXFP4 attention with UOS and PNQ on AMD MI355X (gfx950).

Thin Python binding of ``libmxattn.so`` (C ABI in ``include/mxattn.h``):
argument marshalling only.  Every step of the computation runs in the HIP
kernels of that library; PyTorch is used only to allocate device memory and
to name the current stream.  If the library has not been built, importing the
binding works but every call raises.

Method: "MXAttention: Data-Free Optimal Scaling and Pre-Normalization
Quantization for MXFP4 Attention" (arXiv 2607.24377), abstract.
"""
from __future__ import annotations

import ctypes
import math
import os

MODE_OCP = 0
MODE_UOS = 1
_MODES = {"ocp": MODE_OCP, "uos": MODE_UOS, MODE_OCP: MODE_OCP, MODE_UOS: MODE_UOS}

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxattn.so")
_lib = None


class MXAttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: {status_string(status)} ({status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m mxfp4_quantized_attention_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P, i64, i32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
    L.mxq_status_string.argtypes = [i32]
    L.mxq_status_string.restype = ctypes.c_char_p
    L.mxattn_version.argtypes = []
    L.mxattn_version.restype = i32
    L.mxq_quantize.argtypes = [P, i64, i64, i64, i32, i32, P, P, P]
    L.mxq_quantize.restype = i32
    L.mxattn_kv_tile.argtypes = [i64]
    L.mxattn_kv_tile.restype = i32
    L.mxattn_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.mxattn_workspace_bytes.restype = ctypes.c_size_t
    L.mxattn_fwd.argtypes = [P, P, P, i64, i64, i64, i64, i32, i32, f32, P, P, ctypes.c_size_t, P]
    L.mxattn_fwd.restype = i32
    L.mxattn_fwd_quantized.argtypes = [P, P, P, P, P, P, i64, i64, i64, i64, i32, i32, f32, P, P]
    L.mxattn_fwd_quantized.restype = i32
    L.mxattn_fwd_kv_quantized.argtypes = [P, P, P, P, P, i64, i64, i64, i64, i32, i32, f32, P, P]
    L.mxattn_fwd_kv_quantized.restype = i32
    L.mxgemm_quantized.argtypes = [P, P, P, P, i64, i64, i64, P, P]
    L.mxgemm_quantized.restype = i32
    L.mxgemm_workspace_bytes.argtypes = [i64, i64]
    L.mxgemm_workspace_bytes.restype = ctypes.c_size_t
    L.mxgemm.argtypes = [P, P, P, i64, i64, i64, i32, P, P, ctypes.c_size_t, P]
    L.mxgemm.restype = i32
    L.mxattn_fwd_strided.argtypes = [P, P, P, P, i64, i64, i64, i64, P, P, P, P, i32, i32, f32, P,
                                     ctypes.c_size_t, P]
    L.mxattn_fwd_strided.restype = i32
    L.mxq_quantize_strided.argtypes = [P, i64, i64, i64, i64, P, i32, i32, P, P, P]
    L.mxq_quantize_strided.restype = i32
    L.mxq_dump.argtypes = [ctypes.c_char_p, P, P, i64, i64, i64, i32, i32, P]
    L.mxq_dump.restype = i32
    L.mxattn_varlen_workspace_bytes.argtypes = [i64, i64, i64, i64]
    L.mxattn_varlen_workspace_bytes.restype = ctypes.c_size_t
    L.mxattn_fwd_varlen.argtypes = [P, P, P, P, P, i64, i64, i64, i64, P, i32, i32, f32, P, ctypes.c_size_t, P]
    L.mxattn_fwd_varlen.restype = i32
    L.mxqkv_proj_quantized.argtypes = [P, P, P, P, i64, i64, i64, i64, i32, P, P, P, P, P, P]
    L.mxqkv_proj_quantized.restype = i32
    L.mxqkv_proj.argtypes = [P, P, P, i64, i64, i64, i64, i32, P, P, P, P, P, P, ctypes.c_size_t, P]
    L.mxqkv_proj.restype = i32
    L.mxattn_fwd_noalloc.argtypes = [P, P, P, i64, i64, i64, i64, i32, i32, f32, P, P]
    L.mxattn_fwd_noalloc.restype = i32
    L.mxattn_noalloc_max_bytes.argtypes = []
    L.mxattn_noalloc_max_bytes.restype = ctypes.c_size_t
    _lib = L
    return L


EXPORTS = ("mxq_status_string", "mxattn_version", "mxq_quantize", "mxattn_kv_tile",
           "mxattn_workspace_bytes", "mxattn_fwd", "mxattn_fwd_quantized", "mxattn_fwd_kv_quantized",
           "mxgemm_quantized", "mxgemm_workspace_bytes", "mxgemm", "mxattn_fwd_strided",
           "mxq_quantize_strided", "mxq_dump", "mxattn_varlen_workspace_bytes", "mxattn_fwd_varlen",
           "mxqkv_proj_quantized", "mxqkv_proj", "mxattn_fwd_noalloc", "mxattn_noalloc_max_bytes")


def status_string(status: int) -> str:
    return lib().mxq_status_string(int(status)).decode()


def version() -> int:
    return int(lib().mxattn_version())


def kv_tile(d: int) -> int:
    return int(lib().mxattn_kv_tile(int(d)))


def workspace_bytes(B: int, H: int, N: int, d: int) -> int:
    return int(lib().mxattn_workspace_bytes(B, H, N, d))


def _mode(mode) -> int:
    if mode not in _MODES:
        raise ValueError(f"mode must be 'ocp' or 'uos', got {mode!r}")
    return _MODES[mode]


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise MXAttnError(status, what)


def _bf16_device(t, name):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a bfloat16 CUDA tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


# Argument checks of the binding.  The C ABI sees only pointers, so a host
# tensor, a tensor on another GPU or an undersized output would reach the
# kernels as a bad address; every entry point checks its tensors here first
# and raises before anything is enqueued.

def _on_one_gpu(named):
    """named: (tensor, name) pairs.  Every tensor must be a CUDA tensor, all
    on one device; returns that device."""
    import torch
    dev = None
    for t, n in named:
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise TypeError(f"{n} must be a CUDA tensor")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{n} is on {t.device}, expected {dev} like the other operands")
    return dev


def _u8_operand(t, name, need: int):
    """A quantized operand (codes or scales): contiguous uint8 with at least
    `need` bytes."""
    import torch
    if t.dtype != torch.uint8:
        raise TypeError(f"{name} must be a uint8 tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} bytes, needs {need}")
    return t


def _check_out(out, shape, dev, name="out", dense=True):
    """An output tensor given by the caller: bf16, on `dev`, of `shape`; dense
    entry points also need it contiguous, strided ones a contiguous last dim."""
    import torch
    if not isinstance(out, torch.Tensor) or not out.is_cuda:
        raise TypeError(f"{name} must be a CUDA tensor")
    if out.device != dev:
        raise ValueError(f"{name} is on {out.device}, expected {dev}")
    if out.dtype != torch.bfloat16:
        raise TypeError(f"{name} must be bfloat16")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(out.shape)}, expected {tuple(shape)}")
    if dense and not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not dense and out.dim() > 0 and out.numel() > 0 and out.stride(-1) != 1:
        raise ValueError(f"{name} needs a contiguous last dimension")
    return out


def _workspace(ws, need: int, dev):
    import torch
    if ws is None:
        return torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    if not isinstance(ws, torch.Tensor) or not ws.is_cuda or ws.device != dev:
        raise TypeError(f"workspace must be a CUDA tensor on {dev}")
    if ws.dtype != torch.uint8 or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace holds {ws.numel()} bytes, needs {need}")
    return ws


def n_blocks(L: int) -> int:
    return (L + 31) // 32


def quantize(x, mode="uos", axis: int = 1):
    """MXFP4-quantize a bf16 tensor viewed as [batch][rows][cols].

    x may have any rank >= 2: the last two dimensions are rows and cols, the
    rest is batch.  Returns (codes, scales) as uint8 tensors in the canonical
    layout of ``mxq_quantize`` (axis 1: [batch, rows, nb*16] / [batch, rows, nb];
    axis 0: [batch, cols, nb*16] / [batch, cols, nb]).
    """
    import torch
    x = _bf16_device(x, "x")
    if x.dim() < 2:
        raise ValueError("x needs at least 2 dimensions")
    if axis not in (0, 1):
        raise ValueError(f"axis must be 0 or 1, got {axis!r}")
    rows, cols = x.shape[-2], x.shape[-1]
    batch = x.numel() // max(1, rows * cols) if rows * cols else math.prod(x.shape[:-2])
    nvec, L = (rows, cols) if axis == 1 else (cols, rows)
    nb = n_blocks(L)
    codes = torch.empty((batch, nvec, nb * 16), dtype=torch.uint8, device=x.device)
    scales = torch.empty((batch, nvec, nb), dtype=torch.uint8, device=x.device)
    _check(lib().mxq_quantize(x.data_ptr(), batch, rows, cols, int(axis), _mode(mode),
                              codes.data_ptr(), scales.data_ptr(), _stream(x)), "mxq_quantize")
    return codes, scales


def _qkv4(q, k, v):
    """Dense bf16 [B, H, N, d] Q, K, V on one GPU; returns (B, H, N, d, device)."""
    dev = _on_one_gpu(((q, "q"), (k, "k"), (v, "v")))
    q, k, v = (_bf16_device(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v")))
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    return (*q.shape, dev)


def _kv_operands(kc, ks, vc, vs, B, H, N, d, dev):
    """K quantized along d and V along N in the canonical layouts (batch B*H)."""
    _on_one_gpu(((kc, "kc"), (ks, "ks"), (vc, "vc"), (vs, "vs")))
    for t, n in ((kc, "kc"), (ks, "ks"), (vc, "vc"), (vs, "vs")):
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, expected {dev}")
    BH, nbn = B * H, n_blocks(N)
    _u8_operand(kc, "kc", BH * N * (d // 2))
    _u8_operand(ks, "ks", BH * N * (d // 32))
    _u8_operand(vc, "vc", BH * d * nbn * 16)
    _u8_operand(vs, "vs", BH * d * nbn)


def fwd(q, k, v, mode="uos", pnq: bool = True, softmax_scale: float = 0.0, workspace=None, out=None):
    """Non-causal MXFP4 attention.  q, k, v: bf16 [B, H, N, d] -> o bf16 [B, H, N, d]."""
    import torch
    B, H, N, d, dev = _qkv4(q, k, v)
    workspace = _workspace(workspace, workspace_bytes(B, H, N, d), dev)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, dev)
    _check(lib().mxattn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, _mode(mode),
                            int(bool(pnq)), float(softmax_scale), o.data_ptr(), workspace.data_ptr(),
                            workspace.numel(), _stream(q)), "mxattn_fwd")
    return o


def noalloc_max_bytes() -> int:
    return int(lib().mxattn_noalloc_max_bytes())


def fwd_noalloc(q, k, v, mode="uos", pnq: bool = True, softmax_scale: float = 0.0, out=None):
    """``fwd`` without a workspace: the quantized K and V live in the library's
    own device array (mxattn_fwd_noalloc; the call allocates nothing when
    `out` is given).  Calls on one GPU share that array, so they must not
    overlap in time."""
    import torch
    B, H, N, d, dev = _qkv4(q, k, v)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, dev)
    _check(lib().mxattn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, N, d, _mode(mode),
                                    int(bool(pnq)), float(softmax_scale), o.data_ptr(), _stream(q)),
           "mxattn_fwd_noalloc")
    return o


def fwd_quantized(qc, qs, kc, ks, vc, vs, B: int, H: int, N: int, d: int, mode="uos",
                  pnq: bool = True, softmax_scale: float = 0.0, out=None):
    """The fused kernel on operands already quantized by ``quantize`` (Q, K along
    d with axis 1; V along N with axis 0, batch = B*H)."""
    import torch
    dev = _on_one_gpu(((qc, "qc"), (qs, "qs")))
    _u8_operand(qc, "qc", B * H * N * (d // 2))
    _u8_operand(qs, "qs", B * H * N * (d // 32))
    _kv_operands(kc, ks, vc, vs, B, H, N, d, dev)
    shape = (B, H, N, d)
    o = torch.empty(shape, dtype=torch.bfloat16, device=dev) if out is None else _check_out(out, shape, dev)
    _check(lib().mxattn_fwd_quantized(qc.data_ptr(), qs.data_ptr(), kc.data_ptr(), ks.data_ptr(),
                                      vc.data_ptr(), vs.data_ptr(), B, H, N, d, _mode(mode),
                                      int(bool(pnq)), float(softmax_scale), o.data_ptr(), _stream(qc)),
           "mxattn_fwd_quantized")
    return o


def fwd_kv_quantized(q, kc, ks, vc, vs, mode="uos", pnq: bool = True, softmax_scale: float = 0.0,
                     out=None):
    """The fused kernel of ``fwd`` alone: bf16 Q [B, H, N, d] (quantized in the
    kernel), K and V already quantized by ``quantize`` (K along d with axis 1,
    V along N with axis 0, batch = B*H)."""
    import torch
    dev = _on_one_gpu(((q, "q"),))
    q = _bf16_device(q, "q")
    if q.dim() != 4:
        raise ValueError("q must be a contiguous bf16 [B, H, N, d] tensor")
    B, H, N, d = q.shape
    _kv_operands(kc, ks, vc, vs, B, H, N, d, dev)
    o = torch.empty_like(q) if out is None else _check_out(out, q.shape, dev)
    _check(lib().mxattn_fwd_kv_quantized(q.data_ptr(), kc.data_ptr(), ks.data_ptr(), vc.data_ptr(),
                                         vs.data_ptr(), B, H, N, d, _mode(mode), int(bool(pnq)),
                                         float(softmax_scale), o.data_ptr(), _stream(q)),
           "mxattn_fwd_kv_quantized")
    return o


def _strides3(t, what):
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError(f"{what} must be a [B, H, N, d]-shaped view with contiguous d")
    return (ctypes.c_int64 * 3)(*t.stride()[:3])


def fwd_strided(q, k, v, mode="uos", pnq: bool = True, softmax_scale: float = 0.0, out=None, workspace=None):
    """mxattn_fwd on [B, H, N, d]-shaped views with any strides and contiguous
    d, e.g. a [B, N, H, d] tensor seen through .transpose(1, 2), or slices of
    a packed QKV tensor.  O gets q's strides when q is dense in some order
    (torch.empty_like), else the dense [B, H, N, d] layout."""
    import torch
    dev = _on_one_gpu(((q, "q"), (k, "k"), (v, "v")))
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same [B, H, N, d] shape")
    B, H, N, d = q.shape
    if out is None:
        out = torch.empty_like(q)
        if out.stride(3) != 1:
            out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    else:
        _check_out(out, q.shape, dev, dense=False)
    workspace = _workspace(workspace, workspace_bytes(B, H, N, d), dev)
    _check(lib().mxattn_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, d,
                                    _strides3(q, "q"), _strides3(k, "k"), _strides3(v, "v"), _strides3(out, "out"),
                                    _mode(mode), int(bool(pnq)), float(softmax_scale), workspace.data_ptr(),
                                    workspace.numel(), _stream(q)), "mxattn_fwd_strided")
    return out


def varlen_workspace_bytes(batch: int, T: int, H: int, d: int) -> int:
    return int(lib().mxattn_varlen_workspace_bytes(batch, T, H, d))


def fwd_varlen(q, k, v, cu_seqlens, mode="uos", pnq: bool = True, softmax_scale: float = 0.0, out=None,
               workspace=None):
    """mxattn_fwd_varlen on [T, H, d]-shaped views (token and head strides
    free, d contiguous) with cu_seqlens an int32 device tensor of batch + 1
    prefix offsets.  Each sequence attends to itself only; the result equals
    one mxattn_fwd call per sequence, bit for bit.  O is allocated like q
    (tokens outside every sequence are left as allocated) unless given."""
    import torch
    dev = _on_one_gpu(((q, "q"), (k, "k"), (v, "v"), (cu_seqlens, "cu_seqlens")))
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16:
            raise ValueError(f"{n} must be bf16")
        if t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{n} must be a [T, H, d]-shaped view with contiguous d")
    if q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k and v must have the same [T, H, d] shape")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 tensor")
    if cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens needs at least 2 entries (one sequence)")
    T, H, d = q.shape
    batch = cu_seqlens.numel() - 1
    if out is None:
        out = torch.empty_like(q)
        if out.stride(2) != 1:
            out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    else:
        _check_out(out, q.shape, dev, dense=False)
    workspace = _workspace(workspace, varlen_workspace_bytes(batch, T, H, d), dev)
    st = (ctypes.c_int64 * 8)(q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                              out.stride(0), out.stride(1))
    _check(lib().mxattn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu_seqlens.data_ptr(),
                                   batch, T, H, d, st, _mode(mode), int(bool(pnq)), float(softmax_scale),
                                   workspace.data_ptr(), workspace.numel(), _stream(q)), "mxattn_fwd_varlen")
    return out


def quantize_strided(x, mode="uos", axis: int = 1):
    """mxq_quantize of a [B, H, rows, cols]-shaped view with contiguous cols
    (cols % 32 == 0); returns canonical (codes, scales) with batch B*H."""
    import torch
    _on_one_gpu(((x, "x"),))
    if x.dtype != torch.bfloat16:
        raise TypeError("x must be bfloat16")
    if axis not in (0, 1):
        raise ValueError(f"axis must be 0 or 1, got {axis!r}")
    B, H, R, C = x.shape
    L = C if axis == 1 else R
    nv = R if axis == 1 else C
    nb = (L + 31) // 32
    codes = torch.empty(B * H * nv * nb * 16, dtype=torch.uint8, device=x.device)
    scales = torch.empty(B * H * nv * nb, dtype=torch.uint8, device=x.device)
    _check(lib().mxq_quantize_strided(x.data_ptr(), B, H, R, C, _strides3(x, "x"), int(axis), _mode(mode),
                                      codes.data_ptr(), scales.data_ptr(), _stream(x)), "mxq_quantize_strided")
    return codes, scales


def _gemm_weights(wc, ws, N, K, dev):
    for t, n in ((wc, "wc"), (ws, "ws")):
        _on_one_gpu(((t, n),))
        if t.device != dev:
            raise ValueError(f"{n} is on {t.device}, expected {dev}")
    _u8_operand(wc, "wc", N * (K // 2))
    _u8_operand(ws, "ws", N * (K // 32))


def gemm_quantized(xc, xs, wc, ws, M: int, N: int, K: int, out=None):
    """Y = X W^T on operands quantized by ``quantize`` (X [M][K] and W [N][K],
    batch 1, axis 1); returns bf16 [M, N]."""
    import torch
    dev = _on_one_gpu(((xc, "xc"), (xs, "xs")))
    _u8_operand(xc, "xc", M * (K // 2))
    _u8_operand(xs, "xs", M * (K // 32))
    _gemm_weights(wc, ws, N, K, dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else _check_out(out, (M, N), dev)
    _check(lib().mxgemm_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), ws.data_ptr(), M, N, K,
                                  y.data_ptr(), _stream(xc)), "mxgemm_quantized")
    return y


def gemm(x, wc, ws, N: int, mode="uos", out=None, workspace=None):
    """Y = X W^T with bf16 X [M, K] quantized on the fly and W already
    quantized (codes, scales of W [N][K], axis 1)."""
    import torch
    dev = _on_one_gpu(((x, "x"),))
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous bf16 [M, K] tensor")
    M, K = x.shape
    _gemm_weights(wc, ws, N, K, dev)
    need = int(lib().mxgemm_workspace_bytes(M, K))
    if need == 0:
        raise ValueError(f"unsupported GEMM shape M={M} K={K} (K must be a positive multiple of 128)")
    workspace = _workspace(workspace, need, dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev) if out is None else _check_out(out, (M, N), dev)
    _check(lib().mxgemm(x.data_ptr(), wc.data_ptr(), ws.data_ptr(), M, N, K, _mode(mode), y.data_ptr(),
                        workspace.data_ptr(), workspace.numel(), _stream(x)), "mxgemm")
    return y


def _qkv_outputs(T, H, d, dev):
    import torch
    u8 = dict(dtype=torch.uint8, device=dev)
    nbm = n_blocks(T)
    q = torch.empty((1, H, T, d), dtype=torch.bfloat16, device=dev)
    return (q, torch.empty(H * T * d // 2, **u8), torch.empty(H * T * d // 32, **u8),
            torch.empty(H * d * nbm * 16, **u8), torch.empty(H * d * nbm, **u8))


def qkv_proj_quantized(xc, xs, wc, ws, T: int, C: int, H: int, d: int, mode="uos"):
    """mxqkv_proj_quantized: returns (q [1, H, T, d] bf16, kc, ks, vc, vs) in
    the layouts fwd_kv_quantized takes with B = 1, N = T."""
    dev = _on_one_gpu(((xc, "xc"), (xs, "xs")))
    _u8_operand(xc, "xc", T * (C // 2))
    _u8_operand(xs, "xs", T * (C // 32))
    _gemm_weights(wc, ws, 3 * H * d, C, dev)
    q, kc, ks, vc, vs = _qkv_outputs(T, H, d, dev)
    _check(lib().mxqkv_proj_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), ws.data_ptr(), T, C, H, d,
                                      _mode(mode), q.data_ptr(), kc.data_ptr(), ks.data_ptr(), vc.data_ptr(),
                                      vs.data_ptr(), _stream(xc)), "mxqkv_proj_quantized")
    return q, kc, ks, vc, vs


def qkv_proj(x, wc, ws, H: int, d: int, mode="uos", workspace=None):
    """mxqkv_proj on bf16 x [T, C] (W quantized beforehand with quantize(...,
    axis=1) as [3*H*d, C]); returns (q, kc, ks, vc, vs) as qkv_proj_quantized."""
    dev = _on_one_gpu(((x, "x"),))
    x = _bf16_device(x, "x")
    if x.dim() != 2:
        raise ValueError("x must be a bf16 [T, C] tensor")
    T, C = x.shape
    _gemm_weights(wc, ws, 3 * H * d, C, dev)
    q, kc, ks, vc, vs = _qkv_outputs(T, H, d, dev)
    workspace = _workspace(workspace, int(lib().mxgemm_workspace_bytes(T, C)), dev)
    _check(lib().mxqkv_proj(x.data_ptr(), wc.data_ptr(), ws.data_ptr(), T, C, H, d, _mode(mode), q.data_ptr(),
                            kc.data_ptr(), ks.data_ptr(), vc.data_ptr(), vs.data_ptr(), workspace.data_ptr(),
                            workspace.numel(), _stream(x)), "mxqkv_proj")
    return q, kc, ks, vc, vs


def dump(path: str, codes, scales, batch: int, nvec: int, L: int, axis: int, mode="uos") -> None:
    """Write (codes, scales) in the "MXQ1" reference format (synchronous).
    codes and scales are both CUDA tensors or both host tensors."""
    import torch
    for t, n in ((codes, "codes"), (scales, "scales")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or not t.is_contiguous():
            raise TypeError(f"{n} must be a contiguous uint8 tensor")
    if codes.device != scales.device:
        raise ValueError(f"codes ({codes.device}) and scales ({scales.device}) must be in the same memory")
    nb = n_blocks(L)
    _u8_operand(codes, "codes", batch * nvec * nb * 16)
    _u8_operand(scales, "scales", batch * nvec * nb)
    stream = _stream(codes) if codes.is_cuda else None
    _check(lib().mxq_dump(path.encode(), codes.data_ptr(), scales.data_ptr(), batch, nvec, L,
                          int(axis), _mode(mode), stream), "mxq_dump")
