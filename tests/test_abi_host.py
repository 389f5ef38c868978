"""The C ABI on the host: the library loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no GPU needed)."""
import ctypes
import os
import re

import numpy as np
import pytest

import mxfp4_quantized_attention_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxattn.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP, IO = 0, -1, -2, -3, -4, -5


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(",
                       src, flags=re.M)
    return sorted(set(n for n in names if n not in ("defined",)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 8, names
    raw = ctypes.CDLL(mx.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n
    assert set(mx.EXPORTS) == set(names)


def test_status_strings_and_constants():
    assert mx.status_string(OK) == "MXQ_OK"
    assert mx.status_string(INVALID) == "MXQ_ERR_INVALID_ARG"
    assert mx.status_string(IO) == "MXQ_ERR_IO"
    assert mx.status_string(123) == "MXQ_ERR_UNKNOWN"
    assert mx.version() >= 100
    assert mx.kv_tile(128) == 128 and mx.kv_tile(64) == 128 and mx.kv_tile(96) == 0


def test_workspace_bytes():
    d, N, BH = 128, 32760, 40
    w = mx.workspace_bytes(1, BH, N, d)
    nbn = (N + 31) // 32
    # K codes and scales plus V codes and scales (Q is quantized in the kernel)
    assert w >= (BH * N * d // 2 + BH * N * 4) + BH * d * nbn * 17
    assert w < (BH * N * d // 2 + BH * N * 4) + BH * d * nbn * 17 + 4 * 256
    assert mx.workspace_bytes(1, 1, 0, 128) == 0 and mx.workspace_bytes(1, 1, 10, 96) == 0


def test_quantize_argument_errors():
    L = mx.lib()
    A = 1 << 20  # an aligned fake address: never dereferenced on these paths
    assert L.mxq_quantize(A, 1, 1, 32, 2, 1, A, A, None) == INVALID  # axis
    assert L.mxq_quantize(A, 1, 1, 32, 1, 5, A, A, None) == INVALID  # mode
    assert L.mxq_quantize(A, -1, 1, 32, 1, 1, A, A, None) == INVALID
    assert L.mxq_quantize(None, 1, 1, 32, 1, 1, A, A, None) == INVALID
    assert L.mxq_quantize(A + 2, 1, 1, 32, 1, 1, A, A, None) == INVALID  # misaligned input
    assert L.mxq_quantize(A, 1, 1, 32, 1, 1, A + 4, A, None) == INVALID  # misaligned codes
    assert L.mxq_quantize(None, 0, 5, 32, 1, 1, None, None, None) == OK  # empty: no-op
    assert L.mxq_quantize(A, 1, 1 << 30, 1 << 30, 1, 1, A, A, None) == UNSUPPORTED


def test_attention_argument_errors():
    L = mx.lib()
    A = 1 << 20
    big = 1 << 40
    args = lambda **kw: dict(dict(q=A, k=A, v=A, B=1, H=1, N=64, d=128, mode=1, pnq=1, scale=0.0,
                                  o=A, ws=A, wsb=big), **kw)

    def fwd(**kw):
        a = args(**kw)
        return L.mxattn_fwd(a["q"], a["k"], a["v"], a["B"], a["H"], a["N"], a["d"], a["mode"], a["pnq"],
                            a["scale"], a["o"], a["ws"], a["wsb"], None)

    assert fwd(N=0) == INVALID
    assert fwd(B=0) == INVALID
    assert fwd(d=96) == UNSUPPORTED
    assert fwd(d=256) == UNSUPPORTED
    assert fwd(mode=2) == INVALID
    assert fwd(pnq=2) == INVALID
    assert fwd(q=None) == INVALID
    assert fwd(o=A + 8) == INVALID
    assert fwd(ws=None) == WORKSPACE
    assert fwd(wsb=mx.workspace_bytes(1, 1, 64, 128) - 1) == WORKSPACE
    assert fwd(scale=float("nan")) == INVALID
    assert fwd(H=1 << 21) == UNSUPPORTED
    assert L.mxattn_fwd_quantized(A, A, A, A, A, A, 1, 1, 64, 128, 1, 1, 0.0, None, None) == INVALID
    assert L.mxattn_fwd_quantized(A, A, A, A, A, A, 1, 1, 64, 100, 1, 1, 0.0, A, None) == UNSUPPORTED
    kvq = L.mxattn_fwd_kv_quantized
    assert kvq(A, A, A, A, A, 1, 1, 64, 128, 1, 1, 0.0, None, None) == INVALID
    assert kvq(None, A, A, A, A, 1, 1, 64, 128, 1, 1, 0.0, A, None) == INVALID
    assert kvq(A + 2, A, A, A, A, 1, 1, 64, 128, 1, 1, 0.0, A, None) == INVALID
    assert kvq(A, A, A, A, A, 1, 1, 64, 100, 1, 1, 0.0, A, None) == UNSUPPORTED
    assert kvq(A, A, A, A, A, 1, 1, 0, 128, 1, 1, 0.0, A, None) == INVALID
    assert kvq(A, A, A, A, A, 1, 1, 64, 128, 3, 1, 0.0, A, None) == INVALID
    assert kvq(A, A, A, A, A, 1, 1, 64, 128, 1, 1, float("inf"), A, None) == INVALID


def test_strided_argument_errors():
    import ctypes
    L = mx.lib()
    A = 1 << 20
    s3 = lambda a, b, c: (ctypes.c_int64 * 3)(a, b, c)
    good = s3(4 * 64 * 128, 128, 4 * 128)  # [B][N][H][d] with H=4, N=64, d=128 seen as B,H,N

    def fwd(qs=good, ks=good, vs=good, os_=good, B=1, H=4, N=64, d=128, ws=A, wsb=1 << 40, o=A):
        return L.mxattn_fwd_strided(A, A, A, o, B, H, N, d, qs, ks, vs, os_, 1, 1, 0.0, ws, wsb, None)

    assert fwd(qs=None) == INVALID
    assert fwd(os_=s3(8, 8, 4)) == INVALID          # not a multiple of 8 elements
    assert fwd(ks=s3(-8, 8, 8)) == INVALID         # negative
    assert fwd(o=A + 2) == INVALID
    assert fwd(d=96) == UNSUPPORTED
    assert fwd(B=300, H=300) == UNSUPPORTED        # B*H > 65535
    assert fwd(ws=None) == WORKSPACE
    q = L.mxq_quantize_strided
    assert q(A, 1, 1, 64, 128, None, 1, 1, A, A, None) == INVALID
    assert q(A, 1, 1, 64, 128, s3(0, 0, 12), 1, 1, A, A, None) == INVALID
    assert q(A, 1, 1, 64, 96 + 8, s3(0, 0, 104), 1, 1, A, A, None) == UNSUPPORTED  # cols % 32
    assert q(A, 1, 1, 64, 128, s3(0, 0, 128), 2, 1, A, A, None) == INVALID       # axis
    assert q(None, 0, 1, 64, 128, s3(0, 0, 128), 1, 1, None, None, None) == OK   # empty: no-op


def test_varlen_workspace_and_argument_errors():
    import ctypes
    L = mx.lib()
    A = 1 << 20
    T, H, d, batch = 1000, 4, 128, 3
    w = mx.varlen_workspace_bytes(batch, T, H, d)
    vstride = (T + 31) // 32 + batch
    need = H * T * d // 2 + H * T * 4 + H * d * vstride * 17 + 4 * (batch + 1) * 4
    assert need <= w < need + 5 * 256
    assert mx.varlen_workspace_bytes(0, T, H, d) == 0
    assert mx.varlen_workspace_bytes(batch, T, H, 96) == 0
    assert mx.varlen_workspace_bytes(batch, -1, H, d) == 0
    s8 = lambda *v: (ctypes.c_int64 * 8)(*v)

    def fwd(q=A, o=A, cu=A, batch=batch, T=T, H=H, d=d, st=None, mode=1, pnq=1, scale=0.0, ws=A, wsb=1 << 40):
        return L.mxattn_fwd_varlen(q, A, A, o, cu, batch, T, H, d, st, mode, pnq, scale, ws, wsb, None)

    assert fwd(batch=0) == INVALID
    assert fwd(H=0) == INVALID
    assert fwd(T=-1) == INVALID
    assert fwd(T=0) == OK                      # nothing to do, nothing launched
    assert fwd(d=96) == UNSUPPORTED
    assert fwd(H=70000) == UNSUPPORTED
    assert fwd(T=(1 << 24) + 1) == UNSUPPORTED
    assert fwd(batch=(1 << 20) + 1) == UNSUPPORTED
    assert fwd(cu=None) == INVALID
    assert fwd(cu=A + 2) == INVALID            # cu_seqlens must be 4-byte aligned
    assert fwd(q=A + 2) == INVALID
    assert fwd(mode=5) == INVALID
    assert fwd(pnq=3) == INVALID
    assert fwd(scale=float("nan")) == INVALID
    assert fwd(st=s8(512, 128, 512, 128, 512, 128, 512, 12)) == INVALID  # not a multiple of 8
    assert fwd(st=s8(512, 128, -512, 128, 512, 128, 512, 128)) == INVALID
    assert fwd(ws=None) == WORKSPACE
    assert fwd(wsb=w - 1) == WORKSPACE
    assert fwd(ws=A + 8) == INVALID


def test_qkv_projection_argument_errors():
    L = mx.lib()
    A = 1 << 20
    pq = L.mxqkv_proj_quantized

    def fq(T=300, C=256, H=3, d=64, mode=1, xc=A, xs=A, q=A, vc=A):
        return pq(xc, xs, A, A, T, C, H, d, mode, q, A, A, vc, A, None)

    assert fq(T=0) == INVALID
    assert fq(H=0) == INVALID
    assert fq(d=96) == UNSUPPORTED
    assert fq(C=200) == UNSUPPORTED          # C % 128
    assert fq(mode=4) == INVALID
    assert fq(xc=None) == INVALID
    assert fq(q=A + 2) == INVALID
    assert fq(vc=A + 8) == INVALID
    assert fq(xs=A + 2) == INVALID           # scales need 4-byte alignment
    p = L.mxqkv_proj

    def fb(T=300, C=256, H=3, d=64, ws=A, wsb=1 << 40, x=A):
        return p(x, A, A, T, C, H, d, 1, A, A, A, A, A, ws, wsb, None)

    assert fb(ws=None) == WORKSPACE
    assert fb(wsb=L.mxgemm_workspace_bytes(300, 256) - 1) == WORKSPACE
    assert fb(x=A + 2) == INVALID
    assert fb(C=100) == UNSUPPORTED


def test_dump_from_host_memory(tmp_path):
    import oracle
    import workloads
    from test_oracle_quant import read_mxq1
    g = np.random.default_rng(1)
    x = workloads.f32_to_bf16(g.standard_normal((3, 50)).astype(np.float32))
    c, s = oracle.quantize_bf16(x, 1, 3, 50, 1, oracle.MODE_OCP)
    p1, p2 = str(tmp_path / "lib.mxq"), str(tmp_path / "orc.mxq")
    L = mx.lib()
    assert L.mxq_dump(p1.encode(), c.ctypes.data, s.ctypes.data, 1, 3, 50, 1, 0, None) == OK
    oracle.dump(p2, c, s, 1, 3, 50, 1, oracle.MODE_OCP)
    assert open(p1, "rb").read() == open(p2, "rb").read()
    hdr, c2, s2 = read_mxq1(p1)
    assert hdr["mode"] == "ocp" and hdr["nvec"] == 3 and hdr["L"] == 50
    assert L.mxq_dump(str(tmp_path / "no/dir/x").encode(), c.ctypes.data, s.ctypes.data, 1, 3, 50, 1, 0, None) == IO
    assert L.mxq_dump(None, c.ctypes.data, s.ctypes.data, 1, 3, 50, 1, 0, None) == INVALID
    assert L.mxq_dump(p1.encode(), c.ctypes.data, s.ctypes.data, 1, 3, 50, 3, 0, None) == INVALID


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(mx, "_lib", None)
    monkeypatch.setattr(mx, "LIB_PATH", "/nonexistent/libmxattn.so")
    with pytest.raises(RuntimeError):
        mx.lib()
