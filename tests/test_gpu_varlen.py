"""GPU parity of mxattn_fwd_varlen (sequences of different lengths packed
along one token axis).

  - Every sequence's output is bit-identical to mxattn_fwd on that sequence
    alone (dense [1, H, N_s, d] copies): same codes for Q, K and V, same key
    tiles, same arithmetic.  Length mixes cover empty sequences, one-token
    sequences, lengths on and off the 32-key block and 128-key tile grid, and
    sequences that start off the block grid of the packed axis.
  - Against the oracle (per-sequence attention, pinned on the host) within
    the attention tolerance, on every row of small batches and on sampled
    rows of the Wan-style varlen batch.
  - Strided Q/K/V/O (slices of a packed [T][3][H][d] QKV tensor).
  - Tokens outside every sequence are not written; a malformed cu_seqlens is
    read clamped and made non-decreasing, as the header states.
"""
import numpy as np
import pytest

import oracle
import workloads
from gpu_helpers import HAVE_GPU, compare_attention, to_gpu_bf16, to_np_u16

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not HAVE_GPU, reason="needs a GPU")]

if HAVE_GPU:
    import torch
    import mxfp4_quantized_attention_amd as mx

OMODE = {"uos": oracle.MODE_UOS, "ocp": oracle.MODE_OCP}
MIXES = {
    "mixed": [1, 31, 33, 128, 129, 300, 1000],
    "empties": [0, 5, 0, 200, 0],
    "single": [517],
    "grid": [32, 64, 256, 96],
}


def _inputs(lengths, H, d, seed, dist="tiny"):
    q, k, v, cu = workloads.varlen_qkv(lengths, H, d, seed=seed, dist=dist)
    return q, k, v, cu


def _assert_same(o, ref, cu, what=""):
    a, b = o.view(torch.int16), ref.view(torch.int16)
    if not torch.equal(a, b):
        bad = torch.nonzero(a != b).cpu().numpy()
        seq = np.searchsorted(np.asarray(cu), bad[:, 0], side="right") - 1
        raise AssertionError(f"{what}: {len(bad)} elements differ; first (token, head, channel): {bad[:8].tolist()}, "
                             f"sequences {sorted(set(seq.tolist()))}, cu {list(cu)}")


def _dense_per_sequence(qg, kg, vg, cu, mode, pnq, scale):
    """One mxattn_fwd call per sequence on dense [1, H, N, d] copies."""
    T, H, d = qg.shape
    out = torch.zeros_like(qg)
    for s in range(len(cu) - 1):
        t0, t1 = int(cu[s]), int(cu[s + 1])
        if t1 == t0:
            continue
        dense = [x[t0:t1].permute(1, 0, 2).contiguous().unsqueeze(0) for x in (qg, kg, vg)]
        o = mx.fwd(*dense, mode=mode, pnq=pnq, softmax_scale=scale)
        out[t0:t1] = o[0].permute(1, 0, 2)
    return out


@pytest.mark.parametrize("mix", list(MIXES))
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode,pnq", [("uos", True), ("ocp", False), ("uos", False)])
def test_varlen_bit_identical_to_per_sequence(mix, d, mode, pnq):
    lengths, H = MIXES[mix], 3
    q, k, v, cu = _inputs(lengths, H, d, seed=len(lengths) + d)
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    cug = torch.from_numpy(cu).to("cuda:0")
    o = mx.fwd_varlen(qg, kg, vg, cug, mode=mode, pnq=pnq)
    ref = _dense_per_sequence(qg, kg, vg, cu, mode, pnq, 0.0)
    torch.cuda.synchronize()
    _assert_same(o, ref, cu, f"{mix} d={d} {mode} pnq={pnq}")


@pytest.mark.parametrize("mix", ["mixed", "empties"])
@pytest.mark.parametrize("mode,pnq", [("uos", True), ("ocp", False)])
def test_varlen_matches_oracle(mix, mode, pnq):
    lengths, H, d = MIXES[mix], 2, 64
    q, k, v, cu = _inputs(lengths, H, d, seed=7)
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    o = mx.fwd_varlen(qg, kg, vg, torch.from_numpy(cu).to("cuda:0"), mode=mode, pnq=pnq)
    torch.cuda.synchronize()
    rows = np.array([(t, h) for t in range(int(cu[-1])) for h in range(H)])
    ref = oracle.attn_varlen_rows(q, k, v, cu, H, d, OMODE[mode], pnq, mx.kv_tile(d), 1.0 / np.sqrt(d), rows)
    got = to_np_u16(o)[rows[:, 0], rows[:, 1]]
    compare_attention(got, ref, what=f"varlen {mix} {mode} pnq={pnq}")


def test_varlen_packed_qkv_slices():
    lengths, H, d = [77, 300, 12], 4, 128
    q, k, v, cu = _inputs(lengths, H, d, seed=8)
    T = int(cu[-1])
    qkv = torch.empty((T, 3, H, d), dtype=torch.bfloat16, device="cuda:0")
    for i, x in enumerate((q, k, v)):
        qkv[:, i] = to_gpu_bf16(x)
    out = torch.empty((T, H, 2, d), dtype=torch.bfloat16, device="cuda:0")[:, :, 1]  # strided O
    cug = torch.from_numpy(cu).to("cuda:0")
    o = mx.fwd_varlen(qkv[:, 0], qkv[:, 1], qkv[:, 2], cug, out=out)
    dense = mx.fwd_varlen(*(to_gpu_bf16(x) for x in (q, k, v)), cug)
    torch.cuda.synchronize()
    assert o.data_ptr() == out.data_ptr()
    assert torch.equal(o.view(torch.int16), dense.view(torch.int16))


def test_tokens_outside_sequences_untouched_and_malformed_table():
    H, d, T = 2, 64, 250
    q, k, v, _ = _inputs([T], H, d, seed=9)
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    sentinel = torch.full((T, H, d), 7.0, dtype=torch.bfloat16, device="cuda:0")
    # sequences [5, 100) and [100, 200); tokens 0..4 and 200..249 belong to none
    cu = np.array([5, 100, 200], np.int32)
    o = mx.fwd_varlen(qg, kg, vg, torch.from_numpy(cu).to("cuda:0"), out=sentinel.clone())
    ref = _dense_per_sequence(qg, kg, vg, cu, "uos", True, 0.0)
    torch.cuda.synchronize()
    assert torch.equal(o[:5], sentinel[:5]) and torch.equal(o[200:], sentinel[200:])
    assert torch.equal(o[5:200].view(torch.int16), ref[5:200].view(torch.int16))
    # a decreasing entry is read as the running maximum (an empty sequence),
    # and entries past T as T
    bad = np.array([0, 120, 60, 180, 999], np.int32)
    fixed = np.array([0, 120, 120, 180, 250], np.int32)
    o1 = mx.fwd_varlen(qg, kg, vg, torch.from_numpy(bad).to("cuda:0"))
    o2 = mx.fwd_varlen(qg, kg, vg, torch.from_numpy(fixed).to("cuda:0"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


def test_wan_varlen_sampled_rows():
    """The Wan-style varlen batch (videos of 21, 13, 5 and 1 latent frames,
    T = 62400, H = 40, d = 128): 256 sampled (token, head) rows against the
    oracle, including each sequence's first and last token."""
    cfg = workloads.VARLEN_CONFIGS["wan_varlen"]
    H, d = cfg["H"], cfg["d"]
    q, k, v, cu = workloads.varlen_qkv(cfg["lengths"], H, d, seed=cfg["seed"], dist=cfg["dist"])
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    o = mx.fwd_varlen(qg, kg, vg, torch.from_numpy(cu).to("cuda:0"))
    torch.cuda.synchronize()
    got_all = to_np_u16(o)
    g = np.random.default_rng(11)
    T = int(cu[-1])
    toks = np.concatenate([g.integers(0, T, 240), cu[:-1], cu[1:] - 1])
    rows = np.stack([toks, g.integers(0, H, toks.size)], axis=1)
    ref = oracle.attn_varlen_rows(q, k, v, cu, H, d, oracle.MODE_UOS, True, mx.kv_tile(d), 1.0 / np.sqrt(d), rows)
    compare_attention(got_all[rows[:, 0], rows[:, 1]], ref, what="wan varlen (sampled)")


def test_many_short_sequences():
    """More sequences than the table kernel has threads (1000 > 256), so each
    thread scans a chunk of several entries; lengths 0..40 cover empty,
    one-token and two-block sequences."""
    g = np.random.default_rng(12)
    lengths = [int(n) for n in g.integers(0, 41, 1000)]
    H, d = 2, 64
    q, k, v, cu = _inputs(lengths, H, d, seed=13)
    qg, kg, vg = (to_gpu_bf16(x) for x in (q, k, v))
    o = mx.fwd_varlen(qg, kg, vg, torch.from_numpy(cu).to("cuda:0"))
    ref = _dense_per_sequence(qg, kg, vg, cu, "uos", True, 0.0)
    torch.cuda.synchronize()
    _assert_same(o, ref, cu, "1000 short sequences")
