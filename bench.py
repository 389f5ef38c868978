#!/usr/bin/env python3
"""Benchmark of the MXFP4 attention hot path (MXAttention: UOS + PNQ) on one MI355X.

One step = one pass of the whole path over one batch of synthetic input that
is already resident in HBM: quantize K along d, quantize V along N, and run
the fused MXFP4 attention kernel, which quantizes Q along d itself (exactly
the launches mxattn_fwd makes, issued one by one so each kernel can be
bracketed with HIP events on the stream it runs on).  Default workload: the Wan-style video DiT shape
B=1, H=40, N=32760 (21 x 1560 tokens), d=128, UOS + PNQ, non-causal.

Prints ONE JSON line on stdout; progress goes to stderr.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload wan]

`--workload gemm` times the MXFP4 GEMM of a DiT linear layer instead: a
Wan-style FFN up-projection, Y = X W^T with X [32760][5120] bf16 and W
[13824][5120] quantized once beforehand; one step = quantize X along K, then
the GEMM kernel (mxgemm's launches).

`--workload wan_varlen` times mxattn_fwd_varlen on a varlen batch of four
Wan-style videos (21, 13, 5 and 1 latent frames of 1560 tokens: T = 62400
packed tokens, H=40, d=128, UOS + PNQ); one step = one mxattn_fwd_varlen
call (varlen table, K and V quantization, the fused kernel), and the FLOP
count is 4*H*d*sum(N_s^2).

`--workload wan_block` times the attention block of a Wan-style DiT layer
from its input activations: X [32760][5120] bf16 and W_qkv [15360][5120]
(quantized once beforehand); one step = quantize X, the QKV projection with
the epilogue that writes bf16 Q and MXFP4 K and V in the attention layouts
(mxqkv_proj), and the fused attention kernel.  The same work unfused (bf16
Y from mxgemm, then mxattn_fwd_strided on its Q, K, V slices) is timed
beside it.

`--workload sweep` instead times the quantizer alone (mxq_quantize) over
n = 2^p bf16 values, p = 20..30 (log-uniform magnitudes 2^-20..2^10, random
sign, viewed [n/1024, 1024]), UOS and OCP along the contiguous axis, plus one
run along rows at 2^28; the JSON line's value is the 2^30 UOS figure.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
PEAK_FP4_TFLOPS = 10100.0  # MI355X dense MXFP4 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan_traffic.json")
GEMM_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "gemm_dit_ffn_traffic.json")
UTIL_FILE = os.path.join(ROOT, "profiles", "attn_fwd_wan_utilization.json")
# The vector-unit ceiling of the attention kernel comes from the committed
# instruction-cost probe (bench.py --workload valu_probe, probe.hip): every
# score element needs one fma (scale and max shift), one exponential, half a
# three-input max and half a two-element FP4 convert, and every 2048 scores of
# a wave's key tile take 17 scaled FP4 MFMAs at d = 128 (8 for S, 8 for P.V,
# 1 for the PNQ row sum; 13 at d = 64).  1024 SIMDs.
N_SIMDS = 1024
PROBE_FILE = os.path.join(ROOT, "profiles", "attn_valu_probe.json")
ATTN_SRC = os.path.join(ROOT, "mxfp4_quantized_attention_amd", "csrc", "attention.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash(src: str = "attention.hip") -> str:
    """Identity of one kernel source's binary: the file, the shared device
    header and the compiler flags it is built with (the rest of the build
    script does not shape it)."""
    from mxfp4_quantized_attention_amd import build as hip_build
    h = hashlib.sha256()
    csrc = os.path.dirname(ATTN_SRC)
    headers = () if src == "probe.hip" else ("mx_device.h",)  # the probe includes no header of ours
    for path in (os.path.join(csrc, src), *(os.path.join(csrc, hdr) for hdr in headers)):
        with open(path, "rb") as f:
            h.update(f.read())
    fl = hip_build.flags()
    fl = [f for i, f in enumerate(fl) if f != "-I" and (i == 0 or fl[i - 1] != "-I")]  # paths vary by machine
    h.update(repr((hip_build.ARCH, fl, hip_build.PER_FILE_FLAGS.get(src, []))).encode())
    return h.hexdigest()[:16]


def attn_source_hash() -> str:
    return source_hash("attention.hip")


def measured_traffic(workload: str, path: str = TRAFFIC_FILE, src: str = "attention.hip"):
    """HBM bytes per launch of the dominant kernel from a committed rocprofv3
    counter summary, or None when the counters were taken on another kernel
    version or workload."""
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != source_hash(src) or t.get("workload") != workload:
        return None
    return float(t["bytes_per_launch"])


def copy_calibration(mib: int, dev) -> None:
    """A plain elementwise copy kernel of known size (reads and writes mib MiB
    each): the reference that scales rocprofv3's FETCH_SIZE and WRITE_SIZE
    counters to bytes."""
    import torch
    nbytes = mib << 20
    src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    flush = torch.ones(2 * nbytes // 4, dtype=torch.float32, device=dev)  # evict src from the caches
    del flush
    torch.cuda.synchronize()
    torch.neg(src, out=dst)
    torch.cuda.synchronize()
    log(f"[bench] calibration copy kernel: {nbytes} bytes read, {nbytes} bytes written")
    del src, dst


def measured_probe():
    """The committed instruction-cost probe summary, or None when it was taken
    on another version of the probe kernel."""
    try:
        with open(PROBE_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("probe_sha") != source_hash("probe.hip"):
        return None
    return t


def valu_ceilings(d: int, probe: dict, clock_ghz: float) -> dict:
    """FLOP/s (4 d per score element) at which the per-score vector work alone
    fills every SIMD's issue cycles (MFMA entirely hidden), and with the MFMAs
    serialized behind it, from the probe's cycle costs at `clock_ghz`."""
    cyc = {k: v * probe["clock_ghz"] for k, v in probe["ns_per_wave_instruction"].items()}
    valu = (cyc["fma"] + cyc["exp"] + cyc["cvt"] / 2 + cyc["max3"] / 2) / 64.0  # SIMD cycles per score
    mfma = (17.0 if d == 128 else 13.0) * cyc["mfma"] / 2048.0
    per = lambda c: 4.0 * d * N_SIMDS * clock_ghz * 1e9 / c / 1e12
    return {"valu_cycles_per_score": valu, "mfma_cycles_per_score": mfma,
            "ceiling": per(valu), "ceiling_mfma_serialized": per(valu + mfma)}


def measured_utilization(workload: str):
    """MFMA-busy and VALU-active fractions of the attention launch from the
    committed rocprofv3 counter summary (None if taken on another kernel
    version or workload)."""
    try:
        with open(UTIL_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != attn_source_hash() or t.get("workload") != workload:
        return None
    return t


def valu_bound(achieved: float, d: int, workload: str) -> dict:
    probe = measured_probe()
    util = measured_utilization(workload)
    out = {"bound": "valu", "unit": "TFLOP/s", "source": "profiles/attn_valu_probe.json",
           "valu_active": util["valu_active"] if util else None,
           "mfma_busy": util["mfma_busy"] if util else None,
           "clock_ghz_profiled": util["clock_ghz"] if util else None}
    if probe is None:
        out.update(ceiling=None, frac=None, note="probe summary missing or taken on another probe version")
        return out
    clock = util["clock_ghz"] if util else probe["clock_ghz"]
    c = valu_ceilings(d, probe, clock)
    out.update(c)
    out.update(frac=achieved / c["ceiling"], clock_ghz_used=clock, clock_ghz_probe=probe["clock_ghz"],
               slots_per_score=probe["slots_per_score"], probe_sha=probe["probe_sha"])
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(q, k, v, cfg, mode, pnq, kv_tile, gpu_out, heads=8, rows_per_head=3072):
    """The oracle, timed on this host's cores on a bounded sample of the same
    workload: K/V quantization of `heads` heads plus `rows_per_head` seeded
    query rows of each."""
    import numpy as np
    import oracle
    import workloads
    B, H, N, d = q.shape
    heads, rows_per_head = min(heads, B * H), min(rows_per_head, N)
    rows = []
    g = np.random.default_rng(11)
    for h in range(heads):
        rows.append(h * N + np.sort(g.choice(N, rows_per_head, replace=False)))
    rows = np.concatenate(rows)
    qs, ks, vs = (x.reshape(B * H, N, d)[:heads] for x in (q, k, v))
    t0 = time.perf_counter()
    ref = oracle.attn_rows(qs, ks, vs, heads, N, d, mode, pnq, kv_tile, 1.0 / np.sqrt(d), rows,
                           want_budget=False)
    dt = time.perf_counter() - t0
    flop = 4.0 * N * d * rows.size
    got = oracle.bf16_to_f64(gpu_out.reshape(B * H * N, d)[rows])
    want = oracle.bf16_to_f64(ref["out_bf16"])
    diff = np.abs(got - want)
    # the base parity bound of the tests, max(2e-3, one bf16 ulp of the
    # oracle's value) per element; rows holding decisions near a rounding tie
    # may exceed it by the oracle's flip budget, which the timed oracle run
    # does not compute (the GPU tests check those rows against it)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(want), 1e-30))) - 7)
    ratio = diff / np.maximum(2e-3, ulp)
    flagged = ref["near_tie"].astype(bool)
    # one thread on a small slice of the same rows, for the per-core rate
    threads = oracle.num_threads()
    r1 = rows[:: max(1, rows.size // 256)][:256]
    oracle.set_num_threads(1)
    t1 = time.perf_counter()
    oracle.attn_rows(qs, ks, vs, heads, N, d, mode, pnq, kv_tile, 1.0 / np.sqrt(d), r1, want_budget=False)
    dt1 = time.perf_counter() - t1
    oracle.set_num_threads(threads)
    total_rows = B * H * N
    return {
        "value": flop / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": f"{cfg}: K/V quantization of {heads} heads + {rows.size} seeded query rows "
                  f"({rows_per_head} per head), {dt:.1f} s; FLOP counted as 4*N*d per row",
        "seconds": dt,
        "rows_per_second": rows.size / dt,
        "extrapolated_full_workload_seconds": dt * total_rows / rows.size,
        "single_thread": {"value": 4.0 * N * d * r1.size / dt1 / 1e12, "unit": "TFLOP/s", "rows": int(r1.size),
                          "seconds": dt1},
        "vs_gpu_on_sample": {
            "rel_l2": float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300)),
            "max_diff_over_bound_unflagged_rows": float(ratio[~flagged].max()) if (~flagged).any() else 0.0,
            "near_tie_rows": int(flagged.sum()),
            "near_tie_rows_beyond_base_bound": int(np.sum(np.any(ratio[flagged] > 1.0, axis=1))),
        },
    }


def quality_context(q, k, v, out_uos_pnq, out_ocp, nrows=64):
    """Cosine and relative L2 against unquantized fp64 attention on sampled rows
    (quality context only)."""
    import numpy as np
    import oracle
    B, H, N, d = q.shape
    g = np.random.default_rng(5)
    res = {"rows": nrows}
    cos = {"uos_pnq": [], "ocp": []}
    for r in np.sort(g.choice(B * H * N, nrows, replace=False)):
        h, i = divmod(int(r), N)
        Q = oracle.bf16_to_f64(q.reshape(B * H, N, d)[h, i])
        K = oracle.bf16_to_f64(k.reshape(B * H, N, d)[h])
        V = oracle.bf16_to_f64(v.reshape(B * H, N, d)[h])
        s = K @ Q / np.sqrt(d)
        w = np.exp(s - s.max())
        ref = (w @ V) / w.sum()
        for name, o in (("uos_pnq", out_uos_pnq), ("ocp", out_ocp)):
            x = oracle.bf16_to_f64(o.reshape(B * H, N, d)[h, i])
            cos[name].append(float(x @ ref / np.sqrt((x @ x) * (ref @ ref))))
    for name in cos:
        res["mean_cos_" + name] = float(np.mean(cos[name]))
    return res


def emit(result, checks):
    """Print the JSON line with every in-run correctness check of the run.
    If any failed, the line is marked invalid and the run exits with status 3,
    so a number measured on wrong results is never taken for a valid one."""
    result["checks"] = {name: bool(ok) for name, ok in checks.items()}
    failed = [name for name, ok in checks.items() if not ok]
    result["valid"] = not failed
    print(json.dumps(result), flush=True)
    if failed:
        log(f"[bench] in-run check failed: {', '.join(failed)}; the line above is not a valid measurement")
        sys.exit(3)


def oracle_sample_ok(v):
    """The attention baselines' agreement on their sample: every row not flagged
    near a rounding tie within the base bound, and rel-L2 within 1e-3.  Flagged
    rows may exceed the base bound by a flip budget the timed run does not
    compute; the GPU tests check them against it."""
    return v["max_diff_over_bound_unflagged_rows"] <= 1.0 and v["rel_l2"] <= 1e-3


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=10,
                    help="untimed steps first: the clocks of a fresh process take about 20 ms of steady MFMA load to settle")
    ap.add_argument("--workload", default="wan", choices=["tiny", "small", "wan", "hunyuan", "sweep", "gemm", "wan_varlen",
                                                          "wan_block", "valu_probe"])
    ap.add_argument("--probe-out", default="", help="valu_probe: also write the summary JSON here")
    ap.add_argument("--mode", default="uos", choices=["uos", "ocp"])
    ap.add_argument("--no-pnq", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quality", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device-to-device copy of this many MiB before timing "
                         "(reference for the rocprofv3 FETCH_SIZE/WRITE_SIZE scale factor)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the path shards by head with no communication, "
              "and runs on more than one GPU are not part of this build", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import mxfp4_quantized_attention_amd as mx

    if not torch.cuda.is_available():
        log("no GPU visible")
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.workload == "sweep":
        quantize_sweep(args, dev)
        return
    if args.workload == "gemm":
        gemm_bench(args, dev)
        return
    if args.workload == "wan_varlen":
        varlen_bench(args, dev)
        return
    if args.workload == "wan_block":
        block_bench(args, dev)
        return
    if args.workload == "valu_probe":
        probe_bench(args, dev)
        return
    cfg = workloads.CONFIGS[args.workload]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    BH = B * H
    mode = mx.MODE_UOS if args.mode == "uos" else mx.MODE_OCP
    pnq = 0 if args.no_pnq else 1
    log(f"[bench] generating {args.workload} inputs {B}x{H}x{N}x{d}")
    t0 = time.perf_counter()
    q, k, v = workloads.qkv(args.workload)
    log(f"[bench] generated in {time.perf_counter() - t0:.1f} s; uploading")

    def up(x):
        return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)

    qg, kg, vg = up(q), up(k), up(v)
    L = mx.lib()
    nbn = (N + 31) // 32
    u8 = dict(dtype=torch.uint8, device=dev)
    kc, ks = torch.empty(BH * N * d // 2, **u8), torch.empty(BH * N * d // 32, **u8)
    vc, vs = torch.empty(BH * d * nbn * 16, **u8), torch.empty(BH * d * nbn, **u8)
    o = torch.empty_like(qg)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def launch_k():
        return L.mxq_quantize(kg.data_ptr(), BH, N, d, 1, mode, kc.data_ptr(), ks.data_ptr(), sp)

    def launch_v():
        return L.mxq_quantize(vg.data_ptr(), BH, N, d, 0, mode, vc.data_ptr(), vs.data_ptr(), sp)

    def launch_attn():
        return L.mxattn_fwd_kv_quantized(qg.data_ptr(), kc.data_ptr(), ks.data_ptr(), vc.data_ptr(),
                                         vs.data_ptr(), B, H, N, d, mode, pnq, 0.0, o.data_ptr(), sp)

    launches = (launch_k, launch_v, launch_attn)

    def step(ev=None):
        for i, fn in enumerate(launches):
            if ev is not None:
                ev[i].record(stream)
            st = fn()
            if st != 0:
                raise RuntimeError(f"launch {i} failed: {mx.status_string(st)}")
        if ev is not None:
            ev[len(launches)].record(stream)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, dev)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)]
              for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(events[s])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_kernel = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(len(launches))] for ev in events])
    kk, kvv, ka = per_kernel.mean(axis=0)
    ka_median = float(np.median(per_kernel[:, 2]))
    flop = 4.0 * B * H * N * N * d
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (ka * 1e-3) / 1e12
    log(f"[bench] step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s; attention kernel {ka:.3f} ms "
        f"-> {achieved:.1f} TFLOP/s; quantize K {kk:.3f} V {kvv:.3f} ms (Q in the attention kernel)")

    # the split launches are exactly mxattn_fwd: check bit-equality once
    o_split = o.clone()
    o_fwd = mx.fwd(qg, kg, vg, mode=args.mode, pnq=bool(pnq))
    torch.cuda.synchronize()
    same = bool(torch.equal(o_split.view(torch.int16), o_fwd.view(torch.int16)))
    gpu_out = o_split.view(torch.int16).cpu().numpy().view(np.uint16)

    qbytes = 2.53125 * BH * N * d
    traffic = measured_traffic(args.workload)
    result = {
        "metric": "MXFP4 attention fwd TFLOP/s (4*B*H*N^2*d) and % of MI355X MXFP4 MFMA peak",
        "value": value,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: B={B} H={H} N={N} d={d} non-causal, "
                               f"{args.mode.upper()}{'+PNQ' if pnq else ''}",
                   "B": B, "H": H, "N": N, "d": d, "mode": args.mode, "pnq": bool(pnq),
                   "kv_tile": mx.kv_tile(d), "global_batch": B, "seq_len": N, "parallelism": "single GPU"},
        "pct_of_fp4_peak": 100.0 * value / PEAK_FP4_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP4_TFLOPS, "traffic": traffic,
                     "kernel": "attn_fwd_kernel", "kernel_ms": ka, "kernel_ms_median": ka_median,
                     "algorithmic": f"4*d FLOP per score element x B*H*N^2 = {flop:.4g} FLOP per launch"},
        "valu_bound": valu_bound(achieved, d, args.workload),
        "roofline_quantize": {"bound": "hbm", "unit": "GB/s", "peak": PEAK_HBM_GBS,
                              "bytes_per_launch": qbytes,
                              "k_axis1_ms": kk, "k_axis1_gbs": qbytes / (kk * 1e-3) / 1e9,
                              "v_axis0_ms": kvv, "v_axis0_gbs": qbytes / (kvv * 1e-3) / 1e9},
        "step_equals_mxattn_fwd": same,
    }
    if not args.no_quality:
        log("[bench] quality context")
        o_ocp = mx.fwd(qg, kg, vg, mode="ocp", pnq=False)
        torch.cuda.synchronize()
        out_ocp = o_ocp.view(torch.int16).cpu().numpy().view(np.uint16)
        result["quality"] = quality_context(q, k, v, gpu_out, out_ocp)
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        # the small configurations are timed in full, the large ones on a sample
        full = args.workload in ("tiny", "small")
        result["cpu_baseline"] = cpu_baseline(q, k, v, args.workload, mode, pnq, mx.kv_tile(d), gpu_out,
                                              **({"heads": B * H, "rows_per_head": N} if full else {}))
    checks = {"step_equals_mxattn_fwd": same}
    if "cpu_baseline" in result:
        checks["oracle_agrees_on_sample"] = oracle_sample_ok(result["cpu_baseline"]["vs_gpu_on_sample"])
    emit(result, checks)


PROBE_OPS = {"fma": 1, "exp": 2, "cvt": 3, "max3": 4, "mfma": 5, "mfma32": 6, "mfma_f8": 7}
# FLOP of one wave instruction of each scaled MFMA form the probe times
PROBE_MFMA_FLOP = {"mfma": 2 * 16 * 16 * 128, "mfma32": 2 * 32 * 32 * 64, "mfma_f8": 2 * 16 * 16 * 128}


def probe_bench(args, dev):
    """Issue costs of the attention kernel's per-score instructions and their
    overlap with the scaled FP4 MFMA (libmxprobe.so; see probe.hip).  Prints one
    JSON line; --probe-out also writes it as the summary valu_bound reads."""
    import ctypes
    import numpy as np
    import torch
    from mxfp4_quantized_attention_amd import build as hip_build

    P = ctypes.CDLL(hip_build.PROBE_LIB)
    i32 = ctypes.c_int
    P.mxprobe_launch.argtypes = [i32, i32, i32, i32, i32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    P.mxprobe_launch.restype = i32
    wg = 4  # workgroups per CU: 4 waves of each role per SIMD
    out = torch.zeros(256 * wg * 8, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)

    def run(op_a, it_a, op_b=0, it_b=0, reps=5):
        times = []
        for r in range(reps + 1):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            st = P.mxprobe_launch(op_a, it_a, op_b, it_b, wg, out.data_ptr(), clocks.data_ptr(), stream.cuda_stream)
            e1.record(stream)
            if st != 0:
                raise RuntimeError(f"probe launch failed ({st})")
            torch.cuda.synchronize()
            if r:
                times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    target_ms = 3.0

    def iters_for(op, it0=512):
        t = run(op, it0, reps=2)
        return max(64, int(it0 * target_ms / max(t, 1e-3)))

    log("[probe] costs of each instruction alone (4 waves per SIMD)")
    cost, iters = {}, {}
    for name, op in PROBE_OPS.items():
        iters[name] = iters_for(op)
        t = run(op, iters[name])
        cost[name] = t * 1e6 / (wg * iters[name] * 8)  # ns per wave instruction per SIMD
        log(f"[probe] {name}: {cost[name]:.3f} ns")
    ghz = float(clocks[0].item()) / (float(clocks[1].item()) * 10.0)
    slot = cost["fma"]
    log("[probe] overlap with the scaled FP4 MFMA on other waves of the same SIMD")
    overlap = {}
    for name in ("fma", "exp", "cvt", "max3"):
        ta = run(PROBE_OPS[name], iters[name])
        tb = run(0, 0, PROBE_OPS["mfma"], iters["mfma"])
        tab = run(PROBE_OPS[name], iters[name], PROBE_OPS["mfma"], iters["mfma"])
        overlap[name] = (ta + tb - tab) / min(ta, tb)
        log(f"[probe] {name} + mfma: alone {ta:.3f} / {tb:.3f} ms, together {tab:.3f} ms, overlap {overlap[name]:.2f}")
    log("[probe] overlap with the other MFMA forms on other waves of the same SIMD")
    overlap_forms = {}
    for form in ("mfma32", "mfma_f8"):
        overlap_forms[form] = {}
        tb = run(0, 0, PROBE_OPS[form], iters[form])
        for name in ("fma", "exp", "cvt", "max3"):
            ta = run(PROBE_OPS[name], iters[name])
            tab = run(PROBE_OPS[name], iters[name], PROBE_OPS[form], iters[form])
            overlap_forms[form][name] = (ta + tb - tab) / min(ta, tb)
            log(f"[probe] {name} + {form}: overlap {overlap_forms[form][name]:.2f}")
    log("[probe] one MFMA and R vector instructions interleaved in one wave")
    mixed = {}
    for name in ("fma", "exp", "cvt", "max3"):
        for R in (1, 2, 4, 8):
            op = 16 + 4 * R + (PROBE_OPS[name] & 3)
            it = max(64, int(target_ms * 1e6 / (wg * 8 * (cost["mfma"] + R * cost[name]))))
            t = run(op, it)
            per = t * 1e6 / (wg * it * 8)  # ns per (MFMA + R instructions) per SIMD
            alone = cost["mfma"] + R * cost[name]
            hidden = (alone - per) / min(cost["mfma"], R * cost[name])
            mixed[f"{name}x{R}"] = {"ns": per, "serial_ns": alone, "hidden": hidden}
            log(f"[probe] mfma + {R} {name}: {per:.2f} ns (serial {alone:.2f}), hidden {hidden:.2f}")
    slots = (cost["fma"] + cost["exp"] + cost["cvt"] / 2 + cost["max3"] / 2) / slot
    summary = {
        "probe": "attention per-score instruction costs, gfx950",
        "probe_sha": source_hash("probe.hip"),
        "clock_ghz": ghz,
        "ns_per_wave_instruction": cost,
        "slot_ns": slot,
        "slots": {k: v / slot for k, v in cost.items()},
        "slots_per_score": slots,
        "overlap_with_mfma_other_waves": overlap,
        "mfma_forms": {k: {"ns": cost[k], "pflops_1024_simds": PROBE_MFMA_FLOP[k] * 1024 / cost[k] / 1e6}
                       for k in PROBE_MFMA_FLOP},
        "overlap_with_other_mfma_forms": overlap_forms,
        "mfma_interleaved_same_wave": mixed,
    }
    print(json.dumps(summary), flush=True)
    if args.probe_out:
        with open(args.probe_out, "w") as f:
            json.dump(summary, f, indent=1)


def gemm_bench(args, dev):
    """The MXFP4 GEMM of a DiT linear layer (see the module docstring)."""
    import numpy as np
    import torch
    import workloads
    import mxfp4_quantized_attention_amd as mx

    cfg = workloads.GEMM_CONFIGS["gemm"]
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    mode = mx.MODE_UOS if args.mode == "uos" else mx.MODE_OCP
    log(f"[bench] gemm: generating X [{M}][{K}], W [{N}][{K}]")
    x, w = workloads.gemm_inputs("gemm")
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    xg, wg = up(x), up(w)
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    u8 = dict(dtype=torch.uint8, device=dev)
    wc, ws = torch.empty(N * K // 2, **u8), torch.empty(N * K // 32, **u8)
    if L.mxq_quantize(wg.data_ptr(), 1, N, K, 1, mode, wc.data_ptr(), ws.data_ptr(), sp) != 0:
        raise RuntimeError("weight quantization failed")
    xc, xs = torch.empty(M * K // 2, **u8), torch.empty(M * K // 32, **u8)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def launch_x():
        return L.mxq_quantize(xg.data_ptr(), 1, M, K, 1, mode, xc.data_ptr(), xs.data_ptr(), sp)

    def launch_gemm():
        return L.mxgemm_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), ws.data_ptr(), M, N, K,
                                  y.data_ptr(), sp)

    launches = (launch_x, launch_gemm)

    def step(ev=None):
        for i, fn in enumerate(launches):
            if ev is not None:
                ev[i].record(stream)
            st = fn()
            if st != 0:
                raise RuntimeError(f"launch {i} failed: {mx.status_string(st)}")
        if ev is not None:
            ev[len(launches)].record(stream)

    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib, dev)
    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_kernel = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(len(launches))] for ev in events])
    kx, kg = per_kernel.mean(axis=0)
    flop = 2.0 * M * N * K
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (kg * 1e-3) / 1e12
    log(f"[bench] gemm step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s; gemm kernel {kg:.3f} ms -> "
        f"{achieved:.1f} TFLOP/s; quantize X {kx:.3f} ms")
    y_fwd = mx.gemm(xg, wc, ws, N, mode=args.mode)
    torch.cuda.synchronize()
    same = bool(torch.equal(y.view(torch.int16), y_fwd.view(torch.int16)))
    result = {
        "metric": "MXFP4 GEMM TFLOP/s (2*M*N*K) of a DiT linear layer, and % of MI355X MXFP4 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": f"gemm: Y = X W^T, X [{M}][{K}] bf16 quantized per step, W [{N}][{K}] "
                               f"quantized once, {args.mode.upper()}", "M": M, "N": N, "K": K,
                   "mode": args.mode, "parallelism": "single GPU"},
        "pct_of_fp4_peak": 100.0 * value / PEAK_FP4_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP4_TFLOPS,
                     "traffic": measured_traffic("gemm", GEMM_TRAFFIC_FILE, "gemm.hip"), "kernel": "gemm_kernel",
                     "kernel_ms": kg, "algorithmic": f"2*M*N*K = {flop:.4g} FLOP per launch"},
        "quantize_x_ms": kx,
        "step_equals_mxgemm": same,
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = np.sort(np.random.default_rng(13).choice(M, 8192, replace=False))
        log("[bench] cpu baseline (oracle GEMM on 8192 rows)")
        t0 = time.perf_counter()
        ref = oracle.gemm_rows(x, w, M, N, K, mode, rows)
        dt = time.perf_counter() - t0
        got = oracle.bf16_to_f64(y.view(torch.int16).cpu().numpy().view(np.uint16)[rows])
        g = (K / 128 + 16) * 2.0 ** -24
        err = g * ref["absdot"]
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref["out"]) + err, 1e-30))) - 7)
        result["cpu_baseline"] = {
            "value": 2.0 * rows.size * N * K / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(),
            "kind": "oracle", "seconds": dt,
            "sample": f"quantization of W and of 8192 seeded X rows, their exact product (numpy fp64), "
                      f"{dt:.1f} s; FLOP counted as 2*N*K per row",
            "max_diff_over_bound_on_sample": float((np.abs(got - ref["out"]) / (err + ulp)).max()),
        }
    checks = {"step_equals_mxgemm": same}
    if "cpu_baseline" in result:
        checks["oracle_bound_on_sample"] = result["cpu_baseline"]["max_diff_over_bound_on_sample"] <= 1.0
    emit(result, checks)


def varlen_bench(args, dev):
    """mxattn_fwd_varlen on the Wan-style varlen batch (see the module
    docstring)."""
    import numpy as np
    import torch
    import workloads
    import mxfp4_quantized_attention_amd as mx

    cfg = workloads.VARLEN_CONFIGS[args.workload]
    H, d, lengths = cfg["H"], cfg["d"], list(cfg["lengths"])
    mode = mx.MODE_UOS if args.mode == "uos" else mx.MODE_OCP
    pnq = 0 if args.no_pnq else 1
    log(f"[bench] varlen: generating {len(lengths)} sequences {lengths}, H={H}, d={d}")
    q, k, v, cu = workloads.varlen_qkv(lengths, H, d, seed=cfg["seed"], dist=cfg["dist"])
    T = int(cu[-1])
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    qg, kg, vg = up(q), up(k), up(v)
    cug = torch.from_numpy(cu).to(dev)
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    need = mx.varlen_workspace_bytes(len(lengths), T, H, d)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    o = torch.empty_like(qg)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        st = L.mxattn_fwd_varlen(qg.data_ptr(), kg.data_ptr(), vg.data_ptr(), o.data_ptr(), cug.data_ptr(),
                                 len(lengths), T, H, d, None, mode, pnq, 0.0, ws.data_ptr(), need, sp)
        if st != 0:
            raise RuntimeError(f"mxattn_fwd_varlen failed: {mx.status_string(st)}")
        if ev is not None:
            ev[1].record(stream)

    log(f"[bench] warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    call_ms = float(np.mean([ev[0].elapsed_time(ev[1]) for ev in events]))
    flop = 4.0 * H * d * float(sum(n * n for n in lengths))
    value = flop / (ms_per_step * 1e-3) / 1e12
    achieved = flop / (call_ms * 1e-3) / 1e12
    log(f"[bench] varlen step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s (call {call_ms:.3f} ms)")
    # each sequence alone through mxattn_fwd: bit-identical by design
    same = True
    got = o.clone()
    for s_ in range(len(lengths)):
        t0_, t1_ = int(cu[s_]), int(cu[s_ + 1])
        dense = [x[t0_:t1_].permute(1, 0, 2).contiguous().unsqueeze(0) for x in (qg, kg, vg)]
        od = mx.fwd(*dense, mode=args.mode, pnq=bool(pnq))
        same = same and bool(torch.equal(od[0].permute(1, 0, 2).contiguous().view(torch.int16),
                                         got[t0_:t1_].view(torch.int16)))
    torch.cuda.synchronize()
    result = {
        "metric": "MXFP4 attention fwd TFLOP/s (4*H*d*sum N_s^2) of a varlen batch, and % of MI355X MXFP4 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": f"{args.workload}: {len(lengths)} sequences N={lengths} packed T={T}, H={H}, d={d}, "
                               f"non-causal, {args.mode.upper()}{'+PNQ' if pnq else ''}",
                   "lengths": lengths, "T": T, "H": H, "d": d, "mode": args.mode, "pnq": bool(pnq),
                   "parallelism": "single GPU"},
        "pct_of_fp4_peak": 100.0 * value / PEAK_FP4_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP4_TFLOPS, "traffic": None,
                     "kernel": "mxattn_fwd_varlen call (varlen table, K/V quantize, fused kernel)",
                     "kernel_ms": call_ms,
                     "algorithmic": f"4*d FLOP per score element x H*sum(N_s^2) = {flop:.4g} FLOP per call"},
        "step_equals_per_sequence_mxattn_fwd": same,
    }
    if not args.no_cpu_baseline:
        import oracle
        g = np.random.default_rng(17)
        heads = 8
        toks = np.sort(g.choice(T, 2048, replace=False))
        rows = np.array([(t, h) for t in toks for h in range(heads)], np.int64)
        log(f"[bench] cpu baseline (oracle on {rows.shape[0]} (token, head) rows)")
        t0 = time.perf_counter()
        ref = oracle.attn_varlen_rows(q, k, v, cu, H, d, mode, bool(pnq), mx.kv_tile(d), 1.0 / np.sqrt(d), rows,
                                      want_budget=False)
        dt = time.perf_counter() - t0
        seq = np.searchsorted(cu, rows[:, 0], side="right") - 1
        fl = float(np.sum(4.0 * d * (cu[seq + 1] - cu[seq])))
        gb = got.view(torch.int16).cpu().numpy().view(np.uint16)[rows[:, 0], rows[:, 1]]
        r64 = oracle.bf16_to_f64(ref["out_bf16"])
        diff = np.abs(oracle.bf16_to_f64(gb) - r64)
        # per-element bound max(2e-3, one bf16 ulp of the reference); rows
        # flagged near a rounding tie may legitimately exceed it
        a = np.abs(r64)
        ulp = np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
        over = (diff / np.maximum(2e-3, ulp)).max(axis=1)
        flagged = ref["near_tie"]
        result["cpu_baseline"] = {
            "value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(), "kind": "oracle",
            "seconds": dt,
            "sample": f"{rows.shape[0]} seeded (token, head) rows over heads 0..{heads - 1} with K/V quantization "
                      f"of each touched (sequence, head), {dt:.1f} s; FLOP counted as 4*N_s*d per row",
            "max_abs_diff_on_sample": float(diff.max()),
            "max_diff_over_bound_unflagged_rows": float(over[~flagged].max()) if (~flagged).any() else 0.0,
            "flagged_rows": int(flagged.sum()),
        }
    checks = {"step_equals_per_sequence_mxattn_fwd": same}
    if "cpu_baseline" in result:
        checks["oracle_agrees_on_sample"] = result["cpu_baseline"]["max_diff_over_bound_unflagged_rows"] <= 1.0
    emit(result, checks)


def block_bench(args, dev):
    """The Wan attention block from its input activations (see the module
    docstring)."""
    import numpy as np
    import torch
    import workloads
    import mxfp4_quantized_attention_amd as mx

    T, C, H, d = 32760, 5120, 40, 128
    HD = H * d
    mode = mx.MODE_UOS if args.mode == "uos" else mx.MODE_OCP
    pnq = 0 if args.no_pnq else 1
    log(f"[bench] wan_block: generating X [{T}][{C}], W_qkv [{3 * HD}][{C}]")
    x, w = workloads.gemm_inputs(M=T, N=3 * HD, K=C, seed=7)
    up = lambda a: torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
    xg, wg = up(x), up(w)
    del x, w
    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    u8 = dict(dtype=torch.uint8, device=dev)
    wc, ws = torch.empty(3 * HD * C // 2, **u8), torch.empty(3 * HD * C // 32, **u8)
    if L.mxq_quantize(wg.data_ptr(), 1, 3 * HD, C, 1, mode, wc.data_ptr(), ws.data_ptr(), sp) != 0:
        raise RuntimeError("weight quantization failed")
    xc, xs = torch.empty(T * C // 2, **u8), torch.empty(T * C // 32, **u8)
    nbm = (T + 31) // 32
    q = torch.empty((1, H, T, d), dtype=torch.bfloat16, device=dev)
    kc, ks = torch.empty(H * T * d // 2, **u8), torch.empty(H * T * d // 32, **u8)
    vc, vs = torch.empty(H * d * nbm * 16, **u8), torch.empty(H * d * nbm, **u8)
    o = torch.empty_like(q)

    def launch_x():
        return L.mxq_quantize(xg.data_ptr(), 1, T, C, 1, mode, xc.data_ptr(), xs.data_ptr(), sp)

    def launch_qkv():
        return L.mxqkv_proj_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), ws.data_ptr(), T, C, H, d, mode,
                                      q.data_ptr(), kc.data_ptr(), ks.data_ptr(), vc.data_ptr(), vs.data_ptr(), sp)

    def launch_attn():
        return L.mxattn_fwd_kv_quantized(q.data_ptr(), kc.data_ptr(), ks.data_ptr(), vc.data_ptr(), vs.data_ptr(),
                                         1, H, T, d, mode, pnq, 0.0, o.data_ptr(), sp)

    launches = (launch_x, launch_qkv, launch_attn)

    def run(fns, steps, warmup):
        def step(ev=None):
            for i, fn in enumerate(fns):
                if ev is not None:
                    ev[i].record(stream)
                st = fn()
                if st != 0:
                    raise RuntimeError(f"launch {i} failed: {mx.status_string(st)}")
            if ev is not None:
                ev[len(fns)].record(stream)
        for _ in range(warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
        t0 = time.perf_counter()
        for i in range(steps):
            step(events[i])
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        per = np.array([[ev[i].elapsed_time(ev[i + 1]) for i in range(len(fns))] for ev in events]).mean(axis=0)
        return ms, per

    log(f"[bench] fused block: warmup {args.warmup}, timing {args.steps} steps")
    ms_per_step, per = run(launches, args.steps, args.warmup)
    kx, kq, ka = per
    flop_gemm = 2.0 * T * C * 3 * HD
    flop_attn = 4.0 * H * T * T * d
    flop = flop_gemm + flop_attn
    value = flop / (ms_per_step * 1e-3) / 1e12
    log(f"[bench] wan_block step {ms_per_step:.3f} ms -> {value:.1f} TFLOP/s; quantize X {kx:.3f} ms, "
        f"QKV projection {kq:.3f} ms ({flop_gemm / (kq * 1e-3) / 1e12:.1f} TFLOP/s), attention {ka:.3f} ms")

    # unfused: bf16 Y from the GEMM, then mxattn_fwd_strided on its slices
    y = torch.empty((T, 3 * HD), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty((1, H, T, d), dtype=torch.bfloat16, device=dev)
    wsb = mx.workspace_bytes(1, H, T, d)
    wsp = torch.empty(wsb, **u8)
    import ctypes
    s_qkv = (ctypes.c_int64 * 3)(0, d, 3 * HD)
    s_o = (ctypes.c_int64 * 3)(H * T * d, T * d, d)

    def launch_y():
        return L.mxgemm_quantized(xc.data_ptr(), xs.data_ptr(), wc.data_ptr(), ws.data_ptr(), T, 3 * HD, C,
                                  y.data_ptr(), sp)

    def launch_strided():
        base = y.data_ptr()
        return L.mxattn_fwd_strided(base, base + 2 * HD, base + 4 * HD, o2.data_ptr(), 1, H, T, d, s_qkv, s_qkv, s_qkv,
                                    s_o, mode, pnq, 0.0, wsp.data_ptr(), wsb, sp)

    log("[bench] unfused block")
    ms_unfused, per_u = run((launch_x, launch_y, launch_strided), args.steps, args.warmup)
    same = bool(torch.equal(o.view(torch.int16), o2.view(torch.int16)))
    log(f"[bench] unfused step {ms_unfused:.3f} ms (GEMM to bf16 {per_u[1]:.3f} ms, K/V quantize + attention "
        f"{per_u[2]:.3f} ms); outputs identical: {same}")
    result = {
        "metric": "MXFP4 attention block TFLOP/s (QKV projection 2*T*C*3*H*d + attention 4*H*T^2*d), "
                  "and % of MI355X MXFP4 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "mxfp4", "data": "synthetic",
        "config": {"workload": f"wan_block: X [{T}][{C}] bf16 -> QKV projection ({3 * HD} outputs, W quantized once) "
                               f"-> attention H={H} N={T} d={d} non-causal, {args.mode.upper()}"
                               f"{'+PNQ' if pnq else ''}", "T": T, "C": C, "H": H, "d": d, "mode": args.mode,
                   "pnq": bool(pnq), "parallelism": "single GPU"},
        "pct_of_fp4_peak": 100.0 * value / PEAK_FP4_TFLOPS,
        "roofline": {"bound": "mfma", "achieved": flop_attn / (ka * 1e-3) / 1e12, "peak": PEAK_FP4_TFLOPS,
                     "unit": "TFLOP/s", "frac": flop_attn / (ka * 1e-3) / 1e12 / PEAK_FP4_TFLOPS, "traffic": None,
                     "kernel": "attn_fwd_kernel", "kernel_ms": ka,
                     "algorithmic": f"4*d FLOP per score element x H*T^2 = {flop_attn:.4g} FLOP per launch"},
        "qkv_projection": {"ms": kq, "tflops": flop_gemm / (kq * 1e-3) / 1e12,
                           "frac": flop_gemm / (kq * 1e-3) / 1e12 / PEAK_FP4_TFLOPS},
        "quantize_x_ms": kx,
        "unfused_ms_per_step": ms_unfused,
        "fused_equals_unfused": same,
    }
    emit(result, {"fused_equals_unfused": same})


def quantize_sweep(args, dev):
    """The quantizer alone over the sweep sizes (see the module docstring).
    Each size: `warmup` untimed launches, then `steps` launches, each after a
    512 MiB fill that evicts the input from the caches and bracketed by HIP
    events on the launch stream; the median is reported."""
    import numpy as np
    import torch
    import workloads
    import mxfp4_quantized_attention_amd as mx

    L = mx.lib()
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream
    flush = torch.empty(512 << 18, dtype=torch.float32, device=dev)
    cases = [(p, m, 1) for p in (20, 22, 24, 26, 28, 30) for m in ("uos", "ocp")] + [(28, "uos", 0)]
    rows_out, head = [], None
    xs = {}
    for p, mname, axis in cases:
        n = 1 << p
        if p not in xs:
            xs.clear()
            log(f"[bench] sweep: generating 2^{p}")
            xs[p] = torch.from_numpy(workloads.sweep(p).view(np.int16)).to(dev)
        x = xs[p]
        R, C = n >> 10, 1024
        nb = (C if axis == 1 else R) // 32
        nv = R if axis == 1 else C
        codes = torch.empty(nv * nb * 16, dtype=torch.uint8, device=dev)
        scales = torch.empty(nv * nb, dtype=torch.uint8, device=dev)
        mode = mx.MODE_UOS if mname == "uos" else mx.MODE_OCP

        def launch():
            st = L.mxq_quantize(x.data_ptr(), 1, R, C, axis, mode, codes.data_ptr(), scales.data_ptr(), sp)
            if st != 0:
                raise RuntimeError(mx.status_string(st))

        for _ in range(args.warmup):
            launch()
        ts = []
        for _ in range(args.steps):
            flush.fill_(1.0)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            launch()
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        us = float(np.median(ts)) * 1e3
        gbs = 2.53125 * n / (us * 1e-6) / 1e9
        row = {"p": p, "n": n, "mode": mname, "axis": axis, "us": us, "gbs": gbs,
               "pct_of_hbm_peak": 100.0 * gbs / PEAK_HBM_GBS}
        rows_out.append(row)
        log(f"[bench] sweep 2^{p} {mname} axis {axis}: {us:.1f} us, {gbs:.0f} GB/s")
        if p == 30 and mname == "uos" and axis == 1:
            head = row
            host_codes = codes.cpu().numpy()
            host_scales = scales.cpu().numpy()
        if axis == 0:
            rows_codes, rows_scales = codes.cpu().numpy(), scales.cpu().numpy()
    result = {
        "metric": "MXFP4 quantize GB/s (2.53125 B/element: bf16 in, E2M1 codes + E8M0 scales out) "
                  "and % of MI355X HBM peak",
        "value": head["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["us"] * 1e-3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16->mxfp4", "data": "synthetic",
        "config": {"workload": "quantize sweep: n=2^p bf16, p=20..30, viewed [n/1024, 1024], "
                               "UOS/OCP along the contiguous axis, plus UOS along rows at 2^28; "
                               "value at 2^30 UOS", "parallelism": "single GPU"},
        "sweep": rows_out,
        "roofline": {"bound": "hbm", "achieved": head["gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": head["gbs"] / PEAK_HBM_GBS, "traffic": None,
                     "kernel": "quant_stream_kernel",
                     "algorithmic": "2 B read + 0.5 B codes + 1/32 B scale per element"},
    }
    if not args.no_cpu_baseline:
        import oracle
        log("[bench] cpu baseline (oracle quantizer on the 2^30 input)")
        xh = workloads.sweep(30)
        t0 = time.perf_counter()
        oc, os_ = oracle.quantize_bf16(xh.reshape(1, 1 << 20, 1024), 1, 1 << 20, 1024, 1, oracle.MODE_UOS)
        dt = time.perf_counter() - t0
        same = bool(np.array_equal(oc.reshape(-1), host_codes) and np.array_equal(os_.reshape(-1), host_scales))
        del xh, oc, os_
        # the smaller sizes, each timed in full as well
        per_size = []
        for p in (20, 22, 24, 26, 28):
            xp = workloads.sweep(p)
            t1 = time.perf_counter()
            oracle.quantize_bf16(xp.reshape(1, 1 << (p - 10), 1024), 1, 1 << (p - 10), 1024, 1, oracle.MODE_UOS)
            d1 = time.perf_counter() - t1
            per_size.append({"p": p, "seconds": d1, "value": 2.53125 * (1 << p) / d1 / 1e9})
        per_size.append({"p": 30, "seconds": dt, "value": 2.53125 * (1 << 30) / dt / 1e9})
        result["cpu_baseline"] = {
            "value": 2.53125 * (1 << 30) / dt / 1e9, "unit": "GB/s", "cores": oracle.num_threads(),
            "cpu_model": cpu_model(),
            "kind": "oracle", "sample": f"UOS quantization of the 2^30 sweep values (the whole 2^30 case), {dt:.1f} s",
            "seconds": dt,
            "per_size": per_size,
            "bit_exact_vs_gpu_on_sample": same,
        }
        # the row-axis case (blocks along rows at 2^28) on 8192 seeded
        # (column, block) pairs, every column represented
        R, C = 1 << 18, 1024
        x28 = workloads.sweep(28).reshape(R, C)
        g = np.random.default_rng(2028)
        nb = R // 32
        cols = np.concatenate([np.arange(C), g.integers(0, C, 8192 - C)])
        blks = np.concatenate([g.integers(0, nb, C - 2), [0, nb - 1], g.integers(0, nb, 8192 - C)])
        sub = np.stack([x28[32 * b: 32 * b + 32, c] for c, b in zip(cols, blks)])
        del x28
        ec, es = oracle.quantize_bf16(sub, 1, sub.shape[0], 32, 1, oracle.MODE_UOS)
        flat = cols.astype(np.int64) * nb + blks
        same_rows = bool(np.array_equal(rows_codes.reshape(-1, 16)[flat].reshape(-1), ec.reshape(-1))
                         and np.array_equal(rows_scales.reshape(-1)[flat], es.reshape(-1)))
        result["cpu_baseline"]["rows_axis_2^28_bit_exact_on_sample"] = same_rows
    emit(result, {"oracle_bit_exact_at_2^30": same, "oracle_bit_exact_rows_axis_2^28_sample": same_rows}
         if "cpu_baseline" in result else {})


if __name__ == "__main__":
    main()
