"""Benchmark of the RoLA attention forward (librola on one MI355X).

One step = one fused rola_forward over the whole workload (block pooling and
selection, low-rank state, block-sparse attention with the low-rank apply and
merge), on seeded synthetic Wan-shaped bf16 Q/K/V already resident in HBM.
Default workload: Wan2.1-14B-720P attention shape (B=1, 40 heads, head_dim
128, 21x45x80 latent grid, N=75600 -> 75648), topk 0.03 (35 of 1182 key blocks
kept), rank 32.

Prints one JSON line: value = kept-block TFLOP/s of the whole forward, plus the
per-kernel times measured with HIP events on the call's stream inside the
timed region, the roofline of the dominant kernel and the CPU oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "RoLA fwd ms + kept-block TFLOP/s (% MFMA peak), Wan-14B-720P shape, topk 0.03"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
# fp32 vector FMA: the datasheet's 157.3 TFLOP/s (256 CUs x 4 SIMDs x 32 lanes x 2 flop x 2.4 GHz).
# Plain (unpacked) v_fma_f32 reaches it: with two waves per SIMD a probe of independent FMA chains
# issues one wave64 FMA per about 2.3 cycles per SIMD (one wave alone, one per about 4.6).
PEAK_FP32_FMA_TFLOPS = 157.3


def traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", "attn_sparse_lowrank_%s_traffic.json" % workload)


def linear_traffic_file(workload: str) -> str:
    return os.path.join(ROOT, "profiles", "gemm_w8a8_%s_traffic.json" % workload)


ATTN_SOURCES = ("sparse_rank_attention_amd/csrc/rola_kernels.hip", "sparse_rank_attention_amd/csrc/rola_internal.h",
                "sparse_rank_attention_amd/csrc/rola_device.h")
GEMM_SOURCES = ("sparse_rank_attention_amd/csrc/rola_gemm.hip", "sparse_rank_attention_amd/csrc/rola_internal.h",
                "sparse_rank_attention_amd/csrc/rola_device.h")


def kernel_source_hash(sources=ATTN_SOURCES) -> str:
    h = hashlib.sha256()
    for p in sources:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="wan14b_720p")
    ap.add_argument("--topk", type=float, default=None, help="override the workload's keep ratio")
    ap.add_argument("--gate", action="store_true",
                    help="apply the learned output gate to the low-rank term (seeded synthetic gate)")
    ap.add_argument("--complement", action="store_true",
                    help="low-rank state over each query block's unkept blocks instead of all blocks")
    ap.add_argument("--backward", action="store_true",
                    help="time rola_backward (bf16; with --complement, the complement scope) instead of the forward; its own JSON line")
    ap.add_argument("--e4m3-input", action="store_true",
                    help="fp8 workloads: time rola_forward_e4m3 on pre-quantised Q/K/V codes")
    ap.add_argument("--linear", default=None,
                    help="time a w8a8 linear layer instead (wan14b_720p_qkv, wan14b_720p_out, ...)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the MFMA-probe and copy measurements")
    ap.add_argument("--no-graph", action="store_true", help="skip the timing of the forward replayed as a HIP graph")
    ap.add_argument("--cpu-baseline-child", action="store_true", help=argparse.SUPPRESS)
    ap.add_argument("--sample-stride", type=int, default=32,
                    help="CPU baseline with --complement: every n-th query block of head 0")
    ap.add_argument("--cpu-heads", type=int, default=1, help=argparse.SUPPRESS)
    ap.add_argument("--cpu-threads", type=int, default=1, help=argparse.SUPPRESS)
    ap.add_argument("--gpu-out", default=None, help=argparse.SUPPRESS)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this many MiB (a known-size "
                         "kernel for scaling profiler byte counters)")
    return ap.parse_args()


# --------------------------------------------------------------- CPU baseline
def host_cores() -> int:
    """CPU threads the oracle may use: the affinity mask, capped by OMP_NUM_THREADS when set."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(n, int(env))) if env and env.isdigit() else n


def cpu_baseline_child(args):
    """The oracle on the host cores, in a child process with OMP_NUM_THREADS set.

    Default: the whole forward (selection, both branches, every row) of the first
    ``--cpu-heads`` heads, one head per thread, timed; the time scales linearly to
    all heads (heads are independent and of equal size).  The GPU output of the same
    heads (``--gpu-out``, written by the parent) is compared with it: block map bit
    for bit, and max |error| / RMS of the output; for an fp8 workload also against
    the bf16 oracle (untimed).  With ``--complement`` (whose rows sum every unkept
    block state) only every ``--sample-stride``-th query block of head 0 is run,
    with OpenMP over rows, and scaled to the whole workload."""
    import numpy as np

    import oracle
    from sparse_rank_attention_amd import workloads as W

    w = W.WORKLOADS[args.workload]
    if args.topk is not None:
        import dataclasses
        w = dataclasses.replace(w, topk=args.topk)
    fp8 = w.precision == "fp8"
    kb = oracle.keep_blocks(w.topk, w.nb)
    wq, wk = W.make_proj(w)
    gate_w = W.make_gate(w) if args.gate else None
    oracle.lib()
    if args.complement:
        q, k, v = W.make_qkv(w, heads=[0], threads=args.cpu_threads)
        q, k, v = q[0], k[0], v[0]
        t0 = time.perf_counter()
        bmap = oracle.block_map(q, k, w.n_tokens, kb)
        t1 = time.perf_counter()
        qf, kf, vf = (oracle.widen_bf16(x) for x in (q, k, v))
        Sb, zb = oracle.lowrank_block_states(kf[0], vf[0], wk, w.n_tokens, w.grid)
        t2 = time.perf_counter()
        qbs = list(range(0, w.nb, args.sample_stride))
        rows = np.array([n for qb in qbs for n in range(qb * 64, min(qb * 64 + 64, w.n_tokens))])
        sp = oracle.sparse_rows(qf, kf, vf, bmap, w.n_tokens, rows)
        lr = oracle.lowrank_rows_complement(qf[0], wq, Sb, zb, bmap[0], w.grid, rows, gate_w=gate_w)
        t3 = time.perf_counter()
        assert np.isfinite(sp + lr).all()
        per_head = (t1 - t0) + (t2 - t1) + (t3 - t2) * w.n_tokens / rows.size
        print(json.dumps({"total_s": per_head * w.batch * w.heads, "heads": 1, "rows": int(rows.size),
                          "detail": "head 0: selection %.2f s, block states %.2f s, both branches on every %d-th "
                                    "query block (%d rows) %.2f s" % (t1 - t0, t2 - t1, args.sample_stride, rows.size,
                                                                      t3 - t2)}))
        return
    hs = args.cpu_heads
    q, k, v = W.make_qkv(w, heads=list(range(hs)), threads=args.cpu_threads)
    t0 = time.perf_counter()
    bmap, o_ref = oracle.forward(q[0], k[0], v[0], wq, wk, w.n_tokens, kb, w.grid, fp8=fp8, gate_w=gate_w)
    t1 = time.perf_counter()
    rec = {"total_s": (t1 - t0) * w.batch * w.heads / hs, "heads": hs, "sample_s": t1 - t0,
           "detail": "heads 0-%d of %d, every row, %.2f s" % (hs - 1, w.batch * w.heads, t1 - t0)}
    if args.gpu_out:
        g = np.load(args.gpu_out)
        got = ((g["out"].astype(np.uint32) << 16).view(np.float32)).astype(np.float64)[:, :w.n_tokens]
        rec["map_exact"] = bool(np.array_equal(g["map"], bmap))

        def err(ref):
            ref = ref[:, :w.n_tokens]
            return float(np.abs(got - ref).max() / np.sqrt((ref ** 2).mean()))

        def bound_ratio(ref, tol):
            # the per-element bar for a bf16-stored output: tol * rms * (1 + 2^-8)
            # plus half a bf16 ulp of the element (at most 2^-8 |ref|)
            ref = ref[:, :w.n_tokens]
            rms = np.sqrt((ref ** 2).mean())
            return float((np.abs(got - ref) / (tol * rms * (1 + 2.0 ** -8) + 2.0 ** -8 * np.abs(ref))).max())
        rec["err_rms"] = err(o_ref)
        rec["bar"] = 6e-2 if fp8 else 2e-2
        rec["err_over_bound"] = bound_ratio(o_ref, rec["bar"])
        if fp8:
            _, o16 = oracle.forward(q[0], k[0], v[0], wq, wk, w.n_tokens, kb, w.grid, gate_w=gate_w)
            rec["err_rms_vs_bf16_oracle"] = err(o16)
    print(json.dumps(rec))


def cpu_baseline(args, w, kb, out, bmap):
    """Runs cpu_baseline_child on the host cores; ``out``/``bmap`` are the GPU results
    (bf16 output and block map) whose first heads the child checks."""
    import numpy as np
    import tempfile
    cores = host_cores()
    stride = max(args.sample_stride, 32)
    cmd = [sys.executable, os.path.abspath(__file__), "--cpu-baseline-child", "--workload", args.workload,
           "--cpu-threads", str(cores)] + (["--topk", repr(args.topk)] if args.topk else []) \
        + (["--gate"] if args.gate else [])
    tmp = None
    if args.complement:
        cmd += ["--complement", "--sample-stride", str(stride)]
    else:
        hs = min(cores, w.batch * w.heads)
        tmp = tempfile.NamedTemporaryFile(suffix=".npz", delete=False)
        tmp.close()
        np.savez(tmp.name, out=out[0, :hs].view(torch_int16()).cpu().numpy().view(np.uint16),
                 map=bmap[0, :hs].cpu().numpy())
        cmd += ["--cpu-heads", str(hs), "--gpu-out", tmp.name]
    env = dict(os.environ, OMP_NUM_THREADS=str(cores))
    try:
        res = subprocess.run(cmd, env=env, capture_output=True, text=True, timeout=900)
    finally:
        if tmp is not None:
            os.unlink(tmp.name)
    if res.returncode != 0:
        raise RuntimeError("cpu baseline failed: " + res.stderr[-2000:])
    r = json.loads(res.stdout.strip().splitlines()[-1])
    base = {
        "value": w.kept_block_flop(kb) / r["total_s"] / 1e12,
        "unit": "TFLOP/s (kept-block)",
        "ms": r["total_s"] * 1e3,
        "cores": cores,
        "kind": "oracle",
        "sample": ("oracle (C, fp64 branches, OpenMP on %d host threads) on %s: %s; scaled linearly to all %d heads"
                   % (cores, args.workload, r["detail"], w.batch * w.heads)),
    }
    check = {k_: r[k_] for k_ in ("map_exact", "err_rms", "bar", "err_over_bound", "err_rms_vs_bf16_oracle")
             if k_ in r}
    if check:
        check["heads"] = r["heads"]
    return base, check


def torch_int16():
    import torch
    return torch.int16


# -------------------------------------------------------------- backward
def backward_bench(args, w, rola, torch, np, W, qd, kd, vd, wqd, wkd, gd, stream):
    """rola_backward on the workload: W untimed calls, then K timed ones (HIP events on
    the stream), with the forward's block map and a seeded N(0, 1) dL/dO in bf16."""
    cfg = rola.Config(topk=w.topk, rank=w.rank,
                      lowrank_scope=rola.ROLA_LR_COMPLEMENT if args.complement else rola.ROLA_LR_GLOBAL)
    B, H = w.batch, w.heads
    kb = rola.plan(rola.problem(qd, w.grid), cfg).kb
    bmap = torch.empty((B, H, w.nb, kb), dtype=torch.int32, device="cuda")
    rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg, block_idx_out=bmap, stream=stream, gate=gd)
    print("[bench] generating dL/dO", file=sys.stderr, flush=True)
    dod = torch.from_numpy(W.make_dout(w).view(np.int16)).view(torch.bfloat16).cuda()
    def timed_steps(fn, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    bwd = lambda: rola.rola_backward(qd, kd, vd, wqd, wkd, w.grid, cfg, bmap, dod, gate=gd, stream=stream)
    for _ in range(args.warmup):
        bwd()
    torch.cuda.synchronize()
    print("[bench] timing %d backward steps" % args.steps, file=sys.stderr, flush=True)
    ms = timed_steps(bwd, args.steps)  # no per-kernel events inside the headline
    # per-kernel times from a second pass with events around every kernel
    rola.timing_read()
    rola.timing_enable(True)
    ms_events = timed_steps(bwd, args.steps)
    rola.timing_enable(False)
    kern_ms = {name: tot / n for name, (n, tot) in rola.timing_read().items()}
    # the training pair: the forward that keeps O_s and the log-sum-exp, and
    # the backward that takes them, against rola_forward + rola_backward
    print("[bench] timing the training pair", file=sys.stderr, flush=True)
    fwd = lambda: rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg, block_idx_out=bmap, stream=stream, gate=gd)
    saved = {}
    ftrain = lambda: saved.__setitem__("t", rola.rola_forward_train(qd, kd, vd, wqd, wkd, w.grid, cfg,
                                                                    block_idx_out=bmap, stream=stream, gate=gd))
    ftrain()
    _, os_, lse = saved["t"]
    bsaved = lambda: rola.rola_backward(qd, kd, vd, wqd, wkd, w.grid, cfg, bmap, dod, gate=gd, stream=stream,
                                        saved=(os_, lse))
    for _ in range(max(1, args.warmup)):
        fwd(); ftrain(); bsaved()
    pair = {"fwd_ms": timed_steps(fwd, args.steps), "fwd_train_ms": timed_steps(ftrain, args.steps),
            "bwd_ms": ms, "bwd_saved_ms": timed_steps(bsaved, args.steps)}
    pair = {k_: round(v_, 4) for k_, v_ in pair.items()}
    pair["step_ms_recompute"] = round(pair["fwd_ms"] + pair["bwd_ms"], 4)
    pair["step_ms_saved"] = round(pair["fwd_train_ms"] + pair["bwd_saved_ms"], 4)
    pairs = w.nb * kb * B * H
    unit = 2.0 * 64 * 64 * w.head_dim  # one 64x64xD product
    total = 5 * unit * pairs            # S, dP, dV, dQ, dK per kept block pair
    rec = {
        "metric": "RoLA bwd ms + kept-block TFLOP/s, Wan-14B-720P shape, topk 0.03",
        "value": round(total / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (kept-block, whole backward: 5 products of 2*64*64*D flop per kept block pair)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded Wan-shaped smooth field + noise Q/K, N(0,1) V and dL/dO; no weights)",
        "config": {"workload": w.name, "batch": B, "heads": H, "head_dim": w.head_dim, "grid": list(w.grid),
                   "n_tokens": w.n_tokens, "topk": w.topk, "kb": kb, "nb": w.nb, "rank": w.rank,
                   "output_gate": bool(args.gate), "pass": "backward",
                   "lowrank_scope": "complement" if args.complement else "global"},
        "bwd_ms": round(ms, 4),
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in sorted(kern_ms.items())},
        "kernel_ms_pass": {"steps": args.steps, "bwd_ms": round(ms_events, 4),
                           "how": "second pass with HIP events around every kernel; the headline ms has none"},
        "training_pair": pair,
        "cpu_baseline": None,
    }
    # the two sparse kernels against the bf16 MFMA peak, on their algorithmic
    # products (dq: S, dP, dQ; dkv: S, dP, dV, dK)
    roof = {}
    for name, prods in (("bwd_dq", 3), ("bwd_dkv", 4)):
        if name in kern_ms:
            tf = prods * unit * pairs / (kern_ms[name] * 1e-3) / 1e12
            roof[name] = {"bound": "mfma", "achieved": round(tf, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": None}
    dom = max(roof, key=lambda k_: kern_ms[k_]) if roof else None
    if dom:
        rec["roofline"] = dict(kernel=dom, **roof[dom])
        rec["sparse_rooflines"] = roof
    print(json.dumps(rec), flush=True)


def linear_bench(args, rola, torch, np, W):
    """One w8a8 linear layer per step on the resident bf16 activations: per-token
    quantisation (rola_quant_rows) then the scaled fp8 GEMM (rola_gemm_w8a8),
    with the weights quantised per output channel beforehand (untimed)."""
    lw = W.LINEAR[args.linear]
    print("[bench] generating %s inputs" % lw.name, file=sys.stderr, flush=True)
    xb = W.make_linear_x(lw)
    wb, bias = W.make_linear_w(lw)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    xd, wd, bd = dev(xb), dev(wb), torch.from_numpy(bias).cuda()
    del xb
    stream = torch.cuda.Stream()
    wc, sw = rola.rola_quant_rows(wd, stream=stream)
    xc = torch.empty((lw.tokens, lw.d_in), dtype=torch.uint8, device="cuda")
    sx = torch.empty(lw.tokens, dtype=torch.float32, device="cuda")
    y = torch.empty((lw.tokens, lw.d_out), dtype=torch.bfloat16, device="cuda")

    def step():
        rola.rola_quant_rows(xd, xc, sx, stream=stream)
        rola.rola_gemm_w8a8(xc, sx, wc, sw, bd, out=y, stream=stream)

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: %d bytes read, %d written" % (nbytes, nbytes), file=sys.stderr, flush=True)
        del src, dst

    rola.timing_enable(True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    rola.timing_enable(False)
    rola.timing_read()
    print("[bench] timing %d layer steps" % args.steps, file=sys.stderr, flush=True)
    rola.timing_enable(True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    rola.timing_enable(False)
    ms = e0.elapsed_time(e1) / args.steps
    kern_ms = {name: tot / n for name, (n, tot) in rola.timing_read().items()}
    gemm_tf = lw.flop / (kern_ms["gemm_w8a8"] * 1e-3) / 1e12
    qbytes = lw.tokens * (lw.d_in * 3 + 4)  # bf16 in, e4m3 out, fp32 scale
    traffic = {"gemm_w8a8": None, "quant_rows": None}
    tfile = linear_traffic_file(lw.name)
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash(GEMM_SOURCES) and tr.get("workload") == lw.name:
            traffic = {k_: round(v_["total"]) for k_, v_ in tr["bytes_per_launch"].items()}
    rec = {
        "metric": "w8a8 linear layer TFLOP/s (per-token e4m3 quantisation + fp8 GEMM)",
        "value": round(lw.flop / (ms * 1e-3) / 1e12, 1),
        "unit": "TFLOP/s (2*tokens*d_in*d_out per layer call)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) activations with 1% outlier channels x8, N(0,1/d_in) weights; no checkpoint)",
        "config": {"workload": lw.name, "tokens": lw.tokens, "d_in": lw.d_in, "d_out": lw.d_out,
                   "out_dtype": "bf16", "bias": True},
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in sorted(kern_ms.items())},
        "roofline": {"kernel": "gemm_w8a8", "bound": "mfma", "achieved": round(gemm_tf, 1),
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": round(gemm_tf / PEAK_FP8_TFLOPS, 4),
                     "traffic": traffic["gemm_w8a8"]},
        "quant_roofline": {"kernel": "quant_rows", "bound": "hbm",
                           "achieved": round(qbytes / (kern_ms["quant_rows"] * 1e-3) / 1e9, 1),
                           "peak": PEAK_HBM_GBS, "unit": "GB/s",
                           "frac": round(qbytes / (kern_ms["quant_rows"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                           "traffic": traffic["quant_rows"]},
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        import oracle
        rows = np.arange(0, lw.tokens, max(1, lw.tokens // 2048))[:2048]
        xs = W.make_linear_x(lw, rows)
        t0 = time.perf_counter()
        oracle.linear_w8a8(xs, wb, bias)
        dt = time.perf_counter() - t0
        sample_flop = 2.0 * len(rows) * lw.d_in * lw.d_out
        rec["cpu_baseline"] = {"value": round(sample_flop / dt / 1e12, 6), "unit": "TFLOP/s", "cores": _omp_threads(),
                               "kind": "oracle",
                               "sample": "%d of %d token rows (whole layer incl. weight quantisation), %.1f s"
                                         % (len(rows), lw.tokens, dt)}
    print(json.dumps(rec), flush=True)


def _omp_threads() -> int:
    n = os.environ.get("OMP_NUM_THREADS")
    return int(n) if n and n.isdigit() else (os.cpu_count() or 1)


# -------------------------------------------------------------------- main
def measured_peaks(rola, torch, stream, dtype):
    """Sustained MFMA rate (probe kernel of independent MFMA chains on every
    SIMD) and device-to-device copy bandwidth, timed with events on `stream`;
    best of three runs each.  The shader clock comes from the probe's core and
    reference clock counters (reference clock taken as 100 MHz)."""
    sink = torch.zeros(2048, dtype=torch.float32, device="cuda")
    out = {"mfma_tflops": {}}
    for name, prec, iters in (("bf16", rola.ROLA_PREC_BF16, 20000), ("fp8", rola.ROLA_PREC_FP8, 10000)):
        best = 0.0
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            flop = rola.mfma_probe(prec, iters, sink, stream=stream)
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, flop / (e0.elapsed_time(e1) * 1e-3) / 1e12)
        out["mfma_tflops"][name] = round(best, 1)
        ticks = sink[1024:1026].cpu().tolist()
        out["clock_ghz_" + name] = round(ticks[0] / ticks[1] * 0.1, 3) if ticks[1] > 0 else None
    nbytes = 1 << 30
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    best = 0.0
    with torch.cuda.stream(stream):
        for _ in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            dst.copy_(src)
            e1.record(stream)
            torch.cuda.synchronize()
            best = max(best, 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    out["copy_gbs"] = round(best, 1)
    out["copy_bytes"] = 2 * nbytes
    out["spec"] = {"mfma_tflops": PEAK_FP8_TFLOPS if dtype == "fp8" else PEAK_BF16_TFLOPS, "hbm_gbs": PEAK_HBM_GBS}
    del src, dst
    return out


def main():
    args = parse()
    if args.cpu_baseline_child:
        cpu_baseline_child(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only (use --gpus 1): the RoLA forward shards by heads "
              "with no collective, so N GPUs each run H/N heads of the same kernels.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from sparse_rank_attention_amd import rola, workloads as W

    if args.linear:
        linear_bench(args, rola, torch, np, W)
        return
    w = W.WORKLOADS[args.workload]
    if args.topk is not None:
        import dataclasses
        w = dataclasses.replace(w, topk=args.topk)
    fp8 = w.precision == "fp8"
    print("[bench] generating %s inputs" % w.name, file=sys.stderr, flush=True)
    q, k, v = W.make_qkv(w)
    wq, wk = W.make_proj(w)
    dev = lambda x: torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    qd, kd, vd = dev(q), dev(k), dev(v)
    del q, k, v
    wqd, wkd = torch.from_numpy(wq).cuda(), torch.from_numpy(wk).cuda()
    gd = torch.from_numpy(W.make_gate(w)).cuda() if args.gate else None
    cfg = rola.Config(topk=w.topk, rank=w.rank, precision=rola.ROLA_PREC_FP8 if fp8 else rola.ROLA_PREC_BF16,
                      lowrank_scope=rola.ROLA_LR_COMPLEMENT if args.complement else rola.ROLA_LR_GLOBAL)
    if args.backward:
        if fp8:
            print("bench.py --backward: the backward is bf16", file=sys.stderr)
            sys.exit(2)
        backward_bench(args, w, rola, torch, np, W, qd, kd, vd, wqd, wkd, gd, torch.cuda.current_stream())
        return
    e4m3 = args.e4m3_input
    if e4m3 and not fp8:
        print("bench.py --e4m3-input needs an fp8 workload (e.g. --workload wan14b_720p_fp8)", file=sys.stderr)
        sys.exit(2)
    codes = scales = None
    if e4m3:
        # the caller's side: per-(head, 64-token block) e4m3 codes and scales by
        # the absmax rule, made with torch ops before the timed region
        codes, scales = [], []
        valid = (torch.arange(w.n_pad, device="cuda") < w.n_tokens).view(1, 1, w.nb, 64, 1)
        for x in (qd, kd, vd):
            xf = x.float().view(w.batch, w.heads, w.nb, 64, w.head_dim) * valid
            amax = xf.abs().amax(dim=(3, 4))
            inv = torch.where(amax > 0, 448.0 / torch.where(amax > 0, amax, torch.ones_like(amax)),
                              torch.ones_like(amax))
            scales.append(torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).contiguous())
            codes.append((xf * inv[..., None, None]).to(torch.float8_e4m3fn).view(torch.uint8)
                         .view(w.batch, w.heads, w.n_pad, w.head_dim).contiguous())
            del xf
        torch.cuda.synchronize()

    def fwd(on=None):
        st_ = stream if on is None else on
        if e4m3:
            rola.rola_forward_e4m3(qd, kd, vd, *codes, *scales, wqd, wkd, w.grid, cfg, out=out, stream=st_,
                                   gate=gd)
        else:
            rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg, out=out, stream=st_, gate=gd)

    dominant = "attn8_sparse_lowrank" if fp8 else "attn_sparse_lowrank"
    peak = PEAK_FP8_TFLOPS if fp8 else PEAK_BF16_TFLOPS
    out = torch.empty_like(qd)
    stream = torch.cuda.current_stream()
    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print("[bench] copy calibration: %d bytes read, %d written" % (nbytes, nbytes), file=sys.stderr, flush=True)
        del src, dst
    print("[bench] warmup %d" % args.warmup, file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        fwd()
    torch.cuda.synchronize()

    # the timed region: plain forwards between two stream events (no per-kernel events)
    print("[bench] timing %d steps" % args.steps, file=sys.stderr, flush=True)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        fwd()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps

    # the same forward captured once as a HIP graph and replayed: one graph launch
    # per step instead of the binding's per-kernel launches (the call only
    # launches kernels, so it captures as it is); reported next to the headline
    graph = None
    if not args.no_graph:
        print("[bench] graph capture and %d replays" % args.steps, file=sys.stderr, flush=True)
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            fwd(side)  # the capture stream's workspace, made before the capture
        stream.wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            fwd(side)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eg0, eg1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        eg0.record(stream)
        for _ in range(args.steps):
            g.replay()
        eg1.record(stream)
        torch.cuda.synchronize()
        graph = {"steps": args.steps, "ms_per_step": round(eg0.elapsed_time(eg1) / args.steps, 4)}
        del g

    # per-kernel breakdown: the same number of forwards again, with the library's
    # HIP events around each kernel on the call's stream (event pool made beforehand)
    print("[bench] per-kernel breakdown, %d steps" % args.steps, file=sys.stderr, flush=True)
    rola.timing_enable(True)
    fwd()
    torch.cuda.synchronize()
    rola.timing_read()
    e2, e3 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e2.record(stream)
    for _ in range(args.steps):
        fwd()
    e3.record(stream)
    torch.cuda.synchronize()
    rola.timing_enable(False)
    ms_breakdown = e2.elapsed_time(e3) / args.steps
    kernels = rola.timing_read()
    kern_ms = {name: tot / n for name, (n, tot) in kernels.items()}

    kb = rola.plan(rola.problem(qd, w.grid), cfg).kb
    kept = w.kept_block_flop(kb)
    dense = w.dense_equiv_flop()
    t_attn = kern_ms[dominant] * 1e-3
    achieved = kept / t_attn / 1e12
    traffic = None
    tfile = traffic_file(w.name)
    if os.path.exists(tfile) and args.topk is None and not args.gate and not args.complement and not e4m3:
        with open(tfile) as f:
            tr = json.load(f)
        if tr.get("kernel_source_hash") == kernel_source_hash() and tr.get("workload") == w.name:
            traffic = round(tr["bytes_per_launch"]["total"])
    # algorithmic HBM bytes of the streaming pass: read Q, K, V once; in fp8 mode
    # also write the e4m3 codes of K and V (one byte per element), with bf16
    # operands (and the bf16 output used here) the fp16 copy of V (two bytes)
    n_tok = w.batch * w.heads * w.n_tokens
    # (complement scope: plus the per-block states it writes, bf16 S and fp32 z)
    quant_in_pass1 = fp8 and not e4m3
    pass1_name = "pass1_pool_%s%s" % ("blkstate" if args.complement else "state", "_quant8" if quant_in_pass1 else "")
    pass1_bytes = 3 * n_tok * w.head_dim * 2 + (2 * n_tok * w.head_dim if quant_in_pass1 else 0) \
        + (n_tok * w.head_dim * 2 if not fp8 else 0) \
        + (w.batch * w.heads * w.nb * (w.head_dim * 64 + 128) if args.complement else 0)
    pass1_ms = kern_ms.get(pass1_name)
    rec = {
        "metric": METRIC,
        "value": round(kept / (ms * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s (kept-block, whole forward)",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3" if fp8 else "bf16",
        "data": "synthetic (seeded Wan-shaped smooth field + noise Q/K, N(0,1) V; no weights)",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "head_dim": w.head_dim,
                   "grid": list(w.grid), "n_tokens": w.n_tokens, "topk": w.topk, "kb": kb, "nb": w.nb,
                   "rank": w.rank, "output_gate": bool(args.gate),
                   "lowrank_scope": "complement" if args.complement else "global",
                   **({"input": "pre-quantised e4m3 Q/K/V codes and block scales"} if e4m3 else {})},
        "fwd_ms": round(ms, 4),
        "dense_equiv_tflops": round(dense / (ms * 1e-3) / 1e12, 1),
        "kept_block_tflops": round(kept / (ms * 1e-3) / 1e12, 1),
        "kernel_ms": {k_: round(v_, 4) for k_, v_ in sorted(kern_ms.items())},
        "graph_replay": graph,
        "kernel_ms_pass": {"steps": args.steps, "fwd_ms": round(ms_breakdown, 4),
                           "how": "second pass with HIP events around every kernel; the headline ms has none"},
        "roofline": {"kernel": dominant, "bound": "mfma", "achieved": round(achieved, 1),
                     "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                     "traffic": traffic},
    }
    if e4m3 and "image8" in kern_ms:
        ibytes = 4 * n_tok * w.head_dim  # read K, V codes; write their tile images
        gbs = ibytes / (kern_ms["image8"] * 1e-3) / 1e9
        rec["image8_roofline"] = {"kernel": "image8", "bound": "hbm", "achieved": round(gbs, 1),
                                  "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    if pass1_ms:
        gbs = pass1_bytes / (pass1_ms * 1e-3) / 1e9
        rec["pass1_roofline"] = {"kernel": pass1_name, "bound": "hbm", "achieved": round(gbs, 1),
                                 "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    if "scores" in kern_ms:
        # pooled block scores: one fp32 FMA per (query block, key block, dim), a
        # pinned sequential chain per element, on plain v_fma_f32
        sflop = 2.0 * w.batch * w.heads * w.nb * w.nb * w.head_dim
        tf = sflop / (kern_ms["scores"] * 1e-3) / 1e12
        rec["scores_roofline"] = {"kernel": "scores", "bound": "alu", "achieved": round(tf, 1),
                                  "peak": PEAK_FP32_FMA_TFLOPS, "unit": "TFLOP/s",
                                  "frac": round(tf / PEAK_FP32_FMA_TFLOPS, 4)}
    if not args.no_peaks:
        print("[bench] measured peaks (MFMA probe, device copy)", file=sys.stderr, flush=True)
        rec["measured_peaks"] = measured_peaks(rola, torch, stream, "fp8" if fp8 else "bf16")
        mp = rec["measured_peaks"]
        rec["roofline"]["frac_of_measured"] = round(achieved / mp["mfma_tflops"]["fp8" if fp8 else "bf16"], 4)
        if "pass1_roofline" in rec:
            rec["pass1_roofline"]["frac_of_measured"] = round(rec["pass1_roofline"]["achieved"] / mp["copy_gbs"], 4)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle on %d host threads)" % host_cores(), file=sys.stderr, flush=True)
        bmap = torch.empty((w.batch, w.heads, w.nb, kb), dtype=torch.int32, device="cuda")
        if e4m3:
            rola.rola_forward_e4m3(qd, kd, vd, *codes, *scales, wqd, wkd, w.grid, cfg, out=out, stream=stream,
                                   gate=gd, block_idx_out=bmap)
        else:
            rola.rola_forward(qd, kd, vd, wqd, wkd, w.grid, cfg, out=out, stream=stream, gate=gd, block_idx_out=bmap)
        torch.cuda.synchronize()
        rec["cpu_baseline"], check = cpu_baseline(args, w, kb, out, bmap)
        if check:
            rec["oracle_check"] = check
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
