"""Throughput of the persistent event-tensor MoE kernel on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload prefill]
                    [--mode static|dedicated] [--combine atomic|ordered]
                    [--secondary | --no-secondary] [--no-cpu-baseline]

A step is one call of the library on one batch of synthetic input already resident in
HBM: for the headline "prefill" workload, T=4096 tokens through two chained MoE layers
(H=4096, E=64, k=6, F=1408, bfloat16), i.e. every stage of the path -- RMSNorm,
router, top-k and softmax, counts, scan and permutation, gate/up and down expert tiles
released by the event counters, and the weighted combine -- in one kernel launch.
Steps are timed with HIP events recorded on the stream the kernel is launched on.

Prints one JSON line.  value = tokens per second of the step (T / step time).
roofline: the prefill kernel is MFMA-bound: achieved = algorithmic bfloat16 expert flops
(T*k*6*H*F per layer, no padded rows) / average launch time, against 2.5 PFLOP/s;
decode and fine-grained lines are HBM-bound: algorithmic bytes = expert weights the
run's routing touches + router weights + x and out, against 8 TB/s.
cpu_baseline: the CPU oracle on a bounded sample of the same workload.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from moe_layer_scheduling_amd import binding, synth  # noqa: E402

METRIC = "MoE layer tokens/sec + % of roofline (HBM GB/s decode, MFMA TFLOP/s prefill)"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "moe_kernel_hbm_traffic.txt")
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def time_steps(fn, steps, warmup, flush=None):
    """Run fn warmup times, then time exactly `steps` calls with one event pair per
    call on the current stream.  With `flush`, every timed call is preceded by an
    untimed flush() outside its event pair.  Returns (ms per step from the outer events,
    mean launch ms from the per-call events, list of per-call ms)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    outer0, outer1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    # The GPU spins (untimed) while the host queues the timed calls, so that no event
    # pair waits for the host to submit its kernel: a call shorter than its host-side
    # launch path (split-K's 30 us) would otherwise be timed with that path included.
    torch.cuda._sleep(10_000_000)
    outer0.record(stream)
    for a, b in ev:
        if flush is not None:
            flush()
        a.record(stream)
        fn()
        b.record(stream)
    outer1.record(stream)
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    return outer0.elapsed_time(outer1) / steps, float(np.mean(per)), per


_FLUSH = []


def cache_flush():
    """Read 1 GiB of scratch (a reduction kernel): evicts the 256 MiB Infinity Cache and
    the L2s, so that the next call reads its operands from HBM.  A read rather than a
    write, so that no dirty lines are left whose write-back would compete with the timed
    call's reads."""
    if not _FLUSH:
        _FLUSH.append(torch.ones(1 << 28, dtype=torch.float32, device="cuda"))
    _FLUSH[0].sum()


def cold_times(fn, steps):
    """Median, p10 and p90 (ms) of per-call times, each call after a cache flush."""
    _, _, per = time_steps(fn, steps, 1, flush=cache_flush)
    return {"launch_ms_median": float(np.median(per)), "launch_ms_p10": float(np.percentile(per, 10)),
            "launch_ms_p90": float(np.percentile(per, 90)), "calls": steps}


def moe_inputs(cfg, T, call=0):
    layers = synth.make_layers(cfg)
    x = synth.make_x(cfg, T, call=call)
    ld = [{k: v.cuda() for k, v in l.items()} for l in layers]
    return layers, x, ld


def routed_counts(xd, ld, cfg, ws, mode, combine):
    _, info = binding.moe_layer(xd, ld, cfg.top_k, eps=cfg.eps, mode=mode, combine=combine,
                                workspace=ws, return_routing=True)
    torch.cuda.synchronize()
    return info["expert_counts"].cpu().numpy()


def expert_bytes(cfg):
    es = 2 if cfg.dtype == "bf16" else 4
    return 3 * cfg.hidden * cfg.ffn * es


def algorithmic_work(cfg, T, counts):
    """Algorithmic work of one call (no padded rows, no re-reads): expert flops (every
    (token, slot) pair costs the gate, up and down products, 2*H*F flops each), router
    flops, and the bytes that must move: the weights of every expert that receives a
    token in some layer, the router weights, and x in / out per layer.  counts: the
    per-layer expert counts of the call's routing.  Returns (flops_expert, flops_router,
    bytes, expert-layers touched)."""
    es = 2 if cfg.dtype == "bf16" else 4
    touched = int(sum((np.asarray(c) > 0).sum() for c in counts))
    flops = cfg.layers * T * cfg.top_k * 6 * cfg.hidden * cfg.ffn
    flops_router = cfg.layers * 2 * T * cfg.hidden * cfg.experts
    nbytes = (touched * expert_bytes(cfg) + cfg.layers * cfg.experts * cfg.hidden * es +
              2 * T * cfg.hidden * es * cfg.layers)
    return flops, flops_router, nbytes, touched


def bench_moe(cfg, T, steps, warmup, mode, combine, with_cpu=False, trace_out=None):
    log(f"[bench] {cfg.name}: drawing inputs T={T}")
    layers, x, ld = moe_inputs(cfg, T)
    xd = x.cuda()
    dt = synth.torch_dtype(cfg.dtype)
    ws = binding.MoEWorkspace(T, cfg.hidden, cfg.experts, cfg.top_k, cfg.ffn, cfg.layers, dt,
                              combine)
    counts = routed_counts(xd, ld, cfg, ws, mode, combine)
    out = torch.empty(0)

    def step():
        nonlocal out
        out = binding.moe_layer(xd, ld, cfg.top_k, eps=cfg.eps, mode=mode, combine=combine,
                                workspace=ws)

    log(f"[bench] {cfg.name}: timing {steps} steps")
    ms, launch_ms, per = time_steps(step, steps, warmup)
    cold = cold_times(step, max(5, steps // 2))
    st = ws.status()
    if st != 0:
        raise RuntimeError(f"device status {st}")
    trace_summary = None
    if trace_out:  # one extra call, outside the timed region, with per-task records
        from moe_layer_scheduling_amd import trace

        binding.moe_layer(xd, ld, cfg.top_k, eps=cfg.eps, mode=mode, combine=combine, workspace=ws,
                          flags=binding.FLAG_TRACE)
        rec = ws.read_trace()
        trace_summary = trace.summarize(rec)
        trace.chrome_trace(rec, trace_out)
        with open(trace_out + ".summary.json", "w") as f:
            json.dump(trace_summary, f, indent=1)
    flops_bf16, flops_router, bytes_alg, touched = algorithmic_work(cfg, T, counts)
    res = {
        "tokens": T, "ms_per_step": ms, "launch_ms": launch_ms,
        "launch_ms_p10": float(np.percentile(per, 10)), "launch_ms_p90": float(np.percentile(per, 90)),
        "tokens_per_s": T / (ms / 1e3),
        "tflops_bf16": flops_bf16 / (launch_ms / 1e3) / 1e12,
        "gbs_alg": bytes_alg / (launch_ms / 1e3) / 1e9,
        "flops_bf16": flops_bf16, "flops_router_fp32": flops_router, "bytes_alg": bytes_alg,
        "experts_touched": touched,
        "cold": dict(cold, tokens_per_s=T / cold["launch_ms_median"] * 1e3),
    }
    if trace_summary:
        res["trace"] = trace_summary
    res["mfma_frac"] = res["tflops_bf16"] / PEAK_BF16_TFLOPS
    res["hbm_frac"] = res["gbs_alg"] / PEAK_HBM_GBS
    if with_cpu:
        res["cpu"] = cpu_baseline(cfg, layers, x)
    del ws, ld, xd
    torch.cuda.empty_cache()
    return res


def cpu_baseline(cfg, layers, x, budget_s=20.0):
    """The oracle as it stands, on a bounded sample: the first n tokens through every
    layer (per-token outputs do not depend on the other tokens), n doubled until the
    run takes a few seconds, then extrapolated to tokens/s."""
    from oracle import moe as om

    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover - threadpoolctl missing
        threads = os.cpu_count()
    lnp = synth.layers_as_numpy(layers)
    xn = synth.as_numpy(x)
    n, spent = 4, 0.0
    while True:
        t0 = time.perf_counter()
        om.moe_forward(xn[:n], lnp, cfg.top_k, cfg.eps, cfg.dtype)
        spent = time.perf_counter() - t0
        if spent > budget_s / 3 or n >= x.shape[0]:
            break
        n = min(2 * n, x.shape[0])
    return {"value": n / spent, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {x.shape[0]} tokens through all {cfg.layers} layer(s) "
                      f"of the {cfg.name} workload, numpy float64, {spent:.1f} s"}


def bench_splitk(steps, warmup, mode="static", copies=4):
    cfg = synth.SPLITK
    A, B = synth.make_splitk()
    Ad = A.cuda()
    Bs = [B.cuda()]
    for _ in range(copies - 1):  # rotate B so each call reads it from HBM, not the MALL
        Bs.append(Bs[0].clone())
    ws = binding.SplitKWorkspace(cfg["M"], cfg["N"], cfg["split_k"])
    it = [0]

    def step():
        binding.splitk_gemm(Ad, Bs[it[0] % copies], cfg["split_k"], mode=mode, workspace=ws)
        it[0] += 1

    # every copy of B is touched before the timed calls (first touches pay page-table walks)
    ms, launch_ms, per = time_steps(step, steps, max(warmup, copies))
    cold = cold_times(step, max(5, steps // 2))
    M, N, K = cfg["M"], cfg["N"], cfg["K"]
    nbytes = M * K * 2 + K * N * 2 + M * N * 4
    return {"ms_per_step": ms, "launch_ms": launch_ms, "gbs_alg": nbytes / (launch_ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (launch_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
            "tflops_bf16": 2 * M * N * K / (launch_ms / 1e3) / 1e12, "bytes_alg": nbytes,
            "mode": mode, "cold": cold}


def bench_attention(steps, warmup, mode, lens, label):
    """Variable-context decode attention on one call's worth of synthetic cache: batch,
    heads and lengths from synth.ATTN (or the given lengths).  Algorithmic bytes: every
    request's K and V rows once (L_b * H_kv * 128 * 2 bytes each), q in, out (float32)."""
    cfg = synth.ATTN
    HKV, G, D = cfg["kv_heads"], cfg["group"], cfg["head_dim"]
    lens = torch.as_tensor(lens, dtype=torch.int32)
    B = lens.numel()
    q, k, v, start = synth.make_attention(lens, HKV, G, head_dim=D, seed=cfg["seed"])
    qd, kd, vd, sd, ld = q.cuda(), k.cuda(), v.cuda(), start.cuda(), lens.cuda()
    ws = binding.AttnWorkspace(B, HKV, G, int(lens.sum()), D)
    out = torch.empty(0)

    def step():
        nonlocal out
        out = binding.decode_attention(qd, kd, vd, ld, sd, mode=mode, workspace=ws)

    log(f"[bench] attention {label}: timing {steps} steps")
    ms, launch_ms, _ = time_steps(step, steps, warmup)
    cold = cold_times(step, max(5, steps // 2))
    st = ws.status()
    if st != 0:
        raise RuntimeError(f"device status {st}")
    total = int(lens.sum())
    nbytes = total * HKV * D * 2 * 2 + B * HKV * G * D * 2 + B * HKV * G * D * 4
    del qd, kd, vd, ws
    torch.cuda.empty_cache()
    return {"requests": B, "tokens": total, "launch_ms": launch_ms, "gbs_alg": nbytes / (launch_ms / 1e3) / 1e9,
            "hbm_frac": nbytes / (launch_ms / 1e3) / 1e9 / PEAK_HBM_GBS, "bytes_alg": nbytes,
            "requests_per_s": B / (ms / 1e3), "mode": mode, "cold": cold}


def source_hash():
    """sha256 over the HIP sources of the library (names and contents, sorted): the
    identity of the kernels that counter measurements belong to."""
    import glob
    import hashlib

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_layer_scheduling_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(key):
    """HBM bytes per launch of the MoE kernel for workload `key`, from the committed
    rocprofv3 counter summary (FETCH_SIZE + WRITE_SIZE, scaled by the plain-copy
    calibration); None when there is none or when the kernel sources have changed since
    the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            text = f.read()
        start = text.index("BEGIN-JSON") + len("BEGIN-JSON")
        data = json.loads(text[start:text.index("END-JSON")])
    except (OSError, ValueError):
        return None
    if data.get("source_sha256") != source_hash():
        return None
    entry = data.get("per_launch", {}).get(key)
    return None if entry is None else int(entry["fetch_bytes"] + entry["write_bytes"])


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain device copy of known size (one elementwise kernel reading nbytes and writing
    nbytes per call): the reference against which the L2 fetch/write byte counters of the
    MoE kernel are scaled to HBM bytes."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    ms, launch_ms, _ = time_steps(lambda: torch.mul(src, 1.0, out=dst), reps, 1)
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "calls": reps + 1,
            "launch_ms": launch_ms, "gbs": 2 * nbytes / (launch_ms / 1e3) / 1e9}


def achievable_peaks(cfg, T):
    """Context for the nominal peaks: what the vendor library kernels reach on this GPU.
    A streaming read (one float32 reduction over 1 GiB), a streaming copy (1 GiB read and
    1 GiB written by one elementwise kernel), a square bf16 GEMM (8192^3,
    hipBLASLt through torch.matmul), and the dense GEMMs that hold one call's expert
    arithmetic: every routed row of a layer in one GEMM per projection ([T*k, H] x [H, 2F]
    and [T*k, F] x [F, H]), for every layer, with no routing, gather or combine."""
    reps = 5
    cache_flush()  # allocates the 1 GiB buffer
    buf = _FLUSH[0]
    _, read_ms, _ = time_steps(lambda: buf.sum(), reps, 2)
    dst = torch.empty_like(buf)
    _, copy_ms, _ = time_steps(lambda: torch.mul(buf, 1.0, out=dst), reps, 2)
    del dst
    n = 8192
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    _, sq_ms, _ = time_steps(lambda: torch.matmul(a, b), reps, 2)
    del a, b
    rows, H, F = T * cfg.top_k, cfg.hidden, cfg.ffn
    xg = torch.randn(rows, H, device="cuda").to(torch.bfloat16)
    wgu = torch.randn(H, 2 * F, device="cuda").to(torch.bfloat16)
    hd = torch.randn(rows, F, device="cuda").to(torch.bfloat16)
    wd = torch.randn(F, H, device="cuda").to(torch.bfloat16)
    _, gu_ms, _ = time_steps(lambda: torch.matmul(xg, wgu), reps, 2)
    _, dn_ms, _ = time_steps(lambda: torch.matmul(hd, wd), reps, 2)
    del xg, wgu, hd, wd
    torch.cuda.empty_cache()
    flops_layer = 2.0 * rows * H * 2 * F + 2.0 * rows * F * H
    dense_ms = cfg.layers * (gu_ms + dn_ms)
    return {"read_GBps": buf.numel() * 4 / (read_ms / 1e3) / 1e9,
            "copy_GBps": 2 * buf.numel() * 4 / (copy_ms / 1e3) / 1e9,
            "bf16_gemm_8192_TFLOPs": 2.0 * n ** 3 / (sq_ms / 1e3) / 1e12,
            "dense_equivalent_ms": dense_ms,
            "dense_equivalent_TFLOPs": cfg.layers * flops_layer / (dense_ms / 1e3) / 1e12,
            "how": "library kernels on the same GPU, warm, per-call events (mean of 5)"}


def attention_lines(steps):
    """Decode-attention lines: the serving batch (mixed lengths) and batches of one fixed
    length, each under both schedulers (static: the library's default; dynamic: the
    last-arriver merge), all through the one compiled kernel."""
    cfg = synth.ATTN
    mixed = synth.draw_context_lens(cfg["batch"], cfg["min_len"], cfg["max_len"], cfg["seed"])
    lines = {}
    for m in ("static", "dynamic"):
        lines[f"attention_mixed_{m}"] = bench_attention(steps, 2, m, mixed, f"mixed {m}")
    for L in (1024, 8192, 32768):
        for m in ("static", "dynamic"):
            key = f"attention_L{L}" + ("" if m == "static" else "_dynamic")
            lines[key] = bench_attention(steps, 2, m, [L] * cfg["batch"], f"L={L} {m}")
    keep = ("requests", "tokens", "launch_ms", "gbs_alg", "hbm_frac", "cold")
    return {k: {f: v[f] for f in keep} for k, v in lines.items()}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="prefill", choices=sorted(synth.CONFIGS))
    ap.add_argument("--tokens", type=int, default=0, help="override T (decode: 1/4/16/64)")
    ap.add_argument("--mode", default="static", choices=["static", "dedicated"])
    ap.add_argument("--combine", default="atomic", choices=["atomic", "ordered"])
    ap.add_argument("--secondary", dest="secondary", action="store_true", default=True)
    ap.add_argument("--no-secondary", dest="secondary", action="store_false")
    ap.add_argument("--no-cpu-baseline", dest="cpu", action="store_false", default=True)
    ap.add_argument("--trace-out", default=None,
                    help="also run one traced call and write a Chrome trace here")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB elementwise copy (counter calibration)")
    ap.add_argument("--splitk-only", action="store_true",
                    help="only time the split-K GEMM (for per-kernel profiles)")
    ap.add_argument("--attention-only", action="store_true",
                    help="only time the decode-attention lines (for per-kernel profiles)")
    ap.add_argument("--splitk-copies", type=int, default=4,
                    help="copies of B rotated between split-K calls (4: B streams from HBM)")
    ap.add_argument("--source-hash", action="store_true",
                    help="print the hash that identifies the kernel sources and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.source_hash:
        print(source_hash())
        return
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()), flush=True)
        return
    binding.load_library()
    if args.attention_only:
        print(json.dumps({"attention": attention_lines(args.steps)}), flush=True)
        return
    if args.splitk_only:
        res = {m: bench_splitk(args.steps, args.warmup, m, args.splitk_copies) for m in ("static", "dynamic")}
        print(json.dumps({"splitk": res}), flush=True)
        return

    cfg = synth.CONFIGS[args.workload]
    T = args.tokens or cfg.tokens[-1]
    head = bench_moe(cfg, T, args.steps, args.warmup, args.mode, args.combine, with_cpu=args.cpu,
                     trace_out=args.trace_out)
    mfma_bound = args.workload in ("prefill", "tiny")
    traffic = measured_traffic(f"{cfg.name}_T{T}")
    if mfma_bound:
        roof = {"bound": "mfma", "achieved": head["tflops_bf16"], "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": head["mfma_frac"], "traffic": traffic}
    else:
        roof = {"bound": "hbm", "achieved": head["gbs_alg"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": head["hbm_frac"], "traffic": traffic}
    roof["kernel"] = "etc::moe::moe_kernel<bf16>" if cfg.dtype == "bf16" else "etc::moe::moe_kernel<float>"
    roof["per_launch"] = {"flops_bf16": head["flops_bf16"], "flops_router_fp32": head["flops_router_fp32"],
                          "bytes_alg": head["bytes_alg"], "launch_ms": head["launch_ms"]}

    secondary = {}
    if args.secondary:
        dec = synth.CONFIGS["decode"]
        for t in (1, 64):
            r = bench_moe(dec, t, max(5, args.steps // 2), 2, args.mode, args.combine)
            secondary[f"decode_T{t}"] = {k: r[k] for k in ("tokens_per_s", "launch_ms", "gbs_alg",
                                                          "hbm_frac", "experts_touched", "cold")}
        fg = bench_moe(synth.CONFIGS["finegrained"], 256, max(5, args.steps // 2), 2, args.mode,
                       args.combine)
        secondary["finegrained_T256"] = {k: fg[k] for k in ("tokens_per_s", "launch_ms", "gbs_alg",
                                                           "hbm_frac", "experts_touched", "cold")}
        # the other GPU scheduler of the MoE layer on the same workloads
        other = "dedicated" if args.mode == "static" else "static"
        sched = {}
        for name, c, t in (("decode_T1", dec, 1), ("decode_T64", dec, 64),
                           ("finegrained_T256", synth.CONFIGS["finegrained"], 256),
                           (f"{cfg.name}_T{T}", cfg, T)):
            r = bench_moe(c, t, max(5, args.steps // 2), 2, other, args.combine)
            sched[name] = {k: r[k] for k in ("tokens_per_s", "launch_ms")}
        secondary[f"moe_{other}"] = sched
        for m in ("static", "dynamic"):  # split-K's dynamic mode is a last-arriver reduction
            sk = bench_splitk(max(5, args.steps // 2), 2, m)
            secondary[f"splitk_{m}"] = {k: sk[k] for k in ("launch_ms", "gbs_alg", "hbm_frac", "cold")}
        secondary.update(attention_lines(max(5, args.steps // 2)))

    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} H={cfg.hidden} E={cfg.experts} k={cfg.top_k} "
                               f"F={cfg.ffn}, {cfg.layers} chained layer(s)",
                   "tokens_per_step": T, "layers": cfg.layers, "mode": args.mode,
                   "combine": args.combine, "parallelism": "single GPU"},
        "roofline": roof,
        # the same calls, each after an untimed 1 GiB cache flush (per-call events)
        "cold_cache": head["cold"],
        "cpu_baseline": head.get("cpu"),
        # what vendor library kernels reach on this GPU (context for the nominal peaks)
        "achievable": achievable_peaks(cfg, T) if args.secondary else None,
        "secondary": secondary,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
