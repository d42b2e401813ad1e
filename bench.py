"""Benchmark of the exact-attention backward on one MI355X.

Workload: Llama-3-style causal GQA, B=4, Hq=32, Hkv=8, N_q=N_kv=8192, d=128, bf16,
scale 1/sqrt(128), Q/K/V/dO ~ N(0,1) from the seeded generator (synthetic data).

A step is one pass of the whole hot path on resident inputs: fa_fwd (O, LSE) then
fa_bwd (the dQ pass with the D preprocess of its rows, then the dK/dV kernel; or,
on the atomic path, the preprocess, the fused kernel and the dQ conversion).  The headline value is the
backward's throughput, fa_bwd TFLOP/s, counting 2.5x the forward's 4*Nq*Nkv*d
flops per query head, halved for causal; it is taken from HIP events recorded on
the launch stream around every fa_bwd call of the timed steps.

Also reported: the roofline of the dominant kernel (the dK/dV kernel, timed alone
with events that fa_bwd_ex records around its launch), the forward's rate, and a
CPU baseline: the fp64 oracle's backward on kv-head groups of the same inputs,
timed on the host cores, with the host's CPU model, BLAS library and one-thread
oracle timings of the small workloads.

    python bench.py [--steps K] [--warmup W] [--dq-mode auto|atomic|separate]
                    [--workload NAME[,NAME...]] [--head-dim D] [--bias keys|full] [--dbias]
                    [--dropout P]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16/fp16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk
PEAK_HBM_GBS = 8000.0


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def _threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        return os.cpu_count() or 1


def cpu_baseline(case, x, min_seconds: float = 10.0, max_groups: int = 8) -> dict:
    """The oracle's backward, as it stands, on whole (batch, kv head) groups of the
    same inputs, one group after another until about ``min_seconds`` of CPU work."""
    import oracle.attention_fp64 as orc
    threads = _threads()
    G = case.Hq // case.Hkv
    groups = [(b, g) for b in range(case.B) for g in range(case.Hkv)][:max_groups]
    done, t0 = 0, time.perf_counter()
    for (b, g) in groups:
        s = {"q": x["q"][b:b + 1, g * G:(g + 1) * G], "k": x["k"][b:b + 1, g:g + 1],
             "v": x["v"][b:b + 1, g:g + 1], "do": x["do"][b:b + 1, g * G:(g + 1) * G]}
        orc.backward(s["q"], s["k"], s["v"], s["do"], case.scale, case.causal)
        done += 1
        if time.perf_counter() - t0 >= min_seconds:
            break
    dt = time.perf_counter() - t0
    flops = done * 2.5 * 4.0 * G * case.Nq * case.Nkv * case.d * (0.5 if case.causal else 1.0)
    rate = flops / dt / 1e12
    return {"value": rate, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            # the whole workload at the sample's rate (extrapolated, not measured)
            "extrapolated_full_seconds": round(case.bwd_flops() / (rate * 1e12), 1),
            "sample": f"fp64 oracle backward of {done} (batch, kv head) group(s) of {G} query heads "
                      f"(N={case.Nq}, d={case.d}, {'causal' if case.causal else 'non-causal'}) = "
                      f"{done}/{case.B * case.Hkv} of the workload, {dt:.1f} s; flops counted as "
                      f"the metric counts them",
            "seconds": dt}


def cpu_context() -> dict:
    """The host the oracle runs on (CPU model, BLAS library and its threads), and the
    oracle's backward on one thread for the three small workload families: the
    single head, the ragged family (all 8 cases) and 4 of the 32 (batch, head)
    pairs of the uniform 2048 x 2048 shape."""
    import oracle.attention_fp64 as orc
    from exact_attention_backward_fa_amd import inputs
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        libs = [f"{p.get('internal_api')} {p.get('version')} ({p.get('num_threads')} threads)"
                for p in threadpool_info() if p.get("user_api") == "blas"]
        blas = "; ".join(libs) or blas
    except Exception:
        threadpool_limits = None
    samples = [("single", inputs.cases_of_family(1), None),
               ("ragged (8 cases)", inputs.cases_of_family(2), None),
               ("uniform, 4 of 32 (batch, head)", inputs.cases_of_family(3), 4)]
    rows = []
    for label, cases, heads in samples:
        flops, t = 0.0, 0.0
        for case in cases:
            x = inputs.make_inputs(case)
            if heads is not None:
                x = {k: v[:1, :heads] for k, v in x.items()}
            Hq = x["q"].shape[1]
            ctx = threadpool_limits(limits=1) if threadpool_limits else None
            t0 = time.perf_counter()
            if ctx is not None:
                with ctx:
                    orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal)
            else:
                orc.backward(x["q"], x["k"], x["v"], x["do"], case.scale, case.causal)
            t += time.perf_counter() - t0
            flops += (x["q"].shape[0] * Hq * 10.0 * case.Nq * case.Nkv * case.d
                      * (0.5 if case.causal else 1.0))
        rows.append({"workload": label, "seconds": round(t, 3),
                     "value": round(flops / t / 1e12, 6) if t > 0 else None, "unit": "TFLOP/s",
                     "threads": 1})
    return {"cpu_model": model, "blas": blas, "os_cpus": os.cpu_count(), "single_thread": rows}


def measure(case, args, dev, log_prefix="[bench]") -> tuple:
    """Times args.steps steps of the hot path on one workload; returns the JSON
    object of the line (without the CPU baseline) and the host inputs."""
    import torch
    import exact_attention_backward_fa_amd as fa
    from exact_attention_backward_fa_amd import profiling

    log(f"{log_prefix} workload {case.name}: B={case.B} Hq={case.Hq} Hkv={case.Hkv} N={case.Nq} "
        f"d={case.d} {case.dtype} causal={case.causal}")
    x = inputs_of(case)
    d = {k: v.to(dev) for k, v in x.items()}
    o = torch.empty_like(d["q"])
    lse = torch.empty(case.B, case.Hq, case.Nq, dtype=torch.float32, device=dev)
    dq = torch.empty_like(d["q"])
    dk = torch.empty_like(d["k"])
    dv = torch.empty_like(d["v"])
    mode = args.dq_mode
    if mode == "auto":
        resolved = fa.auto_dq_mode(case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                                   case.causal, case.torch_dtype)
    else:
        resolved = mode
    stream = torch.cuda.current_stream(dev).cuda_stream
    n = args.steps
    features = args.bias != "none" or args.dbias or args.dropout > 0.0
    bias = dbias = None
    if features:
        mode = resolved = "separate"
        g = torch.Generator(device=dev).manual_seed(1234)
        if args.bias == "keys":  # a padding mask: the last 1/8 of every row's keys hidden
            bias = torch.zeros(case.B, 1, 1, (case.Nkv + 7) // 8 * 8, dtype=case.torch_dtype,
                               device=dev)
            bias[..., case.Nkv - case.Nkv // 8:] = float("-inf")
            bias = bias[..., :case.Nkv]
        elif args.bias == "full":
            bias = torch.randn(case.B, case.Hq, case.Nq, (case.Nkv + 7) // 8 * 8, generator=g,
                               device=dev, dtype=torch.float32).to(case.torch_dtype)
            bias = bias[..., :case.Nkv]
        if args.dbias:
            dbias = torch.empty(case.B, case.Hq, case.Nq, case.Nkv, dtype=case.torch_dtype,
                                device=dev)
    ws = torch.empty(max(fa.bwd_workspace_bytes(case.B, case.Hq, case.Hkv, case.Nq, case.Nkv, case.d,
                                                case.causal, case.torch_dtype, mode), 1),
                     dtype=torch.uint8, device=dev)
    ev = {k: [fa.HipEvent() for _ in range(n)] for k in ("f0", "f1", "b0", "b1", "k0", "k1")}

    def step(i=None):
        if i is not None:
            ev["f0"][i].record(stream)
        if features:
            fa.fwd_bias_dropout(d["q"], d["k"], d["v"], case.scale, case.causal, bias=bias,
                                dropout_p=args.dropout, seed=77, o=o, lse=lse)
        else:
            fa.fwd_into(d["q"], d["k"], d["v"], o, lse, case.scale, case.causal)
        if i is not None:
            ev["f1"][i].record(stream)
            ev["b0"][i].record(stream)
        if features:
            fa.bwd_bias_dropout(d["q"], d["k"], d["v"], o, lse, d["do"], case.scale, case.causal,
                                bias=bias, dropout_p=args.dropout, seed=77, dq=dq, dk=dk, dv=dv,
                                dbias=dbias, workspace=ws)
        else:
            fa.bwd_into(d["q"], d["k"], d["v"], o, lse, d["do"], dq, dk, dv, case.scale,
                        case.causal, dq_mode=mode, workspace=ws,
                        events=None if i is None else (ev["k0"][i].handle, ev["k1"][i].handle))
        if i is not None:
            ev["b1"][i].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize(dev)
    log(f"{log_prefix} warmup done ({args.warmup} steps); timing {n} steps, dq path {resolved}")
    t0 = time.perf_counter()
    for i in range(n):
        step(i)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0

    def total(a, b):
        return sum(ev[a][i].elapsed_ms(ev[b][i]) for i in range(n))

    fwd_ms = total("f0", "f1") / n
    bwd_ms = total("b0", "b1") / n
    bwd_each = sorted(ev["b0"][i].elapsed_ms(ev["b1"][i]) for i in range(n))
    bwd_median = bwd_each[n // 2] if n % 2 else 0.5 * (bwd_each[n // 2 - 1] + bwd_each[n // 2])
    # the dK/dV kernel's own events are recorded on the plain path only (the feature
    # runs' per-kernel split comes from a kernel trace)
    kern_ms = None if features else total("k0", "k1") / n
    bwd_flops = case.bwd_flops()
    fwd_flops = case.fwd_flops()
    value = bwd_flops / (bwd_ms * 1e-3) / 1e12
    elt = 2  # fp16 / bf16
    io_bytes = (elt * (4 * case.B * case.Hq * case.Nq * case.d + 4 * case.B * case.Hkv * case.Nkv * case.d)
                + 8 * case.B * case.Hq * case.Nq)
    # Algorithmic flops of the dK/dV kernel per launch: with the atomic dQ path it
    # performs all five products of the backward (10*Nq*Nkv*d per query head, halved
    # for causal); on the separate path it performs four of them (8*Nq*Nkv*d).
    kern_flops = bwd_flops if resolved == "atomic" else bwd_flops * 0.8
    achieved = None if kern_ms is None else kern_flops / (kern_ms * 1e-3) / 1e12
    # HBM bytes per launch of that kernel and its MFMA counters from the committed
    # counter profiles, when they were taken from the kernel code built now.
    dt_id = 1 if case.dtype == "bf16" else 0
    causal = "true" if case.causal else "false"
    kname = (f"bwd_dkdv_atomic_kernel<{dt_id}, {case.d}, {causal}>" if resolved == "atomic"
             else f"bwd_dkdv_kernel<{dt_id}, {case.d}, {causal}, 0>")
    traffic = None if features else profiling.read_traffic(kname)
    mfma = None if features else profiling.read_mfma(kname)
    log(f"{log_prefix} fwd {fwd_ms:.3f} ms ({fwd_flops / fwd_ms / 1e9:.1f} TFLOP/s)  bwd {bwd_ms:.3f} ms "
        f"({value:.1f} TFLOP/s, {100 * value / PEAK_BF16_TFLOPS:.1f}% of peak)"
        + ("" if kern_ms is None else f"  dkdv kernel {kern_ms:.3f} ms ({achieved:.1f} TFLOP/s)"))

    out = {
        "metric": "fa_bwd TFLOP/s and % of MI355X bf16 MFMA peak (causal GQA, d=128)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / n, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": case.dtype,
        "data": (f"synthetic (seeded {'U[0,1)' if case.dist == 'uniform' else 'N(0,1)'} Q, K, V, dO"
                 f"{f'; Q and K x{case.qk_mult:g}' if case.qk_mult != 1.0 else ''})"),
        "config": {"workload": f"{case.name}: {'causal' if case.causal else 'non-causal'} "
                               f"{'GQA' if case.Hq != case.Hkv else 'MHA'} B={case.B} Hq={case.Hq} "
                               f"Hkv={case.Hkv} N_q={case.Nq} N_kv={case.Nkv} d={case.d} {case.dtype}",
                   "global_batch": case.B, "seq_len": case.Nq, "parallelism": "single GPU",
                   "dq_path": resolved},
        "pct_of_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "bwd_ms": round(bwd_ms, 4),
        "bwd_ms_median": round(bwd_median, 4),
        "bwd_ms_min": round(bwd_each[0], 4),
        # inputs and outputs that fit the 256 MB Infinity Cache stay cache-resident
        # from step to step: such timings are warm-cache ones
        "cache": "warm" if io_bytes < (256 << 20) else "cold",
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tflops": round(fwd_flops / (fwd_ms * 1e-3) / 1e12, 2),
        "roofline": {
            "kernel": kname,
            "bound": "mfma",
            "achieved": None if achieved is None else round(achieved, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": None if achieved is None else round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "traffic_gbs": None if traffic is None or kern_ms is None
                           else round(traffic / (kern_ms * 1e-3) / 1e9, 1),
            "kernel_ms": None if kern_ms is None else round(kern_ms, 4),
            # rocprof MfmaUtil (matrix-unit busy share of active SIMD cycles) and the
            # MFMA flops the kernel executes per launch, from the committed counter
            # profile of the kernel code built now; null when that profile is stale.
            "mfma_busy_pct": None if mfma is None else mfma[0],
            "executed_tflop": None if mfma is None else mfma[1],
        },
    }
    if features:
        out["config"]["features"] = {"bias": args.bias, "dbias": bool(args.dbias),
                                     "dropout_p": args.dropout}
    return out, x


def inputs_of(case):
    from exact_attention_backward_fa_amd import inputs
    return inputs.make_inputs(case)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--dq-mode", default="auto", choices=["auto", "atomic", "separate"])
    ap.add_argument("--workload", default=None,
                    help="case name, or several separated by commas (one JSON line each); "
                         "default: the headline workload")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--bias", default="none", choices=["none", "keys", "full"],
                    help="additive score bias: a per-key [B,1,1,N_kv] padding mask, or a "
                         "full [B,Hq,N_q,N_kv] bias (timed through fa_*_bias_dropout)")
    ap.add_argument("--dbias", action="store_true", help="also write dBias [B,Hq,N_q,N_kv]")
    ap.add_argument("--dropout", type=float, default=0.0, help="dropout probability of P")
    ap.add_argument("--head-dim", type=int, default=None,
                    help="run the workload(s) with this head dimension instead (softmax "
                         "scale 1/sqrt(d)); the name gets a _d<D> suffix")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after timing, copy a 512 MiB buffer once (known traffic) so that "
                         "a counter profile of this run can scale FETCH_SIZE/WRITE_SIZE")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(the backward shards by (batch, kv head) group with no communication; "
              "run --gpus 1)", file=sys.stderr, flush=True)
        return 2
    features = args.bias != "none" or args.dbias or args.dropout > 0.0
    if features and args.dq_mode == "atomic":
        log("[bench] bias, dBias and dropout run on the separate dQ path only")
        return 2

    import torch
    from exact_attention_backward_fa_amd import inputs

    names = (args.workload or inputs.HEADLINE).split(",")
    cases = [inputs.case_by_name(nm.strip()) for nm in names]
    if args.head_dim is not None:
        cases = [dataclasses.replace(c, name=f"{c.name}_d{args.head_dim}", d=args.head_dim,
                                     scale=1.0 / math.sqrt(args.head_dim)) for c in cases]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    for case in cases:
        out, x = measure(case, args, dev)
        if args.copy_calibration:
            src = torch.empty(256 << 20, dtype=torch.bfloat16, device=dev).fill_(1.0)
            dst = torch.empty_like(src)
            torch.cuda.synchronize(dev)
            dst.copy_(src)
            torch.cuda.synchronize(dev)
            out["copy_calibration_bytes"] = {"read": src.numel() * 2, "write": dst.numel() * 2}
            del src, dst
        if not args.no_cpu_baseline and not features and len(cases) == 1:
            log("[bench] cpu baseline: fp64 oracle backward on one kv-head group ...")
            out["cpu_baseline"] = cpu_baseline(case, x)
            log(f"[bench] cpu baseline {out['cpu_baseline']['value']:.4f} TFLOP/s "
                f"({out['cpu_baseline']['seconds']:.1f} s, {out['cpu_baseline']['cores']} threads)")
            log("[bench] cpu context: model, BLAS, single-thread oracle on the small families ...")
            out["cpu_baseline"]["context"] = cpu_context()
        print(json.dumps(out), flush=True)
        del x
        torch.cuda.empty_cache()
    return 0


if __name__ == "__main__":
    sys.exit(main())
