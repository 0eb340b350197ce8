"""Benchmark of the group-sparse FFN on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-dense] [--no-decode]

One step = one wide_ffn_forward call (mask reorder, gate/up kernel, down
kernel) over the Llama3.1-8B-shaped prefill workload: T=16384 tokens, d=4096,
d_ff=14336, G=128 (112 groups), bf16, top-50% Gaussian-score mask per token,
inputs resident in HBM. `value` is the effective throughput on active work:
6*d*G*A flops per step (A = active (token, group) pairs) over the step time.

Also reported, on the same line:
  roofline      the dominant kernel's algorithmic TFLOP/s (its share of the
                active flops, timed live with HIP events on its launch stream)
                against the bf16 dense MFMA peak; `traffic` comes from the
                rocprofv3 counter summary under profiles/ when that summary
                was taken on the current kernel source, else null;
  cpu_baseline  the fp64 oracle on a bounded token sample (host cores);
  dense         torch bf16 GEMMs (hipBLASLt) for the unpruned FFN;
  decode        T=1 and T=16 decode steps, active-weight GB/s with the
                weights rotated over 8 copies so each call reads HBM.
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
KERNEL_SOURCES = {
    "gate_up": "group_sparse_ffn_amd/csrc/gemm_mn.hip",
    "down": "group_sparse_ffn_amd/csrc/gemm_k.hip",
    "reorder": "group_sparse_ffn_amd/csrc/reorder.hip",
}


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    with open(os.path.join(ROOT, KERNEL_SOURCES[kernel]), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from profiles/traffic_<kernel>_<workload>.json, if current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_sha") != source_sha(kernel):
        return None  # counters were taken on an older version of the kernel
    return rec.get("bytes_per_launch")


def time_events(torch, fn, steps: int) -> float:
    """Average ms of fn() over `steps` calls, events on the current stream."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_prefill(torch, wide, dg, steps: int, warmup: int):
    w = dg.LLAMA8B_PREFILL
    log(f"generating {w.name}")
    inp = dg.make_inputs(w)
    m = inp["mask"]
    A = int(m.sum())
    ng = w.ngroups
    dev = "cuda:0"
    d = {k: v.to(dev) for k, v in inp.items()}
    call = wide.FfnCall(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G)
    flops = 6.0 * w.d * w.G * A
    log(f"warmup {warmup}")
    for _ in range(warmup):
        call.run()
    torch.cuda.synchronize()
    log(f"timing {steps} forward steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms = time_events(torch, call.run, steps)
    wall = (time.perf_counter() - t0) * 1e3 / steps

    # per-kernel durations: the same stages, events between them on the launch stream
    stages = [("reorder", wide.WIDE_STAGE_REORDER), ("gate_up", wide.WIDE_STAGE_GATE_UP),
              ("down", wide.WIDE_STAGE_DOWN)]
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
          for _ in range(steps)]
    log(f"timing {steps} staged steps")
    torch.cuda.synchronize()
    for s in range(steps):
        ev[s][0].record()
        for i, (_, st) in enumerate(stages):
            call.stage(st)
            ev[s][i + 1].record()
    torch.cuda.synchronize()
    per = {name: sum(ev[s][i].elapsed_time(ev[s][i + 1]) for s in range(steps)) / steps
           for i, (name, _) in enumerate(stages)}
    out = {"workload": w, "A": A, "ng": ng, "ms": ms, "wall_ms": wall, "flops": flops,
           "per_kernel_ms": per, "inputs": inp, "dev_inputs": d, "call": call}
    return out


def dense_baseline(torch, d, steps: int, warmup: int):
    """Unpruned FFN with torch's bf16 GEMMs (hipBLASLt): [X][Wg;Wu]^T, silu*up, [.]Wd^T."""
    Wgu = torch.cat([d["Wg"], d["Wu"]], dim=0)
    dff = d["Wg"].shape[0]

    def step():
        gu = d["X"] @ Wgu.t()
        h = torch.nn.functional.silu(gu[:, :dff]) * gu[:, dff:]
        return h @ d["Wd"].t()

    for _ in range(warmup):
        step()
    ms = time_events(torch, step, steps)
    del Wgu
    return ms


def cpu_baseline(oracle, inp, w, target_s: float = 12.0):
    """fp64 oracle on a seeded token sample, scaled to effective TFLOP/s."""
    import numpy as np
    rng = np.random.default_rng(w.seed + 99)
    m = inp["mask"].numpy()
    x, wg, wu, wd = (inp[k].float().numpy() for k in ("X", "Wg", "Wu", "Wd"))

    def run(rows):
        t0 = time.perf_counter()
        oracle.ffn(x, wg, wu, wd, m, w.G, rows=rows)
        return time.perf_counter() - t0

    probe = rng.choice(w.T, size=32, replace=False)
    tp = run(probe)
    n = int(min(w.T, max(32, 32 * target_s / max(tp, 1e-3))))
    rows = rng.choice(w.T, size=n, replace=False)
    t = run(rows)
    active = int(m[rows].sum())
    flops = 6.0 * w.d * w.G * active
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{n} of {w.T} tokens (seeded), fp64, {t:.1f} s; effective flops of the "
                      f"sampled tokens' active groups"}


def bench_decode(torch, wide, dg, steps: int, copies: int = 8):
    res = {}
    for w in (dg.LLAMA8B_DECODE_T1, dg.LLAMA8B_DECODE_T16):
        log(f"decode {w.name}")
        inp = dg.make_inputs(w)
        dev = "cuda:0"
        X = inp["X"].to(dev)
        mask = inp["mask"].to(dev)
        ws = [{k: inp[k].to(dev) for k in ("Wg", "Wu", "Wd")}]
        for _ in range(copies - 1):
            ws.append({k: v.clone() for k, v in ws[0].items()})
        calls = [wide.FfnCall(X, c["Wg"], c["Wu"], c["Wd"], mask, w.G) for c in ws]
        m = inp["mask"].numpy()
        union = int(m.any(axis=0).sum())
        act_bytes = 3 * w.d * w.G * union * 2
        for c in calls:
            c.run()
        n = max(steps, 4) * copies
        idx = [0]

        def step():
            calls[idx[0] % copies].run()
            idx[0] += 1

        ms = time_events(torch, step, n)
        res[f"T{w.T}"] = {"us_per_step": ms * 1e3, "active_weight_GBps": act_bytes / ms / 1e6,
                          "hbm_frac": act_bytes / ms / 1e6 / PEAK_HBM_GBS,
                          "active_groups": union, "active_weight_MB": act_bytes / 1e6,
                          "weight_copies": copies}
        del calls, ws
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the group-sparse FFN "
              "here has no multi-GPU path", file=sys.stderr)
        sys.exit(2)

    import torch
    import group_sparse_ffn_amd as wide
    from group_sparse_ffn_amd import datagen as dg

    r = bench_prefill(torch, wide, dg, args.steps, args.warmup)
    w = r["workload"]
    per = r["per_kernel_ms"]
    kflops = {"gate_up": 4.0 * w.d * w.G * r["A"], "down": 2.0 * w.d * w.G * r["A"]}
    dom = max(("gate_up", "down"), key=lambda k: per[k])
    achieved = kflops[dom] / (per[dom] * 1e-3) / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 1),
            "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": load_traffic(dom, w.name)}
    value = r["flops"] / (r["ms"] * 1e-3) / 1e12
    line = {
        "metric": "effective TFLOP/s (prefill) & active-weight GB/s (decode), % roofline, vs dense",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Gaussian inputs and weights, top-50% Gaussian-score mask)",
        "config": {"workload": w.name, "T": w.T, "d": w.d, "d_ff": w.d_ff, "G": w.G,
                   "groups": r["ng"], "active_pairs": r["A"],
                   "sparsity": round(1 - r["A"] / (w.T * r["ng"]), 4),
                   "active_tflop_per_step": round(r["flops"] / 1e12, 4)},
        "roofline": roof,
        "per_kernel_ms": {k: round(v, 4) for k, v in per.items()},
        "mfma_frac_of_step": round(value / PEAK_BF16_TFLOPS, 4),
    }
    if not args.no_dense:
        log("dense baseline")
        dms = dense_baseline(torch, r["dev_inputs"], max(5, args.steps // 2), 2)
        line["dense"] = {"ms": round(dms, 4), "impl": "torch bf16 matmul (hipBLASLt)",
                         "speedup": round(dms / r["ms"], 3),
                         "ideal_speedup": round(w.T * r["ng"] / r["A"], 3)}
    del r["call"], r["dev_inputs"]
    torch.cuda.empty_cache()
    if not args.no_decode:
        line["decode"] = bench_decode(torch, wide, dg, args.steps)
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        import oracle
        line["cpu_baseline"] = cpu_baseline(oracle, r["inputs"], w)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
