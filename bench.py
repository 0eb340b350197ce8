"""Benchmark of the group-sparse FFN on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-dense] [--no-decode]
    python bench.py --profile [--steps K]     # short run for rocprofv3 (prefill, decode, a copy)
    python bench.py --summarize DIR [--command CMD]   # rocprofv3 CSVs in DIR -> profiles/*.md

One step = one wide_ffn_forward call (mask reorder, gate/up kernel, down
kernel) over the Llama3.1-8B-shaped prefill workload: T=16384 tokens, d=4096,
d_ff=14336, G=128 (112 groups), bf16, top-50% Gaussian-score mask per token,
inputs resident in HBM. `value` is the effective throughput on active work:
6*d*G*A flops per step (A = active (token, group) pairs) over the step time,
launched eagerly; `graph_ms_per_step` is the same step replayed from a
captured HIP graph (the pages time kernels under graph replay).

Also reported, on the same line:
  roofline      the dominant kernel (the longest): its algorithmic TFLOP/s
                (its share of the active flops) over its average duration,
                timed live with HIP events on the stream it is launched on,
                against the bf16 dense MFMA peak. `traffic` is the HBM bytes
                per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE (scaled by
                the same counters read on a copy of known size), kept in
                profiles/traffic_<kernel>_<workload>.md, or null when that
                summary was taken on other kernel sources;
  per_kernel_ms reorder, gate/up and down, events between the stages;
  dense         torch bf16 GEMMs (hipBLASLt) for the unpruned FFN;
  decode        T=1 and T=16 decode steps: active-weight GB/s against HBM
                peak, weights rotated over 8 copies so each call reads HBM;
  cpu_baseline  the fp64 oracle on a bounded token sample (host cores).
Prints exactly one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP32_TFLOPS = 157.3    # MI355X fp32 vector
CSRC = "group_sparse_ffn_amd/csrc"
# sources that define each kernel (a change to any of them invalidates its counters)
KERNEL_SOURCES = {
    "gate_up": ["gemm_mn.hip", "mfma_core.h", "common.h"],
    "down": ["gemm_k.hip", "mfma_core.h", "common.h"],
    "reorder": ["reorder.hip", "common.h"],
    "decode_gate_up": ["decode.hip", "common.h"],
    "decode_gate_up_xlds": ["decode.hip", "common.h"],
    "down_split_reduce": ["gemm_k.hip", "mfma_core.h", "common.h"],
    "gemm_mn": ["gemm_mn.hip", "mfma_core.h", "common.h"],
    "pack_mask_bits": ["reorder.hip", "common.h"],
    "reorder_bits": ["reorder.hip", "common.h"],
    "router": ["router.hip", "common.h"],
    "router_zpart": ["router.hip", "common.h"],
    "router_decide": ["router.hip", "common.h"],
    "decode_down_splitk": ["decode.hip", "common.h"],
    "decode_gate_up_packed": ["decode.hip", "common.h"],
    "decode_down_splitk_packed": ["decode.hip", "common.h"],
    "decode_down_reduce": ["decode.hip", "common.h"],
    "decode_gate_up_valu": ["decode.hip", "common.h"],
    "decode_down_valu": ["decode.hip", "common.h"],
    "attention_prefill": ["attention.hip", "common.h"],
    "attention_vt": ["attention.hip", "common.h"],
    "attention_decode_split": ["attention_decode.hip", "common.h"],
    "attention_decode_merge": ["attention_decode.hip", "common.h"],
}
# substrings of the device symbol names of each kernel
KERNEL_SYMBOLS = {
    "gate_up": "gate_up_bf16_kernel",
    "down": "down_bf16_kernel",
    "reorder": "reorder_kernel",
    "decode_gate_up": "decode_gate_up_kernel",
    "decode_gate_up_xlds": "decode_gate_up_xlds_kernel",
    "down_split_reduce": "down_split_reduce_kernel",
    "gemm_mn": "gemm_mn_bf16_kernel",
    "pack_mask_bits": "pack_mask_bits_kernel",
    "reorder_bits": "reorder_bits_kernel",
    "router": "router_kernel_",
    "router_zpart": "router_zpart_kernel",
    "router_decide": "router_decide_kernel",
    "decode_down_splitk": "decode_down_splitk_kernel<false, false>",
    "decode_gate_up_packed": "decode_gate_up_packed_kernel",
    "decode_down_splitk_packed": "decode_down_splitk_kernel<false, true>",
    "decode_down_reduce": "decode_down_reduce_kernel",
    "decode_gate_up_valu": "decode_gate_up_valu_kernel",
    "decode_down_valu": "decode_down_valu_kernel",
    "attention_prefill": "attention_prefill_kernel",
    "attention_vt": "attention_vt_kernel",
    "attention_decode_split": "attention_decode_split_kernel",
    "attention_decode_merge": "attention_decode_merge_kernel",
}
COPY_BYTES = 1 << 30  # the calibration copy: 1 GiB read + 1 GiB written


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def source_sha(kernel: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(kernel: str, workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the counter summary, if taken on the current sources."""
    path = traffic_path(kernel, workload)
    if not os.path.exists(path):
        return None
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^- (\w+): (\S+)", line.strip())
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("source_sha") != source_sha(kernel):
        return None  # counters were taken on another version of the kernel
    try:
        return int(float(fields["bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


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


def graph_step_ms(torch, fn, steps: int) -> float:
    """Average ms of fn() replayed from a captured graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    g.replay()
    torch.cuda.synchronize()
    ms = time_events(torch, g.replay, steps)
    del g
    return ms


def bench_prefill(torch, wide, dg, steps: int, warmup: int, graph: bool = True):
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
    gms = None
    if graph:
        log("graph replay")
        gms = graph_step_ms(torch, call.run, steps)
    return {"workload": w, "A": A, "ng": ng, "ms": ms, "wall_ms": wall, "graph_ms": gms,
            "flops": flops, "per_kernel_ms": per, "inputs": inp, "dev_inputs": d, "call": call}


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


def bench_masked_gemms(torch, wide, dg, steps: int):
    """The N-axis and K-axis masked GEMMs at Llama3.1-8B attention shapes.

    Times one library call (mask reorder or bit packing + the GEMM kernel) and
    torch's dense bf16 A @ B^T on the same operands.
    """
    out = {}
    dev = "cuda:0"
    for w in (dg.LLAMA8B_ATTN_Q, dg.LLAMA8B_ATTN_O, dg.LLAMA8B_DEPTH):
        log(f"masked GEMM {w.name}")
        inp = dg.make_gemm_inputs(w)
        act = int(inp["mask"].sum())
        d = {k: v.to(dev) for k, v in inp.items()}
        C = torch.empty((w.M, w.N), dtype=torch.bfloat16, device=dev)
        ws = torch.empty(wide.gemm_workspace_size(w.M, w.ngroups), dtype=torch.uint8, device=dev)
        fn = wide.gemm_mn if w.axis == "mn" else wide.gemm_k
        call = lambda: fn(d["A"], d["B"], d["mask"], w.G, C=C, workspace=ws)
        for _ in range(3):
            call()
        ms = time_events(torch, call, steps)
        Bt = d["B"]
        dense = lambda: d["A"] @ Bt.t()
        for _ in range(3):
            dense()
        dms = time_events(torch, dense, steps)
        # active flops: 2 * (the unpruned extent) * G per active (row, group)
        other = w.K if w.axis == "mn" else w.N
        flops = 2.0 * other * w.G * act
        out[w.name] = {"M": w.M, "N": w.N, "K": w.K, "G": w.G, "axis": w.axis,
                       "density": round(act / (w.M * w.ngroups), 4), "ms": round(ms, 4),
                       "active_tflops": round(flops / (ms * 1e-3) / 1e12, 1),
                       "frac_of_bf16_peak": round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                       "dense_ms": round(dms, 4), "speedup_vs_dense": round(dms / ms, 3),
                       "ideal_speedup": round(w.M * w.ngroups / max(act, 1), 3)}
        del d, C, ws
        torch.cuda.empty_cache()
    return out


def bench_baselines(torch, wide, dg, sizes=(2048, 4096), G: int = 128, p: float = 0.5):
    """Dense GEMM, the naive gather-scatter pipelines, the grouped GEMM on
    reordered masks and the fused kernels on M = N = K = S, for pruning along
    M (one decision per row), N and K (G = 128, random masks with half of
    every token's groups active; M axis: half of the rows).

    Per implementation: ms per call, effective TFLOP/s (the active products'
    flops; dense counts all of them), the bytes the call allocates at its peak
    (for the fused call: nothing, its output and workspace are passed in) and,
    for the naive pipelines, the traffic and materialized storage of the
    pages' closed forms."""
    from group_sparse_ffn_amd import baselines as bl
    out = {}
    dev = "cuda:0"
    try:
        a = torch.ones((4, 16), dtype=torch.bfloat16, device=dev)
        b = torch.ones((2, 16, 16), dtype=torch.bfloat16, device=dev)
        torch._grouped_mm(a, b, offs=torch.tensor([2, 4], dtype=torch.int32, device=dev))
        torch.cuda.synchronize()
        use_gmm = True
    except Exception:  # no grouped GEMM in this torch build for this device
        use_gmm = False

    def measure(fn, reps, graph):
        fn()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        r = fn()
        torch.cuda.synchronize()
        peak = torch.cuda.max_memory_allocated() - base
        del r
        # dense and fused replay from a graph (the pages' protocol); the naive
        # and grouped pipelines read sizes back to the host, so they run eagerly
        ms = graph_step_ms(torch, fn, reps) if graph else time_events(torch, fn, reps)
        return ms, peak

    for S in sizes:
        M = N = K = S
        for axis in ("m", "n", "k"):
            log(f"baselines {axis}-axis {S}^3")
            Gx = N if axis == "m" else G
            w = dg.GemmWorkload(f"baseline-{axis}-{S}", 60 + S % 97, M=M, N=N, K=K, G=Gx,
                                axis="k" if axis == "k" else "mn",
                                mask_kind="bernoulli" if axis == "m" else "topk", density=p)
            inp = dg.make_gemm_inputs(w)
            act = int(inp["mask"].sum())
            A, B, mask = (inp[k].to(dev) for k in ("A", "B", "mask"))
            del inp
            dens = act / mask.numel()
            flops = 2.0 * M * N * K * dens
            impls = {"dense": (lambda: A @ B.t(), 2.0 * M * N * K)}
            if axis == "m":
                impls["naive"] = (lambda: bl.naive_gemm_m(A, B, mask), flops)
                C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                ws = torch.empty(wide.gemm_workspace_size(M, 1), dtype=torch.uint8, device=dev)
                impls["fused"] = (lambda: wide.gemm_mn(A, B, mask, N, C=C, workspace=ws), flops)
            elif axis == "n":
                impls["naive"] = (lambda: bl.naive_gemm_mn(A, B, mask, G), flops)
                impls["grouped"] = (lambda: bl.grouped_gemm_mn(A, B, mask, G, use_gmm), flops)
                C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                ws = torch.empty(wide.gemm_workspace_size(M, N // G), dtype=torch.uint8, device=dev)
                impls["fused"] = (lambda: wide.gemm_mn(A, B, mask, G, C=C, workspace=ws), flops)
            else:
                impls["naive"] = (lambda: bl.naive_gemm_k(A, B, mask, G), flops)
                impls["grouped"] = (lambda: bl.grouped_gemm_k(A, B, mask, G, use_gmm), flops)
                C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
                ws = torch.empty(wide.gemm_workspace_size(M, K // G), dtype=torch.uint8, device=dev)
                impls["fused"] = (lambda: wide.gemm_k(A, B, mask, G, C=C, workspace=ws), flops)
            row = {"M": M, "N": N, "K": K, "G": Gx, "density": round(dens, 4),
                   "table4_traffic_bytes": int(2 * bl.traffic_elements(axis, M, N, K, dens)),
                   "table4_materialized_bytes": int(2 * bl.materialized_elements(axis, M, N, K, dens))}
            for name, (fn, fl) in impls.items():
                eager = name in ("naive", "grouped")
                ms, peak = measure(fn, 3 if eager else 20, not eager)
                row[name] = {"ms": round(ms, 4), "tflops": round(fl / (ms * 1e-3) / 1e12, 2),
                             "peak_alloc_bytes": int(peak), "timing": "eager" if eager else "graph"}
                torch.cuda.empty_cache()
            if "grouped" in row:
                row["grouped"]["impl"] = "torch._grouped_mm" if use_gmm else "one torch.mm per group"
            out[f"{axis}{S}"] = row
            del A, B, mask, C, ws
            torch.cuda.empty_cache()
    return out


def bench_attention(torch, wide, dg, steps: int):
    """Head-group-pruned causal attention at the Llama3.1-8B shape (T = 16384,
    32 query heads, 8 KV heads, dh = 128, half of the (token, group) pairs
    kept): the library call by graph replay, the same call on an all-ones mask,
    and torch's SDPA (causal, GQA; flash or memory-efficient backend only) on
    every head."""
    w = dg.LLAMA8B_ATTN_PREFILL
    dev = "cuda:0"
    log(f"attention {w.name}")
    inp = dg.make_attention_inputs(w)
    alg, exe = attention_work(inp["mask"], w)
    d = {k: v.to(dev) for k, v in inp.items()}
    O = torch.empty((w.T, w.Hq * w.dh), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(wide.attention_workspace_size(w.T, w.Hk, w.dh), dtype=torch.uint8, device=dev)
    call = lambda m: wide.attention_prefill(d["Q"], d["K"], d["V"], m, w.Hq, w.Hk, O=O,  # noqa: E731
                                            workspace=ws)
    call(d["mask"])
    ms = graph_step_ms(torch, lambda: call(d["mask"]), steps)
    ones = torch.ones_like(d["mask"])
    oms = graph_step_ms(torch, lambda: call(ones), max(5, steps // 2))
    dense = 4.0 * w.dh * w.Hq * w.T * (w.T + 1) / 2
    out = {"T": w.T, "Hq": w.Hq, "Hk": w.Hk, "dh": w.dh,
           "density": round(float(inp["mask"].float().mean()), 4),
           "ms": round(ms, 4), "active_tflop": round(alg / 1e12, 4),
           "executed_mfma_tflop": round(exe / 1e12, 4),
           "effective_tflops": round(alg / (ms * 1e-3) / 1e12, 1),
           "frac_of_bf16_peak": round(alg / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
           "all_ones_mask_ms": round(oms, 4),
           "all_ones_tflops": round(dense / (oms * 1e-3) / 1e12, 1),
           "ideal_speedup": round(dense / alg, 3)}
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        q = d["Q"].view(w.T, w.Hq, w.dh).transpose(0, 1).contiguous()[None]
        k = d["K"].view(w.T, w.Hk, w.dh).transpose(0, 1).contiguous()[None]
        v = d["V"].view(w.T, w.Hk, w.dh).transpose(0, 1).contiguous()[None]

        def sdpa():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                return torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True,
                                                                        enable_gqa=True)
        sdpa()
        torch.cuda.synchronize()
        for _ in range(2):
            sdpa()
        sms = time_events(torch, sdpa, max(5, steps // 2))
        out.update({"sdpa_ms": round(sms, 4), "sdpa_tflops": round(dense / (sms * 1e-3) / 1e12, 1),
                    "speedup_vs_sdpa": round(sms / ms, 3)})
        del q, k, v
    except Exception as e:  # no fused SDPA backend for this device / build
        out["sdpa_error"] = f"{type(e).__name__}: {str(e)[:200]}"
    out["decode"] = bench_attention_decode(torch, wide, d, w, steps)
    del d, O, ws
    torch.cuda.empty_cache()
    return out


def bench_attention_decode(torch, wide, d, w, steps: int):
    """One decoding step over the T-token cache (query at position T - 1),
    half of the KV groups kept, against every group kept and torch's SDPA for
    one query. A graph of 16 calls is replayed (the binding's host-side checks
    would otherwise dominate), the calls rotating over 8 copies of the cache so
    each reads HBM rather than the last call's cache lines; bytes = the kept
    groups' K and V rows."""
    dev = "cuda:0"
    q = d["Q"][w.T - 1].contiguous()
    kv = [(d["K"], d["V"])] + [(d["K"].clone(), d["V"].clone()) for _ in range(7)]
    keep = torch.tensor([1, 0] * (w.Hk // 2) + [1] * (w.Hk % 2), dtype=torch.uint8, device=dev)
    ones = torch.ones_like(keep)
    O = torch.empty((w.Hq * w.dh,), dtype=torch.bfloat16, device=dev)
    ws = torch.empty(wide.attention_decode_workspace_size(w.T, w.Hq, w.dh), dtype=torch.uint8,
                     device=dev)
    res = {}
    for name, m in (("half_groups", keep), ("all_groups", ones)):
        for K, V in kv:
            wide.attention_decode(q, K, V, m, w.Hq, w.Hk, O=O, workspace=ws)

        def calls16():
            for i in range(16):
                K, V = kv[i % len(kv)]
                wide.attention_decode(q, K, V, m, w.Hq, w.Hk, O=O, workspace=ws)
        us = graph_step_ms(torch, calls16, max(steps, 10)) / 16 * 1e3
        nbytes = int(m.sum()) * 2 * w.T * w.dh * 2
        res[name] = {"us": round(us, 2), "kv_bytes": nbytes,
                     "GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                     "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / PEAK_HBM_GBS, 4)}
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
        qq = q.view(1, w.Hq, 1, w.dh)
        k = d["K"].view(w.T, w.Hk, w.dh).transpose(0, 1).contiguous()[None]
        v = d["V"].view(w.T, w.Hk, w.dh).transpose(0, 1).contiguous()[None]

        def sdpa():
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION, SDPBackend.EFFICIENT_ATTENTION]):
                return torch.nn.functional.scaled_dot_product_attention(qq, k, v, enable_gqa=True)
        sdpa()
        torch.cuda.synchronize()
        res["sdpa_us"] = round(time_events(torch, sdpa, max(steps, 10)) * 1e3, 2)
        del k, v
    except Exception as e:
        res["sdpa_error"] = f"{type(e).__name__}: {str(e)[:200]}"
    del kv
    return res


def bench_router(torch, wide, dg, steps: int):
    """The bottleneck router (mask production) at the Llama3.1-8B FFN shape:
    D = 4096, r = 32, 112 groups, SiLU, for the prefill length and T = 1,
    over 8 copies of X in turn."""
    out = {}
    dev = "cuda:0"
    D, r, ng = 4096, 32, 112
    rw = dg.make_router_weights(7, D, r, ng)
    W1, W2 = rw["W1"].to(dev), rw["W2"].to(dev)
    for T in (16384, 1):
        X0 = dg.to_dtype(dg.normal_f32(8, (T, D)), "bf16").to(dev)
        # the calls rotate over 8 copies of X, so each reads HBM rather than
        # the previous call's lines in the 256 MB MALL
        xs = [X0] + [X0.clone() for _ in range(7)]
        mask = torch.empty((T, ng), dtype=torch.uint8, device=dev)
        for X in xs:
            wide.router_forward(X, W1, W2, "silu", mask=mask)

        # replay of a graph holding 16 calls: the binding's host-side checks
        # (and one graph launch per call) would dominate at T = 1
        def calls16():
            for i in range(16):
                wide.router_forward(xs[i % len(xs)], W1, W2, "silu", mask=mask)
        ms = graph_step_ms(torch, calls16, max(steps, 10)) / 16
        nbytes = T * D * 2 + T * ng + r * D * 2 + 2 * ng * r * 2
        # router fused with the reorder (wide_router_reorder: X -> packed bits
        # -> row lists) against the unfused chain (router -> mask bytes -> the
        # FFN's pack + partition stage) on the same rotated copies of X
        fused = [wide.RouterReorderCall(X, W1, W2, "silu", wide.WIDE_TOKEN_TILE) for X in xs]
        Z = torch.zeros((T, 64), dtype=torch.bfloat16, device=dev)
        Wz = torch.zeros((ng * 64, 64), dtype=torch.bfloat16, device=dev)
        Wdz = torch.zeros((64, ng * 64), dtype=torch.bfloat16, device=dev)
        reo = wide.FfnCall(Z, Wz, Wz, Wdz, mask, 64, flags=wide.WIDE_FLAG_FORCE_PREFILL)

        def chain16():
            for i in range(16):
                wide.router_forward(xs[i % len(xs)], W1, W2, "silu", mask=mask)
                reo.stage(wide.WIDE_STAGE_REORDER)

        def fused16():
            for i in range(16):
                fused[i % len(fused)].run()
        for f in (chain16, fused16):
            f()
        cms = graph_step_ms(torch, chain16, max(steps, 10)) / 16
        fms = graph_step_ms(torch, fused16, max(steps, 10)) / 16
        out[f"T{T}"] = {"us": round(ms * 1e3, 2), "bytes": nbytes,
                        "GBps": round(nbytes / (ms * 1e-3) / 1e9, 1),
                        "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                        "execute_fraction": round(float(mask.float().mean()), 4),
                        "router_then_reorder_us": round(cms * 1e3, 2),
                        "router_reorder_fused_us": round(fms * 1e3, 2)}
        del xs, X0, mask, fused, reo, Z, Wz, Wdz
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


def achievable_peaks(torch, steps: int = 10):
    """Context for the fixed peaks: hipBLASLt on a dense 8192^3 bf16 GEMM, and
    a 1 GiB device copy (read + write bytes over time)."""
    dev = "cuda:0"
    a = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    b = torch.randn(8192, 8192, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        a @ b
    ms = time_events(torch, lambda: a @ b, steps)
    del a, b
    src = torch.empty(COPY_BYTES // 2, device=dev, dtype=torch.bfloat16)
    dst = torch.empty_like(src)
    dst.copy_(src)
    cms = time_events(torch, lambda: dst.copy_(src), steps)
    del src, dst
    torch.cuda.empty_cache()
    return {"hipblaslt_8192cube_bf16_tflops": round(2 * 8192 ** 3 / (ms * 1e-3) / 1e12, 1),
            "device_copy_GBps": round(2 * COPY_BYTES / (cms * 1e-3) / 1e9, 1)}


def host_cpus():
    """What the host offers: the CPU model, the cores this process may run on
    (sched affinity, as nproc reports) and the logical CPUs of the machine."""
    try:
        nproc = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        nproc = os.cpu_count() or 0
    return {"cpu_model": cpu_model(), "nproc": nproc, "logical_cpus": os.cpu_count(),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def cpu_baseline(oracle, inp, w, target_s: float = 12.0):
    """fp64 oracle on a seeded token sample, scaled to effective TFLOP/s.

    The oracle is rebuilt here with gcc -O3 -march=native (same arithmetic)
    so the baseline uses this host's vector units."""
    import numpy as np
    build = "gcc -O2 (prebuilt)"
    try:
        oracle.use_library(oracle.build_native(tempfile.mkdtemp(prefix="wide_oracle_native_")))
        build = "gcc -O3 -march=native -fopenmp, built on this host"
    except Exception as e:  # noqa: BLE001 - report, keep the -O2 build
        log(f"native oracle build failed ({e}); timing the -O2 build")
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
    out = {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
           "kind": "oracle", "build": build,
           "sample": f"{n} of {w.T} tokens (seeded), fp64, {t:.1f} s; effective flops of the "
                     f"sampled tokens' active groups"}
    out.update(host_cpus())
    return out


def decode_setup(torch, wide, dg, w, copies: int):
    inp = dg.make_inputs(w)
    dev = "cuda:0"
    X = inp["X"].to(dev)
    mask = inp["mask"].to(dev)
    ws = [{k: inp[k].to(dev) for k in ("Wg", "Wu", "Wd")}]
    for _ in range(copies - 1):
        ws.append({k: v.clone() for k, v in ws[0].items()})
    calls = [wide.FfnCall(X, c["Wg"], c["Wu"], c["Wd"], mask, w.G) for c in ws]
    union = int(inp["mask"].numpy().any(axis=0).sum())
    return calls, ws, union


def prepared_calls(wide, calls, ws):
    """The calls of decode_setup on operand-order copies of their weights."""
    out = []
    for c, w in zip(calls, ws):
        X, _, _, _, mask = c.args
        prep = wide.decode_prepare_weights(w["Wg"], w["Wu"], w["Wd"])
        out.append(wide.FfnCall(X, w["Wg"], w["Wu"], w["Wd"], mask, c.G, prepared=prep))
    return out


def bench_decode(torch, wide, dg, steps: int, copies: int = 8):
    res = {}
    for w in (dg.LLAMA8B_DECODE_T1, dg.LLAMA8B_DECODE_T16):
        log(f"decode {w.name}")
        calls, ws, union = decode_setup(torch, wide, dg, w, copies)
        act_bytes = 3 * w.d * w.G * union * 2
        for c in calls:
            c.run()
        n = max(steps, 4) * copies
        idx = [0]

        def step():
            calls[idx[0] % copies].run()
            idx[0] += 1

        ms = time_events(torch, step, n)

        def stage_fn(st):
            def f():
                calls[idx[0] % copies].stage(st)
                idx[0] += 1
            return f
        # the down GEMV reads the H its copy's gate/up wrote on an earlier step
        ms_gu = time_events(torch, stage_fn(wide.WIDE_STAGE_DECODE_GATE_UP), n)
        ms_dn = time_events(torch, stage_fn(wide.WIDE_STAGE_DECODE_DOWN), n)

        # graph replay: one graph holding `copies` steps over the rotated weights
        def all_copies():
            for c in calls:
                c.run()
        gms = graph_step_ms(torch, all_copies, max(steps, 4)) / copies
        gu_bytes = 2 * w.d * w.G * union * 2
        dn_bytes = w.d * w.G * union * 2
        # torch's dense GEMVs on the same rotated weight copies
        X0 = calls[0].args[0]
        dfns = [dense_ffn_fn(torch, X0, c["Wg"], c["Wu"], c["Wd"]) for c in ws]
        for f in dfns:
            f()
        dms = time_events(torch, rotating(dfns), n)
        res[f"T{w.T}"] = {"us_per_step": ms * 1e3, "active_weight_GBps": act_bytes / ms / 1e6,
                          "dense_us": dms * 1e3, "speedup_vs_dense": dms / ms,
                          "hbm_frac": act_bytes / ms / 1e6 / PEAK_HBM_GBS,
                          "graph_us_per_step": gms * 1e3,
                          "graph_hbm_frac": act_bytes / gms / 1e6 / PEAK_HBM_GBS,
                          "active_groups": union, "active_weight_MB": act_bytes / 1e6,
                          "weight_copies": copies,
                          "gate_up_us": ms_gu * 1e3, "gate_up_GBps": gu_bytes / ms_gu / 1e6,
                          "down_us": ms_dn * 1e3, "down_GBps": dn_bytes / ms_dn / 1e6}
        if w is dg.LLAMA8B_DECODE_T16:
            # operand-order weights (wide_ffn_decode_prepared): same results
            # bit for bit, contiguous 1 KB weight operands
            pcalls = prepared_calls(wide, calls, ws)
            for c in pcalls:
                c.run()
            pidx = [0]

            def pstep():
                pcalls[pidx[0] % copies].run()
                pidx[0] += 1
            pms = time_events(torch, pstep, n)

            def all_prepared():
                for c in pcalls:
                    c.run()
            pgms = graph_step_ms(torch, all_prepared, max(steps, 4)) / copies
            res[f"T{w.T}"]["operand_order_weights"] = {
                "us_per_step": pms * 1e3, "active_weight_GBps": act_bytes / pms / 1e6,
                "hbm_frac": act_bytes / pms / 1e6 / PEAK_HBM_GBS,
                "graph_us_per_step": pgms * 1e3,
                "prepared_MB": wide.decode_weights_size(w.d, w.d_ff) / 1e6,
                "entry": "wide_ffn_decode_prepared"}
            del pcalls
        del calls, ws
        torch.cuda.empty_cache()
    return res


def dense_ffn_fn(torch, X, Wg, Wu, Wd):
    """The unpruned FFN with torch's matmuls (hipBLASLt GEMMs / GEMVs)."""
    def f():
        a = X @ Wg.t()
        b = X @ Wu.t()
        return (torch.nn.functional.silu(a) * b) @ Wd.t()
    return f


def rotating(fns):
    """A callable that runs fns[0], fns[1], ... in turn (one per call)."""
    idx = [0]

    def f():
        fns[idx[0] % len(fns)]()
        idx[0] += 1
    return f


def bench_prefill_cell(torch, wide, w, inp, steps: int, dense: bool = True):
    """One prefill-sized workload: the library call (eager, events) next to the
    dense torch FFN on the same operands; effective TFLOP/s of the active
    pairs, roofline fraction against the bf16 (fp32) peak, speedups."""
    dev = "cuda:0"
    d = {k: v.to(dev) for k, v in inp.items()}
    A = int(inp["mask"].sum())
    ng = w.ngroups
    call = wide.FfnCall(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G)
    for _ in range(2):
        call.run()
    ms = time_events(torch, call.run, steps)
    flops = 6.0 * w.d * w.G * A
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_FP32_TFLOPS
    out = {"T": w.T, "G": w.G, "groups": ng, "active_pairs": A,
           "sparsity": round(1 - A / max(w.T * ng, 1), 4), "ms": round(ms, 4),
           "effective_tflops": round(flops / (ms * 1e-3) / 1e12, 2),
           "roofline_frac": round(flops / (ms * 1e-3) / 1e12 / peak, 4),
           "ideal_speedup": round(w.T * ng / A, 3) if A else None}
    if dense:
        f = dense_ffn_fn(torch, d["X"], d["Wg"], d["Wu"], d["Wd"])
        for _ in range(2):
            f()
        dms = time_events(torch, f, steps)
        out["dense_ms"] = round(dms, 4)
        out["speedup_vs_dense"] = round(dms / ms, 3)
    del call, d
    return out


def bench_decode_cell(torch, wide, w, inp, steps: int, copies: int = 8, dense: bool = True):
    """One decode workload (T <= 16): calls rotate over `copies` device copies of
    the weights so every call reads HBM; active-weight GB/s against the HBM
    peak; torch's dense GEMVs on the same rotated copies."""
    dev = "cuda:0"
    X = inp["X"].to(dev)
    mask = inp["mask"].to(dev)
    ws = [{k: inp[k].to(dev) for k in ("Wg", "Wu", "Wd")}]
    for _ in range(copies - 1):
        ws.append({k: v.clone() for k, v in ws[0].items()})
    calls = [wide.FfnCall(X, c["Wg"], c["Wu"], c["Wd"], mask, w.G) for c in ws]
    union = int(inp["mask"].numpy().any(axis=0).sum())
    act_bytes = 3 * w.d * w.G * union * 2
    for c in calls:
        c.run()
    n = max(steps, 4) * copies
    ms = time_events(torch, rotating([c.run for c in calls]), n)
    out = {"T": w.T, "G": w.G, "active_groups": union, "groups": w.ngroups,
           "us": round(ms * 1e3, 2), "active_weight_MB": round(act_bytes / 1e6, 2),
           "active_weight_GBps": round(act_bytes / ms / 1e6, 1),
           "hbm_frac": round(act_bytes / ms / 1e6 / PEAK_HBM_GBS, 4), "weight_copies": copies}
    if dense:
        fns = [dense_ffn_fn(torch, X, c["Wg"], c["Wu"], c["Wd"]) for c in ws]
        for f in fns:
            f()
        dms = time_events(torch, rotating(fns), n)
        out["dense_us"] = round(dms * 1e3, 2)
        out["speedup_vs_dense"] = round(dms / ms, 3)
    del calls, ws, X, mask
    return out


def bench_configs(torch, wide, dg, steps: int):
    """Every workload of the measured set beside the headline: the tiny fp32
    SwiGLU, the Llama3.2-3B-shaped G x sparsity sweep (every G at 50% for
    T = 8192, 2048 and 1, every sparsity level at G = 128), and the
    Qwen3-14B-shaped skewed masks with the all-ones and all-zero limits."""
    import dataclasses
    out = {}
    # tiny fp32 SwiGLU: launch-bound; timed eagerly and by graph replay
    w = dg.TINY
    log(f"config {w.name}")
    inp = dg.make_inputs(w)
    cell = bench_prefill_cell(torch, wide, w, inp, max(steps, 50))
    d = {k: v.to("cuda:0") for k, v in inp.items()}
    call = wide.FfnCall(d["X"], d["Wg"], d["Wu"], d["Wd"], d["mask"], w.G)
    cell["graph_us"] = round(graph_step_ms(torch, call.run, max(steps, 50)) * 1e3, 2)
    cell["note"] = "fp32 VALU path; launch-bound at this size"
    out[w.name] = cell
    del call, d
    # Llama3.2-3B sweep
    cells = {(c.G, round((1 - c.density) * 100), c.T): c for c in dg.llama3b_sweep_cells()}
    want = [(G, 50, T) for T in (8192, 2048, 1) for G in (16, 32, 64, 128, 256, 512)]
    want += [(128, s, 8192) for s in (10, 25, 70)]
    base = cells[(128, 50, 8192)]
    wts = dg.make_inputs(base, T=1)  # weights depend only on the workload id
    xs = {T: dg.make_inputs(base, T=T, weights=False)["X"] for T in (8192, 2048, 1)}
    sweep = []
    for key in want:
        c = cells[key]
        log(f"config {c.name}")
        inp = {"X": xs[c.T], "Wg": wts["Wg"], "Wu": wts["Wu"], "Wd": wts["Wd"],
               "mask": torch.from_numpy(dg.make_mask(c))}
        r = (bench_prefill_cell(torch, wide, c, inp, steps) if c.T > 16
             else bench_decode_cell(torch, wide, c, inp, steps))
        r["target_sparsity"] = key[1] / 100
        sweep.append(r)
        torch.cuda.empty_cache()
    out["llama3.2-3b-sweep"] = sweep
    del wts, xs
    # Qwen3-14B skewed masks and the two limits
    w = dg.QWEN14B_SKEW
    inp = dg.make_inputs(w)
    q = {}
    for kind in ("zipf", "ones", "zeros"):
        log(f"config {w.name} mask={kind}")
        inp["mask"] = torch.from_numpy(dg.make_mask(w, kind))
        q[kind] = bench_prefill_cell(torch, wide, w, inp, steps)
        torch.cuda.empty_cache()
    out[w.name] = q
    del inp
    torch.cuda.empty_cache()
    # where decode hands over to prefill: both paths at small T (Llama3.1-8B shape)
    thr = {}
    w = dg.LLAMA8B_DECODE_T16
    full = dg.make_inputs(w)
    for T in (1, 2, 4, 8, 16):
        wt = dataclasses.replace(w, T=T, name=f"{w.name[:-3]}t{T}")
        inp = dict(full, X=full["X"][:T].contiguous(), mask=full["mask"][:T].contiguous())
        dv = {k: v.to("cuda:0") for k, v in inp.items()}
        row = {}
        for path, flags in (("decode", wide.WIDE_FLAG_FORCE_DECODE),
                            ("prefill", wide.WIDE_FLAG_FORCE_PREFILL)):
            c = wide.FfnCall(dv["X"], dv["Wg"], dv["Wu"], dv["Wd"], dv["mask"], wt.G, flags=flags)
            c.run()
            row[f"{path}_us"] = round(time_events(torch, c.run, max(steps, 10)) * 1e3, 2)
            del c
        thr[f"T{T}"] = row
        del dv
    thr["decode_max_t"] = wide.decode_max_t()
    thr["note"] = ("same weights every call (MALL-warm for both paths); the library takes the "
                   "decode path for T <= decode_max_t")
    out["decode_vs_prefill_small_t"] = thr
    torch.cuda.empty_cache()
    return out


def run_profile(steps: int):
    """Short run for rocprofv3: prefill steps, decode steps, and one copy of known size."""
    import torch
    import group_sparse_ffn_amd as wide
    from group_sparse_ffn_amd import datagen as dg
    r = bench_prefill(torch, wide, dg, steps, 1, graph=False)
    del r["call"], r["dev_inputs"]
    torch.cuda.empty_cache()
    # the Qwen3-14B-shaped prefill on its Zipf-skewed mask
    qw = dg.QWEN14B_SKEW
    qd = {k: v.to("cuda:0") for k, v in dg.make_inputs(qw).items()}
    qc = wide.FfnCall(qd["X"], qd["Wg"], qd["Wu"], qd["Wd"], qd["mask"], qw.G)
    for _ in range(PROFILE_QWEN_CALLS):
        qc.run()
    torch.cuda.synchronize()
    del qc, qd
    torch.cuda.empty_cache()
    for w in (dg.LLAMA8B_DECODE_T1, dg.LLAMA8B_DECODE_T16):
        calls, ws, _ = decode_setup(torch, wide, dg, w, 8)
        for _ in range(2):
            for c in calls:
                c.run()
        torch.cuda.synchronize()
        if w is dg.LLAMA8B_DECODE_T16:
            # the same steps with operand-order weights
            pcalls = prepared_calls(wide, calls, ws)
            for _ in range(2):
                for c in pcalls:
                    c.run()
            torch.cuda.synchronize()
            del pcalls
        del calls, ws
        torch.cuda.empty_cache()
    for w in PROFILE_GEMMS(dg):
        inp = {k: v.to("cuda:0") for k, v in dg.make_gemm_inputs(w).items()}
        # (router calls follow the masked GEMMs)
        fn = wide.gemm_mn if w.axis == "mn" else wide.gemm_k
        for _ in range(PROFILE_GEMM_CALLS):
            fn(inp["A"], inp["B"], inp["mask"], w.G)
        torch.cuda.synchronize()
        del inp
        torch.cuda.empty_cache()
    rw = dg.make_router_weights(7, 4096, 32, 112)
    W1, W2 = rw["W1"].to("cuda:0"), rw["W2"].to("cuda:0")
    for T in PROFILE_ROUTER_T:
        X = dg.to_dtype(dg.normal_f32(8, (T, 4096)), "bf16").to("cuda:0")
        for _ in range(PROFILE_GEMM_CALLS):
            wide.router_forward(X, W1, W2, "silu")
        torch.cuda.synchronize()
        del X
    aw = dg.LLAMA8B_ATTN_PREFILL
    ad = {k: v.to("cuda:0") for k, v in dg.make_attention_inputs(aw).items()}
    for _ in range(PROFILE_GEMM_CALLS):
        wide.attention_prefill(ad["Q"], ad["K"], ad["V"], ad["mask"], aw.Hq, aw.Hk)
    torch.cuda.synchronize()
    # decode steps over the same cache, half of the KV groups kept
    keep = torch.tensor([1, 0] * (aw.Hk // 2), dtype=torch.uint8, device="cuda:0")
    qd = ad["Q"][aw.T - 1].contiguous()
    for _ in range(PROFILE_DECODE_CALLS):
        wide.attention_decode(qd, ad["K"], ad["V"], keep, aw.Hq, aw.Hk)
    torch.cuda.synchronize()
    del ad
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"profile run done: {steps} prefill steps, 16 decode steps per T, "
        f"{PROFILE_GEMM_CALLS} calls per masked GEMM, one {COPY_BYTES} B copy")


PROFILE_GEMM_CALLS = 3
PROFILE_DECODE_CALLS = 16
PROFILE_QWEN_CALLS = 5
T16_PREPARED = "llama3.1-8b-ffn-decode-t16-operand-order-weights"
PROFILE_ROUTER_T = (16384, 1)
ROUTER_WORKLOADS = {16384: "llama3.1-8b-router-prefill", 1: "llama3.1-8b-router-decode-t1"}
ATTN_DECODE_WORKLOAD = "llama3.1-8b-attention-decode-t16384-half-groups"


def PROFILE_GEMMS(dg):
    return (dg.LLAMA8B_ATTN_Q, dg.LLAMA8B_ATTN_O, dg.LLAMA8B_DEPTH)


def profile_plan(dg, steps: int):
    """(workload, kernel, dispatches) in the order `--profile --steps N` launches them."""
    n = 1 + 2 * steps  # warmup, timed and staged prefill steps
    pre = dg.LLAMA8B_PREFILL.name
    # the reorder stage is the mask-bit packing and the per-group partition
    plan = [(pre, "pack_mask_bits", n), (pre, "reorder_bits", n), (pre, "gate_up", n),
            (pre, "down", n)]
    qw = dg.QWEN14B_SKEW.name
    # the Qwen3-14B down projection splits its last round (320 tiles = 256 + 64)
    plan += [(qw, "pack_mask_bits", PROFILE_QWEN_CALLS), (qw, "reorder_bits", PROFILE_QWEN_CALLS),
             (qw, "gate_up", PROFILE_QWEN_CALLS), (qw, "down", PROFILE_QWEN_CALLS),
             (qw, "down_split_reduce", PROFILE_QWEN_CALLS)]
    # T = 1 takes the whole-row VALU GEMVs; T = 16 the MFMA gate/up with the
    # activations in LDS and the split-K down with its reduce
    t1, t16 = dg.LLAMA8B_DECODE_T1.name, dg.LLAMA8B_DECODE_T16.name
    plan += [(t1, "decode_gate_up_valu", PROFILE_DECODE_CALLS),
             (t1, "decode_down_valu", PROFILE_DECODE_CALLS),
             (t16, "decode_gate_up_xlds", PROFILE_DECODE_CALLS),
             (t16, "decode_down_splitk", PROFILE_DECODE_CALLS),
             (t16, "decode_down_reduce", PROFILE_DECODE_CALLS),
             (T16_PREPARED, "decode_gate_up_packed", PROFILE_DECODE_CALLS),
             (T16_PREPARED, "decode_down_splitk_packed", PROFILE_DECODE_CALLS),
             (T16_PREPARED, "decode_down_reduce", PROFILE_DECODE_CALLS)]
    for w in PROFILE_GEMMS(dg):
        if w.axis == "mn":
            plan += [(w.name, "pack_mask_bits", PROFILE_GEMM_CALLS),
                     (w.name, "reorder_bits", PROFILE_GEMM_CALLS),
                     (w.name, "gemm_mn", PROFILE_GEMM_CALLS)]
        else:
            plan += [(w.name, "pack_mask_bits", PROFILE_GEMM_CALLS),
                     (w.name, "down", PROFILE_GEMM_CALLS)]
    plan += [(ROUTER_WORKLOADS[16384], "router", PROFILE_GEMM_CALLS),
             (ROUTER_WORKLOADS[1], "router_zpart", PROFILE_GEMM_CALLS),
             (ROUTER_WORKLOADS[1], "router_decide", PROFILE_GEMM_CALLS)]
    aw = dg.LLAMA8B_ATTN_PREFILL.name
    plan += [(aw, "pack_mask_bits", PROFILE_GEMM_CALLS), (aw, "reorder_bits", PROFILE_GEMM_CALLS),
             (aw, "attention_vt", PROFILE_GEMM_CALLS), (aw, "attention_prefill", PROFILE_GEMM_CALLS),
             (ATTN_DECODE_WORKLOAD, "attention_decode_split", PROFILE_DECODE_CALLS),
             (ATTN_DECODE_WORKLOAD, "attention_decode_merge", PROFILE_DECODE_CALLS)]
    return plan


def split_by_plan(plan, dispatches):
    """dispatches: kernel -> [(dispatch id, value)] -> {(workload, kernel): [values]}.

    Each kernel's dispatches, in dispatch order, are dealt to the plan entries of
    that kernel in plan order."""
    out = {}
    for kernel in {k for _, k, _ in plan}:
        seq = sorted(dispatches.get(kernel, []))
        pos = 0
        for workload, k, n in plan:
            if k != kernel:
                continue
            out[(workload, kernel)] = [v for _, v in seq[pos:pos + n]]
            pos += n
    return out


# flops of one MFMA instruction of each kernel (its instruction shape)
MFMA_FLOPS = {"gate_up": 2 * 32 * 32 * 16, "down": 2 * 32 * 32 * 16, "gemm_mn": 2 * 32 * 32 * 16,
              "decode_gate_up": 2 * 16 * 16 * 32, "decode_down_splitk": 2 * 16 * 16 * 32,
              "decode_gate_up_xlds": 2 * 16 * 16 * 32,
              "decode_gate_up_packed": 2 * 16 * 16 * 32,
              "decode_down_splitk_packed": 2 * 16 * 16 * 32,
              "router": 2 * 16 * 16 * 32, "router_zpart": 2 * 16 * 16 * 32,
              "router_decide": 2 * 16 * 16 * 4,
              "attention_prefill": 2 * 32 * 32 * 16}


def work_closed_forms(dg):
    """(workload, kernel) -> (algorithmic flops, flops the kernel is designed to execute)."""
    pre = dg.LLAMA8B_PREFILL
    A = pre.T * (pre.ngroups // 2)  # top-50% masks: exactly ng/2 groups per token
    out = {(pre.name, "gate_up"): (4.0 * pre.d * pre.G * A, 4.0 * pre.d * pre.G * A),
           (pre.name, "down"): (2.0 * pre.d * pre.G * A, 2.0 * pre.T * pre.d * pre.d_ff)}
    qw = dg.QWEN14B_SKEW
    qa = int(dg.make_mask(qw).sum())
    out[(qw.name, "gate_up")] = (4.0 * qw.d * qw.G * qa, 4.0 * qw.d * qw.G * qa)
    out[(qw.name, "down")] = (2.0 * qw.d * qw.G * qa, 2.0 * qw.T * qw.d * qw.d_ff)
    for w in (dg.LLAMA8B_ATTN_Q, dg.LLAMA8B_ATTN_O, dg.LLAMA8B_DEPTH):
        a = int(dg.make_gemm_mask(w).sum())
        if w.axis == "mn":
            out[(w.name, "gemm_mn")] = (2.0 * w.K * w.G * a, 2.0 * w.K * w.G * a)
        else:
            out[(w.name, "down")] = (2.0 * w.N * w.G * a, 2.0 * w.M * w.N * w.K)
    t16 = dg.LLAMA8B_DECODE_T16
    # 16 token columns per MFMA; every group is live at T = 16
    out[(t16.name, "decode_gate_up_xlds")] = (2.0 * 2 * t16.d_ff * t16.d * 16,) * 2
    out[(t16.name, "decode_down_splitk")] = (2.0 * t16.d_ff * t16.d * 16,) * 2
    out[(T16_PREPARED, "decode_gate_up_packed")] = (2.0 * 2 * t16.d_ff * t16.d * 16,) * 2
    out[(T16_PREPARED, "decode_down_splitk_packed")] = (2.0 * t16.d_ff * t16.d * 16,) * 2
    out[("llama3.1-8b-router-prefill", "router")] = (2.0 * 16384 * 4096 * 32,) * 2
    # T = 1: the first map runs 16 token rows (one MFMA block); the second map
    # 16 rows x 2 N_G columns x r
    out[("llama3.1-8b-router-decode-t1", "router_zpart")] = (2.0 * 16 * 4096 * 32,) * 2
    out[("llama3.1-8b-router-decode-t1", "router_decide")] = (2.0 * 16 * 224 * 32,) * 2
    aw = dg.LLAMA8B_ATTN_PREFILL
    out[(aw.name, "attention_prefill")] = attention_work(dg.make_attention_inputs(aw)["mask"], aw)
    return out


def attention_work(mask, w):
    """(algorithmic flops, flops the kernel executes) of one attention call.

    Algorithmic: 4 dh (t + 1) per kept (token t, query head). Executed: every
    wave with a kept query runs 32 MFMAs of 32x32x16 per 64-key tile up to
    its last query's position (queries in reordered order, 32 per wave)."""
    import numpy as np
    m = mask.numpy().astype(bool)
    T = m.shape[0]
    hpg = w.Hq // w.Hk
    alg = exe = 0.0
    for g in range(w.Hk):
        toks = np.nonzero(m[:, g])[0]  # ascending: the partition's active prefix
        alg += hpg * 4.0 * w.dh * float((toks + 1).sum())
        last = toks[np.minimum(np.arange(31, len(toks) + 31, 32), len(toks) - 1)] if len(toks) else toks
        exe += hpg * float((last // 64 + 1).sum()) * 32 * 2 * 32 * 32 * 16
    return alg, exe


def mfma_summary(directory, command, plan, split_fn):
    """profiles/mfma_work_llama8b.md: MFMA instructions counted by rocprofv3 x
    flops per instruction, against the closed forms of the work."""
    from group_sparse_ffn_amd import datagen as dg
    per_id = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != "SQ_INSTS_MFMA":
                continue
            k = next((kk for kk, v in KERNEL_SYMBOLS.items() if v in r["Kernel_Name"]), None)
            if k is not None:
                per_id.setdefault(k, []).append((int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    if not per_id:
        return
    split = split_fn(plan, per_id)
    forms = work_closed_forms(dg)
    lines = ["# MFMA work per launch: counted vs closed form", "",
             "`SQ_INSTS_MFMA` from a rocprofv3 counter run of the command below, averaged over",
             "each kernel's dispatches for the workload, times the flops of the kernel's MFMA",
             "instruction (32x32x16 bf16 = 32768, 16x16x32 bf16 = 16384). `algorithmic` is the",
             "method's work (active pairs only); `designed` is what the kernel is built to",
             "execute (the down kernel runs the dense product; decode pads tokens to 16).",
             "The router's ratio is not 1: its second map runs v_mfma_f32_16x16x4_f32",
             "(2048 flops), which the counter counts beside the 16x16x32 bf16 instructions of",
             "the first map and this table prices at 16384.", "",
             "```", command.replace("PMC", "SQ_INSTS_MFMA").replace("PASS", "mfma"), "```", CMD_NOTE, "",
             "| kernel | workload | counted TFLOP | algorithmic TFLOP | designed TFLOP | counted / designed |",
             "|---|---|---|---|---|---|"]
    for workload, kernel, _ in plan:
        v = split.get((workload, kernel), [])
        if not v or (workload, kernel) not in forms or kernel not in MFMA_FLOPS:
            continue
        counted = sum(v) / len(v) * MFMA_FLOPS[kernel]
        alg, des = forms[(workload, kernel)]
        lines.append(f"| {kernel} | {workload} | {counted / 1e12:.4f} | {alg / 1e12:.4f} | "
                     f"{des / 1e12:.4f} | {counted / des:.4f} |")
    out = os.path.join(ROOT, "profiles", "mfma_work_llama8b.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def busy_summary(directory, command, plan, split_fn, out_dir=None):
    """profiles/mfma_busy_llama8b.md: from one counter run with SQ_VALU_MFMA_BUSY_CYCLES
    and GRBM_GUI_ACTIVE, the shader clock each kernel ran at and the share of
    SIMD cycles its matrix cores were busy."""
    from group_sparse_ffn_amd import datagen as dg
    agents = glob.glob(os.path.join(directory, "**", "*agent_info.csv"), recursive=True)
    gpu = None
    for path in agents:
        for r in csv.DictReader(open(path)):
            if r.get("Agent_Type") == "GPU":
                gpu = r
    if gpu is None:
        return
    nxcc, nsimd = int(gpu["Num_Xcc"]), int(gpu["Simd_Count"])
    vals = {}  # counter -> kernel -> [(dispatch id, value)]
    durs = {}  # kernel -> [(dispatch id, ns)]
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            name = r["Counter_Name"]
            if name not in ("SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"):
                continue
            k = next((kk for kk, v in KERNEL_SYMBOLS.items() if v in r["Kernel_Name"]), None)
            if k is None:
                continue
            did = int(r["Dispatch_Id"])
            vals.setdefault(name, {}).setdefault(k, []).append((did, float(r["Counter_Value"])))
            if name == "GRBM_GUI_ACTIVE":
                durs.setdefault(k, []).append(
                    (did, int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    if len(vals) < 2:
        return
    busy = split_fn(plan, vals["SQ_VALU_MFMA_BUSY_CYCLES"])
    gui = split_fn(plan, vals["GRBM_GUI_ACTIVE"])
    dur = split_fn(plan, durs)
    forms = work_closed_forms(dg)
    lines = ["# Shader clock and MFMA busy share per launch", "",
             "One rocprofv3 counter run of the command below with SQ_VALU_MFMA_BUSY_CYCLES and",
             f"GRBM_GUI_ACTIVE, averaged over each kernel's dispatches for the workload.",
             f"GRBM_GUI_ACTIVE is summed over the {nxcc} XCDs, so one XCD's active cycles are",
             f"the value / {nxcc}; the clock is those cycles over the dispatch's duration (shown",
             "for kernels of 100 us or more: for shorter ones the counter window is much longer",
             f"than the kernel). MFMA busy = busy cycles summed over the {nsimd} SIMDs /",
             f"({nsimd} x one XCD's active cycles). `peak at clock` scales the 2.5 PFLOP/s",
             "bf16 dense peak (quoted at 2.4 GHz) to the measured clock; `designed TFLOP/s`",
             "is the kernel's designed MFMA work over its duration.", "",
             "```", command.replace("PMC", "SQ_VALU_MFMA_BUSY_CYCLES GRBM_GUI_ACTIVE").replace("PASS", "busy"),
             "```", CMD_NOTE, "",
             "| kernel | workload | duration (us) | clock (GHz) | MFMA busy | peak at clock (TFLOP/s) "
             "| designed TFLOP/s |",
             "|---|---|---|---|---|---|---|"]
    for workload, kernel, _ in plan:
        b, g, t = (busy.get((workload, kernel), []), gui.get((workload, kernel), []),
                   dur.get((workload, kernel), []))
        if not b or not g or not t:
            continue
        ns = sum(t) / len(t)
        cyc = sum(g) / len(g) / nxcc
        clk = cyc / ns
        frac = (sum(b) / len(b)) / (nsimd * cyc)
        des = forms.get((workload, kernel), (0.0, 0.0))[1]
        rate = f"{des / (ns * 1e-9) / 1e12:.0f}" if des else "-"
        if ns < 100e3:  # the counter window dwarfs the kernel: no clock to read
            lines.append(f"| {kernel} | {workload} | {ns / 1e3:.1f} | - | - | - | {rate} |")
            continue
        peak = PEAK_BF16_TFLOPS * clk / 2.4
        lines.append(f"| {kernel} | {workload} | {ns / 1e3:.1f} | {clk:.2f} | {100 * frac:.1f}% | "
                     f"{peak:.0f} | {rate} |")
    out = os.path.join(out_dir or os.path.join(ROOT, "profiles"), "mfma_busy_llama8b.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out}")


CMD_NOTE = "(<repo>: the repository root; <out>: the folder the runs write to, given to --summarize.)"


def profile_commands(steps: int):
    """The kernel-trace command and the counter-run template (PMC: the
    counters, PASS: the output folder) of a profile run on one MI355X. <repo>
    is the repository root, <out> the folder the runs write to (the one later
    given to --summarize)."""
    pre = "cd /tmp && export TMPDIR=/tmp && rocprofv3"
    run = f"-o run -- python3 <repo>/bench.py --profile --steps {steps}"
    return (f"{pre} --kernel-trace --stats --output-format csv -d <out>/ktrace {run}",
            f"{pre} --pmc PMC --output-format csv -d <out>/PASS {run}")


def summarize(directory: str, command: str, steps: int):
    """Turn rocprofv3 CSVs (kernel trace, FETCH_SIZE and WRITE_SIZE counter runs) into profiles/*.md.

    Dispatches are attributed to workloads by their order in the profile run.
    command: the counter-run template (PMC, PASS placeholders); empty = the
    commands of profile_commands(steps)."""
    from group_sparse_ffn_amd import datagen as dg
    ktrace_cmd, pmc_cmd = profile_commands(steps)
    if command:
        ktrace_cmd = pmc_cmd = command
    command = pmc_cmd
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    plan = profile_plan(dg, steps)

    def kernel_of(name):
        return next((k for k, v in KERNEL_SYMBOLS.items() if v in name), None)

    traces = glob.glob(os.path.join(directory, "**", "*kernel_trace.csv"), recursive=True)
    if traces:
        durs = {}
        for r in csv.DictReader(open(traces[0])):
            k = kernel_of(r["Kernel_Name"])
            if k is not None:
                durs.setdefault(k, []).append(
                    (int(r["Dispatch_Id"]),
                     (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3))
        split = split_by_plan(plan, durs)
        lines = ["# Kernel trace: Llama3.1-8B-shaped FFN (prefill T=16384, decode T=1 and T=16) "
                 "and masked GEMMs at its attention shapes",
                 "", "Command (one MI355X):", "", "```", ktrace_cmd, "```", CMD_NOTE, "",
                 "Per-dispatch durations from the kernel trace, attributed to workloads by "
                 "launch order.", "",
                 "| kernel | workload | calls | median (us) | avg (us) | min (us) | max (us) |",
                 "|---|---|---|---|---|---|---|"]
        for workload, kernel, _ in plan:
            v = split.get((workload, kernel), [])
            if not v:
                continue
            med = sorted(v)[len(v) // 2]
            lines.append(f"| {kernel} | {workload} | {len(v)} | {med:.1f} | {sum(v) / len(v):.1f} | "
                         f"{min(v):.1f} | {max(v):.1f} |")
        out = os.path.join(ROOT, "profiles", "kernel_trace_llama8b.md")
        open(out, "w").write("\n".join(lines) + "\n")
        print(f"wrote {out}")
    mfma_summary(directory, command, plan, split_by_plan)
    busy_summary(directory, command, plan, split_by_plan)
    per = {}     # counter -> kernel name -> values (KiB per dispatch), for the copy calibration
    per_id = {}  # counter -> kernel -> [(dispatch id, value)]
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            per.setdefault(r["Counter_Name"], {}).setdefault(r["Kernel_Name"], []).append(
                float(r["Counter_Value"]))
            k = kernel_of(r["Kernel_Name"])
            if k is not None:
                per_id.setdefault(r["Counter_Name"], {}).setdefault(k, []).append(
                    (int(r["Dispatch_Id"]), float(r["Counter_Value"])))
    if not per:
        return
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        if counter not in per:
            raise SystemExit(f"no {counter} rows under {directory}")

    def copy_kib(counter):
        vals = [v for name, vs in per[counter].items() if "copy" in name.lower()
                for v in vs if v > COPY_BYTES / 1024 * 0.5]
        if not vals:
            raise SystemExit("the calibration copy is missing from the counter runs")
        return sum(vals) / len(vals)

    scale = {c: (COPY_BYTES / 1024) / copy_kib(c) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    split = {c: split_by_plan(plan, per_id.get(c, {})) for c in ("FETCH_SIZE", "WRITE_SIZE")}
    for workload, kernel, _ in plan:
        vals = {}
        for counter in ("FETCH_SIZE", "WRITE_SIZE"):
            vs = split[counter].get((workload, kernel), [])
            if vs:
                vals[counter] = sum(vs) / len(vs)
        if len(vals) < 2:
            continue
        fetch = vals["FETCH_SIZE"] * 1024 * scale["FETCH_SIZE"]
        write = vals["WRITE_SIZE"] * 1024 * scale["WRITE_SIZE"]
        text = [f"# HBM traffic per launch: {kernel} ({workload})", "",
                "Two rocprofv3 counter runs of the command below (one with FETCH_SIZE, one with",
                "WRITE_SIZE), averaged over the kernel's dispatches for this workload, in KiB,",
                f"scaled by what the same counter reads for a device copy of {COPY_BYTES} bytes",
                "in the same run.", "",
                "```", command.replace("PMC", "FETCH_SIZE").replace("PASS", "fetch"),
                command.replace("PMC", "WRITE_SIZE").replace("PASS", "write"), "```", CMD_NOTE, "",
                f"- FETCH_SIZE_KiB: {vals['FETCH_SIZE']:.1f}",
                f"- WRITE_SIZE_KiB: {vals['WRITE_SIZE']:.1f}",
                f"- fetch_scale: {scale['FETCH_SIZE']:.4f}",
                f"- write_scale: {scale['WRITE_SIZE']:.4f}",
                f"- fetch_bytes: {fetch:.0f}",
                f"- write_bytes: {write:.0f}",
                f"- bytes_per_launch: {fetch + write:.0f}",
                f"- source_sha: {source_sha(kernel)}", ""]
        out = traffic_path(kernel, workload)
        open(out, "w").write("\n".join(text))
        print(f"wrote {out}")


BASELINE_PROFILE_S = 2048
BASELINE_PROFILE_AXES = ("n", "k")


def run_profile_baselines():
    """Short run for rocprofv3 counters: one naive gather-scatter call per
    axis at S^3, each bracketed by a marker kernel (a 4-element zeta, a name
    nothing else here launches), then the calibration copy."""
    import torch
    from group_sparse_ffn_amd import baselines as bl
    from group_sparse_ffn_amd import datagen as dg
    dev = "cuda:0"
    S, G = BASELINE_PROFILE_S, 128
    marker_x = torch.full((4,), 2.0, device=dev)
    for axis in BASELINE_PROFILE_AXES:
        w = dg.GemmWorkload(f"baseline-{axis}-{S}", 60 + S % 97, M=S, N=S, K=S, G=G,
                            axis="k" if axis == "k" else "mn", mask_kind="topk", density=0.5)
        inp = {k: v.to(dev) for k, v in dg.make_gemm_inputs(w).items()}
        fn = bl.naive_gemm_mn if axis == "n" else bl.naive_gemm_k
        torch.cuda.synchronize()
        torch.special.zeta(marker_x, marker_x)
        C = fn(inp["A"], inp["B"], inp["mask"], G)
        torch.special.zeta(marker_x, marker_x)
        torch.cuda.synchronize()
        del C, inp
        torch.cuda.empty_cache()
    src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    log(f"baseline profile run done: axes {BASELINE_PROFILE_AXES} at {S}^3, one {COPY_BYTES} B copy")


def summarize_baselines(directory: str, command: str):
    """Measured HBM bytes of each naive call (every dispatch between its two
    markers, FETCH_SIZE + WRITE_SIZE scaled by the calibration copy) beside the
    closed form of the pipeline's traffic."""
    from group_sparse_ffn_amd import baselines as bl
    rows = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(path)):
            rows.setdefault(r["Counter_Name"], []).append(
                (int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    lines = ["# Naive gather-scatter pipelines: measured HBM bytes vs the closed forms", "",
             f"One call per axis at M = N = K = {BASELINE_PROFILE_S}, G = 128, half of every "
             "token's groups active (top-k masks: the same count per token).",
             "Measured: FETCH_SIZE and WRITE_SIZE summed over every dispatch between the call's",
             f"two marker kernels, scaled by what each counter reads for a {COPY_BYTES}-byte",
             "device copy in the same run. Closed form: the pipeline's data-tensor traffic",
             "(masks, indices and offsets excluded), bf16 elements.", "",
             "```", command.replace("PMC", "FETCH_SIZE"), command.replace("PMC", "WRITE_SIZE"), "```", CMD_NOTE, "",
             "The gather reads the weight matrix (S * S * 2 bytes, on-chip-cache sized) once per",
             "token, so HBM sees two of the closed form's three p*M*N*K terms (the gathered",
             "subset written, then read by the batched product); the last two columns drop",
             "the gather's read.", "",
             "| axis | kernels | fetch (GB) | write (GB) | measured (GB) | closed form (GB) | measured / closed form "
             "| closed form without the gather's read (GB) | measured / that |",
             "|---|---|---|---|---|---|---|---|---|"]
    meas = {}
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        if counter not in rows:
            raise SystemExit(f"no {counter} rows under {directory}")
        rs = sorted(rows[counter])
        copies = [v for _, n, v in rs if "copy" in n.lower() and v > COPY_BYTES / 1024 * 0.5]
        if not copies:
            raise SystemExit("the calibration copy is missing from the counter runs")
        scale = (COPY_BYTES / 1024) / (sum(copies) / len(copies))
        marks = [i for i, (_, n, _) in enumerate(rs) if "zeta" in n.lower()]
        if len(marks) != 2 * len(BASELINE_PROFILE_AXES):
            raise SystemExit(f"expected {2 * len(BASELINE_PROFILE_AXES)} markers, found {len(marks)}")
        for a, axis in enumerate(BASELINE_PROFILE_AXES):
            seg = rs[marks[2 * a] + 1:marks[2 * a + 1]]
            meas.setdefault(axis, {})[counter] = (len(seg), sum(v for _, _, v in seg) * 1024 * scale)
    S = BASELINE_PROFILE_S
    for axis in BASELINE_PROFILE_AXES:
        n, fetch = meas[axis]["FETCH_SIZE"]
        _, write = meas[axis]["WRITE_SIZE"]
        closed = 2 * bl.traffic_elements(axis, S, S, S, 0.5)
        hbm = closed - 2 * 0.5 * S * S * S
        lines.append(f"| {axis.upper()} | {n} | {fetch / 1e9:.2f} | {write / 1e9:.2f} | "
                     f"{(fetch + write) / 1e9:.2f} | {closed / 1e9:.2f} | {(fetch + write) / closed:.3f} | "
                     f"{hbm / 1e9:.2f} | {(fetch + write) / hbm:.3f} |")
    out = os.path.join(ROOT, "profiles", f"traffic_naive_gather_scatter_{S}.md")
    open(out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {out}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 20; with --summarize: the profile run's, 5)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-gemm", action="store_true")
    ap.add_argument("--no-baselines", action="store_true")
    ap.add_argument("--no-configs", action="store_true")
    ap.add_argument("--profile", action="store_true")
    ap.add_argument("--summarize", metavar="DIR")
    ap.add_argument("--profile-baselines", action="store_true")
    ap.add_argument("--summarize-baselines", metavar="DIR")
    ap.add_argument("--command", default="")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.command, 5 if args.steps is None else args.steps)
        return
    if args.steps is None:
        args.steps = 20
    if args.summarize_baselines:
        summarize_baselines(args.summarize_baselines, args.command)
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the group-sparse FFN "
              "here has no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if args.profile:
        run_profile(args.steps)
        return
    if args.profile_baselines:
        run_profile_baselines()
        return

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
        "graph_ms_per_step": round(r["graph_ms"], 4),
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
        # the same library path on an all-ones mask: the dense limit of these kernels
        dv = r["dev_inputs"]
        ones = torch.ones_like(dv["mask"])
        call1 = wide.FfnCall(dv["X"], dv["Wg"], dv["Wu"], dv["Wd"], ones, w.G)
        call1.run()
        oms = time_events(torch, call1.run, max(5, args.steps // 2))
        del call1
        line["achievable_peaks"] = achievable_peaks(torch)
        line["dense"] = {"ms": round(dms, 4), "impl": "torch bf16 matmul (hipBLASLt)",
                         "speedup": round(dms / r["ms"], 3),
                         "ideal_speedup": round(w.T * r["ng"] / r["A"], 3),
                         "all_ones_mask_ms": round(oms, 4),
                         "speedup_vs_all_ones_mask": round(oms / r["ms"], 3)}
    del r["call"], r["dev_inputs"]
    torch.cuda.empty_cache()
    if not args.no_decode:
        line["decode"] = bench_decode(torch, wide, dg, args.steps)
    if not args.no_gemm:
        line["masked_gemms"] = bench_masked_gemms(torch, wide, dg, args.steps)
        line["router"] = bench_router(torch, wide, dg, args.steps)
        line["attention"] = bench_attention(torch, wide, dg, args.steps)
    if not args.no_configs:
        line["configs"] = bench_configs(torch, wide, dg, max(5, args.steps // 2))
    if not args.no_baselines:
        line["gemm_baselines"] = bench_baselines(torch, wide, dg)
    if not args.no_cpu:
        log("cpu baseline (oracle)")
        import oracle
        line["cpu_baseline"] = cpu_baseline(oracle, r["inputs"], w)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
