"""Benchmark of the log-linear sparse attention hot path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
pool -> select -> sparse attention forward -> index transpose (levels 1..Le+1)
-> backward, each through the C ABI on the current stream.  Inputs are
resident in HBM before the timed region.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload n65536_bf16]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import statistics
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
METRIC = "LLSA fwd+bwd tokens/sec at N=65536, K=8; % bf16 MFMA peak; sel GB/s"


def algorithmic(w, s, grad_bytes=4):
    """Compulsory HBM bytes and useful FLOPs per call (see the derivation in the
    design notes): every tensor the call must read or write, once.  grad_bytes:
    4 for float32 dQ, dK, dV, 2 for bfloat16."""
    bh, N, d = w.bh, w.seq_len, w.head_dim
    e = 2 if str(w.dtype) == "torch.bfloat16" else 4
    L = w.levels
    n = [s.level_tokens[l] for l in range(L + 1)]
    kl = [0] + [s.level_k[l] for l in range(1, L + 1)]
    Le = s.enrich
    pyr = sum(bh * n[l] * d * 4 for l in range(1, L + 1))
    idx = sum(bh * n[l] * kl[l] * 4 for l in range(1, L + 1))
    tok = bh * N * d * e
    coarse_pyr = sum(bh * n[l] * d * 4 for l in range(2, Le + 2))
    B = w.block
    nkv = kl[1] * B + sum(kl[l] for l in range(2, Le + 2))
    out = {}
    out["pool"] = dict(bytes=3 * tok + 3 * pyr, flops=0)
    sel_bytes = 2 * bh * n[L] * d * 4 + bh * n[L] * kl[L] * 4
    sel_flops = 2 * d * bh * n[L] * n[L]
    for l in range(L - 1, 0, -1):
        sel_bytes += 2 * bh * n[l] * d * 4 + bh * n[l + 1] * kl[l + 1] * 4 + bh * n[l] * kl[l] * 4
        sel_flops += 2 * d * bh * n[l] * kl[l + 1] * B
    out["select"] = dict(bytes=sel_bytes, flops=sel_flops)
    out["attn_fwd"] = dict(bytes=4 * tok + bh * N * 4 + 2 * coarse_pyr + idx,
                           flops=4 * bh * N * d * nkv)
    tr = 0
    for l in range(1, Le + 2):
        tr += bh * n[l] * kl[l] * 4 + bh * (n[l] + 1) * 4 + bh * n[l] * kl[l] * 4
    out["transpose"] = dict(bytes=tr, flops=0)
    g = grad_bytes
    # the compulsory bytes of the backward: Q, K, V, O, dO read, dQ, dK, dV
    # written, LSE and D once each.  The kernels never read O (D = sum P dP comes out of the dQ
    # pass), but read the coarse pyramids, the pick lists and the CSR and read
    # D back: "bytes_kernel_inputs".
    out["attn_bwd"] = dict(bytes=5 * tok + 3 * bh * N * d * g + 2 * bh * N * 4,
                           bytes_kernel_inputs=4 * tok + 3 * bh * N * d * g + 3 * bh * N * 4
                           + 2 * coarse_pyr + idx + tr,
                           flops=int(2.5 * 4 * bh * N * d * nkv))
    return out, nkv


def cpu_model():
    """The host CPU's model string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def oracle_threads():
    cores = len(os.sched_getaffinity(0))
    omp = os.environ.get("OMP_NUM_THREADS")
    return min(cores, int(omp)) if omp else cores


def source_hash(paths):
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def cpu_baseline(w, max_heads):
    """The fp64 CPU oracle, untouched, on the first heads of the same workload."""
    import numpy as np
    import torch
    from hierarchical_top_sparse_mean_amd.inputs import make_inputs
    from oracle import oracle as O
    threads = oracle_threads()
    heads = max(1, min(w.heads, max_heads, threads))
    q, k, v, do = make_inputs(1, heads, w.seq_len, w.head_dim, w.dtype, w.sinusoid, True, 0)
    q, k, v, do = (x.double().numpy().reshape(heads, w.seq_len, w.head_dim) for x in (q, k, v, do))
    B, L, K = w.block, w.levels, w.topk
    # whole passes are repeated until about 10 s of work have been timed
    reps = 0
    t0 = time.perf_counter()
    while True:
        pq, pk, pv = O.pool(q, B, L), O.pool(k, B, L), O.pool(v, B, L)
        idx, _ = O.select(pq, pk, B, K)
        O.attn_fwd(q, k, v, pk, pv, idx, B, K, w.enrich, w.scale)
        for l in range(1, w.enrich + 2):
            O.transpose(idx[l - 1], w.seq_len // B ** l)
        O.attn_bwd(q, k, v, pk, pv, idx, do, B, K, w.enrich, w.scale)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= 10.0 or reps >= 20:
            break
    # tokens as the GPU line counts them (batch x sequence, all heads): the
    # sample covers heads / w.heads of a pass
    tokens = reps * w.batch * w.seq_len * heads / w.heads
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{reps} passes over {heads} of {w.heads} heads x {w.seq_len} tokens, "
                      f"pool+select+fwd+transpose+bwd in fp64 ({dt:.1f} s)"}


def oracle_leg(w, g):
    """The CPU-baseline leg of a per-workload record: the oracle, untouched,
    timed over one whole pass of the full workload on the host cores (its own
    pooling, selection, attention and, with a backward, transposes and
    gradients); then, untimed, the parity of the GPU results g against it as
    the parity tests check it: pyramids; picks level by level with the GPU's
    parent picks as the oracle's (near-ties below 1e-5 relative exempt);
    O, LSE and gradients from the oracle over the GPU's own pick lists."""
    import numpy as np
    import torch
    from hierarchical_top_sparse_mean_amd.inputs import workload_inputs
    from oracle import oracle as O
    q, k, v, do = workload_inputs(w)
    bh, N, d = w.bh, w.seq_len, w.head_dim
    f64 = lambda t: t.double().numpy().reshape(bh, N, d)   # noqa: E731
    q, k, v = f64(q), f64(k), f64(v)
    do = f64(do) if do is not None else None
    B, Lv, K, Le = w.block, w.levels, w.topk, w.enrich
    t0 = time.perf_counter()
    pq, pk, pv = O.pool(q, B, Lv), O.pool(k, B, Lv), O.pool(v, B, Lv)
    idx, _ = O.select(pq, pk, B, K)
    O.attn_fwd(q, k, v, pk, pv, idx, B, K, Le, w.scale)
    if do is not None:
        for l in range(1, Le + 2):
            O.transpose(idx[l - 1], N // B ** l)
        O.attn_bwd(q, k, v, pk, pv, idx, do, B, K, Le, w.scale)
    dt = time.perf_counter() - t0
    cpu = {"value": round(w.batch * N / dt, 1), "unit": "tokens/s", "cores": oracle_threads(),
           "cpu_model": cpu_model(), "kind": "oracle",
           "sample": f"one whole pass of the workload in fp64 ({dt:.2f} s)"}
    par = {"pyramids": max(float(np.abs(a - b).max()) for name in ("pq", "pk", "pv")
                           for a, b in zip(g[name], {"pq": pq, "pk": pk, "pv": pv}[name]))}
    agree = exempt = fail = 0
    for l in range(Lv, 0, -1):
        oi, gap = O.select_level(pq[l - 1], pk[l - 1], B, K, None if l == Lv else g["idx"][l])
        same = (oi == g["idx"][l - 1]).all(axis=-1)
        near = (gap > 0) & (gap < 1e-5)
        agree += int(same.sum())
        exempt += int((~same & near).sum())
        fail += int((~same & ~near).sum())
    par.update(picks_agree=agree, picks_exempt=exempt, picks_fail=fail,
               picks_equal_unforced=sum(int((a == b).all(axis=-1).sum()) for a, b in zip(g["idx"], idx)))
    o, lse = O.attn_fwd(q, k, v, pk, pv, g["idx"], B, K, Le, w.scale)
    par["o_max_abs"] = float(np.abs(g["o"] - o).max())
    par["lse_max_abs"] = float(np.abs(g["lse"] - lse).max())
    if do is not None:
        dq, dk, dv = O.attn_bwd(q, k, v, pk, pv, g["idx"], do, B, K, Le, w.scale)
        for name, want in (("dq", dq), ("dk", dk), ("dv", dv)):
            par[name + "_max_abs"] = float(np.abs(g[name] - want).max())
    tol = 1e-4 if w.dtype == torch.float32 else 2e-2
    par["bar"] = tol
    par["pass"] = bool(fail == 0 and all(v <= tol for key, v in par.items() if key.endswith("_max_abs")))
    return cpu, par


def time_workload(L, w, steps, warmup, dev, grad_bf16=False, token_order=0, overlap=False):
    """Runs `warmup` untimed and `steps` timed steps of the whole path on
    workload `w` (inputs resident on the GPU); returns the inputs, problem,
    buffers, sizes, the median per-call milliseconds (HIP events on the stream
    each call runs on) and the wall-clock milliseconds per step.  overlap: the
    index transposes, which only the backward reads, run on a second stream
    (default priority) concurrently with the forward attention."""
    import torch
    from hierarchical_top_sparse_mean_amd.inputs import workload_inputs
    q, k, v, dout = workload_inputs(w)
    q, k, v = q.to(dev), k.to(dev), v.to(dev)
    dout = dout.to(dev) if dout is not None else None
    p = L.problem(w.batch, w.heads, w.seq_len, w.head_dim, w.block, w.levels, w.topk, w.enrich,
                  w.dtype, torch.bfloat16 if grad_bf16 else torch.float32, token_order=token_order)
    B = L.Buffers(p, backward=w.backward)
    s = B.s
    bh = w.bh
    calls = ["pool", "select", "attn_fwd"] + (["transpose", "attn_bwd"] if w.backward else [])
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream() if overlap and w.backward else main

    def transposes(stream):
        L.transpose_levels(B, stream)

    def step(ev=None):
        # ev[c] = (start, end) events of call c, recorded on the call's stream
        def mark(c, i, stream=None):
            if ev is not None:
                ev[c][i].record(stream)
        mark("pool", 0)
        L.llsa_pool(p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v)
        mark("pool", 1)
        mark("select", 0)
        L.llsa_select(p, B.pyr_q, B.pyr_k, B.idx)
        mark("select", 1)
        if w.backward and side is not main:
            side.wait_stream(main)
            mark("transpose", 0, side)
            transposes(side)
            mark("transpose", 1, side)
        mark("attn_fwd", 0)
        L.llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)
        mark("attn_fwd", 1)
        if w.backward:
            if side is main:
                mark("transpose", 0)
                transposes(main)
                mark("transpose", 1)
            else:
                main.wait_stream(side)
            mark("attn_bwd", 0)
            L.llsa_attn_bwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse,
                            dout, B.dq, B.dk, B.dv, B.ws, B.ws.numel())
            mark("attn_bwd", 1)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    events = [{c: [torch.cuda.Event(enable_timing=True) for _ in range(2)] for c in calls}
              for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / steps
    # the median over the timed steps of each call's HIP-event time
    per_call = {c: statistics.median(events[i][c][0].elapsed_time(events[i][c][1]) for i in range(steps))
                for c in calls}
    return q, k, v, dout, p, B, s, per_call, ms_per_step


def step_graph(L, w, p, B, q, k, v, dout):
    """One step of the whole path captured as a HIP graph (torch.cuda.CUDAGraph
    over the same library calls on the capture stream; the library allocates
    nothing and records no memset, so the calls capture as plain kernel
    launches).  Replaying it launches the step's kernels without the host
    calls between them."""
    import torch
    calls = step_calls(L, w, p, B, q, k, v, dout)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _, fn in calls:
            fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    return graph


def time_graph(graph, steps, warmup):
    """Wall-clock milliseconds per replay of a captured step."""
    import torch
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def sweep_workloads():
    """The workload table plus the variations the scaling study asks for, all
    at the 65536-token shape unless named otherwise: more pooling steps,
    no enrichment, wider selection, single-level selection (quadratic in the
    number of blocks), blocks of 64 tokens, bfloat16 gradients, and the 2D
    patch order at every image size."""
    from dataclasses import replace
    from hierarchical_top_sparse_mean_amd.inputs import WORKLOADS
    base = WORKLOADS["n65536_bf16"]
    out = [(w, "") for w in WORKLOADS.values()]
    out += [
        (replace(base, name="n65536_L3_Le2", levels=3, enrich=2), ""),
        (replace(base, name="n65536_Le0", enrich=0), ""),
        (replace(base, name="n65536_K16", topk=16), ""),
        (replace(base, name="n65536_L1_K8", levels=1, enrich=0), ""),
        (replace(base, name="n65536_L1_K20", levels=1, topk=20, enrich=0), ""),
        (replace(base, name="n65536_L1_K32", levels=1, topk=32, enrich=0), ""),
        # blocks of 64 tokens: single level (the large-block single-level setting) and two levels
        (replace(base, name="n65536_B64_L1_K8", block=64, levels=1, enrich=0), ""),
        (replace(base, name="n65536_B64_L2_K8", block=64, levels=2, enrich=1), ""),
        (base, "grad_bf16"),
        # the image tokens read as nested 2D patches, at every image size of the table
        (WORKLOADS["n4096_bf16"], "patch_order"),
        (WORKLOADS["n16384_bf16"], "patch_order"),
        (base, "patch_order"),
        (WORKLOADS["n262144_bf16"], "patch_order"),
    ]
    return out


def transpose_scaling(L, dev, reps):
    """Level-1 key-major lists from real selections at growing N: the sparse
    transpose (count / scan / fill) against the dense bit-mask baseline; then
    the whole backward (key-major lists of every level used + attention
    backward) built either way."""
    import torch
    from hierarchical_top_sparse_mean_amd.inputs import Workload, workload_inputs
    heads = 16
    for N, levels in ((4096, 2), (16384, 2), (65536, 2), (262144, 3), (1048576, 3)):
        w = Workload(f"n{N}", 1, heads, N, 64, torch.bfloat16, 16, levels, 8, levels - 1, True, True)
        q, k, v, dout = (x.to(dev) for x in workload_inputs(w))
        p = L.problem(1, heads, N, levels=levels, topk=8, enrich=levels - 1)
        B = L.Buffers(p, backward=True)
        L.llsa_pool(p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v)
        L.llsa_select(p, B.pyr_q, B.pyr_k, B.idx)
        n1, k1 = B.s.level_tokens[1], B.s.level_k[1]
        ptr, col = B.csr_level(1)
        mws = L.llsa_index_transpose_mask_workspace(heads, n1, n1)
        mw = torch.empty(mws, dtype=torch.uint8, device=dev)
        runs = {
            "csr": lambda: L.llsa_index_transpose(heads, n1, k1, n1, B.index_level(1), ptr, col,
                                                  B.tws, B.tws_bytes),
            "mask": lambda: L.llsa_index_transpose_mask(heads, n1, k1, n1, B.index_level(1), ptr, col,
                                                        mw, mws),
        }
        L.llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse)

        def lists(kind):
            if kind == "csr":   # every level in one call, as the bench step does
                L.transpose_levels(B)
                return
            for l in range(1, B.s.enrich + 2):
                nl, kl = B.s.level_tokens[l], B.s.level_k[l]
                pl, cl = B.csr_level(l)
                L.llsa_index_transpose_mask(heads, nl, kl, nl, B.index_level(l), pl, cl, mw, mws)

        def backward(kind):
            lists(kind)
            L.llsa_attn_bwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr, B.csr_col, B.o, B.lse,
                            dout, B.dq, B.dk, B.dv, B.ws, B.ws.numel())

        runs["csr_backward"] = lambda: backward("csr")
        runs["mask_backward"] = lambda: backward("mask")
        out = {"transpose_scaling_tokens": N, "heads": heads, "key_blocks": n1, "picks": heads * n1 * k1,
               "mask_bytes": mws}
        for name, f in runs.items():
            f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                f()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) * 1e3 / reps
            out[name + "_us"] = round(us, 2)
            if name.endswith("backward"):
                out[name + "_ns_per_token"] = round(us * 1e3 / (heads * N), 4)
            else:
                out[name + "_ns_per_pick"] = round(us * 1e3 / (heads * n1 * k1), 4)
        print(json.dumps(out), flush=True)
        del q, k, v, dout, B, mw
        torch.cuda.empty_cache()


def launch_floor_us(dev, reps=200):
    """Launch-to-completion time of a minimal kernel (a one-element add) issued
    back to back on the current stream, as the HIP events see it: the floor
    under any one of the step's calls."""
    import torch
    x = torch.zeros(1, device=dev)
    for _ in range(20):
        x.add_(1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        x.add_(1.0)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def call_details(alg, per_call):
    """Per-call ms, algorithmic GB/s and HBM fraction, TFLOP/s and bf16 MFMA
    fraction (attention) for measured per-call milliseconds."""
    detail = {}
    for c, ms in per_call.items():
        a = alg[c]
        detail[c] = {"ms": round(ms, 4), "GB/s": round(a["bytes"] / ms / 1e6, 1),
                     "hbm_frac": round(a["bytes"] / ms / 1e6 / HBM_PEAK_GBS, 4)}
        if a["flops"]:
            detail[c]["TFLOP/s"] = round(a["flops"] / ms / 1e9, 2)
        if c in ("attn_fwd", "attn_bwd"):
            detail[c]["bf16_mfma_frac"] = round(detail[c]["TFLOP/s"] / BF16_PEAK_TFLOPS, 4)
            # MFMA fraction this kernel could reach if it ran at the HBM peak
            detail[c]["bf16_mfma_frac_cap_at_hbm_peak"] = round(
                a["flops"] / (a["bytes"] / (HBM_PEAK_GBS * 1e9)) / 1e12 / BF16_PEAK_TFLOPS, 4)
        if "bytes_kernel_inputs" in a:
            detail[c]["GB/s_kernel_inputs"] = round(a["bytes_kernel_inputs"] / ms / 1e6, 1)
    return detail


def step_calls(L, w, p, B, q, k, v, dout):
    """The calls of one step, in order, as (name, function)."""
    calls = [("pool", lambda: L.llsa_pool(p, q, k, v, B.pyr_q, B.pyr_k, B.pyr_v)),
             ("select", lambda: L.llsa_select(p, B.pyr_q, B.pyr_k, B.idx)),
             ("attn_fwd", lambda: L.llsa_attn_fwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.o, B.lse))]
    if w.backward:
        calls += [("transpose", lambda: L.transpose_levels(B)),
                  ("attn_bwd", lambda: L.llsa_attn_bwd(p, q, k, v, B.pyr_k, B.pyr_v, B.idx, B.csr_ptr,
                                                       B.csr_col, B.o, B.lse, dout, B.dq, B.dk, B.dv,
                                                       B.ws, B.ws.numel()))]
    return calls


def time_cold(L, w, p, B, q, k, v, dout, reps, dev):
    """Per-call milliseconds with every call timed on its own right after a
    512 MiB write, which evicts the 256 MB memory-side cache (MALL): the cold
    counterpart of the warm, back-to-back step timing."""
    import torch
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    calls = step_calls(L, w, p, B, q, k, v, dout)
    tot = {c: 0.0 for c, _ in calls}
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for r in range(reps):
        for c, fn in calls:
            flush.fill_(r & 255)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            tot[c] += e0.elapsed_time(e1)
    del flush
    return {c: v / reps for c, v in tot.items()}


def gpu_results(B, w):
    """Host copies of the GPU results of the last step, for the parity leg."""
    bh, N, d, Lv = w.bh, w.seq_len, w.head_dim, w.levels
    host = lambda t: t.detach().double().cpu().numpy()   # noqa: E731
    g = {name: [host(B.pyramid_level(buf, l)) for l in range(1, Lv + 1)]
         for name, buf in (("pq", B.pyr_q), ("pk", B.pyr_k), ("pv", B.pyr_v))}
    g["idx"] = [B.index_level(l).cpu().numpy() for l in range(1, Lv + 1)]
    g["o"] = host(B.o).reshape(bh, N, d)
    g["lse"] = host(B.lse).reshape(bh, N)
    if w.backward:
        for name in ("dq", "dk", "dv"):
            g[name] = host(getattr(B, name)).reshape(bh, N, d)
    return g


def config_records(L, dev, steps, warmup, cold_reps):
    """One JSON line per workload of the table: warm per-call times (and cold,
    after a 512 MiB flush, for the workloads whose working set fits the
    256 MB MALL), the dominant call's roofline, parity against the oracle and
    the oracle's own time on the host cores."""
    import torch
    from hierarchical_top_sparse_mean_amd.inputs import WORKLOADS
    for w in WORKLOADS.values():
        q, k, v, dout, p, B, s, pc, msps = time_workload(L, w, steps, warmup, dev)
        alg, nkv = algorithmic(w, s)
        dom = max(pc, key=lambda c: pc[c])
        ach = alg[dom]["bytes"] / pc[dom] / 1e6
        rec = {"config_record": w.name, "describe": w.describe(), "keys_per_query_block": nkv,
               "ms_per_step": round(msps, 4), "tokens_per_s": round(w.batch * w.seq_len / (msps / 1e3), 1),
               "timing": "warm: calls back to back, inputs resident",
               "steps": steps, "warmup": warmup, "per_call": "median over the timed steps",
               "calls": call_details(alg, pc),
               "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1),
                            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                            "traffic": None, "algorithmic_bytes": alg[dom]["bytes"]}}
        # working set (inputs, pyramids, lists, outputs) within the MALL: time it cold too
        ws_bytes = sum(t.numel() * t.element_size() for t in (q, k, v, B.o, B.pyr_q, B.pyr_k, B.pyr_v))
        if w.name in ("n4096_bf16", "n16384_bf16"):
            rec["working_set_MB"] = round(ws_bytes / 1e6, 1)
            rec["calls_cold"] = call_details(alg, time_cold(L, w, p, B, q, k, v, dout, cold_reps, dev))
            rec["timing_cold"] = f"each call alone after a 512 MiB write (MALL flushed), mean of {cold_reps}"
        # one more step so that every result comes from the same pass, then the oracle
        for _, fn in step_calls(L, w, p, B, q, k, v, dout):
            fn()
        torch.cuda.synchronize()
        g = gpu_results(B, w)
        rec["cpu_baseline"], rec["parity"] = oracle_leg(w, g)
        print(json.dumps(rec), flush=True)
        del q, k, v, dout, B, g
        torch.cuda.empty_cache()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="n65536_bf16")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--overlap", action="store_true",
                    help="run the index transposes on a second stream beside the forward attention "
                         "(measured slower: they wait for the forward's workgroups to drain)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused count-into-select comparison (for profiled runs)")
    ap.add_argument("--cpu-heads", type=int, default=16)
    ap.add_argument("--no-graph", action="store_true",
                    help="time the eager step only (no HIP-graph replay of the step)")
    ap.add_argument("--sweep", action="store_true",
                    help="time every workload and variation (one JSON line each) instead of the bench line")
    ap.add_argument("--transpose-scaling", action="store_true",
                    help="time the level-1 index transpose against the dense-mask baseline for "
                         "4096 .. 1048576 tokens (one JSON line each)")
    ap.add_argument("--configs", action="store_true",
                    help="one record per workload of the table: warm (and, where the working set "
                         "fits the MALL, cold) per-call times, roofline, parity against the oracle "
                         "and the oracle's time")
    ap.add_argument("--cold-reps", type=int, default=10)
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the operator shards by (batch, head) with no "
              "communication, so a step on N GPUs is N independent one-GPU steps; use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from hierarchical_top_sparse_mean_amd import llsa as L
    from hierarchical_top_sparse_mean_amd.inputs import WORKLOADS, workload_inputs

    w = WORKLOADS[args.workload]
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    if args.sweep:
        for sw, var in sweep_workloads():
            _, _, _, _, _, _, ss, pc, msps = time_workload(L, sw, args.steps, args.warmup, dev,
                                                          var == "grad_bf16", int(var == "patch_order"))
            alg, nkv = algorithmic(sw, ss, 2 if var == "grad_bf16" else 4)
            tok = sw.batch * sw.seq_len
            rec = {"sweep": sw.name + ("_" + var if var else ""), "describe": sw.describe(),
                   "keys_per_query_block": nkv, "ms_per_step": round(msps, 4),
                   "tokens_per_s": round(tok / (msps / 1e3), 1),
                   # per token and head: selection + attention forward, the part whose
                   # cost the method makes log-linear in N
                   "ns_per_token_head_select_attn":
                       round((pc["select"] + pc["attn_fwd"]) * 1e6 / (tok * sw.heads), 4),
                   "calls": {c: {"ms": round(v, 4), "GB/s": round(alg[c]["bytes"] / v / 1e6, 1)}
                             for c, v in pc.items()}}
            print(json.dumps(rec), flush=True)
            torch.cuda.empty_cache()
        return
    if args.transpose_scaling:
        transpose_scaling(L, dev, args.steps)
        return
    if args.configs:
        config_records(L, dev, args.steps, args.warmup, args.cold_reps)
        return
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": n * 4, "copy_probe_bytes_written": n * 4,
                          "launches": 3}))
        return
    q, k, v, dout, p, B, s, per_call, ms_per_step = time_workload(L, w, args.steps, args.warmup, dev,
                                                                  overlap=args.overlap)
    bh = w.bh
    calls = list(per_call)
    tokens = w.batch * w.seq_len
    value = tokens / (ms_per_step / 1e3)
    graph_info = None
    if not args.no_graph:
        # the same step captured once as a HIP graph and replayed; it is used
        # for the line's value only if a replay writes the eager step's bytes
        outs = lambda: [t.clone() for t in (B.o, B.lse, B.idx) + ((B.dq, B.dk, B.dv) if w.backward else ())]  # noqa: E731
        torch.cuda.synchronize()
        eager = outs()
        graph = step_graph(L, w, p, B, q, k, v, dout)
        for t in (B.o, B.dq, B.dk, B.dv) if w.backward else (B.o,):
            t.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for a, b in zip(outs(), eager))
        ms_graph = time_graph(graph, args.steps, args.warmup)
        graph_info = {"ms_per_step": round(ms_graph, 4), "matches_eager_bitwise": same,
                      "ms_per_step_eager": round(ms_per_step, 4)}
        if same:
            ms_per_step = ms_graph
            value = tokens / (ms_per_step / 1e3)
        del graph

    alg, nkv = algorithmic(w, s)
    detail = call_details(alg, per_call)

    # dominant call -> roofline (HBM-bound; algorithmic bytes / measured time)
    dom = max(calls, key=lambda c: per_call[c])
    ach = alg[dom]["bytes"] / per_call[dom] / 1e6
    traffic = None
    tfile = os.path.join(ROOT, "profiles", "traffic.json")
    if os.path.exists(tfile):
        with open(tfile) as f:
            tr = json.load(f)
        ent = tr.get(dom)
        if ent and ent.get("workload") == w.name and ent.get("source_hash") == source_hash(ent["sources"]):
            traffic = ent["bytes_per_call"]
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "algorithmic_bytes": alg[dom]["bytes"]}
    if "bytes_kernel_inputs" in alg[dom]:
        # the same time over the bytes the kernels must touch (no O; pyramids, lists, CSR, D read back)
        bk = alg[dom]["bytes_kernel_inputs"]
        roofline["bytes_kernel_inputs"] = bk
        roofline["frac_kernel_inputs"] = round(bk / per_call[dom] / 1e6 / HBM_PEAK_GBS, 4)

    dense = None
    if not args.no_dense and w.dtype == torch.bfloat16:
        o_d = torch.empty_like(q)
        lse_d = torch.empty(bh * w.seq_len, dtype=torch.float32, device=dev)
        L.llsa_dense_attn_fwd(p, q, k, v, o_d, lse_d)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 3
        e0.record()
        for _ in range(reps):
            L.llsa_dense_attn_fwd(p, q, k, v, o_d, lse_d)
        e1.record()
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / reps
        dflops = 4.0 * bh * w.seq_len * w.seq_len * w.head_dim
        llsa_fwd = per_call["pool"] + per_call["select"] + per_call["attn_fwd"]
        dense = {"note": "speedups are against this dense kernel built in the same style, not a tuned "
                         "flash-attention kernel; see its bf16_mfma_frac",
                 "fwd_ms": round(dms, 3), "TFLOP/s": round(dflops / dms / 1e9, 1),
                 "bf16_mfma_frac": round(dflops / dms / 1e9 / BF16_PEAK_TFLOPS, 4),
                 "llsa_fwd_ms": round(llsa_fwd, 4),
                 "speedup_fwd": round(dms / llsa_fwd, 2)}
        if w.backward:
            # dense backward (dQ pass, then dK/dV pass); float32 gradients like the sparse path
            gq, gk, gv = (torch.empty(q.shape, dtype=torch.float32, device=dev) for _ in range(3))
            wsb = L.llsa_dense_attn_bwd_workspace(p)
            wsd = torch.empty(wsb, dtype=torch.uint8, device=dev)
            L.llsa_dense_attn_bwd(p, q, k, v, o_d, lse_d, dout, gq, gk, gv, wsd, wsb)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                L.llsa_dense_attn_bwd(p, q, k, v, o_d, lse_d, dout, gq, gk, gv, wsd, wsb)
            e1.record()
            torch.cuda.synchronize()
            bms = e0.elapsed_time(e1) / reps
            dense.update({"bwd_ms": round(bms, 3),
                          "bwd_TFLOP/s": round(2.5 * dflops / bms / 1e9, 1),
                          "fwd_bwd_ms": round(dms + bms, 3),
                          "llsa_fwd_bwd_ms": round(ms_per_step, 4),
                          "speedup_fwd_bwd": round((dms + bms) / ms_per_step, 2)})
            del gq, gk, gv, wsd
        del o_d, lse_d

    # the launch floor, and the small calls' HBM fraction over the time above it
    floor = launch_floor_us(dev)
    for c in ("select", "transpose"):
        above = per_call[c] * 1e3 - floor
        if above > 0:
            detail[c]["hbm_frac_above_launch_floor"] = round(alg[c]["bytes"] / (above * 1e3) / HBM_PEAK_GBS, 4)

    fused = None
    if w.backward and not args.no_fused:
        # the fused variant: level-1 selection also counts its picks for the transpose
        def separate():
            L.llsa_select(p, B.pyr_q, B.pyr_k, B.idx)
            L.transpose_levels(B)

        def together():
            L.llsa_select_transpose(p, B.pyr_q, B.pyr_k, B.idx, B.csr_ptr, B.csr_col, B.tws, B.tws_bytes)

        fused = {}
        for name, f in (("select_then_transpose_us", separate), ("select_transpose_fused_us", together)):
            f()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(50):
                f()
            e1.record()
            torch.cuda.synchronize()
            fused[name] = round(e0.elapsed_time(e1) * 1e3 / 50, 1)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, args.cpu_heads)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
                   "head_dim": w.head_dim, "block": w.block, "levels": w.levels, "topk": w.topk,
                   "enrich": w.enrich, "keys_per_query_block": nkv,
                   "grad_dtype": "f32", "pass": "fwd+bwd" if w.backward else "fwd"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "calls": detail,
        "select_GB/s": detail["select"]["GB/s"],
        "attn_fwd_bf16_mfma_frac": detail["attn_fwd"].get("bf16_mfma_frac"),
        "dense_comparator": dense,
        "fused_count_into_select": fused,
        "launch_floor_us": round(floor, 2),
        "hip_graph": graph_info,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
