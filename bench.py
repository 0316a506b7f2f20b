#!/usr/bin/env python3
"""Benchmark of the MoE expert path on one MI355X.

One step = the whole path over one batch of seeded synthetic tokens already
resident in HBM: top-k routing -> scatter into the expert layout (FP8: fused
UE8M0 quantisation) -> w13 grouped GEMM -> SiLU-and-mul (FP8: fused requant)
-> w2 grouped GEMM -> weighted combine.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

The default workload is the FP8 DeepSeek-V3-shaped prefill (T=8192, H=7168,
I=2048, 256 experts, top-8, 128x128 block-scaled e4m3 weights).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

METRIC = "MoE-layer tokens/s and grouped-GEMM TFLOP/s (BF16/FP8) as % of MFMA peak, 1 GPU"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8_e4m3": 5000.0}
PEAK_HBM_GBS = 8000.0
# the other seeded workloads, timed after the headline one in the same run
OTHER_WORKLOADS = ("tiny", "bf16_prefill", "fp8_decode", "bf16_skewed")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="fp8_prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target duration of the timed oracle run on the host")
    ap.add_argument("--unfused", action="store_true",
                    help="run w13 and SiLU-and-mul as two kernels")
    ap.add_argument("--weight-format", default=None, choices=["block128", "mxfp8", "mxfp4"],
                    help="FP8 workloads: 128x128 UE8M0 weight blocks (default) or MX e4m3 weights")
    ap.add_argument("--no-mx", action="store_true",
                    help="FP8 workloads: skip the extra MX-weight timings (mxfp8, mxfp4)")
    ap.add_argument("--no-vendor", action="store_true",
                    help="skip the dense vendor-library GEMMs timed for reference")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration)")
    ap.add_argument("--workloads", default=",".join(OTHER_WORKLOADS),
                    help="comma-separated further workloads timed in the same run and reported "
                         "under 'workloads' ('' for none)")
    ap.add_argument("--workload-steps", type=int, default=10)
    return ap.parse_args()


def build_layer(wl, torch, fuse_silu=True, weight_format=None, make_inputs=True):
    from scatter_grouped_gemm_amd import MoELayer, inputs
    layer = MoELayer(hidden=wl.H, intermediate=wl.I, num_experts=wl.E, top_k=wl.k, max_tokens=wl.T,
                     num_local_experts=wl.El, expert_start=wl.expert_start, fp8=wl.fp8,
                     layout=wl.layout, block_e=wl.block_e, max_m=wl.max_m or None,
                     expected_m=wl.expected_m, fuse_silu=fuse_silu, weight_format=weight_format,
                     device="cuda")
    t0 = time.time()
    for e in range(wl.El):
        w13, w2 = inputs.expert_weights(wl, wl.expert_start + e, "cuda")
        layer.set_expert(e, w13, w2)
        del w13, w2
    torch.cuda.synchronize()
    log(f"weights ready for {wl.El} experts in {time.time() - t0:.1f}s")
    if not make_inputs:
        return layer, None, None
    x = inputs.tokens(wl, "cuda")
    logits = inputs.logits(wl, "cuda")
    return layer, x, logits


def gemm_work(wl, layer, torch):
    """Algorithmic FLOPs and HBM bytes of the two grouped GEMMs for the valid
    rows of this batch (padding rows excluded).  With SiLU-and-mul fused into
    w13 its output is the activation (I channels, e4m3 + scales or bf16)
    instead of the bf16 gate/up pair."""
    if layer.layout == "compact":
        counts = layer.num_valid.cpu().to(torch.int64)
    else:
        counts = layer.masked_m.cpu().to(torch.int64)
    A = int(counts.sum())
    active = int((counts > 0).sum())
    ab = 1 if wl.fp8 else 2
    H, I = wl.H, wl.I
    w13_flops = 2.0 * A * (2 * I) * H
    w2_flops = 2.0 * A * H * I
    sc = (1.0 / (128 * 128)) if wl.fp8 else 0.0          # weight block scales
    wb = ab
    if layer.mx:
        sc = 1.0 / 32                                      # one exponent per 32 k
        wb = 0.5 if layer.weight_format == "mxfp4" else 1.0
    asc = (1.0 / 128) if wl.fp8 else 0.0                 # activation scales
    w13_out = (I * (ab + asc)) if layer.fuse_silu else (2 * I * 2)
    w13_bytes = active * 2 * I * H * (wb + sc) + A * H * (ab + asc) + A * w13_out
    w2_bytes = active * H * I * (wb + sc) + A * I * (ab + asc) + A * H * 2
    # rows on which the GEMMs run their MFMAs (whole 16-row blocks of their
    # tiles, padding included), from the library's own tile rule
    from scatter_grouped_gemm_amd import _lib as L
    masked = layer.layout == "masked"
    M = layer.rows if not masked else layer.max_m
    c = counts.numpy()
    rows13 = L.grouped_gemm_rows_executed(layer.wdt, masked, c, layer.expected_m, M, 2 * I, H)
    rows2 = L.grouped_gemm_rows_executed(layer.wdt, masked, c, layer.expected_m, M, H, I)
    return dict(assignments=A, active_experts=active, w13_flops=w13_flops, w2_flops=w2_flops,
                exec_flops=2.0 * (rows13 * 2 * I * H + rows2 * H * I),
                w13_exec_flops=2.0 * rows13 * 2 * I * H, w2_exec_flops=2.0 * rows2 * H * I,
                w13_bytes=w13_bytes, w2_bytes=w2_bytes)


def roofline(flops, nbytes, ms, dtype):
    peak_f = PEAK_TFLOPS[dtype]
    ridge = peak_f * 1e12 / (PEAK_HBM_GBS * 1e9)
    ai = flops / nbytes
    tflops = flops / (ms * 1e-3) / 1e12
    gbs = nbytes / (ms * 1e-3) / 1e9
    if ai < ridge:
        return dict(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                    frac=round(gbs / PEAK_HBM_GBS, 4), traffic=None,
                    tflops=round(tflops, 1), mfma_frac=round(tflops / peak_f, 4),
                    arithmetic_intensity=round(ai, 1))
    return dict(bound="mfma", achieved=round(tflops, 1), peak=peak_f, unit="TFLOP/s",
                frac=round(tflops / peak_f, 4), traffic=None, gbs=round(gbs, 1),
                arithmetic_intensity=round(ai, 1))


# the sources the grouped-GEMM kernels are built from: counter figures taken
# on other sources are not reported
GEMM_SOURCES = ("gemm.hip", "gemm_wreg.hip", "gemm_wreg.h", "gemm_runs.h", "common.h")


def gemm_source_sha256():
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    h = hashlib.sha256()
    for src in GEMM_SOURCES:
        with open(os.path.join(root, "scatter_grouped_gemm_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(wl_name, which):
    """HBM bytes per launch of one grouped GEMM (FETCH_SIZE + WRITE_SIZE, scaled
    by a plain copy's reading) from the rocprofv3 counter summary committed
    under profiles/, or None when there is none for this workload or the GEMM
    source has changed since the counters were taken."""
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", f"traffic_{wl_name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("gemm_source_sha256") != gemm_source_sha256() or which not in d:
        return None
    return int(d[which]["read_bytes"] + d[which]["write_bytes"])


def time_steps(layer, x, logits, steps, warmup, torch, per_step=None):
    """Mean step time (ms) over `steps` after `warmup`, HIP events on the
    stream the layer launches on, plus per-kernel means; `per_step` (a list)
    receives each step's time from an event recorded between steps."""
    for _ in range(warmup):
        layer(x, logits)
    torch.cuda.synchronize()
    layer.marks = {}
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    evs[0].record()
    for i in range(steps):
        layer(x, logits)
        evs[i + 1].record()
    torch.cuda.synchronize()
    ms = evs[0].elapsed_time(evs[-1]) / steps
    if per_step is not None:
        per_step.extend(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    kern = {k: sum(s.elapsed_time(e) for s, e in v) / len(v) for k, v in layer.marks.items()}
    layer.marks = None
    return ms, kern


def memory_kernels(wl, layer, kern, work):
    """Algorithmic HBM bytes and rate of the memory-bound kernels: scatter
    (the bf16 row of every token with a local expert read once; per local
    assignment H*b + H/128 + 8 bytes written: row, scales, row index), combine
    (the 2H-byte rows of the local assignments read, per token a 2H-byte row
    written and 8 bytes of weight and position per slot read) and, when run
    separately, SiLU-and-mul (per valid row 4I read + I*b (+ I/128) written)."""
    import torch
    H, I, k = wl.H, wl.I, wl.k
    A, T = work["assignments"], wl.T
    local = layer.topk_ids[:T].cpu().to(torch.int64) - wl.expert_start
    T_local = int(((local >= 0) & (local < wl.El)).any(dim=1).sum())
    b = 1 if wl.fp8 else 2
    sc = (1.0 / 128) if wl.fp8 else 0.0
    out = {}
    nbytes = {"scatter": T_local * 2 * H + A * (H * b + H * sc + 8),
              "combine": A * 2 * H + T * (2 * H + 8 * k)}
    if "silu_and_mul" in kern:
        nbytes["silu_and_mul"] = A * (4 * I + I * b + I * sc)
    for name, nb in nbytes.items():
        if name in kern and kern[name] > 0:
            gbs = nb / (kern[name] * 1e-3) / 1e9
            out[name] = {"bytes": int(nb), "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4)}
    return out


def graph_steps(layer, x, logits, steps, torch):
    """The same step captured once in a HIP graph and replayed `steps` times
    (launch overhead removed; the whole path runs in every replay)."""
    layer(x, logits)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            layer(x, logits)
    torch.cuda.current_stream().wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(steps):
        graph.replay()
    end.record()
    torch.cuda.synchronize()
    del graph
    return start.elapsed_time(end) / steps


def workload_summary(wl, layer, ms, kern, torch):
    """tokens/s, per-kernel times and both GEMMs' rooflines of one timed run."""
    work = gemm_work(wl, layer, torch)
    dtype = "fp8_e4m3" if wl.fp8 else "bf16"
    w13_key = "gemm_w13_silu" if layer.fuse_silu else "gemm_w13"
    out = {"workload": wl.name, "value": round(wl.T / (ms * 1e-3), 1), "unit": "tokens/s",
           "ms_per_step": round(ms, 4), "dtype": dtype, "layout": layer.layout,
           "assignments": work["assignments"], "kernels_ms": {k: round(v, 4) for k, v in kern.items()}}
    for name, key, flops, nbytes in (("w13", w13_key, work["w13_flops"], work["w13_bytes"]),
                                     ("w2", "gemm_w2", work["w2_flops"], work["w2_bytes"])):
        r = roofline(flops, nbytes, kern[key], dtype)
        r["traffic"] = measured_traffic(wl.name, name)
        r["ms"] = round(kern[key], 4)
        out[f"{name}_roofline"] = r
    gemm_ms = kern[w13_key] + kern["gemm_w2"]
    tf = (work["w13_flops"] + work["w2_flops"]) / (gemm_ms * 1e-3) / 1e12
    out["gemm"] = {"tflops_both": round(tf, 1), "mfma_frac_both": round(tf / PEAK_TFLOPS[dtype], 4),
                   "executed_tflops_both": round(work["exec_flops"] / (gemm_ms * 1e-3) / 1e12, 1)}
    out["memory_kernels"] = memory_kernels(wl, layer, kern, work)
    return out


def other_workloads(names, torch, steps, warmup=3, cpu=True):
    """The further seeded workloads, each built, timed and freed in turn (with
    the oracle's per-stage host timing unless cpu is False)."""
    from scatter_grouped_gemm_amd import inputs
    out = {}
    for name in names:
        wl = inputs.get(name)
        log(f"workload {wl.name}")
        layer, x, logits = build_layer(wl, torch)
        ms, kern = time_steps(layer, x, logits, steps, warmup, torch)
        log(f"{name}: {ms:.3f} ms/step; " + ", ".join(f"{k} {v:.3f}" for k, v in kern.items()))
        out[name] = workload_summary(wl, layer, ms, kern, torch)
        if cpu:
            n_tok, reps = CPU_STAGE_TOKENS.get(wl.name, (min(wl.T, 64), 1))
            out[name]["cpu_stages"] = cpu_stages(wl, x, logits, min(n_tok, wl.T), reps)
        del layer, x, logits
        torch.cuda.empty_cache()
    return out


def mx_variants(wl, x, logits, torch, steps=10, warmup=3):
    """The same batch with MX expert weights (e4m3 and e2m1, one exponent per
    32 k of a weight row), timed like the main run; reported beside it."""
    out = {}
    for wf in ("mxfp8", "mxfp4"):
        layer, _, _ = build_layer(wl, torch, weight_format=wf, make_inputs=False)
        ms, kern = time_steps(layer, x, logits, steps, warmup, torch)
        work = gemm_work(wl, layer, torch)
        roof = roofline(work["w13_flops"], work["w13_bytes"], kern["gemm_w13_silu"], "fp8_e4m3")
        out[wf] = {"value": round(wl.T / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
                   "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
                   "w13_roofline": {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac")}}
        log(f"{wf}: {ms:.3f} ms/step; " + ", ".join(f"{k} {v:.3f}" for k, v in kern.items()))
        del layer
        torch.cuda.empty_cache()
    return out


def requant_weights(wl, torch, reps=5):
    """Time moe_requant_weight_fp8_ue8m0 on block-FP8 checkpoint weights of the
    workload's w13 shape (seeded random e4m3 codes without NaN, fp32 block
    scales log-uniform over 2^-14 .. 2^-4): a load-time step, outside the
    timed path.  Algorithmic bytes: each code read and written once, plus
    4 + 1 scale bytes per 128x128 block."""
    from scatter_grouped_gemm_amd import _lib as L
    G, N, K = wl.El, 2 * wl.I, wl.H
    g = torch.Generator(device="cuda")
    g.manual_seed(12345)
    q = torch.randint(0, 0x7F, (G, N, K), dtype=torch.uint8, device="cuda", generator=g)
    q |= torch.randint(0, 2, (G, N, K), dtype=torch.uint8, device="cuda", generator=g) << 7
    s_in = torch.exp2(torch.rand(G, N // 128, K // 128, device="cuda", generator=g) * 10.0 - 14.0)
    q_out = torch.empty_like(q)
    s_out = torch.empty(G, N // 128, K // 128, dtype=torch.uint8, device="cuda")
    L.moe_requant_weight_fp8_ue8m0(q, s_in, q_out, s_out)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        L.moe_requant_weight_fp8_ue8m0(q, s_in, q_out, s_out)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = 2 * G * N * K + 5 * G * (N // 128) * (K // 128)
    gbs = nbytes / (ms * 1e-3) / 1e9
    del q, q_out, s_in, s_out
    return dict(shape=[G, N, K], ms=round(ms, 4), achieved=round(gbs, 1), peak=PEAK_HBM_GBS,
                unit="GB/s", frac=round(gbs / PEAK_HBM_GBS, 4))


def vendor_dense(wl, work, torch, reps=10, warmup=3):
    """Context, not a step of the path: the vendor library (hipBLASLt through
    torch) on one dense GEMM of the same M x N x K as each grouped GEMM, with
    M = the batch's valid rows and a single weight matrix.  FP8 takes one fp32
    scale per tensor (the library has no 128x128-block UE8M0 mode), BF16 none;
    neither has routing, padding or per-expert weights, so this is an upper
    reference for the grouped kernels, timed on the same GPU."""
    M, H, I = work["assignments"], wl.H, wl.I
    out = {}
    g = torch.Generator(device="cuda").manual_seed(7)
    for name, N, K, flops in (("w13", 2 * I, H, work["w13_flops"]), ("w2", H, I, work["w2_flops"])):
        a = torch.randn(M, K, device="cuda", generator=g)
        w = torch.randn(N, K, device="cuda", generator=g)
        if wl.fp8:
            a, w = a.to(torch.float8_e4m3fn), w.to(torch.float8_e4m3fn)
            one = torch.ones((), device="cuda")
            fn = lambda: torch._scaled_mm(a, w.t(), scale_a=one, scale_b=one, out_dtype=torch.bfloat16)
        else:
            a, w = a.to(torch.bfloat16), w.to(torch.bfloat16)
            fn = lambda: torch.nn.functional.linear(a, w)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(reps):
            fn()
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / reps
        out[name] = {"M": M, "N": N, "K": K, "ms": round(ms, 4),
                     "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
        del a, w
    out["library"] = "hipBLASLt via torch._scaled_mm (fp8, per-tensor scales)" if wl.fp8 \
        else "hipBLASLt via torch.nn.functional.linear (bf16)"
    return out


def cpu_baseline(wl, x, logits, target_s, torch):
    """The oracle, as it stands, on a prefix of the same batch: routing plus the
    layout-free per-token expert path (w13 -> SiLU-mul -> (requant) -> w2 ->
    weighted sum), timed on the host cores.  A first run on a few tokens sizes
    the sample so that the timed run takes about target_s seconds.  Weight
    preparation (copying the needed experts' bf16 weights and, for FP8, the
    oracle's own 128x128 block quantisation) is not timed, as it is not part of
    a step on the GPU either."""
    import numpy as np

    import oracle
    from scatter_grouped_gemm_amd import inputs
    oracle.build(force=False)
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    cache = {}

    def prepare(local):
        t0 = time.time()
        need = sorted({int(e) for e in local.reshape(-1) if 0 <= e < wl.El})
        for e in need:
            if e not in cache:
                a, b = inputs.expert_weights(wl, wl.expert_start + e, "cuda")
                a, b = inputs.bf16_bits(a)[None], inputs.bf16_bits(b)[None]
                if wl.fp8:
                    a, b = oracle.quant_weight_blocks(a), oracle.quant_weight_blocks(b)
                cache[e] = (a, b)
        log(f"oracle weights for {len(need)} experts ready ({time.time() - t0:.1f}s)")
        return need

    def run(n_tok):
        xs = inputs.bf16_bits(x[:n_tok])
        ls = logits[:n_tok].cpu().numpy()
        ids, _ = oracle.route_topk(ls, wl.k)
        local = ids - wl.expert_start
        need = prepare(local)
        remap = np.full(wl.El, -1, np.int32)
        remap[need] = np.arange(len(need), dtype=np.int32)
        inside = (local >= 0) & (local < wl.El)
        ids_c = np.where(inside, remap[np.clip(local, 0, wl.El - 1)], -1).astype(np.int32)
        if wl.fp8:
            W = dict(w13q=np.concatenate([cache[e][0][0] for e in need]),
                     w13s=np.concatenate([cache[e][0][1] for e in need]),
                     w2q=np.concatenate([cache[e][1][0] for e in need]),
                     w2s=np.concatenate([cache[e][1][1] for e in need]))
        else:
            W = dict(w13=np.concatenate([cache[e][0] for e in need]),
                     w2=np.concatenate([cache[e][1] for e in need]))
        t0 = time.perf_counter()
        ids2, w2_ = oracle.route_topk(ls, wl.k)
        out = oracle.moe_dense(xs, ids_c, w2_, 0, len(need), wl.fp8, **W)
        dt = time.perf_counter() - t0
        assert np.array_equal(ids2, ids) and out.shape == (n_tok, wl.H)
        return dt, len(need)

    n0 = min(wl.T, 2 * cores)
    dt0, n_exp0 = run(n0)
    n = min(wl.T, max(n0, int(n0 * target_s / max(dt0, 1e-6))))
    log(f"cpu baseline: {n0} tokens took {dt0:.2f}s; timing {n} tokens")
    dt, n_exp = run(n) if n > n0 else (dt0, n_exp0)
    return dict(value=round(n / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"first {n} of {wl.T} tokens of the batch: routing + per-token expert path "
                       f"({n_exp} experts), {dt:.1f}s on {cores} threads")


def cpu_stages(wl, x, logits, n_tok, reps=1):
    """The oracle's layout path stage by stage on the first n_tok tokens of the
    batch (route -> scatter -> w13 -> SiLU-mul (+ requant) -> w2 -> combine),
    each stage timed with perf_counter on the host cores; the median over
    `reps` runs.  The sample's experts are renumbered densely (experts without
    tokens in the sample are left out of the layout); weight preparation is not
    timed."""
    import numpy as np

    import oracle
    from scatter_grouped_gemm_amd import inputs
    oracle.build(force=False)
    xs = inputs.bf16_bits(x[:n_tok])
    ls = logits[:n_tok].cpu().numpy()
    ids, tw = oracle.route_topk(ls, wl.k)
    local = ids - wl.expert_start
    inside = (local >= 0) & (local < wl.El)
    need = sorted({int(e) for e in local[inside].reshape(-1)})
    remap = np.full(wl.El, -1, np.int32)
    remap[need] = np.arange(len(need), dtype=np.int32)
    ids_c = np.where(inside, remap[np.clip(local, 0, wl.El - 1)], -1).astype(np.int32)
    w13, w2 = [], []
    for e in need:
        a, b = inputs.expert_weights(wl, wl.expert_start + e, x.device)
        w13.append(inputs.bf16_bits(a)[None])
        w2.append(inputs.bf16_bits(b)[None])
    w13, w2 = np.concatenate(w13), np.concatenate(w2)
    if wl.fp8:
        w13, w2 = oracle.quant_weight_blocks(w13), oracle.quant_weight_blocks(w2)
    El = len(need)
    masked = wl.layout == "masked"
    names = ("route", "scatter", "w13", "silu_mul", "w2", "combine")
    runs = []
    for _ in range(reps):
        t = [time.perf_counter()]
        ids2, tw2 = oracle.route_topk(ls, wl.k)
        t.append(time.perf_counter())
        if masked:
            max_m = wl.max_m or n_tok
            sc = oracle.scatter_masked(xs, ids_c, 0, El, max_m, wl.fp8)
            rg = oracle.masked_row_group(sc["masked_m"], max_m)
        else:
            rows = oracle.compact_rows_bound(n_tok * wl.k, El, wl.block_e)
            sc = oracle.scatter_compact(xs, ids_c, 0, El, wl.block_e, rows, wl.fp8)
            rg = sc["m_indices"]
        t.append(time.perf_counter())
        if wl.fp8:
            h1 = oracle.gemm_fp8_rows(sc["x_out"], sc["scale_out"], w13[0], w13[1], rg)
        else:
            h1 = oracle.gemm_bf16_rows(sc["x_out"], w13, rg)
        t.append(time.perf_counter())
        act = oracle.silu_and_mul(h1, rg)
        if wl.fp8:
            aq = np.zeros(act.shape, np.uint8)
            asc = np.zeros((act.shape[0], act.shape[1] // 128), np.uint8)
            valid = rg >= 0
            if valid.any():
                aq[valid], asc[valid] = oracle.quant_rows(act[valid])
        t.append(time.perf_counter())
        if wl.fp8:
            y = oracle.gemm_fp8_rows(aq, asc, w2[0], w2[1], rg)
        else:
            y = oracle.gemm_bf16_rows(act, w2, rg)
        t.append(time.perf_counter())
        out = oracle.combine(y, sc["src2dst"], tw2)
        t.append(time.perf_counter())
        assert np.array_equal(ids2, ids) and out.shape == (n_tok, wl.H)
        runs.append([t[i + 1] - t[i] for i in range(len(names))])
    med = np.median(np.asarray(runs), axis=0)
    res = {f"{n}_s": round(float(v), 5) for n, v in zip(names, med)}
    res.update(tokens=n_tok, experts=El, reps=reps, total_s=round(float(med.sum()), 5),
               tokens_per_s=round(n_tok / float(med.sum()), 2))
    log(f"oracle stages on {n_tok} tokens ({wl.name}): " + ", ".join(f"{n} {v:.3f}s" for n, v in zip(names, med)))
    return res


# tokens of each workload the oracle's stage timing runs on (whole batch and
# median of 3 for the small ones; a few seconds of host time for the others)
CPU_STAGE_TOKENS = {"tiny_bf16_T64_E8": (64, 3), "fp8_masked_decode_T256_E32of256": (256, 3),
                    "fp8_prefill_T8192_H7168_I2048_E256": (256, 1),
                    "bf16_prefill_T4096_H4096_I14336_E8": (128, 1),
                    "bf16_skewed_T16384_H4096_I1536_E128": (256, 1)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the expert path here runs one GPU's share of the "
              f"experts on a single MI355X (--gpus {args.gpus} is not supported).", file=sys.stderr)
        sys.exit(2)
    import torch

    from scatter_grouped_gemm_amd import inputs
    wl = inputs.get(args.workload)
    log(f"workload {wl.name}")
    if args.calib_copy_mib:
        n = args.calib_copy_mib << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda")
        b = torch.empty(n, dtype=torch.uint8, device="cuda")
        a.fill_(1)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        log(f"calibration copy: {args.calib_copy_mib} MiB read + {args.calib_copy_mib} MiB written")
        del a, b
    layer, x, logits = build_layer(wl, torch, fuse_silu=not args.unfused,
                                   weight_format=args.weight_format if wl.fp8 else None)
    per_step = []
    ms, kern = time_steps(layer, x, logits, args.steps, args.warmup, torch, per_step)
    q = sorted(per_step)
    pct = {p: q[min(len(q) - 1, int(round(p / 100 * (len(q) - 1))))] for p in (10, 50, 90)}
    g_ms = graph_steps(layer, x, logits, args.steps, torch)
    log(f"hip graph replay: {g_ms:.3f} ms/step")
    log(f"{ms:.3f} ms/step; " + ", ".join(f"{k} {v:.3f}" for k, v in kern.items()))
    work = gemm_work(wl, layer, torch)
    dtype = "fp8_e4m3" if wl.fp8 else "bf16"
    w13_key = "gemm_w13_silu" if layer.fuse_silu else "gemm_w13"
    roof = roofline(work["w13_flops"], work["w13_bytes"], kern[w13_key], dtype)
    roof["kernel"] = ("grouped_gemm w13 (gate/up) with SiLU-and-mul" if layer.fuse_silu
                      else "grouped_gemm w13 (gate/up)")
    tkey = wl.name if layer.weight_format in ("block128", "bf16") else f"{wl.name}_{layer.weight_format}"
    roof["traffic"] = measured_traffic(tkey, "w13")
    w2_roof = roofline(work["w2_flops"], work["w2_bytes"], kern["gemm_w2"], dtype)
    w2_roof["traffic"] = measured_traffic(tkey, "w2")
    gemm_ms = kern[w13_key] + kern["gemm_w2"]
    gemm_tflops = (work["w13_flops"] + work["w2_flops"]) / (gemm_ms * 1e-3) / 1e12
    res = {
        "metric": METRIC,
        "value": round(wl.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_p10_p50_p90": [round(pct[10], 4), round(pct[50], 4), round(pct[90], 4)],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic (seeded N(0,1) tokens and logits, N(0,0.02) expert weights)",
        "config": {"workload": wl.name, "T": wl.T, "H": wl.H, "I": wl.I, "E": wl.E,
                   "E_local": wl.El, "top_k": wl.k, "layout": layer.layout, "block_e": wl.block_e,
                   "rows": layer.rows, "assignments": work["assignments"],
                   "silu_fused_into_w13": layer.fuse_silu, "weight_format": layer.weight_format},
        "roofline": roof,
        "gemm": {"tflops_both": round(gemm_tflops, 1),
                 "executed_tflops_both": round(work["exec_flops"] / (gemm_ms * 1e-3) / 1e12, 1),
                 "mfma_frac_both": round(gemm_tflops / PEAK_TFLOPS[dtype], 4),
                 "flops": {"w13": work["w13_flops"], "w2": work["w2_flops"]},
                 "executed_flops": {"w13": work["w13_exec_flops"], "w2": work["w2_exec_flops"]},
                 "w2": w2_roof},
        "kernels_ms": {k: round(v, 4) for k, v in kern.items()},
        "memory_kernels": memory_kernels(wl, layer, kern, work),
        "hip_graph": {"ms_per_step": round(g_ms, 4), "value": round(wl.T / (g_ms * 1e-3), 1)},
        "cpu_baseline": None,
    }
    if wl.fp8 and not layer.mx and not args.no_mx:
        res["mx_weights"] = mx_variants(wl, x, logits, torch)
    if wl.fp8:
        res["requant_weights"] = requant_weights(wl, torch)
        log(f"requant of w13-shaped block-FP8 weights: {res['requant_weights']['ms']:.3f} ms, "
            f"{res['requant_weights']['achieved']:.0f} GB/s")
    if not args.no_vendor:
        res["vendor_dense"] = vendor_dense(wl, work, torch)
        log("dense vendor GEMMs of the same sizes: " + ", ".join(
            f"{k} {v['ms']:.3f} ms ({v['tflops']:.0f} TFLOP/s)" for k, v in res["vendor_dense"].items()
            if isinstance(v, dict)))
    if not args.no_cpu_baseline and not layer.mx:
        res["cpu_baseline"] = cpu_baseline(wl, x, logits, args.cpu_seconds, torch)
        n_tok, reps = CPU_STAGE_TOKENS.get(wl.name, (min(wl.T, 64), 1))
        res["cpu_baseline"]["stages"] = cpu_stages(wl, x, logits, min(n_tok, wl.T), reps)
    names = [n for n in args.workloads.split(",") if n and n != args.workload]
    if names:
        del layer, x, logits
        torch.cuda.empty_cache()
        res["workloads"] = other_workloads(names, torch, args.workload_steps,
                                           cpu=not args.no_cpu_baseline)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
