"""Masked versus compact expert layout on one GPU: time the whole expert path
(route -> scatter -> w13 -> SiLU-and-mul -> w2 -> combine) in both layouts
over a sweep of token counts, with the same weights and tokens, and print one
JSON line per (shape, T, layout) plus a markdown table.

The pages leave the choice between the two layouts open beyond a rule on the
local expert count, and report the compact layout as slower than the masked
one up to a crossover in token count ("Support DeepGEMM for standard MoE
dispatch", comments section).  This sweep measures where that crossover lies
for these kernels.

    python layout_study.py [--shapes fp8_e256,fp8_e32,bf16_e128]
        [--tokens 16,64,...] [--steps 10] [--warmup 3] [--md out.md]

The masked layout holds max_m = T rows per local expert, so its buffers grow
as E_local * T; cases whose buffers would pass --max-gib are skipped and
reported as such.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import sys
import time

import torch

from scatter_grouped_gemm_amd import MoELayer, inputs

# (name, H, I, E, E_local, k, fp8, workload whose weight seeds are used)
SHAPES = {
    "fp8_e256": (7168, 2048, 256, 256, 8, True, "fp8_prefill"),
    "fp8_e32": (7168, 2048, 256, 32, 8, True, "fp8_prefill"),
    "bf16_e128": (4096, 1536, 128, 128, 8, False, "bf16_skewed"),
    "bf16_e8": (4096, 14336, 8, 8, 2, False, "bf16_prefill"),
}
DEFAULT_TOKENS = [16, 64, 256, 1024, 1536, 2048, 3072, 4096, 8192, 16384]


def log(*a):
    print("[layout]", *a, file=sys.stderr, flush=True)


def buffer_gib(layout, T, H, I, El, k, fp8):
    """Device bytes of the per-batch buffers (token rows in the expert layout,
    activations, outputs) in GiB."""
    ab = 1 if fp8 else 2
    rows = El * T if layout == "masked" else T * k + El * 127 + 128
    per_row = H * ab + I * ab + H * 2 + (H // 128 + I // 128 if fp8 else 0)
    return rows * per_row / 2**30


def make_layer(layout, T, H, I, E, El, k, fp8):
    return MoELayer(hidden=H, intermediate=I, num_experts=E, top_k=k, max_tokens=T,
                    num_local_experts=El, fp8=fp8, layout=layout,
                    expected_m=max(1, (T * k) // E), device="cuda")


def time_layer(layer, x, logits, steps, warmup):
    for _ in range(warmup):
        layer(x, logits)
    torch.cuda.synchronize()
    layer.marks = {}
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        layer(x, logits)
    e.record()
    torch.cuda.synchronize()
    kern = {n: sum(a.elapsed_time(b) for a, b in v) / len(v) for n, v in layer.marks.items()}
    layer.marks = None
    return s.elapsed_time(e) / steps, kern


def run_shape(name, tokens, steps, warmup, max_gib):
    H, I, E, El, k, fp8, wl_name = SHAPES[name]
    base = dataclasses.replace(inputs.get(wl_name), H=H, I=I, E=E, k=k, fp8=fp8, num_local=El,
                               expert_start=0, skew=False)
    weights = None
    rows = []
    for T in tokens:
        wl = base.with_tokens(T)
        x = inputs.tokens(wl, "cuda")
        logits = inputs.logits(wl, "cuda")
        res = {}
        for layout in ("compact", "masked"):
            gib = buffer_gib(layout, T, H, I, El, k, fp8)
            if gib > max_gib:
                log(f"{name} T={T} {layout}: skipped ({gib:.1f} GiB of buffers)")
                continue
            layer = make_layer(layout, T, H, I, E, El, k, fp8)
            if weights is None:
                t0 = time.time()
                for e in range(El):
                    w13, w2 = inputs.expert_weights(wl, e, "cuda")
                    layer.set_expert(e, w13, w2)
                weights = (layer.w13, layer.w13_scale, layer.w2, layer.w2_scale) if fp8 else \
                    (layer.w13, None, layer.w2, None)
                torch.cuda.synchronize()
                log(f"{name}: weights for {El} experts in {time.time() - t0:.1f}s")
            else:
                layer.w13, layer.w13_scale, layer.w2, layer.w2_scale = weights
            ms, kern = time_layer(layer, x, logits, steps, warmup)
            res[layout] = dict(ms=ms, w13=kern.get("gemm_w13_silu"), gib=gib)
            line = dict(shape=name, T=T, H=H, I=I, E=E, E_local=El, k=k,
                        dtype="fp8_e4m3" if fp8 else "bf16", layout=layout,
                        ms_per_step=round(ms, 4), buffers_gib=round(gib, 2),
                        kernels_ms={n: round(v, 4) for n, v in kern.items()})
            print(json.dumps(line), flush=True)
            del layer
            torch.cuda.empty_cache()
        rows.append(dict(T=T, **{f"{lay}_{f}": v for lay, r in res.items() for f, v in r.items()}))
    return rows


def markdown(results):
    """Table of one sweep: whole-step and w13 times of both layouts, the masked
    buffers' size, and the layout moe_choose_layout picks for the shape."""
    from scatter_grouped_gemm_amd import _lib as L
    out = ["| shape | T | compact ms | masked ms | compact / masked | compact w13 ms | masked w13 ms "
           "| masked buffers GiB | compact buffers GiB | policy |",
           "|---|---|---|---|---|---|---|---|---|---|"]
    f = lambda v, p=4: f"{v:.{p}f}" if v is not None else "-"
    for name, rows in results.items():
        H, I, E, El, k, fp8, _ = SHAPES[name]
        for r in rows:
            T = r["T"]
            c, m = r.get("compact_ms"), r.get("masked_ms")
            ratio = f"{c / m:.3f}" if c is not None and m is not None else "-"
            pick = "masked" if L.moe_choose_layout(T, k, E, El) else "compact"
            out.append(f"| {name} | {T} | {f(c)} | {f(m) if m is not None else 'skipped'} | {ratio} | "
                       f"{f(r.get('compact_w13'), 3)} | {f(r.get('masked_w13'), 3)} | "
                       f"{f(buffer_gib('masked', T, H, I, El, k, fp8), 2)} | "
                       f"{f(buffer_gib('compact', T, H, I, El, k, fp8), 2)} | {pick} |")
    return "\n".join(out)


def from_jsonl(path):
    """Rebuild the per-shape rows of a sweep from the JSON lines it printed."""
    results = {}
    with open(path) as fh:
        for line in fh:
            if not line.startswith("{"):
                continue
            d = json.loads(line)
            rows = results.setdefault(d["shape"], [])
            if not rows or rows[-1]["T"] != d["T"]:
                rows.append(dict(T=d["T"]))
            lay = d["layout"]
            rows[-1][f"{lay}_ms"] = d["ms_per_step"]
            rows[-1][f"{lay}_w13"] = d["kernels_ms"].get("gemm_w13_silu")
    return results


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--shapes", default="fp8_e256,fp8_e32,bf16_e128,bf16_e8")
    ap.add_argument("--tokens", default=",".join(map(str, DEFAULT_TOKENS)))
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--max-gib", type=float, default=120.0)
    ap.add_argument("--md", default=None)
    ap.add_argument("--from-jsonl", default=None,
                    help="only rebuild the markdown table from the JSON lines of an earlier run")
    a = ap.parse_args(argv)
    tokens = [int(t) for t in a.tokens.split(",")]
    if a.from_jsonl:
        results = from_jsonl(a.from_jsonl)
    else:
        results = {}
        for name in a.shapes.split(","):
            results[name] = run_shape(name, tokens, a.steps, a.warmup, a.max_gib)
    md = markdown(results)
    print(md, file=sys.stderr, flush=True)
    if a.md:
        with open(a.md, "w") as f:
            f.write(md + "\n")


if __name__ == "__main__":
    main()
