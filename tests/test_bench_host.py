"""Host-side arithmetic of bench.py, on the CPU: the roofline's bound and
fractions, the algorithmic bytes of the memory-bound kernels, the gate on the
stored HBM counters, and the refusal of more than one GPU."""
import dataclasses
import hashlib
import json
import os
import subprocess
import sys
import types

import pytest
import torch

import bench
from scatter_grouped_gemm_amd import inputs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_roofline_picks_the_bound_by_arithmetic_intensity():
    ridge = bench.PEAK_TFLOPS["fp8_e4m3"] * 1e12 / (bench.PEAK_HBM_GBS * 1e9)  # 625 FLOP/B
    # below the ridge: HBM-bound, achieved in GB/s
    r = bench.roofline(flops=100.0 * 1e9, nbytes=1e9, ms=1.0, dtype="fp8_e4m3")
    assert r["bound"] == "hbm" and r["unit"] == "GB/s"
    assert r["achieved"] == pytest.approx(1000.0)          # 1 GB in 1 ms
    assert r["frac"] == pytest.approx(1000.0 / 8000.0)
    assert r["arithmetic_intensity"] == pytest.approx(100.0)
    # above it: MFMA-bound, achieved in TFLOP/s against the dtype's dense peak
    r = bench.roofline(flops=2 * ridge * 1e9, nbytes=1e9, ms=1.0, dtype="fp8_e4m3")
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s"
    assert r["achieved"] == pytest.approx(2 * ridge, rel=1e-3)
    assert r["frac"] == pytest.approx(2 * ridge / 5000.0, rel=1e-3)
    r = bench.roofline(flops=2000.0 * 1e9, nbytes=1e9, ms=1.0, dtype="bf16")  # bf16 ridge 312.5
    assert r["bound"] == "mfma" and r["peak"] == 2500.0


def _fake_layer(ids):
    return types.SimpleNamespace(topk_ids=torch.as_tensor(ids, dtype=torch.int32))


def test_memory_kernel_bytes_all_experts_local():
    wl = dataclasses.replace(inputs.get("tiny"), T=4, H=256, I=512, E=8, k=2, fp8=True)
    ids = [[0, 1], [2, 3], [4, 5], [6, 7]]
    A = 8
    kern = {"scatter": 1e-5, "combine": 2e-5}  # ms
    out = bench.memory_kernels(wl, _fake_layer(ids), kern, {"assignments": A})
    H, k, T = 256, 2, 4
    assert out["scatter"]["bytes"] == int(T * 2 * H + A * (H * 1 + H / 128 + 8))
    assert out["combine"]["bytes"] == A * 2 * H + T * (2 * H + 8 * k)
    assert out["combine"]["achieved"] == pytest.approx(out["combine"]["bytes"] / 2e-8 / 1e9, rel=1e-3)
    assert out["combine"]["frac"] == pytest.approx(out["combine"]["achieved"] / 8000.0, rel=1e-3)


def test_memory_kernel_bytes_count_only_local_rows():
    # 8 experts, this GPU holds experts 4..5: token 1 has no local expert
    wl = dataclasses.replace(inputs.get("tiny"), T=3, H=128, I=256, E=8, k=2, fp8=False,
                             num_local=2, expert_start=4)
    ids = [[4, 0], [1, 2], [5, 4]]
    A = 3  # local assignments
    out = bench.memory_kernels(wl, _fake_layer(ids), {"scatter": 1.0, "combine": 1.0},
                               {"assignments": A})
    H, k, T = 128, 2, 3
    assert out["scatter"]["bytes"] == 2 * 2 * H + A * (H * 2 + 8)   # two tokens read
    assert out["combine"]["bytes"] == A * 2 * H + T * (2 * H + 8 * k)


def test_stored_traffic_is_reported_only_for_the_source_it_was_taken_on():
    assert bench.measured_traffic("no_such_workload", "w13") is None
    h = hashlib.sha256()
    for src in ("gemm.hip", "gemm_wreg.hip", "gemm_wreg.h", "gemm_runs.h", "common.h"):
        with open(os.path.join(ROOT, "scatter_grouped_gemm_amd", "csrc", src), "rb") as f:
            h.update(f.read())
    assert bench.gemm_source_sha256() == h.hexdigest()
    profiles = os.path.join(ROOT, "profiles")
    names = [n[len("traffic_"):-len(".json")] for n in os.listdir(profiles)
             if n.startswith("traffic_") and n.endswith(".json")]
    assert names
    for name in names:
        with open(os.path.join(profiles, f"traffic_{name}.json")) as f:
            d = json.load(f)
        for which in ("w13", "w2"):
            got = bench.measured_traffic(name, which)
            if d["gemm_source_sha256"] == h.hexdigest():
                assert got == int(d[which]["read_bytes"] + d[which]["write_bytes"])
            else:
                assert got is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single" in r.stderr
    assert r.stdout == ""
