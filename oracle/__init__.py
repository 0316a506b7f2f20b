"""CPU oracle for the routed-token scatter -> grouped GEMM MoE expert path.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow reference the HIP
library is checked against.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does.  It
shares no code with the HIP library: the arithmetic lives in ``moe_oracle.c``
(plain C, no FMA contraction, OpenMP over independent rows only) and this
module only marshals numpy arrays through ctypes.

bf16 arrays are numpy ``uint16`` holding the raw bit patterns; e4m3 and UE8M0
arrays are ``uint8``.  Activation scales are row-major ``[rows, K/128]`` here.

Every function is pinned by the ``-m "not gpu"`` tests in ``tests/`` against
closed forms, brute force, exact rational arithmetic or an independent library
routine; see the docstring of each test for what it pins.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libmoe_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc: no fast-math, no FMA contraction."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
               "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wno-unknown-pragmas",
               _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    sig = {
        "orc_bf16_to_f32": (ctypes.c_float, [ctypes.c_uint16]),
        "orc_f64_to_bf16": (ctypes.c_uint16, [f64]),
        "orc_e4m3_to_f64": (f64, [ctypes.c_uint8]),
        "orc_e4m3_from_f64": (ctypes.c_uint8, [f64]),
        "orc_ue8m0_exponent": (i32, [f64]),
        "orc_compact_rows_bound": (i64, [i64, i32, i32]),
        "orc_use_masked_layout": (i32, [i32, i32]),
        "orc_route_topk": (None, [P, i32, i32, i32, P, P]),
        "orc_quant_rows": (None, [P, i64, i32, i64, P, P]),
        "orc_quant_weight_blocks": (None, [P, i32, i32, i32, P, P]),
        "orc_requant_weight_blocks": (None, [P, P, i32, i32, i32, P, P]),
        "orc_e2m1_to_f64": (f64, [ctypes.c_uint8]),
        "orc_e2m1_from_f64": (ctypes.c_uint8, [f64]),
        "orc_mx_exponent": (i32, [f64, f64]),
        "orc_quant_weight_mx": (None, [P, i32, i32, i32, i32, P, P]),
        "orc_gemm_mx_rows": (None, [P, P, i64, P, P, i32, i32, i32, P, P]),
        "orc_scatter_compact": (i32, [P, i32, i32, P, i32, i32, i32, i32, i64, i32,
                                      P, P, P, P, P, P]),
        "orc_scatter_masked": (i32, [P, i32, i32, P, i32, i32, i32, i32, i32,
                                     P, P, P, P]),
        "orc_gemm_bf16_rows": (None, [P, i64, P, i32, i32, P, P]),
        "orc_gemm_fp8_rows": (None, [P, P, i64, P, P, i32, i32, P, P]),
        "orc_silu_and_mul": (None, [P, i64, i32, P, P]),
        "orc_combine": (None, [P, P, P, i32, i32, i32, P]),
        "orc_moe_dense": (None, [P, i32, i32, i32, P, P, i32, i32, i32, i32,
                                 P, P, P, P, P, P, P]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _c(a: np.ndarray, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _p(a):
    return None if a is None else a.ctypes.data


# --- scalar helpers ------------------------------------------------------------

def bf16_to_f32(b: int) -> float:
    return float(_load().orc_bf16_to_f32(int(b)))


def f64_to_bf16(v: float) -> int:
    return int(_load().orc_f64_to_bf16(float(v)))


def e4m3_to_f64(q: int) -> float:
    return float(_load().orc_e4m3_to_f64(int(q)))


def e4m3_from_f64(v: float) -> int:
    return int(_load().orc_e4m3_from_f64(float(v)))


def ue8m0_exponent(amax: float) -> int:
    return int(_load().orc_ue8m0_exponent(float(amax)))


def compact_rows_bound(num_assignments: int, num_experts: int, block_e: int = 128) -> int:
    return int(_load().orc_compact_rows_bound(num_assignments, num_experts, block_e))


def use_masked_layout(num_experts: int, num_local_experts: int) -> bool:
    return bool(_load().orc_use_masked_layout(num_experts, num_local_experts))


# --- array steps ---------------------------------------------------------------

def route_topk(logits: np.ndarray, k: int):
    L = _c(logits, np.float32)
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _load().orc_route_topk(_p(L), T, E, k, _p(ids), _p(w))
    return ids, w


def quant_rows(x: np.ndarray):
    """Per row, per 128 channels -> (e4m3 [M,K], UE8M0 bytes [M, K/128])."""
    x = _c(x, np.uint16)
    M, K = x.shape
    assert K % 128 == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // 128), np.uint8)
    _load().orc_quant_rows(_p(x), M, K, K, _p(q), _p(s))
    return q, s


def quant_weight_blocks(w: np.ndarray):
    """128x128 blocks of w[G,N,K] -> (e4m3 [G,N,K], UE8M0 [G, N/128, K/128])."""
    w = _c(w, np.uint16)
    G, N, K = w.shape
    assert N % 128 == 0 and K % 128 == 0
    q = np.empty((G, N, K), np.uint8)
    s = np.empty((G, N // 128, K // 128), np.uint8)
    _load().orc_quant_weight_blocks(_p(w), G, N, K, _p(q), _p(s))
    return q, s


def requant_weight_blocks(q: np.ndarray, s: np.ndarray):
    """Block-FP8 weights (e4m3 [G,N,K], fp32 scales [G,N/128,K/128]) -> the
    UE8M0 block format (e4m3 [G,N,K], UE8M0 [G,N/128,K/128]) via bf16."""
    q = _c(q, np.uint8)
    s = _c(s, np.float32)
    G, N, K = q.shape
    assert N % 128 == 0 and K % 128 == 0 and s.shape == (G, N // 128, K // 128)
    qo = np.empty((G, N, K), np.uint8)
    so = np.empty((G, N // 128, K // 128), np.uint8)
    _load().orc_requant_weight_blocks(_p(q), _p(s), G, N, K, _p(qo), _p(so))
    return qo, so


def scatter_compact(x, topk_ids, expert_start, num_local_experts, block_e,
                    rows_capacity, fp8: bool, rows: bool = True):
    """rows=False computes only the indices (no scattered rows)."""
    x = _c(x, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    k = ids.shape[1]
    if not rows:
        x_out = s_out = None
    elif fp8:
        x_out = np.zeros((rows_capacity, H), np.uint8)
        s_out = np.zeros((rows_capacity, H // 128), np.uint8)
    else:
        x_out = np.zeros((rows_capacity, H), np.uint16)
        s_out = None
    m_idx = np.empty(rows_capacity, np.int32)
    start = np.empty(num_local_experts, np.int32)
    nvalid = np.empty(num_local_experts, np.int32)
    src2dst = np.empty((T, k), np.int32)
    rc = _load().orc_scatter_compact(_p(x), T, H, _p(ids), k, expert_start,
                                     num_local_experts, block_e, rows_capacity,
                                     1 if fp8 else 0, _p(x_out), _p(s_out), _p(m_idx),
                                     _p(start), _p(nvalid), _p(src2dst))
    if rc != 0:
        raise ValueError(f"oracle scatter_compact: capacity {rows_capacity} too small")
    return dict(x_out=x_out, scale_out=s_out, m_indices=m_idx,
                expert_start_loc=start, num_valid=nvalid, src2dst=src2dst)


def scatter_masked(x, topk_ids, expert_start, num_local_experts, max_m, fp8: bool,
                   rows: bool = True):
    x = _c(x, np.uint16)
    ids = _c(topk_ids, np.int32)
    T, H = x.shape
    k = ids.shape[1]
    nrows = num_local_experts * max_m
    if not rows:
        x_out = s_out = None
    elif fp8:
        x_out = np.zeros((nrows, H), np.uint8)
        s_out = np.zeros((nrows, H // 128), np.uint8)
    else:
        x_out = np.zeros((nrows, H), np.uint16)
        s_out = None
    masked_m = np.empty(num_local_experts, np.int32)
    src2dst = np.empty((T, k), np.int32)
    rc = _load().orc_scatter_masked(_p(x), T, H, _p(ids), k, expert_start,
                                    num_local_experts, max_m, 1 if fp8 else 0,
                                    _p(x_out), _p(s_out), _p(masked_m), _p(src2dst))
    if rc != 0:
        raise ValueError(f"oracle scatter_masked: max_m {max_m} too small")
    return dict(x_out=x_out, scale_out=s_out, masked_m=masked_m, src2dst=src2dst)


def masked_row_group(masked_m: np.ndarray, max_m: int) -> np.ndarray:
    """Per-row group of a masked layout: g for r < masked_m[g], else -1."""
    G = masked_m.shape[0]
    r = np.arange(max_m)[None, :]
    g = np.where(r < masked_m[:, None], np.arange(G)[:, None], -1)
    return g.reshape(-1).astype(np.int32)


def gemm_bf16_rows(A, B, row_group):
    A = _c(A, np.uint16)
    B = _c(B, np.uint16)
    rg = _c(row_group, np.int32)
    M, K = A.shape
    G, N, K2 = B.shape
    assert K == K2 and rg.shape[0] == M
    C = np.zeros((M, N), np.uint16)
    _load().orc_gemm_bf16_rows(_p(A), M, _p(B), N, K, _p(rg), _p(C))
    return C


def gemm_fp8_rows(A, A_scale, B, B_scale, row_group):
    A = _c(A, np.uint8)
    As = _c(A_scale, np.uint8)
    B = _c(B, np.uint8)
    Bs = _c(B_scale, np.uint8)
    rg = _c(row_group, np.int32)
    M, K = A.shape
    G, N, K2 = B.shape
    assert K == K2 and As.shape == (M, K // 128) and Bs.shape == (G, N // 128, K // 128)
    C = np.zeros((M, N), np.uint16)
    _load().orc_gemm_fp8_rows(_p(A), _p(As), M, _p(B), _p(Bs), N, K, _p(rg), _p(C))
    return C


MX_FORMATS = {"mxfp8": 0, "mxfp4": 1}


def e2m1_to_f64(q: int) -> float:
    return float(_load().orc_e2m1_to_f64(int(q)))


def e2m1_from_f64(v: float) -> int:
    return int(_load().orc_e2m1_from_f64(float(v)))


def mx_exponent(amax: float, fmax: float) -> int:
    return int(_load().orc_mx_exponent(float(amax), float(fmax)))


def quant_weight_mx(w: np.ndarray, fmt: str):
    """MX weights from bf16 w[G,N,K]: (codes, scales [G,N,K/32]); codes are e4m3
    [G,N,K] for "mxfp8", e2m1 two per byte [G,N,K/2] (even k low) for "mxfp4"."""
    w = _c(w, np.uint16)
    G, N, K = w.shape
    assert K % 32 == 0
    f = MX_FORMATS[fmt]
    q = np.zeros((G, N, K if f == 0 else K // 2), np.uint8)
    sc = np.empty((G, N, K // 32), np.uint8)
    _load().orc_quant_weight_mx(_p(w), G, N, K, f, _p(q), _p(sc))
    return q, sc


def gemm_mx_rows(A, A_scale, B, B_scale, fmt: str, row_group):
    """FP8 rows (scales [M, K/128]) times MX weights of format fmt."""
    A = _c(A, np.uint8)
    As = _c(A_scale, np.uint8)
    B = _c(B, np.uint8)
    Bs = _c(B_scale, np.uint8)
    rg = _c(row_group, np.int32)
    f = MX_FORMATS[fmt]
    M, K = A.shape
    G, N, Kb = B.shape
    assert Kb == (K if f == 0 else K // 2) and As.shape == (M, K // 128)
    assert Bs.shape == (G, N, K // 32) and rg.shape[0] == M
    C = np.zeros((M, N), np.uint16)
    _load().orc_gemm_mx_rows(_p(A), _p(As), M, _p(B), _p(Bs), f, N, K, _p(rg), _p(C))
    return C


def silu_and_mul(gateup, row_group):
    gu = _c(gateup, np.uint16)
    rg = _c(row_group, np.int32)
    M, N = gu.shape
    I = N // 2
    out = np.zeros((M, I), np.uint16)
    _load().orc_silu_and_mul(_p(gu), M, I, _p(rg), _p(out))
    return out


def combine(Y, src2dst, topk_weights):
    Y = _c(Y, np.uint16)
    s = _c(src2dst, np.int32)
    w = _c(topk_weights, np.float32)
    T, k = s.shape
    H = Y.shape[1]
    out = np.empty((T, H), np.uint16)
    _load().orc_combine(_p(Y), _p(s), _p(w), T, k, H, _p(out))
    return out


def moe_dense(x, topk_ids, topk_weights, expert_start, num_local_experts, fp8,
              w13=None, w2=None, w13q=None, w13s=None, w2q=None, w2s=None):
    """Layout-free layer: per token and slot, w13 -> SiLU-mul -> w2, summed."""
    x = _c(x, np.uint16)
    ids = _c(topk_ids, np.int32)
    w = _c(topk_weights, np.float32)
    T, H = x.shape
    k = ids.shape[1]
    if fp8:
        w13q, w13s = _c(w13q, np.uint8), _c(w13s, np.uint8)
        w2q, w2s = _c(w2q, np.uint8), _c(w2s, np.uint8)
        assert w13q.shape[0] >= num_local_experts and w2q.shape[0] >= num_local_experts
        I = w2q.shape[2]
    else:
        w13, w2 = _c(w13, np.uint16), _c(w2, np.uint16)
        assert w13.shape[0] >= num_local_experts and w2.shape[0] >= num_local_experts
        I = w2.shape[2]
    out = np.empty((T, H), np.uint16)
    _load().orc_moe_dense(_p(x), T, H, I, _p(ids), _p(w), k, expert_start,
                          num_local_experts, 1 if fp8 else 0, _p(w13), _p(w2),
                          _p(w13q), _p(w13s), _p(w2q), _p(w2s), _p(out))
    return out


def moe_layer(x, logits, k, *, expert_start, num_local_experts, layout, fp8,
              block_e=128, rows_capacity=None, max_m=None,
              w13=None, w2=None, w13q=None, w13s=None, w2q=None, w2s=None, mx=None):
    """The layout path step by step: route -> scatter -> w13 -> SiLU-mul ->
    (requantise) -> w2 -> combine.  Returns the output and every intermediate.
    mx = "mxfp8" / "mxfp4": the FP8 path with MX weights (w13q/w13s and
    w2q/w2s from quant_weight_mx)."""
    ids, tw = route_topk(logits, k)
    T = x.shape[0]
    if layout == "compact":
        if rows_capacity is None:
            rows_capacity = compact_rows_bound(T * k, num_local_experts, block_e)
        sc = scatter_compact(x, ids, expert_start, num_local_experts, block_e,
                             rows_capacity, fp8)
        rg = sc["m_indices"]
    else:
        sc = scatter_masked(x, ids, expert_start, num_local_experts, max_m, fp8)
        rg = masked_row_group(sc["masked_m"], max_m)
    if mx is not None:
        assert fp8

    def wgemm(a, a_s, q, s_):
        if mx is not None:
            return gemm_mx_rows(a, a_s, q, s_, mx, rg)
        return gemm_fp8_rows(a, a_s, q, s_, rg)

    if fp8:
        h1 = wgemm(sc["x_out"], sc["scale_out"], w13q, w13s)
        act = silu_and_mul(h1, rg)
        aq = np.zeros(act.shape, np.uint8)
        asc = np.zeros((act.shape[0], act.shape[1] // 128), np.uint8)
        valid = rg >= 0
        if valid.any():
            q, s = quant_rows(act[valid])
            aq[valid], asc[valid] = q, s
        y = wgemm(aq, asc, w2q, w2s)
    else:
        h1 = gemm_bf16_rows(sc["x_out"], w13, rg)
        act = silu_and_mul(h1, rg)
        y = gemm_bf16_rows(act, w2, rg)
    out = combine(y, sc["src2dst"], tw)
    return dict(out=out, topk_ids=ids, topk_weights=tw, scatter=sc, row_group=rg,
                h1=h1, act=act, y=y)
