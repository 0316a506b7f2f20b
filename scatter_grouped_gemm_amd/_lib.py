"""ctypes binding of libmoe (include/moe.h), one Python function per C entry point.

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, then their data pointers and torch's current HIP stream are handed
to the C call.  Every step of the computation runs in the library's HIP
kernels; there is no fallback.  If libmoe.so has not been built, loading fails
with an error that says how to build it.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")
_lib = None

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ECAPACITY, MOE_EDEVICE = 0, 1, 2, 3, 4
MOE_DTYPE_BF16, MOE_DTYPE_FP8_E4M3_UE8M0, MOE_DTYPE_FP8_E4M3_MXFP8, MOE_DTYPE_FP8_MXFP4 = 0, 1, 2, 3
MOE_MX_E4M3, MOE_MX_E2M1 = 0, 1
MOE_DEVERR_MASKED_OVERFLOW = 1
MOE_SCATTER_NOALLOC_MAX_BYTES = 4 << 20

# name -> (restype, argtypes); the exported symbols of include/moe.h
_P, _I32, _I64, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
SIGNATURES = {
    "moe_compact_rows_bound": (_I64, [_I64, _I32, _I32]),
    "moe_use_masked_layout": (_I32, [_I32, _I32]),
    "moe_choose_layout": (_I32, [_I64, _I32, _I32, _I32, _I32]),
    "moe_scatter_ws_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "moe_status_str": (ctypes.c_char_p, [_I32]),
    "moe_get_device_error": (_I32, [_P, _P, _P]),
    "moe_route_topk": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_scatter_compact": (_I32, [_P, _I32, _I32, _P, _I32, _I32, _I32, _I32, _I64, _I32,
                                   _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_scatter_compact_noalloc": (_I32, [_P, _I32, _I32, _P, _I32, _I32, _I32, _I32, _I64, _I32,
                                           _P, _P, _P, _P, _P, _P, _P]),
    "moe_scatter_masked": (_I32, [_P, _I32, _I32, _P, _I32, _I32, _I32, _I32, _I32,
                                  _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_quant_fp8_ue8m0": (_I32, [_P, _I64, _I32, _I64, _P, _P, _P, _P]),
    "moe_quant_weight_fp8_ue8m0": (_I32, [_P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_requant_weight_fp8_ue8m0": (_I32, [_P, _P, _I32, _I32, _I32, _P, _P, _P]),
    "moe_quant_weight_mx": (_I32, [_P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "moe_mx_scales_tile": (_I32, [_P, _I32, _I32, _I32, _P, _P]),
    "grouped_gemm_rows_executed": (_I64, [_I32, _I32, _P, _I32, _I32, _I64, _I32, _I32]),
    "grouped_gemm_contig": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _I64, _I32, _I32, _I32, _P]),
    "grouped_gemm_masked": (_I32, [_I32, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _P]),
    "grouped_gemm_contig_silu": (_I32, [_I32, _P, _P, _P, _P, _I32, _P, _P, _P, _I64, _I32, _I32,
                                        _I32, _P]),
    "grouped_gemm_masked_silu": (_I32, [_I32, _P, _P, _P, _P, _I32, _P, _P, _P, _I32, _I32, _I32,
                                        _I32, _I32, _P]),
    "silu_and_mul": (_I32, [_P, _I64, _I32, _P, _P, _I32, _I32, _P, _P, _P]),
    "moe_combine": (_I32, [_P, _I64, _P, _P, _I32, _I32, _I32, _P, _P]),
}


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_str(status)})")


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is not built; run `python -m scatter_grouped_gemm_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def lib_path() -> str:
    return _LIB_PATH


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(fn: str, status: int) -> None:
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t):
    if t is None:
        return None
    assert t.is_cuda and t.is_contiguous(), "device tensors must be contiguous"
    return t.data_ptr()


def _stream():
    return torch.cuda.current_stream().cuda_stream


def _dtype_code(fp8: bool) -> int:
    return MOE_DTYPE_FP8_E4M3_UE8M0 if fp8 else MOE_DTYPE_BF16


def _gemm_dtype(fp8) -> int:
    """GEMM operand dtype: False -> BF16, True -> FP8 with 128x128 weight
    blocks, "mxfp8" -> FP8 activations with MX e4m3 weights."""
    if fp8 == "mxfp8":
        return MOE_DTYPE_FP8_E4M3_MXFP8
    if fp8 == "mxfp4":
        return MOE_DTYPE_FP8_MXFP4
    if isinstance(fp8, str):
        raise ValueError(f"unknown GEMM weight format {fp8!r}")
    return _dtype_code(bool(fp8))


# --- host helpers ---------------------------------------------------------------

def moe_compact_rows_bound(num_assignments: int, num_local_experts: int, block_e: int = 128) -> int:
    return int(lib().moe_compact_rows_bound(num_assignments, num_local_experts, block_e))


def moe_use_masked_layout(num_experts: int, num_local_experts: int) -> bool:
    return bool(lib().moe_use_masked_layout(num_experts, num_local_experts))


def moe_choose_layout(max_tokens: int, top_k: int, num_experts: int, num_local_experts: int,
                      block_e: int = 128) -> bool:
    r = lib().moe_choose_layout(max_tokens, top_k, num_experts, num_local_experts, block_e)
    if r < 0:
        raise ValueError("moe_choose_layout: sizes must be positive, num_local_experts <= num_experts "
                         "and top_k <= num_experts")
    return bool(r)


def moe_scatter_ws_bytes(T: int, k: int, num_local_experts: int, H: int) -> int:
    return int(lib().moe_scatter_ws_bytes(T, k, num_local_experts, H))


def moe_get_device_error(ws: torch.Tensor) -> int:
    out = ctypes.c_int32(0)
    _check("moe_get_device_error", lib().moe_get_device_error(_ptr(ws), ctypes.byref(out), _stream()))
    return int(out.value)



def grouped_gemm_rows_executed(fp8, masked: bool, counts, expected_m: int, M: int, N: int, K: int) -> int:
    """Rows the grouped GEMM with these arguments runs its MFMAs on (whole
    16-row blocks of its tiles) for per-expert valid counts."""
    import numpy as np
    c = np.ascontiguousarray(np.asarray(counts, np.int32))
    r = lib().grouped_gemm_rows_executed(_gemm_dtype(fp8), int(bool(masked)),
                                         c.ctypes.data_as(ctypes.c_void_p), len(c), expected_m, M, N, K)
    if r < 0:
        raise ValueError("grouped_gemm_rows_executed: bad arguments")
    return int(r)


# --- device calls ----------------------------------------------------------------

def moe_route_topk(logits: torch.Tensor, k: int, topk_ids: torch.Tensor, topk_weights: torch.Tensor):
    assert logits.dtype == torch.float32 and logits.dim() == 2
    T, E = logits.shape
    assert topk_ids.dtype == torch.int32 and topk_ids.shape == (T, k)
    assert topk_weights.dtype == torch.float32 and topk_weights.shape == (T, k)
    _check("moe_route_topk", lib().moe_route_topk(_ptr(logits), T, E, k, _ptr(topk_ids),
                                                  _ptr(topk_weights), _stream()))


def moe_scatter_compact(x, topk_ids, expert_start, num_local_experts, block_e, rows_capacity,
                        fp8, x_out, scale_out, m_indices, expert_start_loc, num_valid, src2dst, ws):
    assert x.dtype == torch.bfloat16 and x.dim() == 2
    T, H = x.shape
    k = topk_ids.shape[1]
    _check("moe_scatter_compact", lib().moe_scatter_compact(
        _ptr(x), T, H, _ptr(topk_ids), k, expert_start, num_local_experts, block_e, rows_capacity,
        _dtype_code(fp8), _ptr(x_out), _ptr(scale_out), _ptr(m_indices), _ptr(expert_start_loc),
        _ptr(num_valid), _ptr(src2dst), _ptr(ws), ws.numel() * ws.element_size(), _stream()))


def moe_scatter_compact_noalloc(x, topk_ids, expert_start, num_local_experts, block_e, rows_capacity,
                                fp8, x_out, scale_out, m_indices, expert_start_loc, num_valid, src2dst):
    """moe_scatter_compact on the library's static per-device scratch (no ws)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2
    T, H = x.shape
    k = topk_ids.shape[1]
    _check("moe_scatter_compact_noalloc", lib().moe_scatter_compact_noalloc(
        _ptr(x), T, H, _ptr(topk_ids), k, expert_start, num_local_experts, block_e, rows_capacity,
        _dtype_code(fp8), _ptr(x_out), _ptr(scale_out), _ptr(m_indices), _ptr(expert_start_loc),
        _ptr(num_valid), _ptr(src2dst), _stream()))


def moe_scatter_masked(x, topk_ids, expert_start, num_local_experts, max_m, fp8, x_out, scale_out,
                       masked_m, src2dst, ws):
    assert x.dtype == torch.bfloat16 and x.dim() == 2
    T, H = x.shape
    k = topk_ids.shape[1]
    _check("moe_scatter_masked", lib().moe_scatter_masked(
        _ptr(x), T, H, _ptr(topk_ids), k, expert_start, num_local_experts, max_m, _dtype_code(fp8),
        _ptr(x_out), _ptr(scale_out), _ptr(masked_m), _ptr(src2dst), _ptr(ws),
        ws.numel() * ws.element_size(), _stream()))


def moe_quant_fp8_ue8m0(x, q, scale, m_indices=None):
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    M, K = x.shape
    _check("moe_quant_fp8_ue8m0", lib().moe_quant_fp8_ue8m0(
        x.data_ptr(), M, K, x.stride(0), _ptr(m_indices), _ptr(q), _ptr(scale), _stream()))


def moe_quant_weight_fp8_ue8m0(w, q, scale):
    assert w.dtype == torch.bfloat16 and w.dim() == 3
    G, N, K = w.shape
    _check("moe_quant_weight_fp8_ue8m0", lib().moe_quant_weight_fp8_ue8m0(
        _ptr(w), G, N, K, _ptr(q), _ptr(scale), _stream()))


def moe_requant_weight_fp8_ue8m0(q_in, s_in, q_out, s_out):
    """Block-FP8 weights (e4m3 [G,N,K] + fp32 [G,N/128,K/128]) -> e4m3 + UE8M0."""
    G, N, K = q_in.shape
    assert q_in.dtype == torch.uint8 and s_in.dtype == torch.float32 and q_out.shape == (G, N, K)
    assert s_in.shape == (G, N // 128, K // 128) and s_out.shape == s_in.shape and s_out.dtype == torch.uint8
    _check("moe_requant_weight_fp8_ue8m0", lib().moe_requant_weight_fp8_ue8m0(
        _ptr(q_in), _ptr(s_in), G, N, K, _ptr(q_out), _ptr(s_out), _stream()))


def moe_quant_weight_mx(w, fmt, q, scale_tiled):
    """bf16 w [G,N,K] -> MX codes q (e4m3 [G,N,K] or e2m1 pairs [G,N,K/2]) and
    tiled scales scale_tiled [G, N/64, K/128, 256]."""
    G, N, K = w.shape
    f = {"e4m3": MOE_MX_E4M3, "e2m1": MOE_MX_E2M1}[fmt]
    assert w.dtype == torch.bfloat16 and q.dtype == torch.uint8 and scale_tiled.dtype == torch.uint8
    assert q.shape == (G, N, K if f == MOE_MX_E4M3 else K // 2)
    assert scale_tiled.numel() == G * N * (K // 32)
    _check("moe_quant_weight_mx", lib().moe_quant_weight_mx(
        _ptr(w), G, N, K, f, _ptr(q), _ptr(scale_tiled), _stream()))


def moe_mx_scales_tile(scale_plain, scale_tiled):
    """Plain MX scales [G,N,K/32] -> the GEMM's tiled layout."""
    G, N, KB = scale_plain.shape
    assert scale_plain.dtype == torch.uint8 and scale_tiled.dtype == torch.uint8
    assert scale_tiled.numel() == scale_plain.numel()
    _check("moe_mx_scales_tile", lib().moe_mx_scales_tile(
        _ptr(scale_plain), G, N, KB * 32, _ptr(scale_tiled), _stream()))


def _bk(fp8, B):
    """(G, N, K) of a weight tensor: e2m1 weights hold two k per byte."""
    G, N, Kb = B.shape
    return G, N, Kb * 2 if fp8 == "mxfp4" else Kb


def grouped_gemm_contig(fp8, A, A_scale, B, B_scale, C, m_indices):
    M, K = A.shape
    G, N, K2 = _bk(fp8, B)
    assert K == K2 and C.shape == (M, N) and C.dtype == torch.bfloat16
    _check("grouped_gemm_contig", lib().grouped_gemm_contig(
        _gemm_dtype(fp8), _ptr(A), _ptr(A_scale), _ptr(B), _ptr(B_scale), _ptr(C), _ptr(m_indices),
        M, N, K, G, _stream()))


def grouped_gemm_masked(fp8, A, A_scale, B, B_scale, C, masked_m, expected_m):
    G, max_m, K = A.shape
    G2, N, K2 = _bk(fp8, B)
    assert G == G2 and K == K2 and C.shape == (G, max_m, N) and C.dtype == torch.bfloat16
    _check("grouped_gemm_masked", lib().grouped_gemm_masked(
        _gemm_dtype(fp8), _ptr(A), _ptr(A_scale), _ptr(B), _ptr(B_scale), _ptr(C), _ptr(masked_m),
        expected_m, max_m, N, K, G, _stream()))


def grouped_gemm_contig_silu(fp8, A, A_scale, B, B_scale, out, m_indices, out_scale=None):
    """w13 GEMM with SiLU-and-mul fused: out [M][I] is bf16, or e4m3 (uint8)
    with out_scale [I/128][M]."""
    M, K = A.shape
    G, N, K2 = _bk(fp8, B)
    I = N // 2
    q8 = out.dtype == torch.uint8
    assert K == K2 and out.shape == (M, I) and (q8 or out.dtype == torch.bfloat16)
    _check("grouped_gemm_contig_silu", lib().grouped_gemm_contig_silu(
        _gemm_dtype(fp8), _ptr(A), _ptr(A_scale), _ptr(B), _ptr(B_scale), _dtype_code(q8),
        _ptr(out), _ptr(out_scale), _ptr(m_indices), M, I, K, G, _stream()))


def grouped_gemm_masked_silu(fp8, A, A_scale, B, B_scale, out, masked_m, expected_m,
                             out_scale=None):
    """Masked-layout w13 GEMM with SiLU-and-mul fused: out [G][max_m][I];
    FP8 out_scale [G][I/128][max_m]."""
    G, max_m, K = A.shape
    G2, N, K2 = _bk(fp8, B)
    I = N // 2
    q8 = out.dtype == torch.uint8
    assert G == G2 and K == K2 and out.shape == (G, max_m, I) and (q8 or out.dtype == torch.bfloat16)
    _check("grouped_gemm_masked_silu", lib().grouped_gemm_masked_silu(
        _gemm_dtype(fp8), _ptr(A), _ptr(A_scale), _ptr(B), _ptr(B_scale), _dtype_code(q8),
        _ptr(out), _ptr(out_scale), _ptr(masked_m), expected_m, max_m, I, K, G, _stream()))


def silu_and_mul(gateup, out, fp8=False, out_scale=None, m_indices=None, masked_m=None, max_m=0):
    M, N = gateup.shape
    _check("silu_and_mul", lib().silu_and_mul(
        _ptr(gateup), M, N // 2, _ptr(m_indices), _ptr(masked_m), max_m, _dtype_code(fp8),
        _ptr(out), _ptr(out_scale), _stream()))


def moe_combine(Y, src2dst, topk_weights, out):
    T, k = src2dst.shape
    H = Y.shape[-1]
    rows = Y.numel() // H
    _check("moe_combine", lib().moe_combine(_ptr(Y), rows, _ptr(src2dst), _ptr(topk_weights), T, k,
                                            H, _ptr(out), _stream()))
