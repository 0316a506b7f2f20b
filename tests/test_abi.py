"""The C ABI on the host: every symbol declared in include/moe.h is exported by
libmoe.so, the pure host helpers agree with the oracle, and argument
validation rejects bad calls before any device work (no GPU needed: every call
here fails validation, so nothing is launched)."""
import ctypes
import os
import re
import subprocess

import numpy as np
import pytest

from scatter_grouped_gemm_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 4096  # a non-null address that is never dereferenced: each call below fails validation


def _declared():
    src = open(os.path.join(ROOT, "include", "moe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w \*]*?\b(\w+)\s*\(", src, flags=re.M)))


def test_every_declared_symbol_is_exported_and_bound():
    names = _declared()
    assert len(names) >= 14
    out = subprocess.run(["nm", "-D", "--defined-only", L.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if l.strip()}
    for n in names:
        assert n in exported, n
        assert n in L.SIGNATURES, n
        getattr(L.lib(), n)


def test_host_helpers_match_oracle(orc):
    for A, E, B in [(0, 8, 128), (128, 8, 128), (8192, 8, 128), (65536, 256, 128), (7, 128, 128),
                    (131072, 128, 128), (5, 3, 256)]:
        assert L.moe_compact_rows_bound(A, E, B) == orc.compact_rows_bound(A, E, B)
    for E, El in [(256, 32), (256, 33), (8, 8), (64, 1), (32, 32)]:
        assert L.moe_use_masked_layout(E, El) == orc.use_masked_layout(E, El)
    # the measured layout policy: masked while T*k <= 64*E and E_local*T <= 4x
    # the compact bound; the cases are the measured shapes on both sides of
    # their crossovers (T, k, E, E_local, masked?)
    for T, k, E, El, want in [(256, 8, 256, 256, 1), (512, 8, 256, 256, 1), (1024, 8, 256, 256, 0),
                              (1024, 8, 256, 32, 1), (2048, 8, 256, 32, 1), (3072, 8, 256, 32, 0),
                              (256, 8, 128, 128, 1), (1024, 8, 128, 128, 0), (16, 8, 128, 128, 1),
                              (256, 2, 8, 8, 1), (1024, 2, 8, 8, 0), (1, 1, 1, 1, 1)]:
        assert L.moe_choose_layout(T, k, E, El) == bool(want), (T, k, E, El)
    # whatever the shape, a masked pick never holds more than 4x the compact rows
    for T in (1, 7, 64, 300, 1000, 2048, 5000, 20000):
        for k, E, El in [(8, 256, 256), (8, 256, 32), (2, 8, 8), (8, 128, 128), (6, 64, 64), (8, 256, 8)]:
            if L.moe_choose_layout(T, k, E, El):
                assert El * T <= 4 * L.moe_compact_rows_bound(T * k, El, 128), (T, k, E, El)
                assert T * k <= 64 * E
    lib = L.lib()
    for bad in [(0, 8, 256, 256, 128), (8, 0, 256, 256, 128), (8, 8, 0, 1, 128), (8, 8, 256, 0, 128),
                (8, 8, 16, 32, 128), (8, 9, 8, 8, 128), (8, 8, 256, 256, 0)]:
        assert lib.moe_choose_layout(*bad) == -1, bad
    assert L.lib().moe_compact_rows_bound(-1, 8, 128) == -1
    assert L.lib().moe_compact_rows_bound(10, 0, 128) == -1


def test_status_strings():
    for s in range(5):
        assert L.status_str(s)
    assert L.status_str(99) == "unknown status"


def test_ws_bytes_grow_with_problem():
    a = L.moe_scatter_ws_bytes(64, 2, 8, 256)
    b = L.moe_scatter_ws_bytes(16384, 8, 128, 256)
    c = L.moe_scatter_ws_bytes(16384, 8, 128, 7168)
    assert 0 < a < b < c
    # at least the per-row assignment index (4 bytes per assignment) and the
    # staged scale bytes: one per token and 128 channels, each token's row
    # rounded up to whole 8-byte words (56 bytes at H=7168, 8 at H=256)
    assert c - b >= 16384 * (56 - 8)
    assert c >= 16384 * 56 + 16384 * 8 * 4
    assert b >= 16384 * 8 * 4
    assert L.lib().moe_scatter_ws_bytes(-1, 2, 8, 256) == 0
    assert L.lib().moe_scatter_ws_bytes(4, 2, 8, -128) == 0


def test_validation_rejects_before_launch():
    lib = L.lib()
    P = FAKE
    # routing
    assert lib.moe_route_topk(P, 4, 0, 2, P, P, None) == L.MOE_EINVAL          # E = 0
    assert lib.moe_route_topk(P, 4, 8, 9, P, P, None) == L.MOE_EINVAL          # k > E
    assert lib.moe_route_topk(P, 4, 2048, 8, P, P, None) == L.MOE_EINVAL       # E > 1024
    assert lib.moe_route_topk(None, 4, 8, 2, P, P, None) == L.MOE_EINVAL
    ws = L.moe_scatter_ws_bytes(64, 2, 8, 256)
    # compact scatter: capacity below the bound, H not a multiple of 128, block_e, ws too small
    bound = L.moe_compact_rows_bound(128, 8, 128)
    args = lambda T, H, El, be, R, dt, wsb: (P, T, H, P, 2, 0, El, be, R, dt, P, P, P, P, P, P, P, wsb, None)
    assert lib.moe_scatter_compact(*args(64, 256, 8, 128, bound - 1, 0, ws)) == L.MOE_ECAPACITY
    assert lib.moe_scatter_compact(*args(64, 200, 8, 128, bound, 0, ws)) == L.MOE_EUNSUPPORTED
    assert lib.moe_scatter_compact(*args(64, 256, 8, 64, bound, 0, ws)) == L.MOE_EUNSUPPORTED
    assert lib.moe_scatter_compact(*args(64, 256, 8, 128, bound, 0, ws - 1)) == L.MOE_ECAPACITY
    assert lib.moe_scatter_compact(*args(64, 256, 8, 128, bound, 7, ws)) == L.MOE_EUNSUPPORTED
    assert lib.moe_scatter_compact(*args(64, 256, 2000, 128, bound, 0, ws)) == L.MOE_EINVAL
    assert lib.moe_scatter_compact(P, 64, 256, P, 2, 0, 8, 128, bound, 1, P, None, P, P, P, P, P, ws,
                                   None) == L.MOE_EINVAL                       # FP8 without scales
    # masked scatter: max_m below T
    assert lib.moe_scatter_masked(P, 64, 256, P, 2, 0, 8, 63, 0, P, P, P, P, P, ws, None) == L.MOE_ECAPACITY
    assert lib.moe_scatter_masked(P, 64, 256, P, 2, 0, 8, 64, 0, P, P, None, P, P, ws, None) == L.MOE_EINVAL
    # quantisation
    assert lib.moe_quant_fp8_ue8m0(P, 4, 100, 100, None, P, P, None) == L.MOE_EUNSUPPORTED
    assert lib.moe_quant_fp8_ue8m0(P, 4, 128, 64, None, P, P, None) == L.MOE_EINVAL
    assert lib.moe_quant_weight_fp8_ue8m0(P, 2, 128, 96, P, P, None) == L.MOE_EUNSUPPORTED
    assert lib.moe_requant_weight_fp8_ue8m0(P, P, 2, 128, 96, P, P, None) == L.MOE_EUNSUPPORTED
    assert lib.moe_quant_weight_mx(P, 2, 96, 128, 0, P, P, None) == L.MOE_EUNSUPPORTED    # N % 64
    assert lib.moe_quant_weight_mx(P, 2, 128, 96, 0, P, P, None) == L.MOE_EUNSUPPORTED    # K % 128
    assert lib.moe_quant_weight_mx(P, 2, 128, 128, 2, P, P, None) == L.MOE_EUNSUPPORTED   # format
    assert lib.moe_quant_weight_mx(P, 2, 128, 128, 1, P, None, None) == L.MOE_EINVAL
    assert lib.moe_mx_scales_tile(P, 2, 128, 100, P, None) == L.MOE_EUNSUPPORTED
    assert lib.moe_mx_scales_tile(None, 2, 128, 128, P, None) == L.MOE_EINVAL
    assert lib.grouped_gemm_contig(2, P, None, P, P, P, P, 256, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(4, P, P, P, P, P, P, 256, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(3, P, None, P, P, P, P, 256, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.moe_requant_weight_fp8_ue8m0(P, P, -1, 128, 128, P, P, None) == L.MOE_EINVAL
    assert lib.moe_requant_weight_fp8_ue8m0(P, None, 2, 128, 128, P, P, None) == L.MOE_EINVAL
    assert lib.moe_requant_weight_fp8_ue8m0(None, None, 0, 128, 128, None, None, None) == L.MOE_OK
    # grouped GEMMs: dtype follows the weights -> FP8 without scales is an error
    assert lib.grouped_gemm_contig(1, P, None, P, P, P, P, 256, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(1, P, P, P, None, P, P, 256, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(0, P, None, P, None, P, P, 256, 200, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(0, P, None, P, None, P, P, 256, 256, 100, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(5, P, None, P, None, P, P, 256, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig(0, P, None, P, None, P, None, 256, 256, 256, 2, None) == L.MOE_EINVAL
    assert lib.grouped_gemm_contig(0, P, None, P, None, P, P, -1, 256, 256, 2, None) == L.MOE_EINVAL
    assert lib.grouped_gemm_masked(0, P, None, P, None, P, P, 8, 0, 256, 256, 2, None) == L.MOE_EINVAL
    assert lib.grouped_gemm_masked(1, P, None, P, P, P, P, 8, 64, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    # SiLU-and-mul and combine
    assert lib.silu_and_mul(P, 16, 100, None, None, 0, 0, P, None, None) == L.MOE_EUNSUPPORTED
    assert lib.silu_and_mul(P, 16, 128, None, None, 0, 1, P, None, None) == L.MOE_EINVAL
    assert lib.silu_and_mul(P, 16, 128, P, P, 8, 0, P, None, None) == L.MOE_EINVAL
    assert lib.silu_and_mul(P, 15, 128, None, P, 8, 0, P, None, None) == L.MOE_EINVAL
    assert lib.moe_combine(P, 10, P, P, 4, 33, 256, P, None) == L.MOE_EINVAL
    assert lib.moe_combine(P, 10, P, P, 4, 2, 100, P, None) == L.MOE_EUNSUPPORTED
    # the on-chip run table bounds the M-tiles of the compact tile order, and
    # tile positions are 32-bit
    assert lib.grouped_gemm_contig(0, P, None, P, None, P, P, 8177 * 128, 256, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_masked(0, P, None, P, None, P, P, 0, 1 << 30, 256, 256, 1024, None) == L.MOE_EUNSUPPORTED
    # w13 with SiLU-and-mul fused
    assert lib.grouped_gemm_contig_silu(0, P, None, P, None, 0, P, None, P, 256, 100, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig_silu(0, P, None, P, None, 7, P, None, P, 256, 128, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig_silu(0, P, None, P, None, 1, P, None, P, 256, 128, 256, 2, None) == L.MOE_EINVAL
    assert lib.grouped_gemm_contig_silu(1, P, None, P, P, 0, P, None, P, 256, 128, 256, 2, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_contig_silu(0, P, None, P, None, 0, P, None, None, 256, 128, 256, 2, None) == L.MOE_EINVAL
    assert lib.grouped_gemm_masked_silu(0, P, None, P, None, 0, P, None, P, 0, 64, 128, 256, 1025, None) == L.MOE_EUNSUPPORTED
    assert lib.grouped_gemm_masked_silu(0, P, None, P, None, 0, P, None, P, 0, 0, 128, 256, 2, None) == L.MOE_EINVAL
    # masked tile prefix is held on chip for at most 1024 groups
    assert lib.grouped_gemm_masked(0, P, None, P, None, P, P, 8, 64, 256, 256, 1025, None) == L.MOE_EUNSUPPORTED


def test_empty_calls_are_no_ops():
    """Zero-sized work returns OK without touching the device."""
    lib = L.lib()
    assert lib.moe_route_topk(None, 0, 8, 2, None, None, None) == L.MOE_OK
    assert lib.moe_quant_fp8_ue8m0(None, 0, 128, 128, None, None, None, None) == L.MOE_OK
    assert lib.grouped_gemm_contig(0, FAKE, None, FAKE, None, FAKE, None, 0, 256, 256, 2, None) == L.MOE_OK
    assert lib.grouped_gemm_contig_silu(0, FAKE, None, FAKE, None, 0, FAKE, None, None, 0, 128, 256, 2,
                                        None) == L.MOE_OK
    assert lib.moe_combine(None, 0, None, None, 0, 2, 256, None, None) == L.MOE_OK


def test_layer_layout_choice_on_host():
    """The layer's layout follows the measured policy ("auto"), the pages' rule
    ("rule") or the caller; deciding it needs no GPU (buffers on the host)."""
    from scatter_grouped_gemm_amd import MoELayer

    def layer(T, E, El, layout, **kw):
        return MoELayer(hidden=128, intermediate=128, num_experts=E, top_k=2, max_tokens=T,
                        num_local_experts=El, layout=layout, device="cpu", **kw)

    assert layer(256, 256, 32, "auto").layout == "masked"
    assert layer(4096, 256, 32, "auto").layout == "compact"
    assert layer(256, 8, 8, "auto").layout == "masked"          # measured: small batch
    assert layer(256, 8, 8, "rule").layout == "compact"          # pages: all experts local
    assert layer(4096, 256, 32, "rule").layout == "masked"
    assert layer(64, 16, 16, "compact").layout == "compact"
    with pytest.raises(ValueError):
        layer(64, 16, 16, "diagonal")
    with pytest.raises(ValueError):
        layer(64, 16, 16, "auto", fp8=False, weight_format="mxfp8")   # MX needs the FP8 path
    with pytest.raises(ValueError):
        layer(64, 16, 16, "auto", fp8=True, weight_format="nvfp4")


def test_noalloc_scatter_validates_before_device_work():
    """moe_scatter_compact_noalloc rejects bad arguments and scratch needs above
    its static limit on the host, before it looks up its scratch or launches."""
    lib = L.lib()
    P = FAKE
    bound = L.moe_compact_rows_bound(128, 8, 128)
    args = lambda T, H, k, El, be, R: (P, T, H, P, k, 0, El, be, R, 0, P, P, P, P, P, P, None)
    assert lib.moe_scatter_compact_noalloc(*args(64, 256, 2, 8, 64, bound)) == L.MOE_EUNSUPPORTED
    assert lib.moe_scatter_compact_noalloc(*args(64, 200, 2, 8, 128, bound)) == L.MOE_EUNSUPPORTED
    assert lib.moe_scatter_compact_noalloc(*args(64, 256, 2, 8, 128, bound - 1)) == L.MOE_ECAPACITY
    assert lib.moe_scatter_compact_noalloc(*args(64, 256, 2, 0, 128, bound)) == L.MOE_EINVAL
    # 2^23 assignments over 256 experts need more than the 4 MiB static scratch
    T, k, El = 1 << 20, 8, 256
    assert L.moe_scatter_ws_bytes(T, k, El, 128) > L.MOE_SCATTER_NOALLOC_MAX_BYTES
    R = L.moe_compact_rows_bound(T * k, El, 128)
    assert lib.moe_scatter_compact_noalloc(*args(T, 128, k, El, 128, R)) == L.MOE_ECAPACITY
    # the limit the header states
    hdr = open(os.path.join(ROOT, "include", "moe.h")).read()
    assert "#define MOE_SCATTER_NOALLOC_MAX_BYTES (4u << 20)" in hdr
    assert L.MOE_SCATTER_NOALLOC_MAX_BYTES == 4 << 20


def _rows_exec_reference(masked, counts, expected_m, N, wreg):
    """The tile rules written out: masked tiles of 16/32/64/128 rows chosen by
    the hint (16 and 32 only when N % 256 == 0); compact, the register-streamed
    kernel's ceil(z/256) equal tiles rounded up to 16 rows, each running whole
    16-row blocks, else 128-row tiles."""
    total = 0
    for z in counts:
        if masked:
            if 0 < expected_m <= 16 and N % 256 == 0:
                bm = 16
            elif 0 < expected_m <= 32 and N % 256 == 0:
                bm = 32
            elif 0 < expected_m <= 64:
                bm = 64
            else:
                bm = 128
            total += -(-z // bm) * bm
        elif z > 0 and wreg:
            nt = -(-z // 256)
            h = -(-(-(-z // nt)) // 16) * 16
            for t in range(nt):
                r = min(h, z - t * h)
                if r > 0:
                    total += -(-r // 16) * 16
        elif z > 0:
            total += -(-z // 128) * 128
    return total


def test_grouped_gemm_rows_executed_follows_the_tile_rules():
    rng = np.random.default_rng(3)
    for counts in ([0, 1, 15, 16, 17, 255, 256, 257, 511, 512, 513, 1000, 4097],
                   rng.integers(0, 700, 50).tolist()):
        M = sum(-(-c // 128) * 128 for c in counts) + 128
        for em in (0, 8, 16, 24, 32, 50, 64, 65):
            for N in (256, 384, 4096):
                assert L.grouped_gemm_rows_executed(True, True, counts, em, M, N, 512) == \
                    _rows_exec_reference(True, counts, em, N, False), (em, N)
        for fp8 in (False, True, "mxfp8"):
            for N in (256, 384, 4096):
                wreg = fp8 in (False, True) and N % 256 == 0
                assert L.grouped_gemm_rows_executed(fp8, False, counts, 0, M, N, 512) == \
                    _rows_exec_reference(False, counts, 0, N, wreg), (fp8, N)
    # one expert of 257 rows: two tiles of 144 and 113 rows -> 144 + 128
    assert L.grouped_gemm_rows_executed(True, False, [257], 0, 384, 4096, 7168) == 272
    with pytest.raises(ValueError):
        L.grouped_gemm_rows_executed(True, False, [-1], 0, 128, 256, 256)
