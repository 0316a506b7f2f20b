"""Per-kernel parity of the HIP path (through the C ABI) against the CPU oracle.

Bit-exact: routing ids, m_indices (every row), expert_start_loc, num_valid,
masked_m, src2dst, scattered rows, e4m3 codes and UE8M0 scale bytes, combine
(identical inputs).  Tolerance: GEMMs (accumulation order) and SiLU (GPU fp32
exp vs the oracle's fp64), stated in each test.  Inputs are seeded and drawn on
the host, so the oracle and the GPU see the same values; no expected value
comes from the GPU.
"""
import numpy as np
import pytest
import torch

from scatter_grouped_gemm_amd import _lib as L
from scatter_grouped_gemm_amd import inputs
from gpu_util import (DEV, announce, bits, bf16_ulp, compact_layout, distinct_ids, e4m3_table, f32,
                      i32_dev, poison, rel_fro, to_dev_bf16, u8_dev)

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------------------
# routing
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("T,E,k,seed", [(64, 8, 2, 0), (4096, 8, 2, 1), (1000, 256, 8, 2),
                                        (333, 128, 8, 3), (1, 5, 5, 4), (0, 8, 2, 5),
                                        (77, 1024, 32, 6), (500, 256, 1, 7)])
def test_route_topk(orc, T, E, k, seed):
    announce("route", T, E, k, seed)
    g = torch.Generator().manual_seed(seed)
    logits = torch.randn(T, E, generator=g)
    if T > 3 and E > 5:
        logits[::3, 5] = logits[::3, 2]                 # exact ties
        logits[1, :] = 0.25                             # a fully tied row
    ids_ref, w_ref = orc.route_topk(logits.numpy(), k)
    ids = poison((T, k), torch.int32)
    w = poison((T, k), torch.float32)
    L.moe_route_topk(logits.to(DEV), k, ids, w)
    torch.cuda.synchronize()
    assert np.array_equal(ids.cpu().numpy(), ids_ref)
    # fp32 exp/sum/divide on the GPU against the oracle's fp64: <= 8 fp32 ulp
    np.testing.assert_allclose(w.cpu().numpy(), w_ref, rtol=1e-6, atol=0)


# ---------------------------------------------------------------------------
# scatter
# ---------------------------------------------------------------------------

SCATTER_CASES = [
    # T, H, E, El, expert_start, k, fp8
    (64, 256, 8, 8, 0, 2, False),
    (64, 256, 8, 8, 0, 2, True),
    (300, 384, 64, 20, 24, 6, True),
    (1, 128, 8, 8, 0, 2, True),
    (0, 256, 8, 8, 0, 2, False),
    (2000, 128, 128, 128, 0, 8, False),
    (1500, 7168, 256, 256, 0, 8, True),
    (257, 4096, 128, 128, 0, 8, False),
    # more than 16384 assignments: the chunked count / scan / rank kernels.
    # The scan runs one wavefront per expert over ceil(El / 4) workgroups, the
    # last of them scanning the expert sizes: El not a multiple of 4, the
    # 1024-expert maximum (256 workgroups), a single workgroup, uneven chunk
    # runs per lane, and more than 512 chunks (runs longer than the 8 kept in
    # registers take a second pass)
    (2500, 128, 300, 300, 0, 8, True),
    (4100, 256, 1000, 700, 300, 4, False),
    (6000, 128, 3, 3, 0, 3, False),
    (2200, 128, 1024, 1024, 0, 8, False),
    (20000, 128, 64, 16, 8, 8, True),
]


def _scatter_inputs(T, H, E, k, seed):
    rng = np.random.default_rng(seed)
    ids = distinct_ids(rng, T, E, k)
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16)
    return ids, x


@pytest.mark.parametrize("T,H,E,El,start,k,fp8", SCATTER_CASES)
def test_scatter_compact(orc, T, H, E, El, start, k, fp8):
    announce("scatter_compact", T, H, E, El, start, k, fp8)
    ids, x = _scatter_inputs(T, H, E, k, T + H)
    R = L.moe_compact_rows_bound(T * k, El, 128)
    ref = orc.scatter_compact(bits(x), ids, start, El, 128, R, fp8)
    adt = torch.uint8 if fp8 else torch.bfloat16
    x_out = poison((R, H), adt)
    s_out = poison((H // 128, R), torch.uint8) if fp8 else None
    m_idx = poison((R,), torch.int32)
    st = poison((El,), torch.int32)
    nv = poison((El,), torch.int32)
    s2d = poison((T, k), torch.int32)
    ws = torch.empty(L.moe_scatter_ws_bytes(T, k, El, H), dtype=torch.uint8, device=DEV)
    L.moe_scatter_compact(x.to(DEV), i32_dev(ids), start, El, 128, R, fp8, x_out, s_out, m_idx, st,
                          nv, s2d, ws)
    torch.cuda.synchronize()
    m = m_idx.cpu().numpy()
    assert np.array_equal(m, ref["m_indices"])
    assert np.array_equal(st.cpu().numpy(), ref["expert_start_loc"])
    assert np.array_equal(nv.cpu().numpy(), ref["num_valid"])
    assert np.array_equal(s2d.cpu().numpy(), ref["src2dst"])
    valid = m >= 0
    if fp8:
        assert np.array_equal(x_out.cpu().numpy()[valid], ref["x_out"][valid])
        assert np.array_equal(s_out.cpu().numpy().T[valid], ref["scale_out"][valid])
    else:
        assert np.array_equal(bits(x_out)[valid], ref["x_out"][valid])
    assert L.moe_get_device_error(ws) == 0


@pytest.mark.parametrize("T,H,E,El,start,k,fp8", [c for c in SCATTER_CASES if c[3] <= 128])
def test_scatter_masked(orc, T, H, E, El, start, k, fp8):
    announce("scatter_masked", T, H, E, El, start, k, fp8)
    ids, x = _scatter_inputs(T, H, E, k, T + 2 * H)
    max_m = max(T, 1)
    ref = orc.scatter_masked(bits(x), ids, start, El, max_m, fp8)
    adt = torch.uint8 if fp8 else torch.bfloat16
    rows = El * max_m
    x_out = poison((rows, H), adt)
    s_out = poison((El, H // 128, max_m), torch.uint8) if fp8 else None
    mm = poison((El,), torch.int32)
    s2d = poison((T, k), torch.int32)
    ws = torch.empty(L.moe_scatter_ws_bytes(T, k, El, H), dtype=torch.uint8, device=DEV)
    L.moe_scatter_masked(x.to(DEV), i32_dev(ids), start, El, max_m, fp8, x_out, s_out, mm, s2d, ws)
    torch.cuda.synchronize()
    assert np.array_equal(mm.cpu().numpy(), ref["masked_m"])
    assert np.array_equal(s2d.cpu().numpy(), ref["src2dst"])
    valid = orc.masked_row_group(ref["masked_m"], max_m) >= 0
    if fp8:
        assert np.array_equal(x_out.cpu().numpy()[valid], ref["x_out"][valid])
        sc = s_out.cpu().numpy().transpose(0, 2, 1).reshape(rows, H // 128)
        assert np.array_equal(sc[valid], ref["scale_out"][valid])
    else:
        assert np.array_equal(bits(x_out)[valid], ref["x_out"][valid])
    assert L.moe_get_device_error(ws) == 0


def test_scatter_masked_overflow_flag(orc):
    """Repeated ids in one token can push an expert past max_m = T: the device
    error word says so and the overflowing assignments are dropped."""
    announce("scatter_masked_overflow")
    T, H, k, El = 4, 128, 3, 4
    ids = np.array([[1, 1, 1], [1, 2, 3], [1, 0, 2], [1, 1, 0]], np.int32)
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    ws = torch.empty(L.moe_scatter_ws_bytes(T, k, El, H), dtype=torch.uint8, device=DEV)
    s2d = poison((T, k), torch.int32)
    mm = poison((El,), torch.int32)
    L.moe_scatter_masked(x.to(DEV), i32_dev(ids), 0, El, T, False, poison((El * T, H), torch.bfloat16),
                         None, mm, s2d, ws)
    assert L.moe_get_device_error(ws) == L.MOE_DEVERR_MASKED_OVERFLOW
    s = s2d.cpu().numpy()
    ones = s[ids == 1]
    assert (ones >= 0).sum() == T and np.all(np.sort(ones[ones >= 0]) == np.arange(T) + T)
    assert mm.cpu().numpy()[1] == T
    # a clean call afterwards clears the word
    ids2 = np.array([[0, 1, 2], [1, 2, 3], [3, 0, 2], [1, 2, 0]], np.int32)
    L.moe_scatter_masked(x.to(DEV), i32_dev(ids2), 0, El, T, False, poison((El * T, H), torch.bfloat16),
                         None, mm, s2d, ws)
    assert L.moe_get_device_error(ws) == 0


# ---------------------------------------------------------------------------
# quantisation
# ---------------------------------------------------------------------------

def test_quant_rows_exhaustive_bf16(orc):
    """Every finite bf16 pattern passes through the activation quantiser, in
    groups whose maxima span the whole exponent range (including zero,
    subnormal and huge groups), bit-exact against the oracle."""
    announce("quant_rows_exhaustive")
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]
    rng = np.random.default_rng(0)
    b = rng.permutation(b)
    pad = (-len(b)) % 384
    b = np.concatenate([b, np.zeros(pad, np.uint16)]).reshape(-1, 384)
    b[0, :128] = 0                                     # all-zero group
    b[1, :128] = 0x0001                                # subnormal-only group
    b[2, :128] = 0x8000                                # negative zeros
    x = to_dev_bf16(b)
    M, K = b.shape
    q_ref, s_ref = orc.quant_rows(b)
    q = poison((M, K), torch.uint8)
    s = poison((K // 128, M), torch.uint8)
    L.moe_quant_fp8_ue8m0(x, q, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().T, s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_quant_rows_skips_padding_and_honours_ld(orc):
    announce("quant_rows_skip")
    g = torch.Generator().manual_seed(3)
    xfull = torch.randn(200, 640, generator=g).to(torch.bfloat16)
    x = xfull.to(DEV)[:, :512]                          # ld 640, K 512
    m_idx = np.where(np.arange(200) % 5 == 3, -1, 1).astype(np.int32)
    q = poison((200, 512), torch.uint8)
    s = poison((4, 200), torch.uint8)
    L.moe_quant_fp8_ue8m0(x, q, s, m_indices=i32_dev(m_idx))
    torch.cuda.synchronize()
    q_ref, s_ref = orc.quant_rows(bits(xfull[:, :512]))
    v = m_idx >= 0
    assert np.array_equal(q.cpu().numpy()[v], q_ref[v])
    assert np.array_equal(s.cpu().numpy().T[v], s_ref[v])
    assert np.all(q.cpu().numpy()[~v] == 0xFF) and np.all(s.cpu().numpy().T[~v] == 0xFF)


def test_quant_weight_blocks(orc):
    announce("quant_weight_blocks")
    g = torch.Generator().manual_seed(4)
    w = (torch.randn(3, 256, 384, generator=g) * 0.02).to(torch.bfloat16)
    w[1, :128, 128:256] *= 3000
    w[2, 128:, :128] = 0
    q_ref, s_ref = orc.quant_weight_blocks(bits(w))
    q = poison((3, 256, 384), torch.uint8)
    s = poison((3, 2, 3), torch.uint8)
    L.moe_quant_weight_fp8_ue8m0(w.to(DEV), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def _requant_inputs():
    q, s = inputs.block_fp8_checkpoint(3, 256, 384, seed=11)
    q[1, :128, :128] = 0                      # zero block (both signs of zero)
    q[1, :64, :128] = 0x80
    q[1, 128:, 128:256] &= 0x87               # subnormal codes only
    q[2, :128, 256:] = 0x7e                   # every element at the e4m3 maximum
    s[1, 0, 2] = 2.0 ** 100                   # bf16 near its top of range
    s[2, 1, 0] = 2.0 ** -126                  # products in the fp32 subnormal range
    s[2, 1, 1] = 1.0
    return q, s


def test_requant_weight_blocks(orc):
    announce("requant_weight_fp8_ue8m0")
    q_in, s_in = _requant_inputs()
    q_ref, s_ref = orc.requant_weight_blocks(q_in.numpy(), s_in.numpy())
    q = poison((3, 256, 384), torch.uint8)
    s = poison((3, 2, 3), torch.uint8)
    L.moe_requant_weight_fp8_ue8m0(q_in.to(DEV), s_in.to(DEV), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_requant_weight_blocks_in_place(orc):
    announce("requant_weight_fp8_ue8m0 in place")
    q_in, s_in = _requant_inputs()
    q_ref, s_ref = orc.requant_weight_blocks(q_in.numpy(), s_in.numpy())
    q = q_in.to(DEV)
    s = poison((3, 2, 3), torch.uint8)
    L.moe_requant_weight_fp8_ue8m0(q, s_in.to(DEV), q, s)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy(), s_ref)
    assert np.array_equal(q.cpu().numpy(), q_ref)


def test_requant_then_gemm_matches_dequantised_weights(orc):
    """The requantised weights drive the FP8 GEMM like weights quantised from
    their bf16 dequantisation (the two give identical codes and scales)."""
    announce("requant_weight_fp8_ue8m0 vs quant_weight of the dequantised bf16")
    q_in, s_in = inputs.block_fp8_checkpoint(2, 256, 512, seed=12)
    deq = (q_in.view(torch.float8_e4m3fn).float()
           * s_in.repeat_interleave(128, 1).repeat_interleave(128, 2)).to(torch.bfloat16)
    q1, s1 = poison((2, 256, 512), torch.uint8), poison((2, 2, 4), torch.uint8)
    q2, s2 = poison((2, 256, 512), torch.uint8), poison((2, 2, 4), torch.uint8)
    L.moe_requant_weight_fp8_ue8m0(q_in.to(DEV), s_in.to(DEV), q1, s1)
    L.moe_quant_weight_fp8_ue8m0(deq.to(DEV), q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1, s2)


def _mx_tile(s_plain: np.ndarray) -> np.ndarray:
    """Plain MX scales [G,N,K/32] in the GEMM's tiled order
    [G][N/64][K/128][kq][r16][j16] (row 64*b + 16*j16 + r16, k block 4*s + kq)."""
    G, N, KB = s_plain.shape
    t = s_plain.reshape(G, N // 64, 4, 16, KB // 4, 4)          # g, b, j16, r16, s, kq
    return np.ascontiguousarray(t.transpose(0, 1, 4, 5, 3, 2)).reshape(-1)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_quant_weight_mx(orc, fmt):
    announce("quant_weight_mx", fmt)
    g = torch.Generator().manual_seed(8)
    G, N, K = 3, 192, 384
    w = torch.randn(G, N, K, generator=g) * torch.exp2(
        torch.randint(-10, 8, (G, N, K // 32), generator=g).float()).repeat_interleave(32, 2)
    w[1, 5, 64:96] = 0
    w[2, 70, :32] = 6.0 * 2.0 ** -3                  # exactly the e2m1 maximum at a power of two
    w = w.to(torch.bfloat16)
    q_ref, s_ref = orc.quant_weight_mx(bits(w), fmt)
    q = poison(q_ref.shape, torch.uint8)
    st = poison((G * N * K // 32,), torch.uint8)
    L.moe_quant_weight_mx(w.to(DEV), "e4m3" if fmt == "mxfp8" else "e2m1", q, st)
    st2 = poison((G * N * K // 32,), torch.uint8)
    L.moe_mx_scales_tile(torch.from_numpy(s_ref).to(DEV), st2)
    torch.cuda.synchronize()
    assert np.array_equal(q.cpu().numpy(), q_ref)
    assert np.array_equal(st.cpu().numpy(), _mx_tile(s_ref))
    assert np.array_equal(st2.cpu().numpy(), _mx_tile(s_ref))


def _mx_operands(orc, M_counts, N, K, seed, integer_valued=False, fmt="mxfp8"):
    """FP8 activations (128-channel scales) and MX weights (e4m3 or e2m1)."""
    G = len(M_counts)
    m_idx = compact_layout(M_counts)
    M = len(m_idx)
    g = torch.Generator().manual_seed(seed)
    if integer_valued:
        qa = torch.randint(-4, 5, (M, K), generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        if fmt == "mxfp8":
            qb = torch.randint(-4, 5, (G, N, K), generator=g).float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        else:                                                       # every e2m1 code pair
            qb = torch.randint(0, 256, (G, N, K // 2), generator=g).to(torch.uint8).numpy()
        rng = np.random.default_rng(seed)
        # exponents within +-1 keep every partial sum exact in fp32
        sa = rng.integers(126, 129, (M, K // 128)).astype(np.uint8)
        sb = rng.integers(126, 129, (G, N, K // 32)).astype(np.uint8)
    else:
        A = torch.randn(M, K, generator=g).to(torch.bfloat16)
        B = (torch.randn(G, N, K, generator=g) * 0.02).to(torch.bfloat16)
        qa, sa = orc.quant_rows(bits(A))
        qb, sb = orc.quant_weight_mx(bits(B), fmt)
    return dict(m_idx=m_idx, A=qa, As=sa, B=qb, Bs=sb)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("integer_valued", [False, True])
@pytest.mark.parametrize("counts,N,K", [([130, 0, 5, 256, 1, 300], 256, 384), ([64, 129], 384, 512)])
def test_gemm_mx_contig(orc, counts, N, K, integer_valued, fmt):
    """FP8 activations times MX weights (one exponent per 32 k; e4m3, or e2m1
    two per byte): the per-lane scale of the block-scaled MFMA; exact on
    integer-valued codes."""
    announce("gemm_mx_contig", fmt, counts, N, K, integer_valued)
    ops = _mx_operands(orc, counts, N, K, seed=N + K, integer_valued=integer_valued, fmt=fmt)
    ref = orc.gemm_mx_rows(ops["A"], ops["As"], ops["B"], ops["Bs"], fmt, ops["m_idx"])
    M = len(ops["m_idx"])
    C = poison((M, N), torch.bfloat16)
    L.grouped_gemm_contig(fmt, u8_dev(ops["A"]), u8_dev(ops["As"].T.copy()), u8_dev(ops["B"]),
                          u8_dev(_mx_tile(ops["Bs"])), C, i32_dev(ops["m_idx"]))
    torch.cuda.synchronize()
    got = bits(C)
    valid = ops["m_idx"] >= 0
    if integer_valued:
        assert np.array_equal(got[valid], ref[valid])
    else:
        _check_close(got, ref, valid, 2e-2, True)


def _masked_tile_rows(fp8, expected_m, N, K, max_m):
    """The masked kernels' tile height for this hint, from the library (one
    valid row executes one whole tile)."""
    return L.grouped_gemm_rows_executed(fp8, True, [1], expected_m, max_m, N, K)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("expected_m", [0, 8, 24, 50])
def test_gemm_mx_masked(orc, expected_m, fmt):
    """MX weights, masked layout, every tile height (128, 16, 32, 64 rows),
    two N-tiles: bit-exact against the oracle, rows past each group's last
    tile untouched."""
    announce("gemm_mx_masked", fmt, expected_m)
    G, max_m, N, K = 5, 200, 512, 384
    masked = np.array([0, 1, 200, 37, 130], np.int32)
    ops = _mx_operands(orc, [max_m] * G, N, K, seed=31, integer_valued=True, fmt=fmt)
    rg = orc.masked_row_group(masked, max_m)
    A = ops["A"][: G * max_m]
    As = ops["As"][: G * max_m]
    ref = orc.gemm_mx_rows(A, As, ops["B"], ops["Bs"], fmt, rg)
    C = poison((G, max_m, N), torch.bfloat16)
    As_dev = As.reshape(G, max_m, K // 128).transpose(0, 2, 1).copy()
    L.grouped_gemm_masked(fmt, u8_dev(A).view(G, max_m, K), u8_dev(As_dev), u8_dev(ops["B"]),
                          u8_dev(_mx_tile(ops["Bs"])), C, i32_dev(masked), expected_m)
    torch.cuda.synchronize()
    got = bits(C).reshape(G * max_m, N)
    valid = rg >= 0
    assert np.array_equal(got[valid], ref[valid])
    bm = _masked_tile_rows(fmt, expected_m, N, K, max_m)
    assert bm == {0: 128, 8: 16, 24: 32, 50: 64}[expected_m]
    assert np.all(got[_skipped_rows_masked(masked, max_m, bm)] == 0xFFFF)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("out_fp8", [False, True])
def test_gemm_mx_silu_fused_matches_separate(orc, out_fp8, fmt):
    """MX weights through the fused w13 + SiLU-and-mul epilogue (gate and up
    scale slots) equal the plain MX GEMM followed by silu_and_mul, bit for bit."""
    announce("gemm_mx_silu", fmt, out_fp8)
    I, K = 256, 384
    ops = _mx_operands(orc, [130, 0, 5, 256, 1, 300], 2 * I, K, seed=41, fmt=fmt)
    M = len(ops["m_idx"])
    m_dev = i32_dev(ops["m_idx"])
    A, As, B, Bs = u8_dev(ops["A"]), u8_dev(ops["As"].T.copy()), u8_dev(ops["B"]), u8_dev(_mx_tile(ops["Bs"]))
    gu = poison((M, 2 * I), torch.bfloat16)
    L.grouped_gemm_contig(fmt, A, As, B, Bs, gu, m_dev)
    odt = torch.uint8 if out_fp8 else torch.bfloat16
    sep, fus = poison((M, I), odt), poison((M, I), odt)
    ss = poison((I // 128, M), torch.uint8) if out_fp8 else None
    fs = poison((I // 128, M), torch.uint8) if out_fp8 else None
    L.silu_and_mul(gu, sep, out_fp8, ss, m_indices=m_dev)
    L.grouped_gemm_contig_silu(fmt, A, As, B, Bs, fus, m_dev, fs)
    torch.cuda.synchronize()
    valid = ops["m_idx"] >= 0
    assert np.array_equal(fus.view(torch.uint8).cpu().numpy()[valid], sep.view(torch.uint8).cpu().numpy()[valid])
    if out_fp8:
        assert np.array_equal(fs.cpu().numpy()[:, valid], ss.cpu().numpy()[:, valid])
    h1 = orc.gemm_mx_rows(ops["A"], ops["As"], ops["B"], ops["Bs"], fmt, ops["m_idx"])
    _check_close(bits(gu), h1, valid, 2e-2, True)


# ---------------------------------------------------------------------------
# grouped GEMMs
# ---------------------------------------------------------------------------

def _gemm_operands(orc, fp8, M_counts, N, K, seed, integer_valued=False, block_e=128, extra_rows=128,
                   scale_ranges=((125, 130), (124, 129))):
    G = len(M_counts)
    m_idx = compact_layout(M_counts, block_e, extra_rows)
    M = len(m_idx)
    g = torch.Generator().manual_seed(seed)
    if integer_valued:
        A = torch.randint(-4, 5, (M, K), generator=g).to(torch.bfloat16)
        B = torch.randint(-3, 4, (G, N, K), generator=g).to(torch.bfloat16)
    else:
        A = torch.randn(M, K, generator=g).to(torch.bfloat16)
        B = (torch.randn(G, N, K, generator=g) * 0.02).to(torch.bfloat16)
    if not fp8:
        return dict(m_idx=m_idx, A=bits(A), B=bits(B))
    if integer_valued:
        # small integers are exact e4m3 codes; unit and power-of-two scales
        qa = A.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        qb = B.float().to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        rng = np.random.default_rng(seed)
        (a0, a1), (b0, b1) = scale_ranges
        sa = rng.integers(a0, a1, (M, K // 128)).astype(np.uint8)
        sb = rng.integers(b0, b1, (G, N // 128, K // 128)).astype(np.uint8)
        return dict(m_idx=m_idx, A=qa, As=sa, B=qb, Bs=sb)
    qa, sa = orc.quant_rows(bits(A))
    qb, sb = orc.quant_weight_blocks(bits(B))
    return dict(m_idx=m_idx, A=qa, As=sa, B=qb, Bs=sb)


def _ref_gemm(orc, fp8, ops):
    if fp8:
        return orc.gemm_fp8_rows(ops["A"], ops["As"], ops["B"], ops["Bs"], ops["m_idx"])
    return orc.gemm_bf16_rows(ops["A"], ops["B"], ops["m_idx"])


def _run_contig(fp8, ops, N):
    M = len(ops["m_idx"])
    C = poison((M, N), torch.bfloat16)
    if fp8:
        L.grouped_gemm_contig(True, u8_dev(ops["A"]), u8_dev(ops["As"].T.copy()), u8_dev(ops["B"]),
                              u8_dev(ops["Bs"]), C, i32_dev(ops["m_idx"]))
    else:
        L.grouped_gemm_contig(False, to_dev_bf16(ops["A"]), None, to_dev_bf16(ops["B"]), None, C,
                              i32_dev(ops["m_idx"]))
    torch.cuda.synchronize()
    return bits(C)


def _skipped_rows_contig(m_idx, bm=128):
    """Rows of M-tiles whose first row is padding: the GEMM never touches
    them (rows of computed tiles past an expert's valid rows may be written)."""
    first = m_idx[(np.arange(len(m_idx)) // bm) * bm]
    return first < 0


def _skipped_rows_masked(masked, max_m, bm=128):
    """Masked rows at or past masked_m rounded up to bm: never touched."""
    r = np.arange(max_m)
    lim = -(-np.clip(masked, 0, max_m) // bm) * bm
    return (r[None, :] >= lim[:, None]).reshape(-1)


def _check_close(got_bits, ref_bits, valid, tol_rel, fp8=False):
    g = f32(got_bits[valid]).astype(np.float64)
    r = f32(ref_bits[valid]).astype(np.float64)
    assert np.all(np.isfinite(g))
    # BF16: accumulation order only -> within one bf16 ulp of the reference
    # element plus a few fp32 ulp of the row's scale (cancellation).  FP8: the
    # block-scaled MFMA sums e4m3 products internally with less than fp32
    # sequential precision, so the row-scale slack is 2e-4.  Both: relative
    # Frobenius error within tol_rel.
    slack = bf16_ulp(r) + (2e-4 if fp8 else 1e-5) * np.abs(r).max(axis=-1, keepdims=True)
    assert np.all(np.abs(g - r) <= slack), float(np.max(np.abs(g - r) - slack))
    assert rel_fro(g, r) <= tol_rel


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("counts,N,K", [
    ([130, 0, 5, 256, 1, 300], 256, 256),
    ([64, 129], 384, 512),
    ([1000, 17, 0, 0, 333], 512, 1024),
    ([0, 0, 1], 128, 128),
    ([9000, 3, 0, 8300], 128, 128),   # runs of more than 64 M-tiles
])
def test_gemm_contig(orc, fp8, counts, N, K):
    announce("gemm_contig", fp8, counts, N, K)
    ops = _gemm_operands(orc, fp8, counts, N, K, seed=N + K)
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, N)
    valid = ops["m_idx"] >= 0
    _check_close(got, ref, valid, 5e-3 if not fp8 else 2e-2, fp8)
    assert np.all(got[_skipped_rows_contig(ops["m_idx"])] == 0xFFFF)  # padding tiles untouched


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_contig_all_padding(orc, fp8):
    """No expert has a token: every row is padding, each workgroup finds an
    empty tile order and leaves at once, and the output is untouched."""
    announce("gemm_contig_all_padding", fp8)
    ops = _gemm_operands(orc, fp8, [0, 0, 0], 256, 256, seed=11)
    assert len(ops["m_idx"]) > 0 and np.all(ops["m_idx"] < 0)
    got = _run_contig(fp8, ops, 256)
    assert np.all(got == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_contig_wide_padding(orc, fp8):
    """Experts padded to 384 rows leave whole M-tiles of padding between
    experts and 1000 trailing padding rows: those tiles are skipped, every
    valid row is computed once, integer-valued operands make it exact."""
    announce("gemm_contig_wide_padding", fp8)
    ops = _gemm_operands(orc, fp8, [1, 300, 0, 129, 700, 2], 256, 256, seed=5, integer_valued=True,
                         block_e=384, extra_rows=1000)
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, 256)
    valid = ops["m_idx"] >= 0
    assert np.array_equal(got[valid], ref[valid])
    skipped = _skipped_rows_contig(ops["m_idx"])
    assert skipped.sum() >= 1000 + 2 * 128             # the trailing rows and whole padding tiles
    assert np.all(got[skipped] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_contig_blocks_padded_inside_a_run(orc, fp8):
    """The layout contract only asks each 128-row block to hold one expert with
    its valid rows first: an expert may pad a block and continue in the next
    one, and the same expert may reappear later.  Every valid row is computed
    (rows of a run's last block past its tokens are skipped)."""
    announce("gemm_contig_padded_runs", fp8)
    N, K = 256, 256
    ops = _gemm_operands(orc, fp8, [384, 384, 384], N, K, seed=29, integer_valued=True, extra_rows=128)
    m = np.full(len(ops["m_idx"]), -1, np.int32)
    m[0:100] = 0        # expert 0: a padded block ...
    m[128:256] = 0      # ... then a full one in the same run
    m[256:300] = 0      # ... and a short last block
    m[384:512] = 1      # expert 1: one full block
    m[640:650] = 0      # expert 0 again, later
    m[768:770] = 2      # expert 2: 2 rows; a block of padding follows
    ops["m_idx"] = m
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, N)
    valid = m >= 0
    assert np.array_equal(got[valid], ref[valid])
    assert np.all(got[_skipped_rows_contig(m)] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_contig_thousands_of_short_runs(orc, fp8):
    """3000 experts of 1..3 rows: every run is one tile, and the 3001 M-tiles
    spread over the eight XCD shares' run tables."""
    announce("gemm_contig_short_runs", fp8)
    rng = np.random.default_rng(7)
    counts = rng.integers(1, 4, 3000).tolist()
    N, K = 128, 256
    ops = _gemm_operands(orc, fp8, counts, N, K, seed=31, integer_valued=True)
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, N)
    valid = ops["m_idx"] >= 0
    assert np.array_equal(got[valid], ref[valid])


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_contig_integer_exact(orc, fp8):
    """Integer-valued operands make every partial sum exact, so the GPU must
    reproduce the oracle bit for bit whatever its accumulation order; a
    transposed operand, a wrong scale byte or a misplaced output fails here."""
    announce("gemm_contig_exact", fp8)
    ops = _gemm_operands(orc, fp8, [200, 77, 0, 128], 384, 640, seed=9, integer_valued=True)
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, 384)
    valid = ops["m_idx"] >= 0
    assert np.array_equal(got[valid], ref[valid])


def _many_tiles_layout(seed, nblocks=400, G=16):
    """m_indices of `nblocks` 128-row blocks cycling over G experts, each with
    1..24 valid rows, and every 40th run three blocks long: with 256
    persistent workgroups each one processes three or more tiles, so every
    tile after a workgroup's first starts from accumulators cleared by the
    previous tile's epilogue."""
    rng = np.random.default_rng(seed)
    m, j = [], 0
    while j < nblocks:
        e = j % G
        if j % 40 == 39:
            c = 256 + int(rng.integers(1, 129))
            nb = 3
        else:
            c = int(rng.integers(1, 25))
            nb = 1
        m += [e] * c + [-1] * (nb * 128 - c)
        j += nb
    m += [-1] * 128
    return np.array(m, np.int32)


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_contig_many_tiles_per_workgroup(orc, fp8):
    """Several tiles per workgroup (the full-size case) with a k loop whose
    length is not a multiple of the kernel's stage count: integer-valued
    operands, bit-exact against the oracle on every valid row."""
    announce("gemm_contig_many_tiles", fp8)
    N, K = 512, 384
    m = _many_tiles_layout(41)
    G = 16
    ops = _gemm_operands(orc, fp8, [1] * G, N, K, seed=43, integer_valued=True, extra_rows=len(m) - 128 * G)
    ops["m_idx"] = m
    assert len(ops["A"]) == len(m)
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, N)
    valid = m >= 0
    assert np.array_equal(got[valid], ref[valid])
    assert np.all(got[_skipped_rows_contig(m)] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("out_fp8", [False, True])
def test_gemm_silu_fused_many_tiles_per_workgroup(orc, fp8, out_fp8):
    """The fused SiLU epilogue with several tiles per workgroup equals the
    plain GEMM followed by silu_and_mul bit for bit on every valid row."""
    announce("gemm_silu_many_tiles", fp8, out_fp8)
    I, K = 256, 384
    m = _many_tiles_layout(47)
    G = 16
    ops = _gemm_operands(orc, fp8, [1] * G, 2 * I, K, seed=53, extra_rows=len(m) - 128 * G)
    M = len(m)
    m_dev = i32_dev(m)
    if fp8:
        A, As = u8_dev(ops["A"]), u8_dev(ops["As"].T.copy())
        B, Bs = u8_dev(ops["B"]), u8_dev(ops["Bs"])
    else:
        A, As, B, Bs = to_dev_bf16(ops["A"]), None, to_dev_bf16(ops["B"]), None
    C = poison((M, 2 * I), torch.bfloat16)
    L.grouped_gemm_contig(fp8, A, As, B, Bs, C, m_dev)
    odt = torch.uint8 if out_fp8 else torch.bfloat16
    sep = poison((M, I), odt)
    sep_s = poison((I // 128, M), torch.uint8) if out_fp8 else None
    L.silu_and_mul(C, sep, out_fp8, sep_s, m_indices=m_dev)
    fused = poison((M, I), odt)
    fused_s = poison((I // 128, M), torch.uint8) if out_fp8 else None
    L.grouped_gemm_contig_silu(fp8, A, As, B, Bs, fused, m_dev, fused_s)
    torch.cuda.synchronize()
    v = torch.from_numpy(m >= 0)
    a, b = fused.cpu(), sep.cpu()
    if not out_fp8:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a[v], b[v])
    if out_fp8:
        assert np.array_equal(fused_s.cpu().numpy()[:, m >= 0], sep_s.cpu().numpy()[:, m >= 0])
    # and the plain product itself against the oracle on a sample of rows
    ref = _ref_gemm(orc, fp8, dict(ops, m_idx=m))
    got = bits(C)
    _check_close(got, ref, m >= 0, 5e-3 if not fp8 else 2e-2, fp8)


@pytest.mark.parametrize("fp8,counts,N,K", [
    (True, [257, 5, 0, 130], 4096, 7168),     # FP8 w13 of the DeepSeek-V3-shaped prefill
    (False, [130, 3], 28672, 4096),           # BF16 w13 of the Mixtral-shaped prefill
])
def test_gemm_contig_integer_exact_real_shapes(orc, fp8, counts, N, K):
    """The compact GEMM at the workloads' real N and K (many N-tiles, 56 or 64
    k-steps, an expert split into two M-tiles, a one-row-block tile) with
    integer-valued operands: every partial sum is exact in fp32 (BF16:
    |sum| <= 12 K < 2^24; FP8: scale exponents within [-2, 1], so block sums
    of at most 1536 stay within 20 bits), so the result must be bit-exact."""
    announce("gemm_contig_real_shape", fp8, counts, N, K)
    ops = _gemm_operands(orc, fp8, counts, N, K, seed=61, integer_valued=True,
                         scale_ranges=((126, 129), (126, 128)))
    ref = _ref_gemm(orc, fp8, ops)
    got = _run_contig(fp8, ops, N)
    valid = ops["m_idx"] >= 0
    assert np.array_equal(got[valid], ref[valid])
    assert np.all(got[_skipped_rows_contig(ops["m_idx"])] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("integer_valued", [False, True])
def test_gemm_masked_all_tile_heights(orc, fp8, integer_valued):
    """Masked layout; every expected_m hint (tile heights 16, 32, 64 and 128) gives the
    same bits, equal to the oracle (exact for integer-valued operands)."""
    announce("gemm_masked", fp8, integer_valued)
    G, max_m, N, K = 5, 200, 256, 384
    masked = np.array([0, 1, 200, 37, 130], np.int32)
    ops = _gemm_operands(orc, fp8, [max_m] * G, N, K, seed=11, integer_valued=integer_valued)
    rg = orc.masked_row_group(masked, max_m)
    A = ops["A"][: G * max_m]
    if fp8:
        ref = orc.gemm_fp8_rows(A, ops["As"][: G * max_m], ops["B"], ops["Bs"], rg)
    else:
        ref = orc.gemm_bf16_rows(A, ops["B"], rg)
    outs = []
    for em in (0, 8, 24, 50, 200):
        C = poison((G, max_m, N), torch.bfloat16)
        if fp8:
            As = ops["As"][: G * max_m].reshape(G, max_m, K // 128).transpose(0, 2, 1).copy()
            L.grouped_gemm_masked(True, u8_dev(A).view(G, max_m, K), u8_dev(As), u8_dev(ops["B"]),
                                  u8_dev(ops["Bs"]), C, i32_dev(masked), em)
        else:
            L.grouped_gemm_masked(False, to_dev_bf16(A).view(G, max_m, K), None, to_dev_bf16(ops["B"]),
                                  None, C, i32_dev(masked), em)
        torch.cuda.synchronize()
        outs.append(bits(C).reshape(G * max_m, N))
    valid = rg >= 0
    for o in outs[1:]:
        assert np.array_equal(o[valid], outs[0][valid])
    if integer_valued:
        assert np.array_equal(outs[0][valid], ref[valid])
    else:
        _check_close(outs[0], ref, valid, 5e-3 if not fp8 else 2e-2, fp8)
    for o in outs:
        assert np.all(o[_skipped_rows_masked(masked, max_m)] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
def test_gemm_masked_many_groups(orc, fp8):
    """700 groups with random counts (a fifth of them empty): the on-chip tile
    prefix over groups spans every wavefront of the workgroup."""
    announce("gemm_masked_many_groups", fp8)
    G, max_m, N, K = 700, 64, 128, 128
    rng = np.random.default_rng(3)
    masked = rng.integers(1, max_m + 1, G).astype(np.int32)
    masked[rng.random(G) < 0.2] = 0
    ops = _gemm_operands(orc, fp8, [max_m] * G, N, K, seed=13, integer_valued=True)
    rg = orc.masked_row_group(masked, max_m)
    A = ops["A"][: G * max_m]
    C = poison((G, max_m, N), torch.bfloat16)
    if fp8:
        ref = orc.gemm_fp8_rows(A, ops["As"][: G * max_m], ops["B"], ops["Bs"], rg)
        As = ops["As"][: G * max_m].reshape(G, max_m, K // 128).transpose(0, 2, 1).copy()
        L.grouped_gemm_masked(True, u8_dev(A).view(G, max_m, K), u8_dev(As), u8_dev(ops["B"]),
                              u8_dev(ops["Bs"]), C, i32_dev(masked), 0)
    else:
        ref = orc.gemm_bf16_rows(A, ops["B"], rg)
        L.grouped_gemm_masked(False, to_dev_bf16(A).view(G, max_m, K), None, to_dev_bf16(ops["B"]),
                              None, C, i32_dev(masked), 0)
    torch.cuda.synchronize()
    got = bits(C).reshape(G * max_m, N)
    valid = rg >= 0
    assert np.array_equal(got[valid], ref[valid])
    assert np.all(got[_skipped_rows_masked(masked, max_m)] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("expected_m", [0, 8])
def test_gemm_masked_max_groups_long_tail(orc, fp8, expected_m):
    """1024 groups (the maximum), most short, some spanning up to ten tiles,
    the last group full: tiles are found through the group prefix for every
    position of the order (with 64-row tiles the order has 10240 M-tiles)."""
    announce("gemm_masked_max_groups", fp8, expected_m)
    G, max_m, N, K = 1024, 640, 128, 128
    rng = np.random.default_rng(5)
    masked = rng.integers(0, 21, G).astype(np.int32)
    for g, m in ((3, 640), (4, 129), (5, 128), (6, 64), (7, 65), (500, 513), (1022, 0), (1023, 640)):
        masked[g] = m
    ops = _gemm_operands(orc, fp8, [max_m] * G, N, K, seed=17, integer_valued=True)
    rg = orc.masked_row_group(masked, max_m)
    A = ops["A"][: G * max_m]
    C = poison((G, max_m, N), torch.bfloat16)
    if fp8:
        ref = orc.gemm_fp8_rows(A, ops["As"][: G * max_m], ops["B"], ops["Bs"], rg)
        As = ops["As"][: G * max_m].reshape(G, max_m, K // 128).transpose(0, 2, 1).copy()
        L.grouped_gemm_masked(True, u8_dev(A).view(G, max_m, K), u8_dev(As), u8_dev(ops["B"]),
                              u8_dev(ops["Bs"]), C, i32_dev(masked), expected_m)
    else:
        ref = orc.gemm_bf16_rows(A, ops["B"], rg)
        L.grouped_gemm_masked(False, to_dev_bf16(A).view(G, max_m, K), None, to_dev_bf16(ops["B"]),
                              None, C, i32_dev(masked), expected_m)
    torch.cuda.synchronize()
    got = bits(C).reshape(G * max_m, N)
    valid = rg >= 0
    assert np.array_equal(got[valid], ref[valid])
    assert np.all(got[_skipped_rows_masked(masked, max_m)] == 0xFFFF)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("out_fp8", [False, True])
def test_gemm_silu_fused_contig(orc, fp8, out_fp8):
    """w13 with SiLU-and-mul in the epilogue equals grouped_gemm_contig
    followed by silu_and_mul bit for bit on every valid row (activation and,
    for FP8 output, the UE8M0 scales)."""
    announce("gemm_silu_contig", fp8, out_fp8)
    I, K = 256, 384
    ops = _gemm_operands(orc, fp8, [130, 0, 5, 256, 1, 300], 2 * I, K, seed=21)
    M = len(ops["m_idx"])
    m_dev = i32_dev(ops["m_idx"])
    if fp8:
        A, As = u8_dev(ops["A"]), u8_dev(ops["As"].T.copy())
        B, Bs = u8_dev(ops["B"]), u8_dev(ops["Bs"])
    else:
        A, As, B, Bs = to_dev_bf16(ops["A"]), None, to_dev_bf16(ops["B"]), None
    C = poison((M, 2 * I), torch.bfloat16)
    L.grouped_gemm_contig(fp8, A, As, B, Bs, C, m_dev)
    odt = torch.uint8 if out_fp8 else torch.bfloat16
    sep = poison((M, I), odt)
    sep_s = poison((I // 128, M), torch.uint8) if out_fp8 else None
    L.silu_and_mul(C, sep, out_fp8, sep_s, m_indices=m_dev)
    fused = poison((M, I), odt)
    fused_s = poison((I // 128, M), torch.uint8) if out_fp8 else None
    L.grouped_gemm_contig_silu(fp8, A, As, B, Bs, fused, m_dev, fused_s)
    torch.cuda.synchronize()
    v = ops["m_idx"] >= 0
    a, b = fused.cpu(), sep.cpu()
    if not out_fp8:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a[torch.from_numpy(v)], b[torch.from_numpy(v)])
    if out_fp8:
        assert np.array_equal(fused_s.cpu().numpy()[:, v], sep_s.cpu().numpy()[:, v])
    skipped = _skipped_rows_contig(ops["m_idx"])
    untouched = 0xFF if out_fp8 else -1
    assert bool((fused.cpu().view(torch.uint8 if out_fp8 else torch.int16)[torch.from_numpy(skipped)] == untouched).all())


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("out_fp8", [False, True])
@pytest.mark.parametrize("expected_m", [0, 8, 24, 50])
def test_gemm_silu_fused_masked(orc, fp8, out_fp8, expected_m):
    """Masked layout, every tile height (128, 16, 32, 64 rows) and four
    N-tiles: fused equals separate bit for bit; rows past each group's last
    tile are untouched."""
    announce("gemm_silu_masked", fp8, out_fp8, expected_m)
    G, max_m, I, K = 5, 200, 512, 256
    masked = np.array([0, 1, 200, 37, 130], np.int32)
    ops = _gemm_operands(orc, fp8, [max_m] * G, 2 * I, K, seed=23)
    A = ops["A"][: G * max_m]
    if fp8:
        As = ops["As"][: G * max_m].reshape(G, max_m, K // 128).transpose(0, 2, 1).copy()
        Ad, Asd, B, Bs = u8_dev(A).view(G, max_m, K), u8_dev(As), u8_dev(ops["B"]), u8_dev(ops["Bs"])
    else:
        Ad, Asd, B, Bs = to_dev_bf16(A).view(G, max_m, K), None, to_dev_bf16(ops["B"]), None
    mm = i32_dev(masked)
    C = poison((G, max_m, 2 * I), torch.bfloat16)
    L.grouped_gemm_masked(fp8, Ad, Asd, B, Bs, C, mm, expected_m)
    odt = torch.uint8 if out_fp8 else torch.bfloat16
    sep = poison((G * max_m, I), odt)
    sep_s = poison((G, I // 128, max_m), torch.uint8) if out_fp8 else None
    L.silu_and_mul(C.view(G * max_m, 2 * I), sep, out_fp8, sep_s, masked_m=mm, max_m=max_m)
    fused = poison((G, max_m, I), odt)
    fused_s = poison((G, I // 128, max_m), torch.uint8) if out_fp8 else None
    L.grouped_gemm_masked_silu(fp8, Ad, Asd, B, Bs, fused, mm, expected_m, fused_s)
    torch.cuda.synchronize()
    rg = orc.masked_row_group(masked, max_m)
    v = torch.from_numpy(rg >= 0)
    a, b = fused.cpu().view(G * max_m, I), sep.cpu()
    if not out_fp8:
        a, b = a.view(torch.int16), b.view(torch.int16)
    assert torch.equal(a[v], b[v])
    if out_fp8:
        fs, ss = fused_s.cpu().numpy(), sep_s.cpu().numpy()
        for g in range(G):
            assert np.array_equal(fs[g, :, : masked[g]], ss[g, :, : masked[g]])
    bm = _masked_tile_rows(fp8, expected_m, 2 * I, K, max_m)
    assert bm == {0: 128, 8: 16, 24: 32, 50: 64}[expected_m]
    skipped = torch.from_numpy(_skipped_rows_masked(masked, max_m, bm))
    untouched = 0xFF if out_fp8 else -1
    raw = fused.cpu().view(G * max_m, I).view(torch.uint8 if out_fp8 else torch.int16)
    assert bool((raw[skipped] == untouched).all())


# ---------------------------------------------------------------------------
# SiLU-and-mul, combine
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("I", [128, 512, 1536])
def test_silu_and_mul_bf16(orc, I):
    announce("silu_bf16", I)
    M = 300
    g = torch.Generator().manual_seed(I)
    gu = (torch.randn(M, 2 * I, generator=g) * 3).to(torch.bfloat16)
    m_idx = np.where(np.arange(M) % 7 == 6, -1, 0).astype(np.int32)
    ref = orc.silu_and_mul(bits(gu), m_idx)
    out = poison((M, I), torch.bfloat16)
    L.silu_and_mul(gu.to(DEV), out, m_indices=i32_dev(m_idx))
    torch.cuda.synchronize()
    got = bits(out)
    v = m_idx >= 0
    r = f32(ref[v]).astype(np.float64)
    d = np.abs(f32(got[v]).astype(np.float64) - r)
    # GPU fp32 exp/divide vs fp64: at most one bf16 ulp, and rarely
    assert np.all(d <= bf16_ulp(r))
    assert (d > 0).mean() < 2e-3
    assert np.all(got[~v] == 0xFFFF)


def test_silu_and_mul_fp8_and_masked(orc):
    announce("silu_fp8_masked")
    G, max_m, I = 3, 50, 256
    masked = np.array([50, 0, 17], np.int32)
    g = torch.Generator().manual_seed(5)
    gu = (torch.randn(G * max_m, 2 * I, generator=g) * 3).to(torch.bfloat16)
    rg = orc.masked_row_group(masked, max_m)
    act_ref = orc.silu_and_mul(bits(gu), rg)
    v = rg >= 0
    q_ref = np.zeros((G * max_m, I), np.uint8)
    s_ref = np.zeros((G * max_m, I // 128), np.uint8)
    q_ref[v], s_ref[v] = orc.quant_rows(act_ref[v])
    q = poison((G * max_m, I), torch.uint8)
    s = poison((G, I // 128, max_m), torch.uint8)
    L.silu_and_mul(gu.to(DEV), q, True, s, masked_m=i32_dev(masked), max_m=max_m)
    # the bf16 output of the same masked call
    a = poison((G * max_m, I), torch.bfloat16)
    L.silu_and_mul(gu.to(DEV), a, masked_m=i32_dev(masked), max_m=max_m)
    torch.cuda.synchronize()
    sg = s.cpu().numpy().transpose(0, 2, 1).reshape(G * max_m, I // 128)
    qg = q.cpu().numpy()
    ag = bits(a)
    # rows whose bf16 activation matches the oracle bit for bit must quantise
    # to the same bytes; the rest differ by one bf16 ulp somewhere
    same = np.all(ag == act_ref, axis=1) & v
    assert same.sum() >= 0.9 * v.sum()
    assert np.array_equal(qg[same], q_ref[same]) and np.array_equal(sg[same], s_ref[same])
    tab = e4m3_table()
    deq = lambda qq, ss: tab[qq] * np.repeat(np.ldexp(1.0, ss.astype(np.int64) - 127), 128, axis=1)
    assert rel_fro(deq(qg[v], sg[v]), deq(q_ref[v], s_ref[v])) < 1e-2
    assert np.all(qg[~v] == 0xFF)


@pytest.mark.parametrize("T,k,H,R", [(50, 8, 7168, 500), (33, 2, 256, 80), (1, 1, 128, 3), (7, 32, 512, 300),
                                       (5, 4, 16384, 40), (3, 32, 7168, 100)])
def test_combine_bit_exact(orc, T, k, H, R):
    announce("combine", T, k, H, R)
    g = torch.Generator().manual_seed(T * k)
    Y = torch.randn(R, H, generator=g).to(torch.bfloat16)
    rng = np.random.default_rng(T)
    s2d = np.array([rng.permutation(R)[:k] for _ in range(T)], np.int32).reshape(T, k)
    s2d[::4, 0] = -1
    if T > 2:
        s2d[2, :] = -1
    w = rng.random((T, k)).astype(np.float32)
    ref = orc.combine(bits(Y), s2d, w)
    out = poison((T, H), torch.bfloat16)
    L.moe_combine(Y.to(DEV), i32_dev(s2d), torch.from_numpy(w).to(DEV), out)
    torch.cuda.synchronize()
    assert np.array_equal(bits(out), ref)
