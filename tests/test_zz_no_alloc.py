"""The allocation-free compact scatter (moe_scatter_compact_noalloc) against
the workspace entry point (moe_scatter_compact) on the same inputs, through the
C ABI: two calls in a row on the shared static scratch, the second smaller, so
a stale count or error word left by the first call would show."""
import numpy as np
import pytest
import torch

from scatter_grouped_gemm_amd import _lib as L
from gpu_util import DEV, announce, distinct_ids, i32_dev, poison

pytestmark = pytest.mark.gpu


def _outputs(T, H, E, El, start, k, fp8, seed, noalloc):
    rng = np.random.default_rng(seed)
    ids = distinct_ids(rng, T, E, k)
    x = torch.randn(T, H, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16).to(DEV)
    R = L.moe_compact_rows_bound(T * k, El, 128)
    adt = torch.uint8 if fp8 else torch.bfloat16
    out = dict(x_out=poison((R, H), adt), s_out=poison((H // 128, R), torch.uint8) if fp8 else None,
               m_idx=poison((R,), torch.int32), st=poison((El,), torch.int32),
               nv=poison((El,), torch.int32), s2d=poison((T, k), torch.int32))
    args = (x, i32_dev(ids), start, El, 128, R, fp8, out["x_out"], out["s_out"], out["m_idx"],
            out["st"], out["nv"], out["s2d"])
    if noalloc:
        L.moe_scatter_compact_noalloc(*args)
    else:
        ws = torch.empty(L.moe_scatter_ws_bytes(T, k, El, H), dtype=torch.uint8, device=DEV)
        L.moe_scatter_compact(*args, ws)
    torch.cuda.synchronize()
    return {n: (t.view(torch.uint8).cpu().numpy() if t is not None and t.dtype == torch.bfloat16
                else t.cpu().numpy() if t is not None else None) for n, t in out.items()}


def _same(a, b):
    for n in ("m_idx", "st", "nv", "s2d"):
        assert np.array_equal(a[n], b[n]), n
    valid = a["m_idx"] >= 0
    assert np.array_equal(a["x_out"][valid], b["x_out"][valid])
    if a["s_out"] is not None:
        assert np.array_equal(a["s_out"].T[valid], b["s_out"].T[valid])


# (T, H, E, El, start, k): the first call of each pair takes the chunked
# count / scan / rank kernels (more than 16384 assignments), the second the
# one-workgroup path, with fewer experts.
PAIRS = [((4100, 256, 256, 256, 0, 8), (300, 256, 64, 48, 8, 4)),
         ((3000, 512, 300, 200, 50, 8), (1, 128, 8, 8, 0, 2))]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_workspace_entry(first, second, fp8):
    for i, case in enumerate((first, second)):
        announce("scatter_compact_noalloc", i, *case, fp8)
        ref = _outputs(*case, fp8, seed=17 + i, noalloc=False)
        got = _outputs(*case, fp8, seed=17 + i, noalloc=True)
        _same(got, ref)


def test_noalloc_rejects_oversize():
    T, k, El = 1 << 20, 8, 256
    assert L.moe_scatter_ws_bytes(T, k, El, 128) > L.MOE_SCATTER_NOALLOC_MAX_BYTES
    x = torch.empty(1, 128, dtype=torch.bfloat16, device=DEV)
    P = x.data_ptr()
    st = L.lib().moe_scatter_compact_noalloc(P, T, 128, P, k, 0, El, 128, 1 << 30, 0, P, None, P,
                                             P, P, P, None)
    assert st == L.MOE_ECAPACITY
