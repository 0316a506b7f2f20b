"""Full-size parity on the five seeded workloads, in the launch configuration
bench.py times (the same MoELayer construction).

At full size the oracle cannot run the whole batch in seconds, so: routing and
every layout index are compared bit-exactly for ALL tokens; a sample of
scattered rows is compared bit-exactly; the outputs of a sample of tokens are
compared with the oracle's layout-free per-token path (valid because each
token's output depends only on its own row, which the batch-invariance checks
confirm on the GPU)."""
import numpy as np
import pytest
import torch

from scatter_grouped_gemm_amd import MoELayer, inputs
from gpu_util import DEV, announce, bits, f32, rel_fro

pytestmark = pytest.mark.gpu

SAMPLE = {"tiny": 64, "bf16_prefill": 8, "fp8_prefill": 6, "fp8_decode": 256, "bf16_skewed": 12}


def _build(wl):
    layer = MoELayer(hidden=wl.H, intermediate=wl.I, num_experts=wl.E, top_k=wl.k, max_tokens=wl.T,
                     num_local_experts=wl.El, expert_start=wl.expert_start, fp8=wl.fp8,
                     layout=wl.layout, block_e=wl.block_e, max_m=wl.max_m or None,
                     expected_m=wl.expected_m, device=DEV)
    for e in range(wl.El):
        a, b = inputs.expert_weights(wl, wl.expert_start + e, DEV)
        layer.set_expert(e, a, b)
    return layer


def _oracle_tokens(orc, wl, xs_bits, ids, w):
    """Oracle output rows for a token sample, with only the experts it needs."""
    local = ids - wl.expert_start
    need = sorted({int(e) for e in local.reshape(-1) if 0 <= e < wl.El})
    remap = np.full(wl.El, -1, np.int32)
    remap[need] = np.arange(len(need), dtype=np.int32)
    inside = (local >= 0) & (local < wl.El)
    ids_c = np.where(inside, remap[np.clip(local, 0, wl.El - 1)], -1).astype(np.int32)
    parts13, parts2 = [], []
    for e in need:
        a, b = inputs.expert_weights(wl, wl.expert_start + e, DEV)
        a, b = bits(a)[None], bits(b)[None]
        parts13.append(orc.quant_weight_blocks(a) if wl.fp8 else a)
        parts2.append(orc.quant_weight_blocks(b) if wl.fp8 else b)
    if not need:
        return np.zeros((len(xs_bits), wl.H), np.uint16)
    if wl.fp8:
        W = dict(w13q=np.concatenate([p[0] for p in parts13]), w13s=np.concatenate([p[1] for p in parts13]),
                 w2q=np.concatenate([p[0] for p in parts2]), w2s=np.concatenate([p[1] for p in parts2]))
    else:
        W = dict(w13=np.concatenate(parts13), w2=np.concatenate(parts2))
    return orc.moe_dense(xs_bits, ids_c, w, 0, len(need), wl.fp8, **W)


@pytest.mark.parametrize("name", ["tiny", "bf16_prefill", "fp8_prefill", "fp8_decode", "bf16_skewed"])
def test_workload_full_size(orc, name):
    wl = inputs.get(name)
    announce("workload", wl.name)
    layer = _build(wl)
    x = inputs.tokens(wl, DEV)
    logits = inputs.logits(wl, DEV)
    out = layer(x, logits)
    torch.cuda.synchronize()
    T, k = wl.T, wl.k
    # routing, all tokens
    ids_ref, w_ref = orc.route_topk(logits.cpu().numpy(), k)
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ids_ref)
    np.testing.assert_allclose(layer.topk_weights[:T].cpu().numpy(), w_ref, rtol=1e-6, atol=0)
    xb = bits(x)
    # layout indices, all rows
    if layer.layout == "compact":
        sc = orc.scatter_compact(xb, ids_ref, wl.expert_start, wl.El, wl.block_e, layer.rows, wl.fp8,
                                 rows=False)
        assert np.array_equal(layer.m_indices.cpu().numpy(), sc["m_indices"])
        assert np.array_equal(layer.expert_start_loc.cpu().numpy(), sc["expert_start_loc"])
        assert np.array_equal(layer.num_valid.cpu().numpy(), sc["num_valid"])
        counts = sc["num_valid"]
    else:
        sc = orc.scatter_masked(xb, ids_ref, wl.expert_start, wl.El, layer.max_m, wl.fp8, rows=False)
        assert np.array_equal(layer.masked_m.cpu().numpy(), sc["masked_m"])
        counts = sc["masked_m"]
    s2d = sc["src2dst"]
    assert np.array_equal(layer.src2dst[:T].cpu().numpy(), s2d)
    if wl.skew:
        assert (counts == 0).sum() >= 8                 # dead experts receive nothing
    # sampled scattered rows, bit-exact
    rng = np.random.default_rng(0)
    ts, js = np.nonzero(s2d >= 0)
    pick = rng.choice(len(ts), size=min(64, len(ts)), replace=False)
    rows = s2d[ts[pick], js[pick]]
    if wl.fp8:
        q, s = orc.quant_rows(xb[ts[pick]])
        xg = layer.x_buf[torch.from_numpy(rows).long().to(DEV)].cpu().numpy()
        assert np.array_equal(xg, q)
        if layer.layout == "compact":
            sg = layer.x_scale.view(wl.H // 128, layer.rows)[:, torch.from_numpy(rows).long().to(DEV)]
            assert np.array_equal(sg.cpu().numpy().T, s)
    else:
        xg = bits(layer.x_buf[torch.from_numpy(rows).long().to(DEV)])
        assert np.array_equal(xg, xb[ts[pick]])
    # sampled token outputs against the oracle's per-token path
    n = min(SAMPLE[name], T)
    tok = np.sort(rng.choice(T, size=n, replace=False))
    ref = _oracle_tokens(orc, wl, xb[tok], ids_ref[tok], w_ref[tok])
    got = f32(bits(out)[tok]).astype(np.float64)
    assert np.all(np.isfinite(got))
    err = rel_fro(got, f32(ref))
    assert err <= (2e-2 if wl.fp8 else 5e-3), err
    # batch invariance at the workload's own shape (the skewed workload is
    # specified with T = 1, 7, 33 as well)
    full = bits(out).copy()
    for Tp in (1, 7, 33):
        part = bits(layer(x[:Tp].contiguous(), logits[:Tp].contiguous()))
        assert np.array_equal(part, full[:Tp]), Tp
