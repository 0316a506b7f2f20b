"""Full-size parity on the five seeded workloads, in the launch configuration
bench.py times (the same MoELayer construction).

At full size the oracle cannot run the whole batch in seconds, so: routing and
every layout index are compared bit-exactly for ALL tokens; a sample of
scattered rows is compared bit-exactly; the outputs of 256 tokens (all of them
when the batch is smaller) are compared element by element with the oracle's
layout-free per-token path (valid because each token's output depends only on
its own row, which the batch-invariance checks confirm on the GPU).  The
sample always holds tokens routed to the hottest and to the coldest live
expert and tokens whose rows are the last rows of an expert (the last,
partial M-tile of its run), the rest drawn at random."""
import numpy as np
import pytest
import torch

from scatter_grouped_gemm_amd import MoELayer, inputs
from gpu_util import DEV, announce, bf16_ulp, bits, f32, rel_fro

pytestmark = pytest.mark.gpu

N_SAMPLE = 256


def _build(wl):
    layer = MoELayer(hidden=wl.H, intermediate=wl.I, num_experts=wl.E, top_k=wl.k, max_tokens=wl.T,
                     num_local_experts=wl.El, expert_start=wl.expert_start, fp8=wl.fp8,
                     layout=wl.layout, block_e=wl.block_e, max_m=wl.max_m or None,
                     expected_m=wl.expected_m, device=DEV)
    for e in range(wl.El):
        a, b = inputs.expert_weights(wl, wl.expert_start + e, DEV)
        layer.set_expert(e, a, b)
    return layer


# Element-wise slack (fraction of the row's largest output) beyond one bf16
# ulp.  The GPU and the oracle sum in different orders, so an intermediate
# bf16 (the w13 output, the SiLU product) can land one ulp apart; FP8 then
# requantises the activation to e4m3, where such a difference occasionally
# moves a code by one e4m3 step (up to 1/8 of that element), and the w2 sum
# carries it into every output of the token.  Measured worst cases over the
# 256-token samples on MI355X: 3.8e-3 (BF16 workloads) and 6.4e-3 (FP8); the
# bounds leave about a factor three.  The relative-Frobenius bounds are the
# method's stated tolerances (5e-3 BF16, 2e-2 FP8).
ELEMENT_SLACK = {False: 1e-2, True: 2e-2}


def _pick_tokens(wl, s2d, counts, rng):
    """N_SAMPLE tokens: those routed to the hottest and to the coldest live
    expert (up to 16 each), those holding the last 4 rows of up to 16 live
    experts, then random ones."""
    T = s2d.shape[0]
    if T <= N_SAMPLE:
        return np.arange(T)
    # assignments in destination-row order: both layouts keep an expert's rows
    # contiguous, experts in increasing order, so the sorted sequence is
    # counts[0] rows of expert 0, then counts[1] of expert 1, ...
    flat = s2d.reshape(-1)
    order = np.argsort(flat, kind="stable")
    order = order[flat[order] >= 0]
    tok_sorted = order // s2d.shape[1]
    exp_of = np.repeat(np.arange(len(counts)), counts)
    assert len(exp_of) == len(tok_sorted)
    starts = np.concatenate([[0], np.cumsum(counts)])
    live = np.nonzero(counts > 0)[0]
    hot, cold = live[np.argmax(counts[live])], live[np.argmin(counts[live])]
    pick = []
    for e in (hot, cold):
        pick += list(tok_sorted[exp_of == e][:16])
    for e in rng.choice(live, size=min(16, len(live)), replace=False):
        pick += list(tok_sorted[starts[e + 1] - min(4, counts[e]):starts[e + 1]])
    pick = list(dict.fromkeys(int(t) for t in pick))[:N_SAMPLE]
    rest = np.setdiff1d(np.arange(T), pick)
    pick += [int(t) for t in rng.choice(rest, size=N_SAMPLE - len(pick), replace=False)]
    return np.sort(np.array(pick, np.int64))


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
    tok = _pick_tokens(wl, s2d, counts, rng)
    ref = f32(_oracle_tokens(orc, wl, xb[tok], ids_ref[tok], w_ref[tok])).astype(np.float64)
    got = f32(bits(out)[tok]).astype(np.float64)
    assert np.all(np.isfinite(got))
    err = rel_fro(got, ref)
    # element-wise: one bf16 ulp of the reference element plus a slack scaled
    # by the row's largest element (see ELEMENT_SLACK)
    rowmax = np.abs(ref).max(axis=1, keepdims=True)
    idle = rowmax[:, 0] == 0              # tokens with no local expert: exactly zero
    assert np.all(got[idle] == 0)
    excess = np.abs(got - ref) - bf16_ulp(ref)
    worst = float(np.max(excess[~idle] / rowmax[~idle])) if (~idle).any() else 0.0
    print(f"[parity] {wl.name}: {len(tok)} tokens, rel-Frobenius {err:.3e}, "
          f"worst element excess over 1 ulp / row max {worst:.3e}", flush=True)
    assert err <= (2e-2 if wl.fp8 else 5e-3), err
    assert worst <= ELEMENT_SLACK[wl.fp8], worst
    # batch invariance at the workload's own shape (the skewed workload is
    # specified with T = 1, 7, 33 as well)
    full = bits(out).copy()
    for Tp in (1, 7, 33):
        part = bits(layer(x[:Tp].contiguous(), logits[:Tp].contiguous()))
        assert np.array_equal(part, full[:Tp]), Tp
