"""Layer-level parity of the HIP path against the oracle at small sizes, plus
the invariances the pages ask for: masked and compact layouts agree, a token's
output bits do not depend on its batch, and uninitialised (poisoned) buffers
do not leak into results."""
import zlib

import numpy as np
import pytest
import torch

from scatter_grouped_gemm_amd import MoELayer, inputs
from gpu_util import DEV, announce, bits, f32, rel_fro

pytestmark = pytest.mark.gpu


def _layer(T, H, I, E, k, *, El=None, start=0, fp8=False, layout="auto", expected_m=0):
    return MoELayer(hidden=H, intermediate=I, num_experts=E, top_k=k, max_tokens=T,
                    num_local_experts=El, expert_start=start, fp8=fp8, layout=layout,
                    expected_m=expected_m, device=DEV)


def _oracle_weights(orc, w13, w2, fp8):
    if not fp8:
        return dict(w13=bits(w13), w2=bits(w2))
    a, b = orc.quant_weight_blocks(bits(w13))
    c, d = orc.quant_weight_blocks(bits(w2))
    return dict(w13q=a, w13s=b, w2q=c, w2s=d)


def _fill(layer, byte):
    for name in ("x_buf", "x_scale", "gateup", "act", "act_scale", "y", "out", "src2dst",
                 "m_indices", "masked_m", "topk_ids", "topk_weights"):
        t = getattr(layer, name, None)
        if t is not None:
            t.view(torch.uint8).fill_(byte)


CASES = [
    # name, T, H, I, E, El, start, k, fp8, layout
    ("tiny_bf16", 64, 256, 512, 8, None, 0, 2, False, "compact"),
    ("bf16_e16", 300, 256, 384, 16, None, 0, 4, False, "compact"),
    ("fp8_compact", 200, 384, 256, 16, None, 0, 4, True, "compact"),
    ("fp8_masked_share", 150, 256, 256, 64, 8, 8, 6, True, "masked"),
    ("bf16_masked_share", 97, 256, 256, 40, 12, 20, 5, False, "masked"),
]


@pytest.mark.parametrize("name,T,H,I,E,El,start,k,fp8,layout", CASES)
def test_layer_matches_oracle(orc, name, T, H, I, E, El, start, k, fp8, layout):
    announce("layer", name)
    x, logits, w13, w2 = inputs.small_case(zlib.crc32(name.encode()) % 1000, T, H, I, E, k, El=El or E)
    layer = _layer(T, H, I, E, k, El=El, start=start, fp8=fp8, layout=layout,
                   expected_m=max(1, T * k // E))
    layer.set_weights(w13.to(DEV), w2.to(DEV))
    _fill(layer, 0xFF)
    out = layer(x.to(DEV), logits.to(DEV))
    torch.cuda.synchronize()
    W = _oracle_weights(orc, w13, w2, fp8)
    ref = orc.moe_layer(bits(x), logits.numpy(), k, expert_start=start, num_local_experts=El or E,
                        layout=layout, fp8=fp8, max_m=T, **W)
    assert np.array_equal(layer.topk_ids[:T].cpu().numpy(), ref["topk_ids"])
    sc = ref["scatter"]
    if layout == "compact":
        assert np.array_equal(layer.m_indices.cpu().numpy(), sc["m_indices"])
        valid = sc["m_indices"] >= 0
    else:
        assert np.array_equal(layer.masked_m.cpu().numpy(), sc["masked_m"])
        valid = orc.masked_row_group(sc["masked_m"], T) >= 0
    assert np.array_equal(layer.src2dst[:T].cpu().numpy(), sc["src2dst"])
    if fp8:
        assert np.array_equal(layer.x_buf.cpu().numpy()[valid], sc["x_out"][valid])
    else:
        assert np.array_equal(bits(layer.x_buf)[valid], sc["x_out"][valid])
    got = f32(bits(out)).astype(np.float64)
    assert np.all(np.isfinite(got))
    err = rel_fro(got, f32(ref["out"]))
    assert err <= (2e-2 if fp8 else 5e-3), err
    no_local = np.all(sc["src2dst"] < 0, axis=1)
    assert np.all(got[no_local] == 0)


@pytest.mark.parametrize("fp8", [False, True])
def test_masked_equals_compact(fp8):
    """Same routing through both layouts gives the same output bits (the
    end-to-end agreement "Support DeepGEMM for standard MoE dispatch" tests)."""
    announce("masked_eq_compact", fp8)
    T, H, I, E, El, start, k = 256, 384, 256, 64, 16, 16, 8
    x, logits, w13, w2 = inputs.small_case(21, T, H, I, E, k, El=El)
    outs = []
    for layout, em in (("compact", 0), ("masked", 8), ("masked", 100)):
        layer = _layer(T, H, I, E, k, El=El, start=start, fp8=fp8, layout=layout, expected_m=em)
        layer.set_weights(w13.to(DEV), w2.to(DEV))
        outs.append(bits(layer(x.to(DEV), logits.to(DEV))))
    assert np.array_equal(outs[0], outs[1])
    assert np.array_equal(outs[0], outs[2])


@pytest.mark.parametrize("fp8", [False, True])
def test_batch_invariance(fp8):
    """A token's output bits do not depend on how many other tokens share the
    batch or where it sits ("[Feature] Support BF16 and batch-invariant
    inference with DeepEP v2": atol = 0, rtol = 0)."""
    announce("batch_invariance", fp8)
    T, H, I, E, k = 700, 256, 384, 32, 8
    x, logits, w13, w2 = inputs.small_case(33, T, H, I, E, k)
    layer = _layer(T, H, I, E, k, fp8=fp8)
    layer.set_weights(w13.to(DEV), w2.to(DEV))
    xd, ld = x.to(DEV), logits.to(DEV)
    full = bits(layer(xd, ld)).copy()
    for Tp in (1, 7, 33, 129):
        part = bits(layer(xd[:Tp].contiguous(), ld[:Tp].contiguous()))
        assert np.array_equal(part, full[:Tp]), Tp
    perm = torch.randperm(T, generator=torch.Generator().manual_seed(1))
    shuffled = bits(layer(xd[perm.to(DEV)].contiguous(), ld[perm.to(DEV)].contiguous()))
    assert np.array_equal(shuffled, full[perm.numpy()])


@pytest.mark.parametrize("fp8,layout", [(False, "compact"), (True, "compact"), (True, "masked")])
def test_empty_batch_then_full_batch(fp8, layout):
    """A batch of zero tokens runs every kernel of the path on empty inputs
    (no routed rows, all-padding layouts) and returns an empty output; the
    next full batch is unaffected."""
    announce("empty_batch", fp8, layout)
    T, H, I, E, k = 64, 256, 256, 16, 4
    x, logits, w13, w2 = inputs.small_case(55, T, H, I, E, k)
    layer = _layer(T, H, I, E, k, fp8=fp8, layout=layout)
    layer.set_weights(w13.to(DEV), w2.to(DEV))
    xd, ld = x.to(DEV), logits.to(DEV)
    before = bits(layer(xd, ld)).copy()
    empty = layer(xd[:0].contiguous(), ld[:0].contiguous())
    torch.cuda.synchronize()
    assert tuple(empty.shape) == (0, H)
    assert np.array_equal(bits(layer(xd, ld)), before)


@pytest.mark.parametrize("fp8", [False, True])
def test_uninitialised_buffers_do_not_leak(fp8):
    """Buffers are allocated uninitialised ("Support DeepGEMM for standard MoE
    dispatch", implementation breakdown item 4): whatever they hold, the
    output is the same."""
    announce("poison", fp8)
    T, H, I, E, k = 100, 256, 256, 16, 4
    x, logits, w13, w2 = inputs.small_case(44, T, H, I, E, k)
    layer = _layer(T, H, I, E, k, fp8=fp8)
    layer.set_weights(w13.to(DEV), w2.to(DEV))
    res = []
    for byte in (0x00, 0xFF, 0x7F):
        _fill(layer, byte)
        res.append(bits(layer(x.to(DEV), logits.to(DEV))).copy())
    assert np.array_equal(res[0], res[1]) and np.array_equal(res[0], res[2])


@pytest.mark.parametrize("layout", ["compact", "masked"])
def test_layer_block_fp8_checkpoint(orc, layout):
    """Block-FP8 checkpoint weights requantised in the library drive the layer
    like the oracle's requantisation of the same codes and scales."""
    announce("layer_block_fp8_checkpoint", layout)
    T, H, I, E, k = 160, 256, 384, 16, 4
    x, logits, _, _ = inputs.small_case(77, T, H, I, E, k)
    w13q, w13s = inputs.block_fp8_checkpoint(E, 2 * I, H, seed=78)
    w2q, w2s = inputs.block_fp8_checkpoint(E, H, I, seed=79)
    layer = _layer(T, H, I, E, k, fp8=True, layout=layout, expected_m=T * k // E)
    layer.set_block_fp8_weights(w13q.to(DEV), w13s.to(DEV), w2q.to(DEV), w2s.to(DEV))
    out = layer(x.to(DEV), logits.to(DEV))
    torch.cuda.synchronize()
    a, b = orc.requant_weight_blocks(w13q.numpy(), w13s.numpy())
    c, d = orc.requant_weight_blocks(w2q.numpy(), w2s.numpy())
    assert np.array_equal(layer.w13.cpu().numpy(), a) and np.array_equal(layer.w13_scale.cpu().numpy(), b)
    assert np.array_equal(layer.w2.cpu().numpy(), c) and np.array_equal(layer.w2_scale.cpu().numpy(), d)
    ref = orc.moe_layer(bits(x), logits.numpy(), k, expert_start=0, num_local_experts=E,
                        layout=layout, fp8=True, max_m=T, w13q=a, w13s=b, w2q=c, w2s=d)
    err = rel_fro(f32(bits(out)).astype(np.float64), f32(ref["out"]))
    assert err <= 2e-2, err


def test_fp8_layer_rejects_bf16_mix():
    announce("dtype_follows_weights")
    layer = _layer(8, 128, 128, 4, 2, fp8=False)
    with pytest.raises(ValueError):
        layer.set_quantized_weights(None, None, None, None)
    with pytest.raises(ValueError):
        layer.set_block_fp8_weights(None, None, None, None)


@pytest.mark.parametrize("name,T,H,I,E,El,start,k,fp8,layout", CASES)
def test_layer_fused_silu_matches_unfused(name, T, H, I, E, El, start, k, fp8, layout):
    """SiLU-and-mul fused into the w13 GEMM gives the same output bits as the
    two separate kernels."""
    announce("layer_fused", name)
    x, logits, w13, w2 = inputs.small_case(zlib.crc32(name.encode()) % 1000, T, H, I, E, k, El=El or E)
    outs = []
    for fuse in (True, False):
        layer = MoELayer(hidden=H, intermediate=I, num_experts=E, top_k=k, max_tokens=T,
                         num_local_experts=El, expert_start=start, fp8=fp8, layout=layout,
                         expected_m=max(1, T * k // E), fuse_silu=fuse, device=DEV)
        layer.set_weights(w13.to(DEV), w2.to(DEV))
        outs.append(bits(layer(x.to(DEV), logits.to(DEV))))
    torch.cuda.synchronize()
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("layout", ["compact", "masked"])
@pytest.mark.parametrize("fuse", [True, False])
def test_layer_mx_weights(orc, layout, fuse, fmt):
    """MX weights (one exponent per 32 k of a weight row; e4m3 or e2m1)
    quantised in the library drive the FP8 layer like the oracle's MX weights."""
    announce("layer_mx", fmt, layout, fuse)
    T, H, I, E, k = 160, 256, 384, 16, 4
    x, logits, w13, w2 = inputs.small_case(91, T, H, I, E, k)
    layer = MoELayer(hidden=H, intermediate=I, num_experts=E, top_k=k, max_tokens=T, fp8=True,
                     layout=layout, expected_m=T * k // E, fuse_silu=fuse, weight_format=fmt,
                     device=DEV)
    layer.set_weights(w13.to(DEV), w2.to(DEV))
    out = layer(x.to(DEV), logits.to(DEV))
    torch.cuda.synchronize()
    a, b = orc.quant_weight_mx(bits(w13), fmt)
    c, d = orc.quant_weight_mx(bits(w2), fmt)
    assert np.array_equal(layer.w13.cpu().numpy(), a) and np.array_equal(layer.w2.cpu().numpy(), c)
    ref = orc.moe_layer(bits(x), logits.numpy(), k, expert_start=0, num_local_experts=E,
                        layout=layout, fp8=True, max_m=T, w13q=a, w13s=b, w2q=c, w2s=d, mx=fmt)
    err = rel_fro(f32(bits(out)).astype(np.float64), f32(ref["out"]))
    assert err <= 2e-2, err


@pytest.mark.parametrize("fp8,layout", [(True, "compact"), (True, "masked"), (False, "compact")])
def test_layer_hip_graph_replays_match_eager(fp8, layout):
    """The forward allocates nothing, reads nothing back and records no memset,
    so it can be captured in a HIP graph: every replay (with new tokens copied
    into the captured input, and eager work between replays) gives the eager
    forward's bits."""
    announce("layer_hip_graph", fp8, layout)
    T, H, I, E, k = 96, 256, 256, 16, 4
    layer = _layer(T, H, I, E, k, fp8=fp8, layout=layout, expected_m=T * k // E)
    x0, logits0, w13, w2 = inputs.small_case(5, T, H, I, E, k)
    layer.set_weights(w13.to(DEV), w2.to(DEV))
    x_in = x0.to(DEV).clone()
    l_in = logits0.to(DEV).clone()
    layer(x_in, l_in)                                   # first launches outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            out_g = layer(x_in, l_in)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for seed in (6, 7, 8):
        x1, l1, _, _ = inputs.small_case(seed, T, H, I, E, k)
        x_in.copy_(x1.to(DEV))
        l_in.copy_(l1.to(DEV))
        graph.replay()
        torch.cuda.synchronize()
        got = bits(out_g).copy()
        eager = bits(layer(x_in, l_in)).copy()          # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), seed
