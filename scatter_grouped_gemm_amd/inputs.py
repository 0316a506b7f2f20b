"""Seeded synthetic inputs for the MoE expert path.

This module only draws random numbers with fixed distributions; it performs
none of the method's arithmetic (no routing, no layout, no quantisation, no
products).  Both the HIP path (tests, smoke check, benchmark) and the CPU oracle
take their inputs from here, and nothing else is shared between them.

Distributions (the plain reading of the workloads these kernels are sized for):
  x        ~ N(0, 1), rounded to bf16            [T, H]
  logits   ~ N(0, 1) in fp32                     [T, E]; the skewed workload adds
             a per-expert bias -1.2*ln(rank) (Zipf-like popularity, s = 1.2)
             over a seeded random ranking, and -1e4 for 8 "dead" experts so
             some experts receive no tokens.
  w13, w2  ~ N(0, 0.02), rounded to bf16         [2I, H] and [H, I] per expert;
             each expert is drawn from its own stream keyed by its GLOBAL id, so
             a 32-expert share equals experts expert_start.. of the full model.

Values depend on the device they are drawn on (torch's CPU and GPU generators
differ); a test always draws every input for one comparison on one device.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import torch

BASE_SEED = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int               # experts in the model (global)
    k: int
    fp8: bool
    layout: str          # "compact" or "masked"
    num_local: int = 0   # experts held by this GPU (0 -> all)
    expert_start: int = 0
    block_e: int = 128
    max_m: int = 0       # masked layout rows per expert
    expected_m: int = 0  # masked layout hint
    skew: bool = False
    model_key: str = ""  # workloads with the same key share expert weights
    index: int = 0

    @property
    def El(self) -> int:
        return self.num_local or self.E

    def with_tokens(self, T: int) -> "Workload":
        return dataclasses.replace(self, T=T)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_bf16_T64_E8", T=64, H=256, I=512, E=8, k=2, fp8=False,
                 layout="compact", model_key="tiny", index=0),
        Workload("bf16_prefill_T4096_H4096_I14336_E8", T=4096, H=4096, I=14336, E=8,
                 k=2, fp8=False, layout="compact", model_key="bf16_e8", index=1),
        Workload("fp8_prefill_T8192_H7168_I2048_E256", T=8192, H=7168, I=2048,
                 E=256, k=8, fp8=True, layout="compact", model_key="fp8_e256", index=2),
        Workload("fp8_masked_decode_T256_E32of256", T=256, H=7168, I=2048, E=256, k=8,
                 fp8=True, layout="masked", num_local=32, expert_start=0, max_m=256,
                 expected_m=8, model_key="fp8_e256", index=3),
        Workload("bf16_skewed_T16384_H4096_I1536_E128", T=16384, H=4096, I=1536,
                 E=128, k=8, fp8=False, layout="compact", skew=True,
                 model_key="bf16_e128", index=4),
    ]
}

# short aliases used by the tests and the benchmark command line
ALIASES = {
    "tiny": "tiny_bf16_T64_E8",
    "bf16_prefill": "bf16_prefill_T4096_H4096_I14336_E8",
    "fp8_prefill": "fp8_prefill_T8192_H7168_I2048_E256",
    "fp8_decode": "fp8_masked_decode_T256_E32of256",
    "bf16_skewed": "bf16_skewed_T16384_H4096_I1536_E128",
}


def get(name: str) -> Workload:
    return WORKLOADS[ALIASES.get(name, name)]


def _seed(*keys) -> int:
    parts = [BASE_SEED] + [int.from_bytes(str(k).encode(), "little") % (2**31)
                           if not isinstance(k, int) else k for k in keys]
    return int(np.random.SeedSequence(parts).generate_state(1, dtype=np.uint64)[0]
               & np.uint64(2**63 - 1))


def _gen(device, *keys) -> torch.Generator:
    g = torch.Generator(device=torch.device(device))
    g.manual_seed(_seed(*keys))
    return g


def tokens(wl: Workload, device="cpu") -> torch.Tensor:
    """x [T, H] bf16 for the workload's own T.  A batch-size sweep takes the
    first T' rows of one full draw (a draw at T' itself holds other values)."""
    g = _gen(device, "x", wl.index)
    return torch.randn(wl.T, wl.H, generator=g, device=device).to(torch.bfloat16)


def expert_bias(wl: Workload, device="cpu") -> torch.Tensor:
    """Per-expert logit bias: 0 unless the workload is skewed."""
    if not wl.skew:
        return torch.zeros(wl.E, dtype=torch.float32, device=device)
    g = _gen("cpu", "rank", wl.index)
    perm = torch.randperm(wl.E, generator=g)          # rank of expert e = perm[e] + 1
    live = wl.E - 8
    rank = (perm + 1).to(torch.float64)
    bias = torch.where(rank <= live, -1.2 * torch.log(rank), torch.full_like(rank, -1e4))
    return bias.to(torch.float32).to(device)


def logits(wl: Workload, device="cpu") -> torch.Tensor:
    """Router logits [T, E] fp32."""
    g = _gen(device, "logits", wl.index)
    L = torch.randn(wl.T, wl.E, generator=g, device=device, dtype=torch.float32)
    return L + expert_bias(wl, device)[None, :]


def expert_weights(wl: Workload, global_expert: int, device="cpu"):
    """(w13 [2I, H], w2 [H, I]) bf16 for one expert, keyed by its global id."""
    g = _gen(device, "w13", wl.model_key, global_expert)
    w13 = (torch.randn(2 * wl.I, wl.H, generator=g, device=device) * 0.02).to(torch.bfloat16)
    g = _gen(device, "w2", wl.model_key, global_expert)
    w2 = (torch.randn(wl.H, wl.I, generator=g, device=device) * 0.02).to(torch.bfloat16)
    return w13, w2


def local_weights(wl: Workload, device="cpu"):
    """All local experts' bf16 weights stacked: w13 [El, 2I, H], w2 [El, H, I]."""
    w13 = torch.empty(wl.El, 2 * wl.I, wl.H, dtype=torch.bfloat16, device=device)
    w2 = torch.empty(wl.El, wl.H, wl.I, dtype=torch.bfloat16, device=device)
    for e in range(wl.El):
        a, b = expert_weights(wl, wl.expert_start + e, device)
        w13[e].copy_(a)
        w2[e].copy_(b)
    return w13, w2


def small_case(seed: int, T: int, H: int, I: int, E: int, k: int, *, El=None,
               expert_start=0, device="cpu", integer_valued=False):
    """A free-form small case for parity tests: x, logits and local weights.

    integer_valued=True draws small integers (x in [-4, 4], weights in [-2, 2])
    so every partial sum of a product is exact in fp32."""
    El = El or E
    g = _gen(device, "small", seed, T, H, I, E, k)
    if integer_valued:
        x = torch.randint(-4, 5, (T, H), generator=g, device=device).to(torch.bfloat16)
        w13 = torch.randint(-2, 3, (El, 2 * I, H), generator=g, device=device).to(torch.bfloat16)
        w2 = torch.randint(-2, 3, (El, H, I), generator=g, device=device).to(torch.bfloat16)
    else:
        x = torch.randn(T, H, generator=g, device=device).to(torch.bfloat16)
        w13 = (torch.randn(El, 2 * I, H, generator=g, device=device) * 0.02).to(torch.bfloat16)
        w2 = (torch.randn(El, H, I, generator=g, device=device) * 0.02).to(torch.bfloat16)
    L = torch.randn(T, E, generator=g, device=device, dtype=torch.float32)
    return x, L, w13, w2


def block_fp8_checkpoint(G: int, N: int, K: int, seed: int, device="cpu"):
    """Synthetic block-FP8 expert weights as a checkpoint stores them: e4m3
    codes [G,N,K] (uint8, bell-shaped over the code range, no NaN codes) and one
    positive fp32 scale per 128x128 block [G,N/128,K/128], log-uniform over
    2^-14 .. 2^-4 and not powers of two."""
    g = torch.Generator().manual_seed(seed)
    v = (torch.randn(G, N, K, generator=g) * 96.0).clamp_(-448.0, 448.0)
    codes = v.to(torch.float8_e4m3fn).view(torch.uint8)
    scales = torch.exp2(torch.rand(G, N // 128, K // 128, generator=g) * 10.0 - 14.0)
    return codes.to(device), scales.to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Raw bf16 bit patterns of a tensor as a numpy uint16 array (on the host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)


def from_bf16_bits(a: np.ndarray, device="cpu") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)


def zipf_reference_shares(E_live: int, s: float = 1.2) -> np.ndarray:
    """Zipf(s) shares over E_live ranks (documentation of the skew target)."""
    r = np.arange(1, E_live + 1, dtype=np.float64)
    p = r ** (-s)
    return p / p.sum()


__all__ = ["Workload", "WORKLOADS", "ALIASES", "get", "tokens", "logits", "expert_bias",
           "expert_weights", "local_weights", "small_case", "block_fp8_checkpoint", "bf16_bits", "from_bf16_bits",
           "zipf_reference_shares"]
