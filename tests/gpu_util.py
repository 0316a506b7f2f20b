"""Helpers shared by the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np
import torch

from scatter_grouped_gemm_amd import inputs

DEV = "cuda"


def announce(*what):
    """Name the case on stdout before a GPU step, flushed, so a run that dies
    mid-step still says which case it was."""
    print("[case]", *what, flush=True)
    sys.stdout.flush()


def bits(t: torch.Tensor) -> np.ndarray:
    return inputs.bf16_bits(t)


def f32(b: np.ndarray) -> np.ndarray:
    return inputs.from_bf16_bits(b).float().numpy()


def to_dev_bf16(b: np.ndarray) -> torch.Tensor:
    return inputs.from_bf16_bits(b, DEV)


def u8_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(DEV)


def i32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).to(DEV)


def poison(shape, dtype) -> torch.Tensor:
    """A device buffer filled with a value no kernel would produce (0xFF bytes:
    bf16 NaN, e4m3 NaN, int32 -1 ... replaced by 0x7F7F7F7F for int32)."""
    if dtype == torch.int32:
        return torch.full(shape, 0x7F7F7F7F, dtype=torch.int32, device=DEV)
    t = torch.empty(shape, dtype=dtype, device=DEV)
    t.view(torch.uint8).fill_(0xFF)
    return t


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.frexp(ax)[1] - 8)


def e4m3_table() -> np.ndarray:
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def compact_layout(counts, block_e=128, extra_rows=128):
    """m_indices of a compact layout with the given per-expert counts, padded to
    block_e, plus `extra_rows` trailing -1 rows."""
    m = []
    for e, c in enumerate(counts):
        p = -(-c // block_e) * block_e
        m += [e] * c + [-1] * (p - c)
    m += [-1] * extra_rows
    return np.array(m, np.int32)


def distinct_ids(rng, T, E, k):
    return np.array([rng.permutation(E)[:k] for _ in range(T)], np.int32).reshape(T, k)
