"""Seeded synthetic inputs shaped like the workloads on the pages.

This module holds only random-number recipes: no step of the quantizer's
arithmetic lives here. The CPU oracle's tests, the GPU parity tests and the
benchmark all draw their inputs from it, on the host, and move them where
they need them.

Every tensor is generated in float32 from ``torch.Generator('cpu')`` and then
cast to its storage dtype (round to nearest even). Offsets and per-group
factors use ``numpy.random.default_rng``. The families follow the pages'
descriptions: training activations and weights, the four data families the
fused-QDQ validation mirrors, a list of discrete expert weights, and a packed
MoE token tensor with uneven groups and an over-allocated tail.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16, "fp32": torch.float32}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator("cpu")
    g.manual_seed(int(seed))
    return g


def sha256(t: torch.Tensor) -> str:
    """SHA-256 of a tensor's raw bytes (for run logs)."""
    t = t.detach().contiguous().cpu()
    return hashlib.sha256(t.view(torch.uint8).numpy().tobytes()).hexdigest()


def normal(M: int, K: int, seed: int, dtype: str = "bf16", std: float = 1.0) -> torch.Tensor:
    """N(0, std^2), drawn in float32 (std applied as one float32 multiply)."""
    x = torch.randn(M, K, generator=_gen(seed), dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(TORCH_DTYPES[dtype])


def activation_family(family: str, M: int, K: int, seed: int, dtype: str = "bf16") -> torch.Tensor:
    """The four dense-activation data families.

    normal:   N(0, 1)
    uniform:  U(-1, 1) = 2 * rand - 1
    outlier:  N(0, 1) with round(0.001 * M * K) positions (seeded randperm) scaled x1000
    special:  per 1x16 block a type drawn uniformly from {all +0; random +-0;
              one N(0,1) constant repeated; that constant with about half the
              entries replaced by +-0; N(0,1) with about a quarter replaced by
              +-0}; rows 0-7 are entirely +-0 (rows whose amax is zero).
    """
    g = _gen(seed)
    if family == "normal":
        x = torch.randn(M, K, generator=g, dtype=torch.float32)
    elif family == "uniform":
        x = 2.0 * torch.rand(M, K, generator=g, dtype=torch.float32) - 1.0
    elif family == "outlier":
        x = torch.randn(M, K, generator=g, dtype=torch.float32)
        n_out = int(round(0.001 * M * K))
        idx = torch.randperm(M * K, generator=g)[:n_out]
        flat = x.view(-1)
        flat[idx] = flat[idx] * 1000.0
    elif family == "special":
        assert K % 16 == 0
        nb = K // 16
        kind = torch.randint(0, 5, (M, nb, 1), generator=g)
        normal_v = torch.randn(M, nb, 16, generator=g, dtype=torch.float32)
        const = torch.randn(M, nb, 1, generator=g, dtype=torch.float32).expand(M, nb, 16)
        zero_sign = torch.randint(0, 2, (M, nb, 16), generator=g).to(torch.float32) * -2.0 + 1.0
        signed_zero = torch.zeros(M, nb, 16) * zero_sign  # +0 or -0
        half = torch.rand(M, nb, 16, generator=g) < 0.5
        quarter = torch.rand(M, nb, 16, generator=g) < 0.25
        x = torch.zeros(M, nb, 16, dtype=torch.float32)
        x = torch.where(kind == 1, signed_zero, x)
        x = torch.where(kind == 2, const, x)
        x = torch.where(kind == 3, torch.where(half, signed_zero, const), x)
        x = torch.where(kind == 4, torch.where(quarter, signed_zero, normal_v), x)
        x = x.reshape(M, K)
        x[: min(8, M)] = signed_zero.reshape(M, K)[: min(8, M)]
    else:
        raise ValueError(family)
    return x.to(TORCH_DTYPES[dtype])


ACTIVATION_FAMILIES = ("normal", "uniform", "outlier", "special")


def weight(M: int, K: int, seed: int, dtype: str = "bf16") -> torch.Tensor:
    """Weights drawn from N(0, 0.02^2)."""
    return normal(M, K, seed, dtype, std=0.02)


def expert_weight_list(n: int, M: int, K: int, seed_base: int, dtypes=("bf16", "fp16")) -> dict:
    """n discrete expert weights, each an FP32 master 0.02 * randn with 1% of
    the entries (seeded randperm) scaled x50, cast to each dtype in ``dtypes``
    from the same master. Returns {dtype: [tensor, ...]}."""
    out = {d: [] for d in dtypes}
    for i in range(n):
        g = _gen(seed_base + i)
        w = torch.randn(M, K, generator=g, dtype=torch.float32) * 0.02
        n_big = int(round(0.01 * M * K))
        idx = torch.randperm(M * K, generator=g)[:n_big]
        flat = w.view(-1)
        flat[idx] = flat[idx] * 50.0
        for d in dtypes:
            out[d].append(w.to(TORCH_DTYPES[d]))
    return out


def group_offsets(G: int, M: int, seed: int, alpha: float = 0.5, multiple: int = 16) -> np.ndarray:
    """Cumulative end offsets of G token groups over M rows: group sizes
    from Dirichlet(alpha), rounded to multiples of ``multiple``; the last
    offset is M; empty groups are allowed."""
    rng = np.random.default_rng(seed)
    p = rng.dirichlet([alpha] * G)
    offs = np.round(np.cumsum(p) * M / multiple).astype(np.int64) * multiple
    offs[-1] = M
    offs = np.maximum.accumulate(np.minimum(offs, M))
    return offs.astype(np.int32)


def group_factors(G: int, seed: int, lo: float = -2.0, hi: float = 2.0) -> np.ndarray:
    """Per-group scale factors drawn log-uniformly from [10^lo, 10^hi]."""
    rng = np.random.default_rng(seed)
    return (10.0 ** rng.uniform(lo, hi, size=G)).astype(np.float32)


def grouped_tokens(M: int, pad: int, K: int, G: int, seeds=(51, 52, 53, 54), dtype: str = "bf16"):
    """Packed MoE token tensor of M logical rows plus ``pad`` over-allocated
    rows. Group g's rows are N(0,1) * f_g; the padding rows hold seeded
    garbage (N(0,1) * 1e4 with some NaN) that a correct quantizer never reads.
    Returns (x[M + pad, K], offs[G] int32, factors[G] float32)."""
    s_offs, s_fac, s_data, s_pad = seeds
    offs = group_offsets(G, M, s_offs)
    fac = group_factors(G, s_fac)
    x = torch.randn(M + pad, K, generator=_gen(s_data), dtype=torch.float32)
    starts = np.concatenate([[0], offs[:-1]])
    row_fac = np.zeros(M, np.float32)
    for g in range(G):
        row_fac[starts[g]:offs[g]] = fac[g]
    x[:M] = x[:M] * torch.from_numpy(row_fac)[:, None]
    if pad:
        gp = _gen(s_pad)
        garbage = torch.randn(pad, K, generator=gp, dtype=torch.float32) * 1e4
        nan_mask = torch.rand(pad, K, generator=gp) < 0.01
        garbage[nan_mask] = float("nan")
        x[M:] = garbage
    return x.to(TORCH_DTYPES[dtype]), offs, fac


def random_packed_codes(M: int, K: int, seed: int) -> np.ndarray:
    """uint8 [M, K/2] of uniformly random bytes (two random 4-bit codes each)."""
    return np.random.default_rng(seed).integers(0, 256, (M, K // 2), dtype=np.uint8)


def random_block_scales(M: int, K: int, seed: int) -> np.ndarray:
    """uint8 [M, K/16] of uniformly random finite non-negative E4M3 codes (0x00..0x7E)."""
    return np.random.default_rng(seed).integers(0, 0x7F, (M, K // 16), dtype=np.uint8)


def raw_bits(t: torch.Tensor) -> np.ndarray:
    """Host numpy view of a tensor's raw element bits: uint16 for bfloat16
    and float16, float32 for float32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


def from_bits(a: np.ndarray, dtype: str) -> torch.Tensor:
    """Inverse of raw_bits."""
    if dtype == "fp32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).view(TORCH_DTYPES[dtype])
