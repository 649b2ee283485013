"""Comparison helpers for the GPU-vs-oracle parity tests.

Output tolerance (bf16 output, fp32 accumulation on the GPU, fp64 in the
oracle): |gpu - ref| <= 2e-4 + 8e-3 * |ref|.  One bf16 ulp is at most
2^-7 |v| = 7.8e-3 |v|, so a single disagreement in the final rounding always
passes, while a dropped or misplaced tap of the benchmark's N(0,1)*0.02
inputs generally does not (the exact-valued tests pin tap placement
bit-exactly).  State and cache writes are bit copies and must be identical.
"""
from __future__ import annotations

import sys

import torch

ATOL = 2e-4
RTOL = 8e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(gpu: torch.Tensor, ref: torch.Tensor, what: str = "out"):
    g = gpu.detach().to("cpu", torch.float64)
    r = ref.detach().to("cpu", torch.float64)
    assert g.shape == r.shape, (what, g.shape, r.shape)
    both_nan = torch.isnan(g) & torch.isnan(r)
    bad = ((g - r).abs() > ATOL + RTOL * r.abs()) & ~both_nan
    bad |= torch.isnan(g) ^ torch.isnan(r)
    if bad.any():
        idx = bad.nonzero()[0].tolist()
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.numel()} elements out of tolerance; "
            f"first at {idx}: gpu={g[tuple(idx)].item()!r} ref={r[tuple(idx)].item()!r}")


def assert_bits(gpu: torch.Tensor, ref: torch.Tensor, what: str = "state"):
    g = gpu.detach().cpu()
    r = ref.detach().cpu()
    assert g.shape == r.shape, (what, g.shape, r.shape)
    gb = g.contiguous().view(torch.int16)
    rb = r.contiguous().view(torch.int16)
    if not torch.equal(gb, rb):
        bad = (gb != rb)
        idx = bad.nonzero()[0].tolist()
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.numel()} elements differ bitwise; "
            f"first at {idx}: gpu={g[tuple(idx)].item()!r} ref={r[tuple(idx)].item()!r}")


def sample_channels(dim: int, n: int = 48, seed: int = 0) -> torch.Tensor:
    """Channel sample for full-size checks: the edges of the channel range
    and of 8-wide vectors / 512-wide slabs, plus random channels."""
    fixed = {0, 1, 7, 8, 9, 255, 256, 511, 512, 513, dim - 9, dim - 8, dim - 1}
    fixed = {c for c in fixed if 0 <= c < dim}
    g = torch.Generator().manual_seed(seed)
    rnd = torch.randperm(dim, generator=g)[:max(0, n - len(fixed))].tolist()
    return torch.tensor(sorted(fixed | set(rnd)), dtype=torch.long)
