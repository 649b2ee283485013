"""Seeded synthetic inputs for the causal depthwise short convolution.

This module only draws inputs; it computes nothing the convolution computes.
Both the CPU oracle's tests and the GPU path's tests and benchmark take their
inputs from here, so that the two sides see identical bytes.

Workloads follow the pages' own shapes and value distribution:
  * atrex-bench operator #003 "causal_conv1d", section "Input Generation":
    x (dim, T), weight (dim, width), bias (dim,), initial_state
    (1, dim, width-1), every tensor drawn as randn in bf16 and scaled by 0.02,
    in that order; the "Shapes" table gives the (T, dim) pairs.
  * tokenspeed causal_conv1d.py (causal_conv1d_fn docstring): a packed varlen
    batch described by query_start_loc, cache_indices with a pad id, and
    has_initial_state.
  * Inkling sconv.py (module docstring, fused_sconv): a paged cache
    [num_blocks, H, N, D] holding each stream at a D sub-range, a
    block_table, absolute positions and slot_mapping with negative pads.

Every generator is deterministic for a given seed and device.  Large inputs
can be drawn directly on the GPU (``device="cuda"``); values then differ from
the CPU draw of the same seed but are still reproducible.
"""
from __future__ import annotations

import torch

BF16 = torch.bfloat16
PAD_SLOT_ID = -1

# Named workloads (sizes from the pages' tables and the paged-cache docstring).
SINGLE_SEQ_SMALL = dict(dim=256, T=16, width=4)                     # smallest case
PREFILL_SWEEP_DIM4096 = dict(dim=4096, Ts=(1, 128, 256, 514, 1024), width=4)
LONG_PREFILL_DIM8192 = dict(dim=8192, Ts=(4195, 11027, 14807), width=4)
VARLEN_BATCH = dict(dim=8192, nseq=64, max_len=2048, num_lines=256, n_pad=4,
                    widths=(2, 3, 4, 5))
SPEC_DECODE = dict(batch=64, dim=8192, width=4, seqlen=4, num_lines=256, n_pad=4)
PAGED_MIXED = dict(H=32, ws=128, N=16, D=512, off_s=128, num_blocks=4096,
                   width=4, n_decode=32, n_prefill=8, chunk=512, max_pos=8191,
                   pad_frac=0.05)
PAGED_MULTI_OFFSETS = (0, 128, 256, 384)      # four streams filling D = 512


def seed_for(config: int, variant: int = 0) -> int:
    """Seed convention: 1000 + 100 * config + variant."""
    return 1000 + 100 * config + variant


def _gen(seed: int, device) -> torch.Generator:
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(int(seed))
    return g


def _draw(shape, g, device, values: str):
    """One bf16 tensor: 'normal' is randn(bf16) * 0.02 (the benchmark page's
    recipe); 'exact' draws k/8 with k uniform in -4..4, values whose products
    and short sums are exactly representable in bf16 and fp32."""
    if values == "normal":
        return torch.randn(*shape, dtype=BF16, generator=g, device=device) * 0.02
    if values == "exact":
        k = torch.randint(-4, 5, tuple(shape), generator=g, device=device)
        return (k.to(torch.float32) / 8.0).to(BF16)
    raise ValueError(f"unknown value distribution {values!r}")


def to_layout(x_dim_tok: torch.Tensor, layout: str) -> torch.Tensor:
    """Return the same logical (dim, T) tensor stored either token-contiguous
    ('dim_tok', strides (T, 1)) or channel-contiguous ('tok_dim', strides
    (1, dim))."""
    if layout == "dim_tok":
        return x_dim_tok.contiguous()
    if layout == "tok_dim":
        return x_dim_tok.t().contiguous().t()
    raise ValueError(f"unknown layout {layout!r}")


def qsl_from_lengths(lengths) -> torch.Tensor:
    """query_start_loc: int32 offsets with a leading 0 (prefix sums of the
    lengths), as in the varlen docstring's example [5,1,1,1] -> [0,5,6,7,8]."""
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    out = torch.zeros(lengths.numel() + 1, dtype=torch.int64)
    out[1:] = torch.cumsum(lengths, 0)
    return out.to(torch.int32)


def single_sequence(dim: int, T: int, width: int = 4, seed: int = 0,
                    layout: str = "dim_tok", device="cpu",
                    values: str = "normal") -> dict:
    """One sequence exactly as the benchmark page's input generator draws it
    (x, weight, bias, initial_state in that order), plus the varlen
    description of a batch of one (query_start_loc [0, T], has_initial_state
    [True], no cache_indices)."""
    g = _gen(seed, device)
    x = _draw((dim, T), g, device, values)
    weight = _draw((dim, width), g, device, values)
    bias = _draw((dim,), g, device, values)
    state = _draw((1, dim, width - 1), g, device, values)
    return dict(
        x=to_layout(x, layout), weight=weight, bias=bias, conv_states=state,
        query_start_loc=torch.tensor([0, T], dtype=torch.int32, device=device),
        cache_indices=None,
        has_initial_state=torch.ones(1, dtype=torch.bool, device=device),
    )


def varlen_batch(lengths=None, dim: int = 8192, width: int = 4, seed: int = 0,
                 nseq: int = 64, min_len: int = 1, max_len: int = 2048,
                 num_lines: int = 256, n_pad: int = 4, p_init: float = 0.5,
                 layout: str = "tok_dim", device="cpu", values: str = "normal",
                 with_bias: bool = True) -> dict:
    """A packed continuous batch: sequence lengths uniform in
    [min_len, max_len] (or the given list), x logical (dim, total_T), a
    conv_states cache of num_lines lines x [dim, width-1], cache_indices a
    random selection of distinct lines with n_pad entries set to the pad id,
    and has_initial_state drawn Bernoulli(p_init)."""
    g_host = _gen(seed, "cpu")
    if lengths is None:
        lengths = torch.randint(min_len, max_len + 1, (nseq,), generator=g_host)
    lengths = torch.as_tensor(lengths, dtype=torch.int64)
    nseq = lengths.numel()
    if nseq > num_lines:
        raise ValueError("need at least one cache line per sequence")
    qsl = qsl_from_lengths(lengths)
    total = int(qsl[-1])
    lines = torch.randperm(num_lines, generator=g_host)[:nseq].to(torch.int32)
    if n_pad:
        lines[torch.randperm(nseq, generator=g_host)[:n_pad]] = PAD_SLOT_ID
    has_init = torch.rand(nseq, generator=g_host) < p_init

    g = _gen(seed + 1, device)
    x = _draw((dim, total), g, device, values)
    weight = _draw((dim, width), g, device, values)
    bias = _draw((dim,), g, device, values) if with_bias else None
    states = _draw((num_lines, dim, width - 1), g, device, values)
    return dict(
        x=to_layout(x, layout), weight=weight, bias=bias, conv_states=states,
        query_start_loc=qsl.to(device), cache_indices=lines.to(device),
        has_initial_state=has_init.to(device), lengths=lengths,
    )


def decode_batch(batch: int = 1, dim: int = 4096, width: int = 4,
                 seqlen: int = 1, seed: int = 0, num_lines: int | None = None,
                 n_pad: int = 0, device="cpu", values: str = "normal",
                 with_bias: bool = True) -> dict:
    """Decode-step inputs: x (batch, dim, seqlen) stored channel-contiguous per
    token, a state cache of num_lines x [dim, width-1], and cache_indices
    drawn as distinct lines (n_pad of them set to the pad id)."""
    num_lines = batch if num_lines is None else num_lines
    g_host = _gen(seed, "cpu")
    lines = torch.randperm(num_lines, generator=g_host)[:batch].to(torch.int32)
    if n_pad:
        lines[torch.randperm(batch, generator=g_host)[:n_pad]] = PAD_SLOT_ID
    g = _gen(seed + 1, device)
    x = _draw((batch, seqlen, dim), g, device, values).permute(0, 2, 1)
    weight = _draw((dim, width), g, device, values)
    bias = _draw((dim,), g, device, values) if with_bias else None
    state = _draw((num_lines, dim, width - 1), g, device, values)
    return dict(x=x, weight=weight, bias=bias, conv_state=state,
                cache_indices=lines.to(device))


def spec_decode_batch(batch: int = 64, dim: int = 8192, width: int = 4,
                      seqlen: int = 4, state_len: int | None = None, seed: int = 0,
                      num_lines: int = 256, n_pad: int = 0, mode: str = "roll",
                      device="cpu", values: str = "normal",
                      with_bias: bool = True, state_layout: str = "dim_contig") -> dict:
    """A speculative-decoding verify step (tokenspeed causal_conv1d.py,
    causal_conv1d_update with num_accepted_tokens): every entry feeds seqlen
    tokens whose history window starts at column num_accepted - 1 of its
    state line.  num_accepted is uniform over the values that keep the window
    inside the line.  mode "roll": the state line (default length
    width-2+seqlen) is rewritten in place; mode "scatter": the state lines
    are width-1 long and the call saves per-step windows into `intermediate`
    (batch, seqlen, dim, width-1) and into the lines named by
    `output_state_indices` (batch, seqlen), distinct lines outside the ones
    being read, about a quarter of them -1 (no write).  x is
    channel-contiguous per token and, by default, so is the state
    ("dim_contig", unit stride along dim, as the page asks of it)."""
    if mode not in ("roll", "scatter"):
        raise ValueError(f"unknown mode {mode!r}")
    hist = width - 1
    if state_len is None:
        state_len = hist - 1 + seqlen if mode == "roll" else hist
    state_len = max(state_len, hist)
    g_host = _gen(seed, "cpu")
    perm = torch.randperm(num_lines, generator=g_host).to(torch.int32)
    lines = perm[:batch].clone()
    if n_pad:
        lines[torch.randperm(batch, generator=g_host)[:n_pad]] = PAD_SLOT_ID
    hi = state_len - hist + 1
    num_acc = torch.randint(1, hi + 1, (batch,), generator=g_host).to(torch.int32)
    osi = None
    if mode == "scatter":
        free = perm[batch:]
        if free.numel() < batch * seqlen:
            raise ValueError("need num_lines >= batch * (seqlen + 1) for scatter mode")
        osi = free[:batch * seqlen].reshape(batch, seqlen).clone()
        osi[torch.rand(batch, seqlen, generator=g_host) < 0.25] = -1

    g = _gen(seed + 1, device)
    x = _draw((batch, seqlen, dim), g, device, values).permute(0, 2, 1)
    weight = _draw((dim, width), g, device, values)
    bias = _draw((dim,), g, device, values) if with_bias else None
    if state_layout == "dim_contig":
        state = _draw((num_lines, state_len, dim), g, device, values).permute(0, 2, 1)
    elif state_layout == "tok_contig":
        state = _draw((num_lines, dim, state_len), g, device, values)
    else:
        raise ValueError(f"unknown state layout {state_layout!r}")
    out = dict(x=x, weight=weight, bias=bias, conv_state=state,
               cache_indices=lines.to(device), num_accepted_tokens=num_acc.to(device),
               state_len=state_len)
    if mode == "scatter":
        out["intermediate"] = torch.zeros(batch, seqlen, dim, hist, dtype=BF16, device=device)
        out["output_state_indices"] = osi.to(device)
    return out


def ring_decode_batch(batch: int = 64, dim: int = 8192, width: int = 4,
                      seqlen: int = 1, state_len: int = 8, seed: int = 0,
                      num_lines: int = 256, n_pad: int = 0, max_seen: int = 64,
                      device="cpu", values: str = "normal",
                      with_bias: bool = True, state_layout: str = "tok_contig") -> dict:
    """A decode step on ring-buffer states (the cache_seqlens option of
    tokenspeed causal_conv1d_update's docstring): each line holds state_len
    inputs, input n of a stream at column n mod state_len, and
    cache_seqlens counts the inputs seen so far (uniform in [0, max_seen]).
    The state is stored token-contiguous by default, or with unit stride
    along dim ("dim_contig")."""
    g_host = _gen(seed, "cpu")
    lines = torch.randperm(num_lines, generator=g_host)[:batch].to(torch.int32)
    if n_pad:
        lines[torch.randperm(batch, generator=g_host)[:n_pad]] = PAD_SLOT_ID
    seen = torch.randint(0, max_seen + 1, (batch,), generator=g_host).to(torch.int32)
    g = _gen(seed + 1, device)
    x = _draw((batch, seqlen, dim), g, device, values).permute(0, 2, 1)
    weight = _draw((dim, width), g, device, values)
    bias = _draw((dim,), g, device, values) if with_bias else None
    if state_layout == "tok_contig":
        state = _draw((num_lines, dim, state_len), g, device, values)
    elif state_layout == "dim_contig":
        state = _draw((num_lines, state_len, dim), g, device, values).permute(0, 2, 1)
    else:
        raise ValueError(f"unknown state layout {state_layout!r}")
    return dict(x=x, weight=weight, bias=bias, conv_state=state,
                cache_indices=lines.to(device), cache_seqlens=seen.to(device),
                state_len=state_len)


def paged_batch(H: int = 32, ws: int = 128, N: int = 16, D: int = 512,
                off_s: int = 128, num_blocks: int = 4096, width: int = 4,
                n_decode: int = 32, n_prefill: int = 8, chunk: int = 512,
                max_pos: int = 8191, pad_frac: float = 0.05,
                trailing_pad: int = 0, seed: int = 0, device="cpu",
                values: str = "normal", with_bias: bool = False,
                min_pos: int | None = None) -> dict:
    """A mixed paged step: n_decode one-token requests at positions uniform in
    [width-1, max_pos], then n_prefill chunks of `chunk` tokens continuing
    from positions uniform in [width-1, max_pos+1-chunk].  Each request's
    touched logical blocks (from the first tap position to the last written
    position) are dealt distinct physical blocks from one random permutation;
    the rest of block_table holds valid, never-read block ids.  slot_mapping =
    block * N + position % N; a random pad_frac of the rows get slot -1, and
    `trailing_pad` extra rows past the last request are appended as pads.
    The cache is drawn like every other tensor (it is large: 2 GiB at the
    default sizes)."""
    g_host = _gen(seed, "cpu")
    lo = width - 1 if min_pos is None else min_pos
    reqs = []   # (first position, length)
    for _ in range(n_decode):
        reqs.append((int(torch.randint(lo, max_pos + 1, (1,), generator=g_host)), 1))
    for _ in range(n_prefill):
        hi = max(lo, max_pos + 1 - chunk)
        reqs.append((int(torch.randint(lo, hi + 1, (1,), generator=g_host)), chunk))
    num_reqs = len(reqs)
    max_blocks = (max_pos + N) // N
    perm = torch.randperm(num_blocks, generator=g_host)
    bt = torch.randint(0, num_blocks, (max(num_reqs, 1), max_blocks),
                       generator=g_host, dtype=torch.int64)
    used = 0
    positions, slots, lengths = [], [], []
    for r, (p0, n) in enumerate(reqs):
        first_blk = max(p0 - (width - 1), 0) // N
        last_blk = (p0 + n - 1) // N
        k = last_blk - first_blk + 1
        if used + k > num_blocks:
            raise ValueError("not enough physical blocks for the requests")
        bt[r, first_blk:last_blk + 1] = perm[used:used + k]
        used += k
        pos = torch.arange(p0, p0 + n, dtype=torch.int64)
        positions.append(pos)
        slots.append(bt[r, pos // N] * N + pos % N)
        lengths.append(n)
    positions = torch.cat(positions) if positions else torch.zeros(0, dtype=torch.int64)
    slots = torch.cat(slots) if slots else torch.zeros(0, dtype=torch.int64)
    T_actual = positions.numel()
    n_pad = int(round(pad_frac * T_actual))
    if n_pad:
        slots[torch.randperm(T_actual, generator=g_host)[:n_pad]] = -1
    if trailing_pad:
        positions = torch.cat([positions, torch.zeros(trailing_pad, dtype=torch.int64)])
        slots = torch.cat([slots, torch.full((trailing_pad,), -1, dtype=torch.int64)])
    qsl = qsl_from_lengths(lengths)
    T = positions.numel()
    C = H * ws

    g = _gen(seed + 1, device)
    x = _draw((T, C), g, device, values)
    weight = _draw((C, width), g, device, values)
    bias = _draw((C,), g, device, values) if with_bias else None
    cache = _draw((num_blocks, H, N, D), g, device, values)
    return dict(
        x=x, weight=weight, bias=bias, cache=cache,
        positions=positions.to(device), slot_mapping=slots.to(device),
        query_start_loc=qsl.to(device),
        block_table=bt.to(torch.int32).to(device),
        off_s=off_s, ws=ws, block_size=N, requests=reqs,
    )


def paged_multi_batch(offsets=PAGED_MULTI_OFFSETS, seed: int = 0, device="cpu",
                      values: str = "normal", with_bias: bool = False, **paged_kw) -> dict:
    """Several conv streams sharing one paged step (the paged page's module
    docstring: K, V, attention output and MLP output at their own D
    sub-ranges of the same cache).  The shared metadata, the cache and the
    first stream come from paged_batch (with off_s = offsets[0]); every
    further stream gets its own x, weight and (optionally) bias, drawn from
    a generator seeded with seed + 2.  Returns the paged_batch dict plus
    lists xs, weights, biases, offs."""
    base = paged_batch(off_s=offsets[0], seed=seed, device=device, values=values,
                       with_bias=with_bias, **paged_kw)
    T, C = base["x"].shape
    width = base["weight"].shape[1]
    g = _gen(seed + 2, device)
    xs, weights, biases = [base["x"]], [base["weight"]], [base["bias"]]
    for _ in offsets[1:]:
        xs.append(_draw((T, C), g, device, values))
        weights.append(_draw((C, width), g, device, values))
        biases.append(_draw((C,), g, device, values) if with_bias else None)
    return dict(base, xs=xs, weights=weights, biases=biases, offs=list(offsets))
