"""Randomised GPU parity sweep: seeded random configurations of every entry
point, each compared with the oracle -- exact-valued inputs (k/8) bit for
bit without activation, and within the tolerance with SiLU.

The configurations mix what the fixed cases cover one at a time: batch
sizes, zero-length and very short sequences, pads, missing state / bias /
has_initial_state / cache_indices, widths 2..5, ragged channel counts, both
storages, paged block sizes, stream offsets and request mixes, and, for
the single-sequence kernels, every row-length regime
(per-row, short-row and long-row kernels)."""
import pytest
import torch

import causal_depthwise_short_conv1d_amd as S
import oracle
import workloads as W
from tests.parity import assert_bits, assert_close, say
from tests.test_gpu_fwd import check_full, to_dev

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def place_x(g, x, layout):
    """x (dim, T) on the device in the given storage; channel-contiguous rows
    get a pitch rounded up to 8 elements (16-byte aligned rows)."""
    dim, T = x.shape
    if layout == "tok_dim":
        pitch = (dim + 7) // 8 * 8
        buf = torch.zeros(T, pitch, dtype=BF, device=DEV)
        buf[:, :dim] = x.t().to(DEV)
        g["x"] = buf[:, :dim].t()
    else:
        g["x"] = x.contiguous().to(DEV)
    return g


@pytest.mark.parametrize("case", range(48))
def test_random_varlen_forward(case):
    r = torch.Generator().manual_seed(5000 + case)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=r))
    width = ri(2, 5)
    layout = ("dim_tok", "tok_dim")[case % 2]
    single = case % 3 == 0
    if single:
        # one sequence: per-row (T < 16), short-row (16..2047) and long-row
        # (>= 2048) regimes of the token-contiguous path
        T = (ri(1, 15), ri(16, 2047), ri(2048, 5000))[case % 9 // 3]
        lens = [T]
        dim = ri(1, 96)
    else:
        nseq = ri(2, 40)
        lens = [ri(0, 3) if ri(0, 3) == 0 else ri(0, 300) for _ in range(nseq)]
        if case % 4 == 1:
            lens.append(ri(2048, 3000))          # rows long enough for the streaming varlen kernel
        dim = ri(1, 80)
    n_pad = 0 if len(lens) < 3 else ri(0, 2)
    d = W.varlen_batch(lengths=lens, dim=dim, width=width, seed=6000 + case,
                       num_lines=len(lens) + ri(0, 4), n_pad=n_pad, layout="dim_tok",
                       values="exact", with_bias=ri(0, 1) == 1)
    if ri(0, 4) == 0:
        d["has_initial_state"] = None
    if ri(0, 5) == 0:
        d["conv_states"] = None
        d["has_initial_state"] = None
    elif ri(0, 5) == 0 and n_pad == 0:
        d["cache_indices"] = None
        d["conv_states"] = d["conv_states"][:len(lens)].contiguous()
    x = d.pop("x")
    g = place_x(to_dev(d), x, layout)
    label = f"random fwd {case}: {layout} dim {dim} W{width} lens {lens[:6]}{'...' if len(lens) > 6 else ''}"
    check_full(g, activation=None, exact=True, label=label)
    check_full(g, activation="silu", label=label + " silu")


@pytest.mark.parametrize("case", range(24))
def test_random_update(case):
    """Plain decode update: random batch, channel count (whole four-channel
    groups in half the cases), token count, width, pads, bias and out
    storage, bit for bit with exact values."""
    r = torch.Generator().manual_seed(7000 + case)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=r))
    width = ri(2, 5)
    batch, dim, seqlen = ri(1, 12), ri(1, 700), ri(1, 6)
    if case % 2 == 0:
        dim = 4 * ri(1, 400)              # whole four-channel groups
    n_pad = ri(0, 2) if batch > 2 else 0
    d = W.decode_batch(batch=batch, dim=dim, width=width, seqlen=seqlen, seed=7100 + case,
                       num_lines=batch + ri(0, 3), n_pad=n_pad, values="exact",
                       with_bias=ri(0, 1) == 1)
    x, ci = d["x"], d["cache_indices"]
    st_ref = d["conv_state"].clone()
    out_ref = torch.full(x.shape, -5.0, dtype=BF)
    oracle.update_decode(x, st_ref, d["weight"], d["bias"], out_ref, cache_indices=ci,
                         activation=None)
    st_gpu = d["conv_state"].to(DEV)
    x_dev = x.to(DEV)
    # out contiguous, or laid out like x (channel-contiguous)
    out = (torch.full_like(x_dev, -5.0) if ri(0, 1) == 1
           else torch.full(x.shape, -5.0, dtype=BF, device=DEV))
    S.conv1d_update(x_dev, st_gpu, d["weight"].to(DEV),
                    None if d["bias"] is None else d["bias"].to(DEV), activation=None,
                    cache_indices=ci.to(DEV), out=out)
    torch.cuda.synchronize()
    say(f"[update] random {case}: batch {batch} dim {dim} seqlen {seqlen} W{width} pads {n_pad}")
    assert_bits(out, out_ref, f"random update {case} out")
    assert_bits(st_gpu, st_ref, f"random update {case} state")


@pytest.mark.parametrize("case", range(16))
def test_random_paged(case):
    """Paged insert + conv: random heads, stream width and offset, block
    size, head dim, request mix (decode tokens, prefill chunks), pads, bias,
    residual and width, bit for bit with exact values and no activation."""
    from tests.test_gpu_paged import run_both
    r = torch.Generator().manual_seed(8000 + case)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=r))
    width = ri(2, 5)
    H = ri(1, 12)
    ws = 8 * ri(1, 6)
    D = ws + 8 * ri(0, 4)
    off_s = 8 * ri(0, (D - ws) // 8)
    N = (1, 2, 4, 8, 16)[ri(0, 4)]
    n_decode, n_prefill, chunk = ri(0, 12), ri(0, 4), ri(1, 70)
    if n_decode + n_prefill == 0:
        n_decode = 1
    max_pos = ri(chunk + width, 400)
    blocks_needed = n_decode * (width // N + 2) + n_prefill * ((chunk + width) // N + 2)
    d = W.paged_batch(H=H, ws=ws, N=N, D=D, off_s=off_s, num_blocks=blocks_needed + ri(1, 20),
                      width=width, n_decode=n_decode, n_prefill=n_prefill, chunk=chunk,
                      max_pos=max_pos, pad_frac=0.1 * ri(0, 2), trailing_pad=ri(0, 3),
                      seed=8100 + case, values="exact", with_bias=ri(0, 1) == 1, min_pos=0)
    run_both(d, activation=None, residual=ri(0, 1) == 1, exact=True,
             label=f"random paged {case}: H{H} ws{ws} D{D} off{off_s} N{N} W{width} "
                   f"dec {n_decode} pre {n_prefill}x{chunk}")


@pytest.mark.parametrize("case", range(24))
def test_random_spec_and_ring(case):
    """conv1d_update with the speculative options (state roll, or saved
    windows and lines in either subset) or ring-buffer states: random batch,
    channel count, token count, width, state length, pads, bias, and the
    storage of the states, the windows and out (channel-contiguous storage
    with whole four-channel groups takes the four-channel kernel), bit for
    bit with exact values, and with SiLU within the tolerance."""
    from tests.test_gpu_update import both
    r = torch.Generator().manual_seed(9000 + case)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=r))
    width = ri(2, 5)
    batch, dim, seqlen = ri(1, 12), ri(1, 700), ri(1, 6)
    if case % 2 == 0:
        dim = 4 * ri(1, 400)              # whole four-channel groups
    n_pad = ri(0, 2) if batch > 2 else 0
    kind = ("roll", "scatter", "ring")[case % 3]
    bias = ri(0, 1) == 1
    layout = ("dim_contig", "tok_contig")[ri(0, 1)]
    if kind == "ring":
        d = W.ring_decode_batch(batch=batch, dim=dim, width=width, seqlen=seqlen,
                                state_len=width - 1 + ri(0, 6), num_lines=batch + ri(0, 4),
                                n_pad=n_pad, max_seen=ri(0, 40), seed=9100 + case,
                                values="exact", with_bias=bias, state_layout=layout)
        use = ("cache_seqlens",)
    else:
        extra = ri(0, 3)
        state_len = (width - 2 + seqlen if kind == "roll" else width - 1) + extra
        lines = batch * (seqlen + 1) + ri(0, 5) if kind == "scatter" else batch + ri(0, 4)
        d = W.spec_decode_batch(batch=batch, dim=dim, width=width, seqlen=seqlen,
                                state_len=state_len, num_lines=lines, n_pad=n_pad, mode=kind,
                                seed=9100 + case, values="exact", with_bias=bias,
                                state_layout=layout)
        use = ("num_accepted_tokens",) + (
            (("intermediate", "output_state_indices"), ("intermediate",),
             ("output_state_indices",))[ri(0, 2)] if kind == "scatter" else ())
    kw = dict(use=use, out_like_x=ri(0, 1) == 1, windows_dim_contig=ri(0, 1) == 1)
    say(f"[update] random {kind} {case}: batch {batch} dim {dim} seqlen {seqlen} W{width} "
        f"state_len {d['conv_state'].shape[2]} {layout} pads {n_pad} {kw}")
    both(d, activation=None, exact=True, **kw)
    both(d, activation="silu", **kw)


@pytest.mark.parametrize("case", range(12))
def test_random_paged_multi(case):
    """Several streams in one sconv_paged_fused_multi launch: random stream
    count, order and spacing of the D sub-ranges, block size, request mix,
    pads, bias, residual and width, bit for bit with exact values."""
    from tests.test_gpu_paged import run_multi
    r = torch.Generator().manual_seed(9500 + case)
    ri = lambda lo, hi: int(torch.randint(lo, hi + 1, (1,), generator=r))
    width = ri(2, 5)
    k = ri(2, 4)
    ws = 8 * ri(1, 4)
    gaps = [8 * ri(0, 2) for _ in range(k)]
    starts, at = [], 0
    for gp in gaps:
        starts.append(at + gp)
        at += gp + ws
    D = at + 8 * ri(0, 2)
    order = torch.randperm(k, generator=r).tolist()
    offsets = tuple(starts[i] for i in order)
    N = (1, 2, 4, 8, 16)[ri(0, 4)]
    n_decode, n_prefill, chunk = ri(0, 10), ri(0, 3), ri(1, 60)
    if n_decode + n_prefill == 0:
        n_prefill = 1
    blocks_needed = n_decode * (width // N + 2) + n_prefill * ((chunk + width) // N + 2)
    d = W.paged_multi_batch(offsets=offsets, seed=9600 + case, values="exact",
                            with_bias=ri(0, 1) == 1, H=ri(1, 6), ws=ws, N=N, D=D,
                            num_blocks=blocks_needed + ri(1, 10), width=width,
                            n_decode=n_decode, n_prefill=n_prefill, chunk=chunk,
                            max_pos=ri(chunk + width, 300), pad_frac=0.1 * ri(0, 2),
                            trailing_pad=ri(0, 2), min_pos=0)
    run_multi(d, activation=None, residual=ri(0, 1) == 1, exact=True,
              label=f"random multi {case}: offs {offsets} ws{ws} D{D} N{N} W{width} "
                    f"dec {n_decode} pre {n_prefill}x{chunk}")
