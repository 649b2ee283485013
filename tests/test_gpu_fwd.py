"""GPU parity for conv1d_fwd_varlen (through the C ABI) against the oracle.

Sizes: every named workload at full size (the long prefill and the width-4
varlen batch compare every output with the oracle; the other varlen widths
compare a channel sample and check the state of every channel), plus many
small seeded cases that span several tiles, the ragged tail and every edge
case: widths 2..5, both storages, pads, zero and short sequences, missing
optional tensors, strided states.
"""
import pytest
import torch

import causal_depthwise_short_conv1d_amd as S
import oracle
import workloads as W
from tests.parity import assert_bits, assert_close, sample_channels, say

pytestmark = pytest.mark.gpu
BF = torch.bfloat16
DEV = "cuda"


def to_dev(d):
    r = {}
    for k, v in d.items():
        if isinstance(v, torch.Tensor):
            t = v.to(DEV)
            assert t.stride() == v.stride() or v.numel() <= 1
            r[k] = t
        else:
            r[k] = v
    return r


def run_gpu(d, activation="silu", pad_slot_id=-1, out_fill=None):
    out = S.new_output(d["x"])
    if out_fill is not None:
        out.fill_(out_fill)
    cs = d["conv_states"].clone() if d.get("conv_states") is not None else None
    S.conv1d_fwd_varlen(d["x"], d["weight"], d.get("bias"), cs, d["query_start_loc"],
                        cache_indices=d.get("cache_indices"),
                        has_initial_state=d.get("has_initial_state"),
                        activation=activation, pad_slot_id=pad_slot_id, out=out)
    torch.cuda.synchronize()
    return out, cs


def run_oracle(d, activation="silu", pad_slot_id=-1, out_fill=None, channels=None):
    """Oracle on CPU copies; with `channels`, only those channels (all tokens)."""
    def cpu(t):
        return None if t is None else t.cpu()
    x, w, b, cs = d["x"], d["weight"], d.get("bias"), d.get("conv_states")
    if channels is not None:                   # select on the device: only those rows move
        x, w = x[channels.to(x.device)], w[channels.to(w.device)]
        b = b[channels.to(b.device)] if b is not None else None
        cs = cs[:, channels.to(cs.device)] if cs is not None else None
    x, w, b, cs = cpu(x), cpu(w), cpu(b), cpu(cs)
    cs = cs.clone() if cs is not None else None
    out = torch.full(x.shape, 0.0 if out_fill is None else out_fill, dtype=BF)
    oracle.fwd_varlen(x, w, b, cs, cpu(d["query_start_loc"]), out,
                      cache_indices=cpu(d.get("cache_indices")),
                      has_initial_state=cpu(d.get("has_initial_state")),
                      activation=activation, pad_slot_id=pad_slot_id)
    return out, cs


def check_full(d, activation="silu", pad_slot_id=-1, exact=False, label=""):
    say(f"[fwd] {label} x{tuple(d['x'].shape)} strides={d['x'].stride()} W={d['weight'].shape[1]}")
    g_out, g_cs = run_gpu(d, activation, pad_slot_id, out_fill=-7.0)
    r_out, r_cs = run_oracle(d, activation, pad_slot_id, out_fill=-7.0)
    if exact:
        assert_bits(g_out, r_out, f"{label} out")
    else:
        assert_close(g_out, r_out, f"{label} out")
    if g_cs is not None:
        assert_bits(g_cs, r_cs, f"{label} state")


# ------------------------------------------------------- named workloads --

def test_smallest_single_sequence():
    d = to_dev(W.single_sequence(**W.SINGLE_SEQ_SMALL, seed=W.seed_for(1)))
    check_full(d, label="dim256 T16")


@pytest.mark.parametrize("T", W.PREFILL_SWEEP_DIM4096["Ts"])
@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_prefill_sweep_dim4096(T, layout):
    d = to_dev(W.single_sequence(dim=4096, T=T, width=4, seed=W.seed_for(2, T % 97),
                                 layout=layout))
    check_full(d, label=f"dim4096 T{T} {layout}")


@pytest.mark.parametrize("T", W.LONG_PREFILL_DIM8192["Ts"])
def test_long_prefill_dim8192(T):
    """The benchmark launch: token-contiguous (dim, T), dim 8192, width 4 --
    every output and every state value compared with the oracle."""
    d = W.single_sequence(dim=8192, T=T, width=4, seed=W.seed_for(3, T % 97), device=DEV)
    say(f"[fwd] dim8192 T{T} full-size launch, full comparison")
    g_out, g_cs = run_gpu(d)
    r_out, r_cs = run_oracle(d)
    assert_close(g_out, r_out, f"T{T} out")
    assert_bits(g_cs, r_cs, f"T{T} state")


# Row lengths for the long-row kernel (rows of at least 2048 tokens).  Its
# waves hold 1536 elements (three rounds) for 3072 <= T < 10000 and 2048
# (four rounds) otherwise; T = k * wave - 1 puts the head of row c at
# offset wave - c inside a wave, so rows 1..3 have heads whose first width-1
# tokens cross into the next wave (4607 and 10239 for the two wave sizes).
LONG_ROW_TS = [2048, 2049, 2050, 3075, 4093, 4095, 4096, 4607, 10239]
LONG_ROW_DIM = 72


def long_wave_elems(T):
    return 1536 if 3072 <= T < 10000 else 2048


def test_long_row_cases_cross_every_wave_size():
    """Each wave size and width 3..5 has a case with a row head that crosses
    into the next wave (width 2 has a single history token, which cannot)."""
    for elems in (1536, 2048):
        for width in (3, 4, 5):
            assert any((c * T) % elems > elems - (width - 1)
                       for T in LONG_ROW_TS if long_wave_elems(T) == elems
                       for c in range(1, LONG_ROW_DIM)), (elems, width)


@pytest.mark.parametrize("T", LONG_ROW_TS)
@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("init", [True, False])
def test_long_rows_every_head_position(T, width, init):
    """Rows of at least one wave: row heads land at every offset inside the
    waves of both wave sizes, including heads whose first width-1 tokens
    cross into the next wave and waves that start inside another wave's
    head."""
    d = W.single_sequence(dim=LONG_ROW_DIM, T=T, width=width, seed=T * 10 + width, values="exact")
    if not init:
        d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    g = to_dev(d)
    check_full(g, activation=None, exact=True, label=f"long rows T{T} W{width} init={init}")
    check_full(g, activation="silu", label=f"long rows T{T} W{width} silu")


def lead_and_cut_waves(T, dim, width):
    """Long-row waves that start at most width-2 tokens into a row (they own
    that row's head, whose first tokens lie just before them) and end inside
    the next row's head, whose first tokens the next wave owns."""
    elems, H, n = long_wave_elems(T), width - 1, dim * T
    hits = []
    for w in range((n + elems - 1) // elems):
        e0 = w * elems
        e_last = min(e0 + elems, n) - 1
        c = e0 // T
        row_end = (c + 1) * T
        if e0 - c * T <= H - 1 and row_end <= e_last and row_end + H - 1 > e_last:
            hits.append(w)
    return hits


@pytest.mark.parametrize("width", [4, 5])
def test_long_rows_wave_with_head_before_and_cut_after(width):
    """T 2049, dim 2048: waves 2046-2047 start 2-3 tokens into a row and end
    1-2 tokens into the next one -- both boundary spans of one wave."""
    T, dim = 2049, 2048
    assert lead_and_cut_waves(T, dim, width)
    d = W.single_sequence(dim=dim, T=T, width=width, seed=T + width, values="exact")
    g = to_dev(d)
    check_full(g, activation=None, exact=True, label=f"lead+cut T{T} dim{dim} W{width}")
    check_full(g, activation="silu", label=f"lead+cut T{T} dim{dim} W{width} silu")


@pytest.mark.parametrize("T", [16, 17, 18, 19, 20, 23, 24, 25, 31, 33, 100, 127, 128, 129,
                               514, 1000, 1023, 1024, 2047])
@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_short_rows_every_head_position(T, width):
    """Rows of 16..2047 tokens: a chunk holds at most one row start; the
    row's owner computes the head outputs that spill into the next chunk."""
    d = W.single_sequence(dim=72, T=T, width=width, seed=T * 10 + width + 7, values="exact")
    g = to_dev(d)
    check_full(g, activation=None, exact=True, label=f"short rows T{T} W{width}")
    check_full(g, activation="silu", label=f"short rows T{T} W{width} silu")
    g["has_initial_state"] = torch.zeros(1, dtype=torch.bool, device=DEV)
    check_full(g, activation=None, exact=True, label=f"short rows T{T} W{width} no init")


@pytest.mark.parametrize("T,dim", [(33, 130000), (47, 96000), (1000, 4200), (100, 170000),
                                   (2047, 8200)])
def test_short_rows_two_and_four_rounds(T, dim):
    """Sizes that select the two- and four-round short-row variants (a wave
    spans up to 64 rows), ragged row lengths, every output compared."""
    d = W.single_sequence(dim=dim, T=T, width=4, seed=T + dim, values="exact", device=DEV)
    say(f"[fwd] short rows T{T} dim{dim}")
    check_full(d, activation=None, exact=True, label=f"short rows T{T} dim{dim}")
    check_full(d, activation="silu", label=f"short rows T{T} dim{dim} silu")


@pytest.mark.parametrize("T", list(range(1, 16)))
@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_very_short_rows(T, width):
    d = W.single_sequence(dim=300, T=T, width=width, seed=T * 10 + width + 9, values="exact")
    g = to_dev(d)
    check_full(g, activation=None, exact=True, label=f"very short rows T{T} W{width}")
    check_full(g, activation="silu", label=f"very short rows T{T} W{width} silu")
    g["has_initial_state"] = torch.zeros(1, dtype=torch.bool, device=DEV)
    check_full(g, activation=None, exact=True, label=f"very short rows T{T} W{width} no init")


# One sequence in token-contiguous rows of at least 2048 tokens (the long-row
# kernel): every way of describing the sequence -- a cache line other than 0,
# a pad, no history, no state, no bias, no has_initial_state array, and a
# sequence that ends before T -- at every width.
ONE_TOK_CASES = [
    (2051, 40, 4, "line5"), (2500, 24, 2, "pad"), (3000, 33, 3, "no_init"),
    (2049, 16, 5, "no_state"), (4099, 20, 4, "no_bias"), (2100, 36, 5, "no_has_init"),
    (2048, 8, 3, "end_short"), (4096, 12, 2, "line5"),
]


@pytest.mark.parametrize("T,dim,width,variant", ONE_TOK_CASES)
def test_one_sequence_long_rows_variants(T, dim, width, variant):
    d = W.single_sequence(dim=dim, T=T, width=width, seed=T * 3 + dim + width, values="exact")
    if variant == "line5":
        d["conv_states"] = W._draw((8, dim, width - 1), W._gen(T, "cpu"), "cpu", "exact")
        d["cache_indices"] = torch.tensor([5], dtype=torch.int32)
    elif variant == "pad":
        d["cache_indices"] = torch.tensor([-1], dtype=torch.int32)
    elif variant == "no_init":
        d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    elif variant == "no_state":
        d["conv_states"] = None
        d["has_initial_state"] = None
    elif variant == "no_bias":
        d["bias"] = None
    elif variant == "no_has_init":
        d["has_initial_state"] = None
    elif variant == "end_short":
        d["query_start_loc"] = torch.tensor([0, T - 3], dtype=torch.int32)
    say(f"[fwd] one sequence (dim,T) long rows T{T} dim{dim} W{width} {variant}")
    g = to_dev(d)
    check_full(g, activation=None, exact=True, label=f"long one seq T{T} dim{dim} W{width} {variant}")
    check_full(g, activation="silu", label=f"long one seq T{T} dim{dim} W{width} {variant} silu")


def strided_taps(g, width):
    """The weights as a (dim, width) view with row stride width + 3 that starts
    one element into its storage, and the bias one element in: taps whose
    rows start at every 2-byte alignment, read through each kernel's general
    path."""
    dim = g["weight"].shape[0]
    wide = torch.zeros(dim, width + 3, dtype=BF, device=DEV)
    wide[:, 1:1 + width] = g["weight"]
    g["weight"] = wide[:, 1:1 + width]
    if g.get("bias") is not None:
        b = torch.zeros(dim + 1, dtype=BF, device=DEV)
        b[1:] = g["bias"]
        g["bias"] = b[1:]
    assert g["weight"].stride() == (width + 3, 1)
    return g


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("case", ["long_dim_tok", "varlen_dim_tok", "varlen_tok_dim", "one_tok_dim"])
def test_strided_misaligned_weights(width, case):
    if case == "long_dim_tok":
        d = W.single_sequence(dim=24, T=2300, width=width, seed=900 + width, values="exact")
    elif case == "one_tok_dim":
        d = W.single_sequence(dim=264, T=300, width=width, seed=910 + width, values="exact",
                              layout="tok_dim")
    else:
        lens = [700, 1, 2, 3, 2500, 9, 1200]
        d = W.varlen_batch(lengths=lens, dim=40, width=width, seed=920 + width, num_lines=12,
                           n_pad=1, values="exact",
                           layout="dim_tok" if case == "varlen_dim_tok" else "tok_dim")
    g = strided_taps(to_dev(d), width)
    say(f"[fwd] strided weights {case} W{width}")
    check_full(g, activation=None, exact=True, label=f"strided weights {case} W{width}")
    check_full(g, activation="silu", label=f"strided weights {case} W{width} silu")


@pytest.mark.parametrize("T,start", [(100, 5), (10, 3), (3000, 2)])
def test_single_sequence_not_starting_at_zero(T, start):
    """query_start_loc [start, T] (outside the documented contract, which
    asks for a leading 0): the kernels still follow the oracle, which covers
    tokens [start, T) only."""
    d = W.single_sequence(dim=40, T=T, width=4, seed=T + start, values="exact")
    d["query_start_loc"] = torch.tensor([start, T], dtype=torch.int32)
    check_full(to_dev(d), activation=None, exact=True, label=f"start {start} T{T}")


def test_prefill_dim8192_T1024_four_round_short_rows():
    """Large enough for the four-round short-row variant."""
    d = W.single_sequence(dim=8192, T=1024, width=4, seed=W.seed_for(3, 1), device=DEV)
    g_out, g_cs = run_gpu(d)
    r_out, r_cs = run_oracle(d)
    assert_close(g_out, r_out, "dim8192 T1024 out")
    assert_bits(g_cs, r_cs, "dim8192 T1024 state")


def test_long_prefill_channel_contiguous():
    T = 4195
    d = W.single_sequence(dim=8192, T=T, width=4, seed=W.seed_for(3, 50), device=DEV,
                          layout="tok_dim")
    g_out, g_cs = run_gpu(d)
    ch = sample_channels(8192, 64, seed=5)
    r_out, r_cs = run_oracle(d, channels=ch)
    assert_close(g_out[ch.to(DEV)], r_out, "T4195 (T,dim) sampled out")
    assert_bits(g_cs[0], d["x"][:, T - 3:], "T4195 (T,dim) state")


@pytest.mark.parametrize("layout,T", [("dim_tok", (2 ** 32 - 1) // 8192), ("tok_dim", 300000)])
def test_largest_single_sequence(layout, T):
    """The largest (dim, T) sequence the 32-bit element indexing of the
    token-contiguous kernels accepts (dim 8192, T 524287: 2^32 - 8192
    elements, 8.6 GB per tensor), and a (T, dim) sequence past 2^31 elements:
    sampled channels against the oracle, every state value against the
    sequence's last width-1 inputs."""
    dim = 8192
    d = W.single_sequence(dim=dim, T=T, width=4, seed=W.seed_for(3, 77), device=DEV, layout=layout)
    say(f"[fwd] largest single sequence {layout} dim{dim} T{T}")
    g_out, g_cs = run_gpu(d)
    ch = sample_channels(dim, 24, seed=T % 1000)
    r_out, r_cs = run_oracle(d, channels=ch)
    assert_close(g_out[ch.to(DEV)], r_out, f"{layout} T{T} sampled out")
    assert_bits(g_cs[0], d["x"][:, T - 3:], f"{layout} T{T} state")
    del d, g_out, g_cs
    torch.cuda.empty_cache()


def test_largest_varlen_token_contiguous():
    """A 64-sequence batch in token-contiguous rows at the 32-bit element
    limit (dim 8192, 524287 tokens): pads, mixed history, sampled channels
    against the oracle in every sequence and the state property of every
    line."""
    dim, total = 8192, (2 ** 32 - 1) // 8192
    g = torch.Generator().manual_seed(4242)
    cuts = torch.sort(torch.randperm(total - 1, generator=g)[:63] + 1).values
    lens = torch.diff(torch.cat([torch.tensor([0]), cuts, torch.tensor([total])])).tolist()
    d = W.varlen_batch(lengths=lens, dim=dim, width=4, seed=W.seed_for(4, 77), layout="dim_tok",
                       device=DEV)
    say(f"[fwd] largest varlen (dim,T) dim{dim} total_T {total}")
    g_out, g_cs = run_gpu(d, out_fill=-3.0)
    ch = sample_channels(dim, 16, seed=11)
    r_out, r_cs = run_oracle(d, out_fill=-3.0, channels=ch)
    assert_close(g_out[ch.to(DEV)], r_out, "largest varlen sampled out")
    assert_bits(g_cs[:, ch.to(DEV)], r_cs, "largest varlen sampled state")
    del d, g_out, g_cs
    torch.cuda.empty_cache()


# One sequence in (T, dim) rows: four 8-row tiles per workgroup with the
# halos passed on chip; cases for partial last groups (waves past T), idle
# lanes, every width, with and without history or state, a padded sequence,
# row pitches wider than dim (one of them with dim % 4 != 0, which takes the
# general kernel), and sequences that do not cover [0, T) (the general tile
# routine inside the same launch).
ONE_CL_CASES = [
    (64, 256, 4, "plain"), (65, 264, 2, "plain"), (95, 8, 3, "plain"), (97, 520, 5, "plain"),
    (100, 1032, 4, "no_init"), (1000, 264, 4, "no_state"), (333, 256, 5, "pad"),
    (257, 256, 4, "pitch"), (301, 13, 3, "pitch"), (4096, 200, 3, "plain"),
    (130, 8, 2, "start5"), (130, 16, 4, "end_short"), (63, 256, 4, "plain"),
]


@pytest.mark.parametrize("T,dim,width,variant", ONE_CL_CASES)
def test_one_sequence_channel_contiguous(T, dim, width, variant):
    d = W.single_sequence(dim=dim, T=T, width=width, seed=T * 7 + dim + width,
                          layout="tok_dim" if variant != "pitch" else "dim_tok", values="exact")
    if variant == "no_init":
        d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    elif variant == "no_state":
        d["conv_states"] = None
        d["has_initial_state"] = None
    elif variant == "pad":
        d["cache_indices"] = torch.tensor([-1], dtype=torch.int32)
    elif variant == "start5":
        d["query_start_loc"] = torch.tensor([5, T], dtype=torch.int32)
    elif variant == "end_short":
        d["query_start_loc"] = torch.tensor([0, T - 3], dtype=torch.int32)
    gd = to_dev(d)
    if variant == "pitch":                     # rows wider than dim, built on the device
        pitch = (dim + 7) // 8 * 8 + 8
        wide = torch.zeros(T, pitch, dtype=BF, device=DEV)
        wide[:, :dim] = gd["x"].t()
        gd["x"] = wide[:, :dim].t()
    assert gd["x"].stride(0) == 1
    say(f"[fwd] one sequence (T,dim) T{T} dim{dim} W{width} {variant}")
    check_full(gd, activation=None, exact=True, label=f"one seq T{T} dim{dim} W{width} {variant}")
    check_full(gd, activation="silu", label=f"one seq T{T} dim{dim} W{width} {variant} silu")


def varlen_state_property(d, g_cs, width):
    """New state of every channel of every processed line: the last width-1
    entries of (history ++ sequence); untouched lines unchanged."""
    before = d["conv_states"]
    qsl = d["query_start_loc"].tolist()
    lines = d["cache_indices"].tolist()
    init = d["has_initial_state"].tolist()
    want = before.clone()
    for s in range(len(lines)):
        L = qsl[s + 1] - qsl[s]
        if lines[s] == -1 or L == 0:
            continue
        h = before[lines[s]] if init[s] else torch.zeros_like(before[lines[s]])
        u = torch.cat([h, d["x"][:, qsl[s]:qsl[s + 1]]], dim=1)
        want[lines[s]] = u[:, L:L + width - 1]
    assert_bits(g_cs, want, "varlen state (all channels)")


@pytest.mark.parametrize("width", W.VARLEN_BATCH["widths"])
@pytest.mark.parametrize("layout", ["tok_dim", "dim_tok"])
def test_varlen_batch(width, layout):
    d = W.varlen_batch(dim=8192, width=width, seed=W.seed_for(4, width), layout=layout,
                       device=DEV)
    total = int(d["query_start_loc"][-1])
    say(f"[fwd] varlen 64 seqs total_T={total} W={width} {layout}")
    g_out, g_cs = run_gpu(d, out_fill=-7.0)
    if width == 4:
        # every output and state of every channel (about 12 s of oracle time)
        r_out, r_cs = run_oracle(d, out_fill=-7.0)
        assert_close(g_out, r_out, f"varlen W{width} out (all channels)")
        assert_bits(g_cs, r_cs, f"varlen W{width} state (all channels)")
    else:
        ch = sample_channels(8192, 40, seed=width)
        r_out, r_cs = run_oracle(d, out_fill=-7.0, channels=ch)
        assert_close(g_out[ch.to(DEV)], r_out, f"varlen W{width} sampled out")
        assert_bits(g_cs[:, ch.to(DEV)], r_cs, f"varlen W{width} sampled state")
    varlen_state_property(d, g_cs, width)
    # pad sequences' rows untouched in every channel
    qsl = d["query_start_loc"].tolist()
    for s, line in enumerate(d["cache_indices"].tolist()):
        if line == -1:
            assert torch.all(g_out[:, qsl[s]:qsl[s + 1]] == -7.0)


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("seed,dim", [(0, 24), (1, 37)])
def test_varlen_long_rows_token_contiguous(width, seed, dim):
    """A batch in token-contiguous rows of at least one wave: hundreds of
    sequences of 0..24 tokens (starts at every chunk offset, two and more
    starts per chunk, heads shorter than the window) plus a few long ones,
    pads, mixed initial state, and (dim 37) a ragged last chunk; every output
    and state compared bit for bit with exact values."""
    g = torch.Generator().manual_seed(800 + 10 * width + seed)
    lens = torch.randint(0, 25, (300,), generator=g).tolist() + [300, 1000, 7, 0, 513]
    perm = torch.randperm(len(lens), generator=g).tolist()
    lens = [lens[i] for i in perm]
    d = W.varlen_batch(lengths=lens, dim=dim, width=width, seed=810 + width + seed,
                       num_lines=len(lens) + 8, n_pad=12, layout="dim_tok", values="exact")
    assert int(d["query_start_loc"][-1]) >= 2048
    say(f"[fwd] varlen long rows W{width} T={int(d['query_start_loc'][-1])}")
    gd = to_dev(d)
    check_full(gd, activation=None, exact=True, label=f"varlen long rows W{width}")
    check_full(gd, activation="silu", label=f"varlen long rows W{width} silu")


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("lead", [2045, 2046, 2047, 2048])
@pytest.mark.parametrize("init", ["all", "none", "mixed", "null", "no_state", "strided_state"])
def test_varlen_long_starts_at_wave_edges(lead, width, init):
    """Token-contiguous rows of 4101 tokens (2048-token waves, so several
    waves cross a row end): a sequence of 64 tokens starting 3, 2, 1 or 0
    tokens before a wave boundary (its first outputs spill into the next
    wave), one of 63 (the shortest and longest lengths either side of the
    split between the stream and head launches), the next row's first
    sequence starting inside a wave, and a short one across a wave
    boundary; a padded sequence next to the long ones.  Exact values, every
    output and state compared bit for bit."""
    lens = [lead, 64, 63, 1920 + (2047 - lead), 7]
    assert sum(lens) == 4101
    d = W.varlen_batch(lengths=lens, dim=7, width=width, seed=930 + lead + width, num_lines=9,
                       n_pad=0, layout="dim_tok", values="exact")
    d["cache_indices"][2] = W.PAD_SLOT_ID if lead % 2 else d["cache_indices"][2]
    hi = torch.ones(len(lens), dtype=torch.bool)
    if init == "none":
        hi[:] = False
    elif init == "mixed":
        hi[1::2] = False
    d["has_initial_state"] = None if init in ("null", "no_state") else hi
    if init == "no_state":
        d["conv_states"] = None
    elif init == "strided_state":
        # a [lines, width-1, dim] buffer viewed as [lines, dim, width-1]
        cs = d["conv_states"]
        d["conv_states"] = cs.transpose(1, 2).contiguous().transpose(1, 2)
    say(f"[fwd] long starts at wave edges lead {lead} W{width} init {init}")
    gd = to_dev(d)
    check_full(gd, activation=None, exact=True, label=f"wave edges {lead} W{width} {init}")
    check_full(gd, activation="silu", label=f"wave edges {lead} W{width} {init} silu")


@pytest.mark.parametrize("nseq", [63, 64, 65])
@pytest.mark.parametrize("width", [2, 4, 5])
def test_varlen_padded_runs_either_side_of_64_sequences(nseq, width):
    """Token-contiguous rows of 64 and 65 sequences -- either side of the
    batch size up to which a wave keeps the table in its lanes -- with runs
    of adjacent padded sequences (long, short and empty ones), so that chunks
    lie wholly in padded tokens, straddle two padded sequences, or mix padded
    and live tokens.  Exact values; every output (padded rows keep their
    fill) and state compared bit for bit."""
    g = torch.Generator().manual_seed(4000 + 10 * nseq + width)
    lens = torch.randint(1, 90, (nseq,), generator=g).tolist()
    lens[3:7] = [700, 5, 0, 301]                  # a padded run in the middle
    lens[-3:] = [9, 400, 2]                       # and at the end
    d = W.varlen_batch(lengths=lens, dim=11, width=width, seed=4100 + nseq + width,
                       num_lines=nseq + 4, n_pad=0, layout="dim_tok", values="exact")
    for i in (3, 4, 5, 6, nseq - 3, nseq - 2, 20):
        d["cache_indices"][i] = W.PAD_SLOT_ID
    assert int(d["query_start_loc"][-1]) >= 2048
    say(f"[fwd] padded runs nseq {nseq} W{width} T={int(d['query_start_loc'][-1])}")
    gd = to_dev(d)
    check_full(gd, activation=None, exact=True, label=f"padded runs {nseq} W{width}")
    check_full(gd, activation="silu", label=f"padded runs {nseq} W{width} silu")


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
@pytest.mark.parametrize("nseq", [2047, 2048])
def test_varlen_batch_size_at_lds_table_limit(nseq, layout):
    """2047 sequences fill the LDS copy of query_start_loc exactly; 2048 take
    the kernels' global-table path.  Lengths 0..3 (most sequences shorter
    than the window), pads, mixed initial state; every output and state
    compared bit for bit with exact values."""
    g = torch.Generator().manual_seed(nseq)
    lens = torch.randint(0, 4, (nseq,), generator=g).tolist()
    dim = 5 if layout == "dim_tok" else 8              # (T, dim) rows: a multiple of 8
    d = W.varlen_batch(lengths=lens, dim=dim, width=4, seed=nseq + 1, num_lines=nseq + 3,
                       n_pad=40, layout=layout, values="exact")
    assert int(d["query_start_loc"][-1]) >= 2048
    say(f"[fwd] varlen {nseq} sequences {layout}")
    check_full(to_dev(d), activation=None, exact=True, label=f"varlen {nseq} seqs {layout}")


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
@pytest.mark.parametrize("total", [2047, 2048])
def test_varlen_total_tokens_at_wave_limit(total, layout):
    """A batch whose rows are one wave (2048 tokens) long, and one token
    shorter: the two sides of the token-contiguous varlen dispatch."""
    lens = [700, 3, 0, 1, 900, 2, total - 1606]
    d = W.varlen_batch(lengths=lens, dim=67 if layout == "dim_tok" else 72, width=4, seed=total,
                       num_lines=12, n_pad=1, layout=layout, values="exact")
    assert int(d["query_start_loc"][-1]) == total
    check_full(to_dev(d), activation=None, exact=True, label=f"varlen T={total} {layout}")
    check_full(to_dev(d), activation="silu", label=f"varlen T={total} {layout} silu")


# ------------------------------------------------------------ small cases --

SMALL_CASES = []
_rng = torch.Generator().manual_seed(2024)
for i in range(40):
    width = 2 + i % 4
    dim = [1, 3, 8, 13, 64, 520, 1030, 24][i % 8]
    nseq = 1 + int(torch.randint(0, 9, (1,), generator=_rng))
    lens = torch.randint(0, 70, (nseq,), generator=_rng).tolist()
    if i % 5 == 0:
        lens = [int(l) % 4 for l in lens]          # many sequences shorter than the window
    if sum(lens) == 0:
        lens[0] = 5
    SMALL_CASES.append(dict(i=i, width=width, dim=dim, lens=lens,
                            layout="dim_tok" if i % 2 else "tok_dim"))


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: f"c{c['i']}-W{c['width']}-d{c['dim']}-{c['layout']}")
def test_small_varlen_cases(case):
    i = case["i"]
    d = W.varlen_batch(lengths=case["lens"], dim=case["dim"], width=case["width"],
                       seed=300 + i, num_lines=len(case["lens"]) + 3,
                       n_pad=1 if len(case["lens"]) > 2 else 0, layout=case["layout"],
                       with_bias=(i % 3 != 0))
    if i % 7 == 3:
        d["has_initial_state"] = None
    if i % 11 == 4:
        d["cache_indices"] = None
        d["conv_states"] = d["conv_states"][:len(case["lens"])].contiguous()
    act = None if i % 4 == 1 else "silu"
    x = d.pop("x")
    g = to_dev(d)
    if case["layout"] == "tok_dim":
        # channel-contiguous rows must be 16-byte aligned: pad the row pitch
        pitch = (case["dim"] + 7) // 8 * 8
        buf = torch.zeros(x.shape[1], pitch, dtype=BF, device=DEV)
        buf[:, :case["dim"]] = x.t().to(DEV)
        g["x"] = buf[:, :case["dim"]].t()
    else:
        g["x"] = x.contiguous().to(DEV)
    check_full(g, activation=act, label=f"small{i}")


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_exact_values_bit_exact(width, layout):
    """Exact-valued inputs (k/8): every sum is exact in fp32 and bf16, so the
    GPU must reproduce the oracle bit for bit -- this pins tap placement."""
    d = W.varlen_batch(lengths=[1, 2, 700, 3, 0, 1501, 5, 260], dim=520, width=width,
                       seed=400 + width, num_lines=12, n_pad=1, layout=layout,
                       values="exact")
    check_full(to_dev(d), activation=None, exact=True, label=f"exact W{width} {layout}")


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_no_state_no_bias(layout):
    d = W.varlen_batch(lengths=[33, 1, 64, 9], dim=40, width=4, seed=501, num_lines=8,
                       n_pad=0, layout=layout, with_bias=False)
    d["conv_states"] = None
    d["has_initial_state"] = None
    d["cache_indices"] = None
    check_full(to_dev(d), label=f"nostate {layout}")


def test_dim_contiguous_state_storage():
    # the cache stored (lines, width-1, dim) and viewed as (lines, dim, width-1)
    d = W.varlen_batch(lengths=[20, 3, 41], dim=96, width=4, seed=601, num_lines=6,
                       n_pad=0, layout="tok_dim")
    d["conv_states"] = d["conv_states"].transpose(1, 2).contiguous().transpose(1, 2)
    assert d["conv_states"].stride(1) == 1
    check_full(to_dev(d), label="dim-contiguous state")


def test_custom_pad_id():
    d = W.varlen_batch(lengths=[10, 10, 10], dim=16, width=3, seed=701, num_lines=5,
                       n_pad=0, layout="dim_tok")
    d["cache_indices"] = torch.tensor([2, 77, 0], dtype=torch.int32)
    check_full(to_dev(d), pad_slot_id=77, label="pad id 77")


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_split_sequence_bit_identical(layout):
    T, dim = 3000, 1024
    d = to_dev(W.single_sequence(dim=dim, T=T, width=4, seed=801, layout=layout))
    full, st_full = run_gpu(d)
    for k in (1, 2, 3, 1000, 2999):
        cs = d["conv_states"].clone()
        parts = []
        for lo, hi in ((0, k), (k, T)):
            xs = W.to_layout(d["x"][:, lo:hi], layout)
            o = S.conv1d_fwd_varlen(xs, d["weight"], d["bias"], cs,
                                    torch.tensor([0, hi - lo], dtype=torch.int32, device=DEV),
                                    has_initial_state=torch.ones(1, dtype=torch.bool, device=DEV))
            parts.append(o)
        torch.cuda.synchronize()
        assert_bits(torch.cat(parts, dim=1), full, f"split at {k}")
        assert_bits(cs, st_full, f"split state at {k}")


@pytest.mark.parametrize("width", [2, 4, 5])
def test_split_long_rows_chain(width):
    """A (dim, T) sequence cut into pieces of at least 2048 tokens, each run
    by the long-row kernel with the state the previous call wrote (read back
    through the scalar cache by the next launch): outputs and the final
    state bit-identical to one call."""
    T, dim = 7000, 96
    d = to_dev(W.single_sequence(dim=dim, T=T, width=width, seed=830 + width))
    full, st_full = run_gpu(d)
    for cuts in ((2500,), (2048, 4096), (2400, 4700)):
        cs = d["conv_states"].clone()
        parts = []
        bounds = (0,) + cuts + (T,)
        for lo, hi in zip(bounds[:-1], bounds[1:]):
            assert hi - lo >= 2048
            o = S.conv1d_fwd_varlen(d["x"][:, lo:hi].contiguous(), d["weight"], d["bias"], cs,
                                    torch.tensor([0, hi - lo], dtype=torch.int32, device=DEV),
                                    has_initial_state=torch.ones(1, dtype=torch.bool, device=DEV))
            parts.append(o)
        torch.cuda.synchronize()
        assert_bits(torch.cat(parts, dim=1), full, f"W{width} cuts {cuts}")
        assert_bits(cs, st_full, f"W{width} cuts {cuts} state")


def test_repeat_is_deterministic():
    d = W.varlen_batch(dim=2048, nseq=16, max_len=600, width=4, seed=901, device=DEV)
    a, sa = run_gpu(d, out_fill=0.0)      # pad rows are left untouched
    b, sb = run_gpu(d, out_fill=0.0)
    assert_bits(a, b, "repeat out")
    assert_bits(sa, sb, "repeat state")


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_bound_forward_equals_the_call(layout):
    """bind_fwd_varlen marshals once and then launches exactly what
    conv1d_fwd_varlen launches: outputs and states bit-identical over
    repeated steps, each step carrying the state the previous one wrote."""
    d = W.varlen_batch(lengths=[300, 0, 5, 2100, 1], dim=520, width=4, seed=990, num_lines=8,
                       n_pad=1, layout=layout, device=DEV)
    st_a, st_b = d["conv_states"].clone(), d["conv_states"].clone()
    oa = torch.full_like(S.new_output(d["x"]), -3.0)
    ob = torch.full_like(oa, -3.0)
    kw = dict(cache_indices=d["cache_indices"], has_initial_state=d["has_initial_state"],
              activation="silu")
    launch = S.bind_fwd_varlen(d["x"], d["weight"], d["bias"], st_b, d["query_start_loc"],
                               out=ob, **kw)
    assert launch.out is ob
    for step in range(3):
        S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"], st_a, d["query_start_loc"],
                            out=oa, **kw)
        launch()
        torch.cuda.synchronize()
        assert_bits(ob, oa, f"bound forward {layout} step {step} out")
        assert_bits(st_b, st_a, f"bound forward {layout} step {step} state")
