"""GPU parity for the layouts outside the vector kernels' storage classes,
through the C ABI, against the oracle: sliced, pitched, offset, transposed
and broadcast views of x, out, the weights and the paged cache, compact
channel-contiguous batches whose dim is not a multiple of 8, and arrays of
2^32 elements or more (the token-contiguous forward in channel groups, and a
sliced view through the general-stride kernel's 64-bit offsets).

Every view is built on the device around a storage filled with a sentinel;
the elements outside the view must keep it.  Exact-valued inputs (k/8) are
compared bit for bit with the oracle, N(0,1)*0.02 inputs with SiLU within
the output tolerance; states and caches always bit for bit.
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
SENT = -7.0


def view_of(x, kind, fill=0.0):
    """The logical (dim, T) tensor x (any device) as a device view of the
    given kind inside a larger storage filled with `fill`.  Returns
    (view, storage)."""
    dim, T = x.shape
    if kind == "dim_tok":                      # compact token-contiguous
        buf = torch.full((dim, T), fill, dtype=BF, device=DEV)
        v = buf
    elif kind == "tok_dim":                    # compact channel-contiguous (any dim)
        buf = torch.full((T, dim), fill, dtype=BF, device=DEV)
        v = buf.t()
    elif kind == "slice_dim_tok":              # x[:, a:b] of a wider (dim, T) array, odd offset
        buf = torch.full((dim, T + 13), fill, dtype=BF, device=DEV)
        v = buf[:, 5:5 + T]
    elif kind == "pitch_tok_dim":              # (T, dim) rows with an odd pitch, odd offset
        buf = torch.full((T, dim + 3), fill, dtype=BF, device=DEV)
        v = buf[:, 1:1 + dim].t()
    elif kind == "offset_dim_tok":             # compact (dim, T) one element into its storage
        buf = torch.full((dim * T + 1,), fill, dtype=BF, device=DEV)
        v = buf[1:].view(dim, T)
    elif kind == "offset_tok_dim":             # compact (T, dim), 16-byte pitch, 2-byte base
        pitch = (dim + 7) // 8 * 8
        buf = torch.full((T * pitch + 1,), fill, dtype=BF, device=DEV)
        v = buf[1:].view(T, pitch)[:, :dim].t()
    elif kind == "every_other":                # both strides above 1
        buf = torch.full((2 * dim, 3 * T), fill, dtype=BF, device=DEV)
        v = buf[::2, ::3]
    elif kind == "every_other_t":              # the same, channel axis the smaller stride
        buf = torch.full((3 * T, 2 * dim), fill, dtype=BF, device=DEV)
        v = buf[::3, ::2].t()
    else:
        raise ValueError(kind)
    v.copy_(x.to(DEV))
    return v, buf


def outside(buf, view):
    """Mask of the storage elements that the view does not cover."""
    m = torch.ones(buf.numel(), dtype=torch.bool, device=buf.device)
    idx = torch.as_strided(torch.arange(buf.numel(), device=buf.device), view.shape,
                           view.stride(), view.storage_offset() - buf.storage_offset())
    m[idx.reshape(-1)] = False
    return m.view(buf.shape)


def run_oracle(d, activation, pad_slot_id=-1, channels=None):
    cpu = lambda t: None if t is None else t.cpu()
    x, w, b, cs = d["x"], d["weight"], d.get("bias"), d.get("conv_states")
    if channels is not None:
        ch = channels.to(x.device)
        x, w = x[ch], w[ch]
        b = b[ch] if b is not None else None
        cs = cs[:, ch] if cs is not None else None
    x, w, b, cs = cpu(x), cpu(w), cpu(b), cpu(cs)
    cs = cs.clone() if cs is not None else None
    out = torch.full(x.shape, SENT, dtype=BF)
    oracle.fwd_varlen(x.contiguous(), w.contiguous(), b, cs, cpu(d["query_start_loc"]), out,
                      cache_indices=cpu(d.get("cache_indices")),
                      has_initial_state=cpu(d.get("has_initial_state")),
                      activation=activation, pad_slot_id=pad_slot_id)
    return out, cs


def check(d, x_kind, out_kind, activation, exact, label):
    """d: inputs on the CPU (or the device).  x and out are placed as views of
    the given kinds; everything else is moved to the device as is."""
    say(f"[general] {label}: x {x_kind} out {out_kind} W{d['weight'].shape[1]} act={activation}")
    x, _ = view_of(d["x"], x_kind)
    out, obuf = view_of(torch.zeros_like(d["x"]), out_kind, fill=SENT)
    obuf.fill_(SENT)
    dv = lambda t: None if t is None else t.to(DEV)
    cs = dv(d.get("conv_states"))
    cs = cs.clone() if cs is not None else None
    w = d["weight"] if d["weight"].device.type == "cuda" else dv(d["weight"])
    S.conv1d_fwd_varlen(x, w, dv(d.get("bias")), cs, dv(d["query_start_loc"]),
                        cache_indices=dv(d.get("cache_indices")),
                        has_initial_state=dv(d.get("has_initial_state")),
                        activation=activation, out=out)
    torch.cuda.synchronize()
    r_out, r_cs = run_oracle(d, activation)
    (assert_bits if exact else assert_close)(out, r_out, f"{label} out")
    if cs is not None:
        assert_bits(cs, r_cs, f"{label} state")
    assert torch.all(obuf[outside(obuf, out)] == SENT), f"{label}: write outside the out view"


LAYOUTS = [("slice_dim_tok", "slice_dim_tok"), ("pitch_tok_dim", "pitch_tok_dim"),
           ("offset_dim_tok", "offset_dim_tok"), ("offset_tok_dim", "offset_tok_dim"),
           ("dim_tok", "tok_dim"), ("tok_dim", "dim_tok"), ("every_other", "every_other_t"),
           ("every_other_t", "slice_dim_tok")]


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("x_kind,out_kind", LAYOUTS)
def test_varlen_batch_general_layouts(x_kind, out_kind, width):
    """A varlen batch (sequences of 0..700 tokens, several shorter than the
    window, pads, mixed history) in every view kind, exact values bit for
    bit and SiLU within tolerance."""
    lens = [700, 1, 2, 3, 0, 260, 9, 1200, 4, 33]
    d = W.varlen_batch(lengths=lens, dim=37, width=width, seed=1500 + width, num_lines=14,
                       n_pad=2, values="exact")
    check(d, x_kind, out_kind, None, True, f"varlen {x_kind}->{out_kind}")
    dn = W.varlen_batch(lengths=lens, dim=37, width=width, seed=1510 + width, num_lines=14,
                        n_pad=2)
    check(dn, x_kind, out_kind, "silu", False, f"varlen {x_kind}->{out_kind} silu")


@pytest.mark.parametrize("dim,T", [(1, 300), (5, 1), (300, 1), (8, 2500), (1030, 70)])
@pytest.mark.parametrize("x_kind", ["slice_dim_tok", "pitch_tok_dim", "every_other"])
def test_single_sequence_general_edges(dim, T, x_kind):
    """One channel, one token, rows spanning several tiles and a ragged
    tail; no state, no bias and no history variants."""
    for variant in ("plain", "no_state", "no_init"):
        d = W.single_sequence(dim=dim, T=T, width=4, seed=dim * 7 + T, values="exact")
        if variant == "no_state":
            d["conv_states"], d["has_initial_state"], d["bias"] = None, None, None
        elif variant == "no_init":
            d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
        check(d, x_kind, x_kind, None, True, f"one seq dim{dim} T{T} {variant}")


@pytest.mark.parametrize("dim", [37, 1030, 4100])
@pytest.mark.parametrize("width", [2, 4, 5])
def test_compact_channel_contiguous_any_dim(dim, width):
    """A (T, dim) batch stored compactly when dim % 8 != 0 (row pitch = dim,
    the layout the tokenspeed launcher takes)."""
    d = W.varlen_batch(lengths=[300, 5, 2, 999, 64], dim=dim, width=width, seed=1600 + dim,
                       num_lines=8, n_pad=1)
    check(d, "tok_dim", "tok_dim", "silu", False, f"compact (T,dim) dim{dim}")


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_broadcast_and_overlapping_weights(layout, width):
    """One set of taps broadcast to every channel (weight stride 0) and
    weight rows that overlap (stride 1 < width): read-only views, so the
    general kernel takes them in either storage."""
    d = W.varlen_batch(lengths=[500, 3, 1, 800], dim=40, width=width, seed=1700 + width,
                       num_lines=6, n_pad=1, values="exact")
    base = d["weight"][0].to(DEV)
    d["weight"] = base.unsqueeze(0).expand(40, width)
    assert d["weight"].stride() == (0, 1)
    check(d, layout, layout, None, True, f"broadcast taps {layout}")
    store = W._draw((40 + width,), W._gen(1710 + width, "cpu"), "cpu", "exact").to(DEV)
    d["weight"] = torch.as_strided(store, (40, width), (1, 1))
    check(d, layout, layout, None, True, f"overlapping tap rows {layout}")


def test_decode_broadcast_weights():
    """The decode update with taps broadcast to every channel (stride 0)."""
    d = W.decode_batch(batch=6, dim=300, width=4, seqlen=3, seed=1720, num_lines=8, n_pad=1,
                       values="exact")
    st_ref = d["conv_state"].clone()
    w = d["weight"][:1].expand(300, 4)
    out_ref = torch.full(d["x"].shape, SENT, dtype=BF)
    oracle.update_decode(d["x"], st_ref, w.contiguous(), d["bias"], out_ref,
                         cache_indices=d["cache_indices"])
    x = d["x"].to(DEV)
    st = d["conv_state"].to(DEV)
    out = torch.full(x.shape, SENT, dtype=BF, device=DEV)
    wd = d["weight"][:1].to(DEV).expand(300, 4)
    S.conv1d_update_decode(x, st, wd, d["bias"].to(DEV), cache_indices=d["cache_indices"].to(DEV),
                           out=out)
    torch.cuda.synchronize()
    assert_bits(out, out_ref, "decode broadcast taps out")
    assert_bits(st, st_ref, "decode broadcast taps state")


def test_token_contiguous_past_2_32_elements_in_channel_groups():
    """A compact (dim, T) sequence of more than 2^32 elements (dim 8192,
    T 525001): the token-contiguous kernels run it as channel groups of
    fewer than 2^32 elements.  Sampled channels (including both sides of
    the group edge, channel 8176) against the oracle; every state value
    against the sequence's last width-1 inputs."""
    dim, T = 8192, 525001
    assert dim * T >= 2 ** 32
    d = W.single_sequence(dim=dim, T=T, width=4, seed=W.seed_for(3, 78), device=DEV)
    say(f"[general] (dim,T) dim{dim} T{T}: {dim * T} elements")
    cs = d["conv_states"].clone()
    out = S.conv1d_fwd_varlen(d["x"], d["weight"], d["bias"], cs, d["query_start_loc"],
                              has_initial_state=d["has_initial_state"])
    torch.cuda.synchronize()
    ch = torch.unique(torch.cat([sample_channels(dim, 20, seed=3),
                                 torch.tensor([8175, 8176, 8177])]))
    r_out, r_cs = run_oracle(d, "silu", channels=ch)
    assert_close(out[ch.to(DEV)], r_out, "past 2^32 sampled out")
    assert_bits(cs[0], d["x"][:, T - 3:], "past 2^32 state")
    del d, out, cs
    torch.cuda.empty_cache()


def test_sliced_view_past_2_32_elements():
    """A (dim, T) slice of a wider array, more than 2^32 elements in the
    view: the general-stride kernel with 64-bit offsets."""
    dim, T = 8192, 524300
    assert dim * T >= 2 ** 32
    d = W.single_sequence(dim=dim, T=8, width=4, seed=W.seed_for(3, 79), device=DEV)
    buf = torch.empty((dim, T + 8), dtype=BF, device=DEV)
    g = torch.Generator(device=DEV).manual_seed(W.seed_for(3, 79))
    for c0 in range(0, dim, 1024):                      # drawn in slabs to bound the temporaries
        buf[c0:c0 + 1024].normal_(0.0, 0.02, generator=g)
    x = buf[:, 3:3 + T]
    d["x"] = x
    d["query_start_loc"] = torch.tensor([0, T], dtype=torch.int32, device=DEV)
    say(f"[general] sliced (dim,T) view dim{dim} T{T}: {dim * T} elements")
    cs = d["conv_states"].clone()
    out = torch.empty((dim, T), dtype=BF, device=DEV)
    S.conv1d_fwd_varlen(x, d["weight"], d["bias"], cs, d["query_start_loc"],
                        has_initial_state=d["has_initial_state"], out=out)
    torch.cuda.synchronize()
    ch = sample_channels(dim, 16, seed=4)
    r_out, r_cs = run_oracle(d, "silu", channels=ch)
    assert_close(out[ch.to(DEV)], r_out, "sliced past 2^32 sampled out")
    assert_bits(cs[0], x[:, T - 3:], "sliced past 2^32 state")
    del d, out, cs, buf, x
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- paged --

def paged_views(d, x_pitch_extra=3, c_extra=(1, 2, 3), offset=1):
    """The step's x as rows with an odd pitch at an odd element offset, an
    out buffer of the same kind filled with the sentinel, and the cache as a
    view with odd strides inside a larger storage (also filled with the
    sentinel outside the view).  Returns (x, out, out_buf, cache, cache_buf)."""
    T, C = d["x"].shape
    xb = torch.zeros(T * (C + x_pitch_extra) + offset, dtype=BF, device=DEV)
    x = torch.as_strided(xb, (T, C), (C + x_pitch_extra, 1), offset)
    x.copy_(d["x"].to(DEV))
    ob = torch.full((T * (C + x_pitch_extra + 2) + offset,), SENT, dtype=BF, device=DEV)
    out = torch.as_strided(ob, (T, C), (C + x_pitch_extra + 2, 1), offset)
    nb, H, N, D = d["cache"].shape
    sn, sh, sb = D + c_extra[0], N * (D + c_extra[0]) + c_extra[1], 0
    sb = H * sh + c_extra[2]
    cb = torch.full((nb * sb + offset,), SENT, dtype=BF, device=DEV)
    cache = torch.as_strided(cb, (nb, H, N, D), (sb, sh, sn, 1), offset)
    cache.copy_(d["cache"].to(DEV))
    return x, out, ob, cache, cb


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("ws,off_s", [(20, 6), (13, 0), (16, 5), (8, 40)])
def test_paged_general_layouts(width, ws, off_s):
    """Stream widths and D offsets that are not multiples of 8, odd row
    pitches, odd cache strides and 2-byte aligned bases: exact values bit
    for bit (residual, no activation) and SiLU within tolerance; the cache
    bit for bit, and nothing written outside the views."""
    for values, act in (("exact", None), ("normal", "silu")):
        d = W.paged_batch(H=4, ws=ws, N=4, D=48, off_s=off_s, num_blocks=96, n_decode=5,
                          n_prefill=3, chunk=37, max_pos=60, width=width, pad_frac=0.1,
                          trailing_pad=2, seed=1800 + width + ws, values=values,
                          with_bias=width % 2 == 0, min_pos=0)
        say(f"[general] paged ws{ws} off{off_s} W{width} {values}")
        cache_ref = d["cache"].clone()
        out_ref = torch.full(d["x"].shape, float("nan"), dtype=BF)
        oracle.paged(d["x"], d["weight"], d["bias"], cache_ref, d["positions"],
                     d["slot_mapping"], d["query_start_loc"], d["block_table"], off_s, ws,
                     out_ref, activation=act, use_residual=True)
        x, out, ob, cache, cb = paged_views(d)
        dv = lambda t: None if t is None else t.to(DEV)
        S.sconv_paged_fused(x, dv(d["weight"]), cache, dv(d["positions"]),
                            dv(d["slot_mapping"]), dv(d["query_start_loc"]),
                            dv(d["block_table"]), off_s, ws, activation=act,
                            use_residual=True, bias=dv(d["bias"]), out=out)
        torch.cuda.synchronize()
        (assert_bits if values == "exact" else assert_close)(out, out_ref, "paged general out")
        assert_bits(cache, cache_ref, "paged general cache")
        assert torch.all(ob[outside(ob, out)] == SENT), "write outside the out view"
        assert torch.all(cb[outside(cb, cache)] == SENT), "write outside the cache view"


@pytest.mark.parametrize("width", [3, 4])
def test_paged_multi_general_layouts(width):
    """Two streams of widths 20 and 12 at D offsets 0 and 20 (not multiples
    of 8) in one launch; each equals its own oracle step."""
    d = W.paged_multi_batch(offsets=(0, 20), H=4, ws=20, N=4, D=48, num_blocks=96,
                            n_decode=5, n_prefill=3, chunk=37, max_pos=60, width=width,
                            pad_frac=0.1, seed=1900 + width, values="exact", min_pos=0)
    # the second stream is 12 channels wide per head
    d["xs"][1] = d["xs"][1][:, :4 * 12].contiguous()
    d["weights"][1] = d["weights"][1][:4 * 12].contiguous()
    wss = [20, 12]
    cache_ref = d["cache"].clone()
    refs = []
    for i in range(2):
        o = torch.full(d["xs"][i].shape, float("nan"), dtype=BF)
        oracle.paged(d["xs"][i], d["weights"][i], None, cache_ref, d["positions"],
                     d["slot_mapping"], d["query_start_loc"], d["block_table"], d["offs"][i],
                     wss[i], o, activation=None, use_residual=True)
        refs.append(o)
    dv = lambda t: t.to(DEV)
    cache = dv(d["cache"])
    outs = S.sconv_paged_fused_multi([dv(x) for x in d["xs"]], [dv(w) for w in d["weights"]],
                                     cache, dv(d["positions"]), dv(d["slot_mapping"]),
                                     dv(d["query_start_loc"]), dv(d["block_table"]), d["offs"],
                                     wss, activation=None, use_residual=True)
    torch.cuda.synchronize()
    for i in range(2):
        assert_bits(outs[i], refs[i], f"multi general stream {i}")
    assert_bits(cache, cache_ref, "multi general cache")
