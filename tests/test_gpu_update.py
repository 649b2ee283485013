"""GPU parity for conv1d_update (through the C ABI) against the oracle: the
speculative-decoding options (num_accepted_tokens, intermediate windows,
output_state_indices) and ring-buffer states (cache_seqlens)."""
import pytest
import torch

import causal_depthwise_short_conv1d_amd as S
import oracle
import workloads as W
from tests.parity import assert_bits, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16

OPTS = ("cache_seqlens", "num_accepted_tokens", "output_state_indices")


def gpu(t):
    return None if t is None else t.to(DEV)


def windows(shape, device, dim_contig):
    """Saved-window buffer (batch, steps, dim, width-1) filled with 2.5,
    stored with unit stride along dim when dim_contig."""
    if not dim_contig:
        return torch.full(shape, 2.5, dtype=BF, device=device)
    b, n, dim, h = shape
    return torch.full((b, n, h, dim), 2.5, dtype=BF, device=device).permute(0, 1, 3, 2)


def both(d, activation="silu", exact=False, in_place=False, use=OPTS + ("intermediate",),
         windows_dim_contig=False, out_like_x=False, w_pitch=None):
    """Run the oracle and the library on the same inputs with the options of
    `d` named in `use`; compare out (tolerance, or bits when exact), the whole
    state cache and the intermediate windows (bits).  The GPU's out is
    contiguous, or laid out like x when out_like_x; the GPU's weights are
    packed, or rows of a (dim, w_pitch) buffer."""
    opts = {k: d[k] for k in OPTS if k in use and d.get(k) is not None}
    inter0 = d.get("intermediate") if "intermediate" in use else None
    x_cpu = d["x"]
    st_ref = d["conv_state"].clone()
    out_ref = torch.full(x_cpu.shape, -3.0, dtype=BF)
    inter_ref = None if inter0 is None else windows(inter0.shape, "cpu", windows_dim_contig)
    oracle.update_general(x_cpu, st_ref, d["weight"], d["bias"], out_ref,
                          cache_indices=d["cache_indices"], intermediate=inter_ref,
                          activation=activation, **opts)
    x = x_cpu.to(DEV)
    st = d["conv_state"].to(DEV)       # keeps the strides of the CPU tensor
    assert st.stride() == d["conv_state"].stride()
    inter = None if inter0 is None else windows(inter0.shape, DEV, windows_dim_contig)
    if in_place:
        out = x
        for bi, line in enumerate(d["cache_indices"].tolist()):
            if out_ref[bi].eq(-3.0).all():      # skipped entry keeps x
                out_ref[bi] = x_cpu[bi]
    elif out_like_x:
        out = torch.full_like(x, -3.0)
        assert out.stride() == x.stride()
    else:
        out = torch.full(x.shape, -3.0, dtype=BF, device=DEV)
    w = gpu(d["weight"])
    if w_pitch is not None:
        buf = torch.zeros(w.shape[0], w_pitch, dtype=BF, device=DEV)
        buf[:, :w.shape[1]] = w
        w = buf[:, :w.shape[1]]
        assert w.stride(0) == w_pitch
    S.conv1d_update(x, st, w, gpu(d["bias"]), activation=activation,
                    cache_indices=gpu(d["cache_indices"]), intermediate=inter, out=out,
                    **{k: gpu(v) for k, v in opts.items()})
    torch.cuda.synchronize()
    if exact:
        assert_bits(out, out_ref, "update out")
    else:
        assert_close(out, out_ref, "update out")
    assert_bits(st, st_ref, "update state")
    if inter is not None:
        assert_bits(inter, inter_ref, "update windows")


# ------------------------------------------------------ speculative: roll --

@pytest.mark.parametrize("state_layout", ["dim_contig", "tok_contig"])
def test_spec_roll_full_size(state_layout):
    """64 entries x dim 8192, width 4, 4 tokens each (4 of them pads), 256
    lines: the speculative verify step at the size of the long prefill."""
    cfg = W.SPEC_DECODE
    d = W.spec_decode_batch(batch=cfg["batch"], dim=cfg["dim"], width=cfg["width"],
                            seqlen=cfg["seqlen"], num_lines=cfg["num_lines"],
                            n_pad=cfg["n_pad"], seed=W.seed_for(6, 0), mode="roll",
                            state_layout=state_layout)
    say(f"[update] spec roll full size {state_layout}")
    both(d)
    if state_layout == "dim_contig":
        # out laid out like x, as the benchmark launches it: the four-channel kernel
        say("[update] spec roll full size, out like x")
        both(d, out_like_x=True)


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("seqlen", [1, 2, 5, 7])
def test_spec_roll_ragged(width, seqlen):
    d = W.spec_decode_batch(batch=23, dim=300, width=width, seqlen=seqlen,
                            state_len=width + seqlen + 1, num_lines=40, n_pad=3,
                            seed=500 + 10 * width + seqlen, mode="roll")
    both(d)


def test_spec_roll_exact_values_bit_exact():
    d = W.spec_decode_batch(batch=16, dim=777, width=4, seqlen=3, num_lines=20, n_pad=2,
                            seed=531, mode="roll", values="exact")
    both(d, activation=None, exact=True)


def test_spec_roll_in_place():
    d = W.spec_decode_batch(batch=9, dim=1000, width=5, seqlen=3, num_lines=12, n_pad=2,
                            seed=532, mode="roll")
    both(d, in_place=True)


def test_spec_chain_on_gpu():
    """Verify pass, then accept a prefix and verify more, with the state kept
    on the GPU between the calls, against the oracle doing the same."""
    d = W.spec_decode_batch(batch=12, dim=520, width=4, seqlen=4, num_lines=16, n_pad=1,
                            seed=533, mode="roll")
    d2 = W.spec_decode_batch(batch=12, dim=520, width=4, seqlen=4, num_lines=16, n_pad=1,
                             seed=534, mode="roll")
    ones = torch.ones(12, dtype=torch.int32)
    st_ref = d["conv_state"].clone()
    st = d["conv_state"].to(DEV)
    outs = []
    for x_cpu, nacc in ((d["x"], ones), (d2["x"], d2["num_accepted_tokens"])):
        o_ref = torch.full(x_cpu.shape, -3.0, dtype=BF)
        oracle.update_general(x_cpu, st_ref, d["weight"], d["bias"], o_ref,
                              cache_indices=d["cache_indices"], num_accepted_tokens=nacc,
                              activation="silu")
        o = torch.full(x_cpu.shape, -3.0, dtype=BF, device=DEV)
        S.conv1d_update(x_cpu.to(DEV), st, gpu(d["weight"]), gpu(d["bias"]),
                        activation="silu", cache_indices=gpu(d["cache_indices"]),
                        num_accepted_tokens=nacc.to(DEV), out=o)
        outs.append((o, o_ref))
    torch.cuda.synchronize()
    for o, o_ref in outs:
        assert_close(o, o_ref, "chain out")
    assert_bits(st, st_ref, "chain state")


def test_spec_invalid_entries_are_skipped():
    d = W.spec_decode_batch(batch=6, dim=200, width=4, seqlen=2, state_len=5, num_lines=8,
                            seed=535, mode="roll")
    d["num_accepted_tokens"] = torch.tensor([0, 1, 4, 3, -7, 2], dtype=torch.int32)
    both(d)


# --------------------------------------------------- speculative: scatter --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_spec_scatter_windows_and_lines(width):
    d = W.spec_decode_batch(batch=20, dim=650, width=width, seqlen=4, state_len=width + 2,
                            num_lines=128, n_pad=2, seed=540 + width, mode="scatter")
    d["output_state_indices"][0, 1] = 10_000          # out of range: no write
    both(d)


def test_spec_scatter_full_size():
    cfg = W.SPEC_DECODE
    d = W.spec_decode_batch(batch=cfg["batch"], dim=cfg["dim"], width=cfg["width"],
                            seqlen=cfg["seqlen"], num_lines=512, n_pad=cfg["n_pad"],
                            seed=W.seed_for(6, 1), mode="scatter")
    say("[update] spec scatter full size")
    both(d)


def test_spec_intermediate_only_and_lines_only():
    d = W.spec_decode_batch(batch=10, dim=333, width=4, seqlen=3, state_len=5,
                            num_lines=64, n_pad=1, seed=546, mode="scatter")
    both(d, use=("num_accepted_tokens", "intermediate"))
    both(d, use=("num_accepted_tokens", "output_state_indices"))
    both(d, use=("intermediate",))                    # windows without acceptance offsets


def test_spec_scatter_exact_values_bit_exact():
    d = W.spec_decode_batch(batch=8, dim=129, width=5, seqlen=3, state_len=6, num_lines=40,
                            seed=547, mode="scatter", values="exact")
    both(d, activation=None, exact=True)


# ------------------------------------------------------------------- ring --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("extra,seqlen", [(0, 1), (3, 1), (4, 3), (2, 11)])
def test_ring(width, extra, seqlen):
    d = W.ring_decode_batch(batch=19, dim=260, width=width, seqlen=seqlen,
                            state_len=width - 1 + extra, num_lines=32, n_pad=2,
                            seed=560 + 10 * width + extra)
    both(d)


def test_ring_full_size_and_negative_counts():
    d = W.ring_decode_batch(batch=64, dim=8192, width=4, seqlen=1, state_len=8,
                            num_lines=256, n_pad=4, seed=W.seed_for(6, 2))
    d["cache_seqlens"][5] = -1
    say("[update] ring full size")
    both(d)


def test_ring_exact_values_bit_exact():
    d = W.ring_decode_batch(batch=7, dim=100, width=3, seqlen=5, state_len=4, num_lines=9,
                            seed=571, values="exact")
    both(d, activation=None, exact=True)


# ------------------------------------------------- channel-contiguous --
# x, out, the state lines and the saved windows all with unit stride along
# dim and dim % 4 == 0: the kernel then moves four channels per lane.  Two
# workgroups of channels (the second partial), one and six tokens (two
# groups of inputs), every mode.

MODES = ("plain", "roll", "roll_in_place", "scatter_windows", "scatter_lines", "ring")


def channel_contiguous_batch(mode, width, seqlen, values):
    seed = 590 + 10 * width + seqlen + MODES.index(mode) * 100
    dim, batch = 1156, 7
    if mode == "ring":
        return W.ring_decode_batch(batch=batch, dim=dim, width=width, seqlen=seqlen,
                                   state_len=width + 2, num_lines=10, n_pad=1, seed=seed,
                                   values=values, state_layout="dim_contig")
    kind = "scatter" if mode.startswith("scatter") else "roll"
    lines = batch * (seqlen + 1) + 3 if kind == "scatter" else 10
    return W.spec_decode_batch(batch=batch, dim=dim, width=width, seqlen=seqlen,
                               state_len=width - 2 + seqlen + 1 if kind == "roll" else width,
                               num_lines=lines, n_pad=1, seed=seed, mode=kind, values=values,
                               state_layout="dim_contig")


@pytest.mark.parametrize("seqlen", [1, 6])
@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("mode", MODES)
def test_channel_contiguous_layouts(mode, width, seqlen):
    use = {"plain": (), "roll": ("num_accepted_tokens",),
           "roll_in_place": ("num_accepted_tokens",),
           "scatter_windows": ("num_accepted_tokens", "intermediate", "output_state_indices"),
           "scatter_lines": ("num_accepted_tokens", "output_state_indices"),
           "ring": ("cache_seqlens",)}[mode]
    # six tokens: taps from a pitched weight buffer (the per-channel tap loads)
    kw = dict(use=use, in_place=mode == "roll_in_place",
              windows_dim_contig=mode == "scatter_windows", out_like_x=True,
              w_pitch=width + 3 if seqlen == 6 else None)
    d = channel_contiguous_batch(mode, width, seqlen, "exact")
    assert d["x"].stride(1) == 1 and d["conv_state"].stride(1) == 1
    both(d, activation=None, exact=True, **kw)
    d = channel_contiguous_batch(mode, width, seqlen, "normal")
    both(d, activation="silu", **kw)


# ------------------------------------------------------------ plain mode --

def test_plain_update_equals_decode_entry_point():
    d = W.decode_batch(batch=33, dim=4096, width=4, seqlen=2, seed=580, num_lines=40,
                       n_pad=3)
    x = d["x"].to(DEV)
    w, b, ci = gpu(d["weight"]), gpu(d["bias"]), gpu(d["cache_indices"])
    st1 = d["conv_state"].to(DEV)
    st2 = st1.clone()
    o1 = torch.full(x.shape, -3.0, dtype=BF, device=DEV)
    o2 = o1.clone()
    S.conv1d_update(x, st1, w, b, activation="silu", cache_indices=ci, out=o1)
    S.conv1d_update_decode(x, st2, w, b, activation="silu", cache_indices=ci, out=o2)
    torch.cuda.synchronize()
    assert_bits(o1, o2, "plain vs decode out")
    assert_bits(st1, st2, "plain vs decode state")
    both(d)
