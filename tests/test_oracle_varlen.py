"""Pins for the oracle's varlen forward (prefill) and decode update.

Each check ties the oracle to something other than itself:
  * the benchmark page's reference Model.forward (torch conv1d, run in fp64);
  * an exact rational brute force written in "lag" form over tiny inputs;
  * closed forms (width 1, impulse responses), invariants (split sequence,
    power-of-two scaling) and the varlen docstring's structural examples.
"""
import itertools
import json
import os
from fractions import Fraction

import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as W
from tests.exact_ref import (bf16_ulp_half, bits_to_fraction,
                             fraction_to_bf16_bits, tensor_bits)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
BF = torch.bfloat16


def run_fwd(d, activation="silu", out_fill=None, pad_slot_id=-1):
    x = d["x"]
    out = torch.full(x.shape, float("nan") if out_fill is None else out_fill, dtype=BF)
    cs = d["conv_states"].clone() if d.get("conv_states") is not None else None
    oracle.fwd_varlen(x, d["weight"], d.get("bias"), cs, d["query_start_loc"], out,
                      cache_indices=d.get("cache_indices"),
                      has_initial_state=d.get("has_initial_state"),
                      activation=activation, pad_slot_id=pad_slot_id)
    return out, cs


def windowed_reference_fp64(x, weight, bias, history, activation):
    """The forward that the benchmark page's reference implementation
    defines (atrex-bench #003 "causal_conv1d", section "Reference
    Implementation"), evaluated in float64 through torch's window view
    instead of a convolution: with u = (the last width-1 state columns) ++ x,
    output t of channel c is bias[c] + sum_j weight[c, j] * u[c, t + j],
    followed by SiLU y * sigmoid(y)."""
    width = weight.shape[1]
    h = history[0].double()
    u = torch.cat([h[:, h.shape[1] - (width - 1):], x.double()], dim=1)
    win = u.unfold(1, width, 1)                     # win[c, t, j] = u[c, t + j]
    y = (win * weight.double().unsqueeze(1)).sum(dim=-1)
    if bias is not None:
        y = y + bias.double().unsqueeze(1)
    if activation in ("silu", "swish"):
        y = y * torch.sigmoid(y)
    return y


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("T", [1, 2, 3, 7, 33])
@pytest.mark.parametrize("activation", ["silu", None])
@pytest.mark.parametrize("init", [True, False])
def test_matches_benchmark_reference_in_fp64(width, T, activation, init):
    d = W.single_sequence(dim=9, T=T, width=width, seed=100 + T + width)
    if not init:
        d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    out, _ = run_fwd(d, activation)
    state = d["conv_states"] if init else torch.zeros_like(d["conv_states"])
    ref = windowed_reference_fp64(d["x"], d["weight"], d["bias"], state, activation)
    o = out.double()
    # the oracle's bf16 value must be the correctly rounded fp64 result
    assert torch.all((o - ref).abs() <= bf16_ulp_half(ref) * (1 + 1e-9))


@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_layouts_agree(layout):
    d = W.single_sequence(dim=16, T=40, width=4, seed=5)
    base, base_state = run_fwd(d)
    d2 = dict(d, x=W.to_layout(d["x"], layout))
    out, st = run_fwd(d2)
    assert torch.equal(out.contiguous(), base.contiguous())
    assert torch.equal(st, base_state)


# ------------------------------------------------------------------ brute --

def brute_varlen(x, w, b, states, qsl, lines, has_init, width, silu):
    """Exact rational evaluation in lag form: the weight of tap width-1-lag
    multiplies the input `lag` steps back; steps before the sequence start
    come from the history (state column width-1+tau) or are zero."""
    dim = len(x)
    out, new_states = {}, {}
    for s in range(len(qsl) - 1):
        start, L = qsl[s], qsl[s + 1] - qsl[s]
        line = lines[s]
        if line == -1 or L == 0:
            continue
        init = has_init[s]

        def val(c, tau):
            if tau >= 0:
                return bits_to_fraction(x[c][start + tau])
            return bits_to_fraction(states[line][c][width - 1 + tau]) if init else Fraction(0)

        def val_bits(c, tau):
            if tau >= 0:
                return x[c][start + tau]
            return states[line][c][width - 1 + tau] if init else 0

        for c in range(dim):
            for t in range(L):
                acc = bits_to_fraction(b[c]) if b is not None else Fraction(0)
                for lag in range(width):
                    acc += bits_to_fraction(w[c][width - 1 - lag]) * val(c, t - lag)
                out[(c, start + t)] = acc
            for k in range(width - 1):
                new_states[(line, c, k)] = val_bits(c, L - (width - 1) + k)
    return out, new_states


def _tiny_case(dim, lengths, width, lines, has_init, seed, with_bias, num_lines=3):
    g = torch.Generator().manual_seed(seed)
    total = sum(lengths)
    k = lambda *s: (torch.randint(-4, 5, s, generator=g).float() / 8).to(BF)
    x = k(dim, total)
    w = k(dim, width)
    b = k(dim) if with_bias else None
    st = k(num_lines, dim, width - 1)
    return dict(x=x, weight=w, bias=b, conv_states=st,
                query_start_loc=W.qsl_from_lengths(lengths),
                cache_indices=torch.tensor(lines, dtype=torch.int32),
                has_initial_state=torch.tensor(has_init, dtype=torch.bool))


@pytest.mark.parametrize("width", [1, 2, 3, 4, 5])
def test_brute_force_exhaustive_tiny(width):
    """Exhaustive over two-sequence batches: lengths 0..7 each, init on/off,
    pad on/off for the first sequence, bias on/off, dim 2.  Exact-valued
    inputs make every sum exact, so outputs must be bit-identical to the
    rational result; states are bit copies."""
    case = 0
    for L0, L1 in itertools.product(range(8), range(0, 8, 3)):
        for init0, init1, pad0, with_bias in itertools.product((0, 1), (0, 1), (0, 1), (0, 1)):
            case += 1
            lines = [-1 if pad0 else 2, 0]
            d = _tiny_case(2, [L0, L1], width, lines, [init0, init1], seed=case,
                           with_bias=with_bias)
            out, st = run_fwd(d, activation=None, out_fill=7.0)
            ref_out, ref_st = brute_varlen(
                tensor_bits(d["x"]), tensor_bits(d["weight"]),
                tensor_bits(d["bias"]) if with_bias else None,
                tensor_bits(d["conv_states"]), d["query_start_loc"].tolist(),
                lines, [init0, init1], width, False)
            ob = tensor_bits(out)
            sentinel = tensor_bits(torch.tensor([7.0], dtype=BF))[0]
            for c in range(2):
                for t in range(L0 + L1):
                    if (c, t) in ref_out:
                        assert ob[c][t] == fraction_to_bf16_bits(ref_out[(c, t)])
                    else:
                        assert ob[c][t] == sentinel      # pad rows untouched
            sb, s0 = tensor_bits(st), tensor_bits(d["conv_states"])
            for line in range(3):
                for c in range(2):
                    for k in range(width - 1):
                        want = ref_st.get((line, c, k), s0[line][c][k])
                        assert sb[line][c][k] == want


@pytest.mark.parametrize("width", [2, 4, 5])
def test_brute_force_with_silu(width):
    d = _tiny_case(3, [6, 1, 0, 4], width, [1, -1, 2, 0], [1, 0, 1, 0], seed=9,
                   with_bias=True)
    out, _ = run_fwd(d, activation="silu")
    ref_out, _ = brute_varlen(tensor_bits(d["x"]), tensor_bits(d["weight"]),
                              tensor_bits(d["bias"]), tensor_bits(d["conv_states"]),
                              d["query_start_loc"].tolist(), [1, -1, 2, 0],
                              [1, 0, 1, 0], width, True)
    import math
    for (c, t), acc in ref_out.items():
        a = float(acc)
        y = a / (1 + math.exp(-a))
        got = bits_to_fraction(tensor_bits(out)[c][t])
        want = bits_to_fraction(fraction_to_bf16_bits(Fraction(y)))
        assert got == want


# ------------------------------------------------------------ closed forms --

def test_width_one_is_elementwise():
    d = W.single_sequence(dim=8, T=20, width=1, seed=3)
    out, st = run_fwd(d, activation="silu")
    assert st.shape[2] == 0
    x, w, b = d["x"].double(), d["weight"].double(), d["bias"].double()
    ref = F.silu(b[:, None] + w[:, :1] * x)
    assert torch.all((out.double() - ref).abs() <= bf16_ulp_half(ref) * (1 + 1e-9))


@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_impulse_response_is_reversed_taps(width):
    dim, T = 6, 9
    d = W.single_sequence(dim=dim, T=T, width=width, seed=21)
    d["x"] = torch.zeros(dim, T, dtype=BF)
    d["x"][:, 0] = 1.0
    d["bias"] = None
    d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    out, _ = run_fwd(d, activation=None)
    w = d["weight"]
    for t in range(T):
        want = w[:, width - 1 - t] if t < width else torch.zeros(dim, dtype=BF)
        assert torch.equal(out[:, t], want)


@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_impulse_in_state_slot(width):
    dim, T = 4, 8
    for k in range(width - 1):
        d = W.single_sequence(dim=dim, T=T, width=width, seed=22 + k)
        d["x"] = torch.zeros(dim, T, dtype=BF)
        d["bias"] = None
        st = torch.zeros(1, dim, width - 1, dtype=BF)
        st[0, :, k] = 1.0
        d["conv_states"] = st
        out, _ = run_fwd(d, activation=None)
        w = d["weight"]
        for t in range(T):
            want = w[:, k - t] if 0 <= k - t < width else torch.zeros(dim, dtype=BF)
            assert torch.equal(out[:, t], want)


# -------------------------------------------------------------- invariants --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("layout", ["dim_tok", "tok_dim"])
def test_split_sequence_equals_one_call(width, layout):
    T = 13
    d = W.single_sequence(dim=5, T=T, width=width, seed=31 + width, layout=layout)
    full, full_state = run_fwd(d)
    for k in range(0, T + 1):
        cs = d["conv_states"].clone()
        out = torch.empty(5, T, dtype=BF)
        for lo, hi in ((0, k), (k, T)):
            piece = W.to_layout(d["x"][:, lo:hi].contiguous(), layout)
            o = torch.empty(5, hi - lo, dtype=BF)
            oracle.fwd_varlen(piece, d["weight"], d["bias"], cs,
                              torch.tensor([0, hi - lo], dtype=torch.int32), o,
                              has_initial_state=torch.ones(1, dtype=torch.bool))
            out[:, lo:hi] = o
        assert torch.equal(out, full.contiguous()), k
        assert torch.equal(cs, full_state), k


def test_split_without_initial_state():
    T = 10
    d = W.single_sequence(dim=3, T=T, width=4, seed=41)
    d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    full, full_state = run_fwd(d)
    for k in range(1, T + 1):
        cs = d["conv_states"].clone()
        out = torch.empty(3, T, dtype=BF)
        for (lo, hi), init in (((0, k), False), ((k, T), True)):
            o = torch.empty(3, hi - lo, dtype=BF)
            oracle.fwd_varlen(d["x"][:, lo:hi].contiguous(), d["weight"], d["bias"], cs,
                              torch.tensor([0, hi - lo], dtype=torch.int32), o,
                              has_initial_state=torch.tensor([init]))
            out[:, lo:hi] = o
        assert torch.equal(out, full), k
        assert torch.equal(cs, full_state), k


@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_power_of_two_scaling(width):
    d = W.varlen_batch(lengths=[9, 1, 4, 0, 17], dim=7, width=width, seed=51,
                       num_lines=8, n_pad=1, layout="dim_tok", with_bias=False)
    out, st = run_fwd(d, activation=None, out_fill=0.0)
    d2 = dict(d, x=d["x"] * 2, conv_states=d["conv_states"] * 2)
    out2, st2 = run_fwd(d2, activation=None, out_fill=0.0)
    assert torch.equal(out2, out * 2)
    assert torch.equal(st2, st * 2)


def test_zero_length_and_pad_sequences_write_nothing():
    d = W.varlen_batch(lengths=[0, 5, 0, 3], dim=4, width=4, seed=61, num_lines=6,
                       n_pad=0, layout="dim_tok")
    d["cache_indices"] = torch.tensor([0, 1, 2, -1], dtype=torch.int32)
    out, st = run_fwd(d, out_fill=3.0)
    before = d["conv_states"]
    assert torch.equal(st[0], before[0])          # zero length: untouched
    assert torch.equal(st[2], before[2])
    assert torch.equal(st[3:], before[3:])        # pad line / unreferenced
    assert not torch.equal(st[1], before[1])
    assert torch.all(out[:, 5:8] == 3.0)          # pad sequence's rows untouched


def test_short_sequence_shifts_state():
    # L < width-1: the new state is the old tail followed by x
    d = W.single_sequence(dim=3, T=1, width=4, seed=71)
    _, st = run_fwd(d)
    old = d["conv_states"]
    assert torch.equal(st[0, :, :2], old[0, :, 1:])
    assert torch.equal(st[0, :, 2], d["x"][:, 0])
    d["has_initial_state"] = torch.zeros(1, dtype=torch.bool)
    _, st = run_fwd(d)
    assert torch.equal(st[0, :, :2], torch.zeros(3, 2, dtype=BF))
    assert torch.equal(st[0, :, 2], d["x"][:, 0])


def test_out_of_range_line_is_skipped():
    d = W.varlen_batch(lengths=[3, 3], dim=2, width=3, seed=81, num_lines=2,
                       n_pad=0, layout="dim_tok")
    d["cache_indices"] = torch.tensor([5, 1], dtype=torch.int32)
    out, st = run_fwd(d, out_fill=2.0)
    assert torch.all(out[:, :3] == 2.0)
    assert torch.equal(st[0], d["conv_states"][0])


# ------------------------------------------------ docstring structure pins --

def test_docstring_query_start_loc_examples():
    g = json.load(open(os.path.join(GOLDEN, "varlen_docstring_examples.json")))
    for ex in g["query_start_loc_examples"]:
        assert W.qsl_from_lengths(ex["lengths"]).tolist() == ex["query_start_loc"]


def test_docstring_pad_example():
    g = json.load(open(os.path.join(GOLDEN, "varlen_docstring_examples.json")))["pad_example"]
    lines = g["cache_indices"]
    d = W.varlen_batch(lengths=[2, 3, 4, 1], dim=4, width=4, seed=91, num_lines=24,
                       n_pad=0, layout="dim_tok")
    d["cache_indices"] = torch.tensor(lines, dtype=torch.int32)
    d["has_initial_state"] = torch.ones(4, dtype=torch.bool)
    out, st = run_fwd(d, out_fill=5.0, pad_slot_id=g["pad_slot_id"])
    qsl = d["query_start_loc"].tolist()
    for s in g["skipped"]:
        assert torch.all(out[:, qsl[s]:qsl[s + 1]] == 5.0)
    for s in g["processed"]:
        assert not torch.any(out[:, qsl[s]:qsl[s + 1]] == 5.0)
    changed = [l for l in range(24) if not torch.equal(st[l], d["conv_states"][l])]
    assert changed == sorted(lines[s] for s in g["processed"])


# ------------------------------------------------------------------ decode --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("seqlen", [1, 2, 5])
def test_decode_equals_forward_with_state(width, seqlen):
    d = W.decode_batch(batch=5, dim=6, width=width, seqlen=seqlen, seed=101,
                       num_lines=9, n_pad=1)
    out = torch.full(d["x"].shape, 9.0, dtype=BF)
    st = d["conv_state"].clone()
    oracle.update_decode(d["x"], st, d["weight"], d["bias"], out,
                         cache_indices=d["cache_indices"], activation="silu")
    for b in range(5):
        line = int(d["cache_indices"][b])
        if line == -1:
            assert torch.all(out[b] == 9.0)
            continue
        o = torch.empty(6, seqlen, dtype=BF)
        s1 = d["conv_state"][line:line + 1].clone()
        oracle.fwd_varlen(d["x"][b], d["weight"], d["bias"], s1,
                          torch.tensor([0, seqlen], dtype=torch.int32), o,
                          has_initial_state=torch.ones(1, dtype=torch.bool))
        assert torch.equal(out[b], o)
        assert torch.equal(st[line], s1[0])


def test_decode_single_token_matches_benchmark_reference():
    d = W.decode_batch(batch=1, dim=16, width=4, seqlen=1, seed=111)
    out = torch.empty_like(d["x"])
    st = d["conv_state"].clone()
    oracle.update_decode(d["x"], st, d["weight"], d["bias"], out, activation="silu")
    ref = windowed_reference_fp64(d["x"][0], d["weight"], d["bias"], d["conv_state"], "silu")
    assert torch.all((out[0].double() - ref).abs() <= bf16_ulp_half(ref) * (1 + 1e-9))
    # state: shifted left by one with the new input at the end
    assert torch.equal(st[0, :, :2], d["conv_state"][0, :, 1:])
    assert torch.equal(st[0, :, 2], d["x"][0, :, 0])


def test_decode_in_place():
    d = W.decode_batch(batch=3, dim=5, width=4, seqlen=2, seed=121)
    ref = torch.empty_like(d["x"])
    st_ref = d["conv_state"].clone()
    oracle.update_decode(d["x"], st_ref, d["weight"], d["bias"], ref, activation="silu")
    x = d["x"].clone()
    st = d["conv_state"].clone()
    oracle.update_decode(x, st, d["weight"], d["bias"], x, activation="silu")
    assert torch.equal(x, ref)
    assert torch.equal(st, st_ref)
