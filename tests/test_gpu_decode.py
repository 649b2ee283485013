"""GPU parity for conv1d_update_decode (through the C ABI) against the oracle."""
import pytest
import torch

import causal_depthwise_short_conv1d_amd as S
import oracle
import workloads as W
from tests.parity import assert_bits, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


def both(d, activation="silu", in_place=False, values_exact=False, out_like_x=False):
    x_cpu = d["x"]
    st_ref = d["conv_state"].clone()
    out_ref = torch.full(x_cpu.shape, -3.0, dtype=BF)
    oracle.update_decode(x_cpu, st_ref, d["weight"], d["bias"], out_ref,
                         cache_indices=d["cache_indices"], activation=activation)
    x = x_cpu.to(DEV)
    st = d["conv_state"].to(DEV)
    w = d["weight"].to(DEV)
    b = d["bias"].to(DEV) if d["bias"] is not None else None
    ci = d["cache_indices"].to(DEV) if d["cache_indices"] is not None else None
    if in_place:
        # pads keep x as it was
        S.conv1d_update_decode(x, st, w, b, activation=activation, cache_indices=ci, out=x)
        out = x
        for bi, line in enumerate(d["cache_indices"].tolist()):
            if line == -1:
                out_ref[bi] = x_cpu[bi]
    else:
        out = torch.full_like(x, -3.0) if out_like_x else torch.full(x.shape, -3.0, dtype=BF, device=DEV)
        S.conv1d_update_decode(x, st, w, b, activation=activation, cache_indices=ci, out=out)
    torch.cuda.synchronize()
    if values_exact:
        assert_bits(out, out_ref, "decode out")
    else:
        assert_close(out, out_ref, "decode out")
    assert_bits(st, st_ref, "decode state")


@pytest.mark.parametrize("seqlen", [1, 6])
@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_decode_four_channel_runs(width, seqlen):
    """Channel-contiguous x and out, (lines, dim, width-1) states and dim %
    4 == 0: four channels' histories are one run per lane.  Two workgroups
    of channels (the second partial), pads, one and six tokens; exact values
    bit for bit, and SiLU."""
    for values, act in (("exact", None), ("normal", "silu")):
        d = W.decode_batch(batch=9, dim=1156, width=width, seqlen=seqlen, seed=560 + width,
                           num_lines=12, n_pad=2, values=values)
        assert d["x"].stride(1) == 1 and d["conv_state"].is_contiguous()
        say(f"[decode] four-channel runs W{width} seqlen {seqlen} {values}")
        both(d, activation=act, values_exact=values == "exact", out_like_x=True)
        both(d, activation=act, values_exact=values == "exact", in_place=True)


@pytest.mark.parametrize("values", ["normal", "exact"])
def test_decode_serving_batch_full_size(values):
    """64 entries x dim 8192, one token each, 128 lines, out laid out like x:
    the decode step the benchmark times at a serving batch."""
    d = W.decode_batch(batch=64, dim=8192, width=4, seed=W.seed_for(2, 2), num_lines=128,
                       values=values)
    say(f"[decode] 64 x 8192 T1 {values}")
    if values == "exact":
        both(d, activation=None, values_exact=True, out_like_x=True)
    else:
        both(d, out_like_x=True)


@pytest.mark.parametrize("width", [2, 3, 4, 5])
def test_decode_single_token_dim4096(width):
    """The T=1 row of the prefill sweep, through the decode entry point."""
    d = W.decode_batch(batch=1, dim=4096, width=width, seed=W.seed_for(2, 1))
    say(f"[decode] dim4096 T1 W{width}")
    both(d)


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("seqlen", [1, 2, 3, 7])
def test_decode_batch_with_pads(width, seqlen):
    d = W.decode_batch(batch=37, dim=300, width=width, seqlen=seqlen, seed=50 + width,
                       num_lines=64, n_pad=5)
    both(d)


@pytest.mark.parametrize("width", [2, 4, 5])
def test_decode_in_place(width):
    d = W.decode_batch(batch=9, dim=1000, width=width, seqlen=2, seed=60 + width,
                       num_lines=12, n_pad=2)
    both(d, in_place=True)


def test_decode_exact_values_no_activation():
    d = W.decode_batch(batch=16, dim=777, width=4, seqlen=3, seed=70, num_lines=20,
                       n_pad=3, values="exact")
    both(d, activation=None, values_exact=True)


def test_decode_without_cache_indices_and_bias():
    d = W.decode_batch(batch=8, dim=96, width=3, seqlen=1, seed=80, with_bias=False)
    d["cache_indices"] = None
    both(d)


def test_decode_equals_forward_on_gpu():
    """Cross-entry-point check: decode == varlen forward of T=1 with state."""
    d = W.decode_batch(batch=1, dim=4096, width=4, seed=90)
    x = d["x"].to(DEV)
    st1 = d["conv_state"].to(DEV)
    st2 = st1.clone()
    w, b = d["weight"].to(DEV), d["bias"].to(DEV)
    o1 = S.conv1d_update_decode(x, st1, w, b, activation="silu")
    o2 = S.conv1d_fwd_varlen(x[0], w, b, st2,
                             torch.tensor([0, 1], dtype=torch.int32, device=DEV),
                             has_initial_state=torch.ones(1, dtype=torch.bool, device=DEV))
    torch.cuda.synchronize()
    assert_bits(o1[0], o2, "decode vs fwd out")
    assert_bits(st1, st2, "decode vs fwd state")


@pytest.mark.parametrize("in_place", [False, True])
def test_bound_decode_equals_the_call(in_place):
    """bind_update_decode marshals once and then launches exactly what
    conv1d_update_decode launches: outputs and states bit-identical over
    repeated steps, in place and out of place."""
    d = W.decode_batch(batch=5, dim=520, width=4, seed=577, num_lines=8, n_pad=1)
    x = d["x"].to(DEV)
    w, b, ci = d["weight"].to(DEV), d["bias"].to(DEV), d["cache_indices"].to(DEV)
    st_a, st_b = d["conv_state"].to(DEV), d["conv_state"].to(DEV)
    xa, xb = x.clone(), x.clone()
    oa = xa if in_place else torch.full_like(x, -3.0)
    ob = xb if in_place else torch.full_like(x, -3.0)
    launch = S.bind_update_decode(xb, st_b, w, b, activation="silu", cache_indices=ci, out=ob)
    for step in range(3):
        S.conv1d_update_decode(xa, st_a, w, b, activation="silu", cache_indices=ci, out=oa)
        launch()
        torch.cuda.synchronize()
        assert_bits(ob, oa, f"bound decode step {step} out")
        assert_bits(st_b, st_a, f"bound decode step {step} state")
