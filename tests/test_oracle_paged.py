"""Pins for the oracle's paged sliding-window step and token metadata.

The brute force below is written as a per-request timeline (absolute
position -> input) built from the pre-call cache for positions before the
request's first row and from x for positions inside this forward; the oracle
instead decides tap by tap from the row index, as the Inkling sconv.py kernel
does.  Cross-API checks tie a prefill chunk to the varlen forward and a decode
token to the decode update.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.exact_ref import bits_to_fraction, fraction_to_bf16_bits, tensor_bits

BF = torch.bfloat16
SMALL = dict(H=2, ws=8, N=4, D=24, off_s=8, num_blocks=64, n_decode=3,
             n_prefill=2, chunk=6, max_pos=40)


def run_paged(d, activation=None, residual=True, cache=None):
    out = torch.full(d["x"].shape, float("nan"), dtype=BF)
    cache = d["cache"].clone() if cache is None else cache
    oracle.paged(d["x"], d["weight"], d.get("bias"), cache, d["positions"],
                 d["slot_mapping"], d["query_start_loc"], d["block_table"],
                 d["off_s"], d["ws"], out, activation=activation,
                 use_residual=residual)
    return out, cache


def brute_paged(d, width, residual):
    x = tensor_bits(d["x"])
    w = tensor_bits(d["weight"])
    b = tensor_bits(d["bias"]) if d.get("bias") is not None else None
    cache = d["cache"]
    bt = d["block_table"].tolist()
    pos = d["positions"].tolist()
    slot = d["slot_mapping"].tolist()
    qsl = d["query_start_loc"].tolist()
    ws, off, N = d["ws"], d["off_s"], d["block_size"]
    C = len(x[0])
    outs = {}
    for r in range(len(qsl) - 1):
        rows = range(qsl[r], qsl[r + 1])
        if not rows:
            continue
        p_first = pos[qsl[r]]
        for t in rows:
            if slot[t] < 0:
                continue
            p = pos[t]
            for c in range(C):
                def value(q):
                    if q < 0:
                        return Fraction(0)
                    if q >= p_first:                       # inside this forward
                        return bits_to_fraction(x[qsl[r] + (q - p_first)][c])
                    blk = bt[r][q // N]
                    v = cache[blk, c // ws, q % N, off + c % ws]
                    return bits_to_fraction(int(v.view(torch.int16)) & 0xFFFF)
                acc = bits_to_fraction(b[c]) if b is not None else Fraction(0)
                for lag in range(width):
                    acc += bits_to_fraction(w[c][width - 1 - lag]) * value(p - lag)
                if residual:
                    acc += bits_to_fraction(x[t][c])
                outs[(t, c)] = acc
    return outs


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("residual", [True, False])
@pytest.mark.parametrize("with_bias", [False, True])
def test_brute_force_small_paged(width, residual, with_bias):
    d = W.paged_batch(**SMALL, width=width, pad_frac=0.15, trailing_pad=2,
                      seed=200 + width, values="exact", with_bias=with_bias, min_pos=0)
    out, cache = run_paged(d, residual=residual)
    ref = brute_paged(d, width, residual)
    ob = tensor_bits(out)
    xb = tensor_bits(d["x"])
    T, C = d["x"].shape
    for t in range(T):
        for c in range(C):
            if (t, c) in ref:
                assert ob[t][c] == fraction_to_bf16_bits(ref[(t, c)]), (t, c)
            else:   # pad row: not convolved, out = x with residual else 0
                assert ob[t][c] == (xb[t][c] if residual else 0)
    # cache: exactly the non-pad rows inserted, everything else unchanged
    want = d["cache"].clone()
    H, ws, off, N = SMALL["H"], d["ws"], d["off_s"], d["block_size"]
    for t, s in enumerate(d["slot_mapping"].tolist()):
        if s >= 0:
            want[s // N, :, s % N, off:off + ws] = d["x"][t].view(H, ws)
    assert torch.equal(cache, want)


def test_silu_and_residual_rounding_once():
    d = W.paged_batch(**SMALL, width=4, pad_frac=0.1, seed=301)
    out, _ = run_paged(d, activation="silu", residual=True)
    ref = brute_paged(d, 4, residual=False)
    import math
    ob = tensor_bits(out)
    xb = tensor_bits(d["x"])
    for (t, c), acc in ref.items():
        a = float(acc)
        y = Fraction(a / (1 + math.exp(-a))) + bits_to_fraction(xb[t][c])
        assert ob[t][c] == fraction_to_bf16_bits(y)


def test_idempotent_step():
    d = W.paged_batch(**SMALL, width=4, pad_frac=0.1, seed=311)
    out1, cache1 = run_paged(d, activation="silu")
    out2, cache2 = run_paged(d, activation="silu", cache=cache1.clone())
    assert torch.equal(out1, out2)
    assert torch.equal(cache1, cache2)


@pytest.mark.parametrize("width", [2, 4, 5])
def test_prefill_chunk_equals_varlen_forward(width):
    cfg = dict(SMALL, n_decode=0, n_prefill=3, chunk=7)
    d = W.paged_batch(**cfg, width=width, pad_frac=0.0, seed=321, with_bias=True)
    out, _ = run_paged(d, activation="silu", residual=False)
    qsl = d["query_start_loc"].tolist()
    N, ws, off = d["block_size"], d["ws"], d["off_s"]
    C = d["x"].shape[1]
    for r in range(len(qsl) - 1):
        p0 = int(d["positions"][qsl[r]])
        hist = torch.zeros(1, C, width - 1, dtype=BF)
        for k in range(width - 1):
            q = p0 - (width - 1) + k
            if q >= 0:
                blk = int(d["block_table"][r, q // N])
                hist[0, :, k] = d["cache"][blk, :, q % N, off:off + ws].reshape(C)
        xs = d["x"][qsl[r]:qsl[r + 1]].t()
        o = torch.empty(xs.shape, dtype=BF)
        oracle.fwd_varlen(xs, d["weight"], d["bias"], hist,
                          torch.tensor([0, xs.shape[1]], dtype=torch.int32), o,
                          has_initial_state=torch.ones(1, dtype=torch.bool),
                          activation="silu")
        assert torch.equal(out[qsl[r]:qsl[r + 1]], o.t())


def test_decode_token_equals_decode_update():
    cfg = dict(SMALL, n_decode=4, n_prefill=0)
    d = W.paged_batch(**cfg, width=4, pad_frac=0.0, seed=331, with_bias=True)
    out, _ = run_paged(d, activation="silu", residual=False)
    N, ws, off = d["block_size"], d["ws"], d["off_s"]
    C = d["x"].shape[1]
    for t in range(4):
        p = int(d["positions"][t])
        st = torch.zeros(1, C, 3, dtype=BF)
        for k in range(3):
            q = p - 3 + k
            blk = int(d["block_table"][t, q // N])
            st[0, :, k] = d["cache"][blk, :, q % N, off:off + ws].reshape(C)
        o = torch.empty(1, C, 1, dtype=BF)
        oracle.update_decode(d["x"][t].view(1, C, 1), st, d["weight"], d["bias"], o,
                             activation="silu")
        assert torch.equal(out[t], o.view(C))


def test_positions_before_zero_contribute_nothing():
    cfg = dict(SMALL, n_decode=2, n_prefill=1)
    d = W.paged_batch(**cfg, width=5, pad_frac=0.0, seed=341, min_pos=0)
    d["positions"][0] = 0            # decode at position 0: only its own input
    blk = int(d["block_table"][0, 0])
    d["slot_mapping"][0] = blk * d["block_size"]
    d["weight"] = torch.ones_like(d["weight"])
    out, _ = run_paged(d, residual=False)
    assert torch.equal(out[0], d["x"][0])


def test_trailing_rows_are_pads():
    d = W.paged_batch(**SMALL, width=4, pad_frac=0.0, trailing_pad=3, seed=351)
    T = d["x"].shape[0]
    d["slot_mapping"][T - 1] = 0     # even with a slot, rows past the last request are pads
    out, cache = run_paged(d, residual=True)
    assert torch.equal(out[T - 3:], d["x"][T - 3:])
    assert torch.equal(cache[0, :, 0], d["cache"][0, :, 0])


# --------------------------------------------------------------- metadata --

def test_seq_metadata_matches_searchsorted():
    rng = np.random.default_rng(5)
    lengths = rng.integers(0, 6, 30)
    qsl = W.qsl_from_lengths(lengths.tolist())
    total = int(qsl[-1])
    seq_idx, qstart = oracle.seq_metadata(qsl, total, total + 7)
    tok = np.arange(total)
    want = np.searchsorted(qsl.numpy()[:-1], tok, side="right") - 1
    assert np.array_equal(seq_idx.numpy()[:total], want)
    assert np.array_equal(qstart.numpy()[:total], qsl.numpy()[want])
    assert np.all(seq_idx.numpy()[total:] == 0) and np.all(qstart.numpy()[total:] == 0)


def test_seq_metadata_rejects_short_padding():
    qsl = W.qsl_from_lengths([3, 2])
    with pytest.raises(RuntimeError):
        oracle.seq_metadata(qsl, 5, 4)
