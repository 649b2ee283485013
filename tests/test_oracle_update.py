"""Pins for the oracle's general decode update: the speculative-decoding
options (num_accepted_tokens, intermediate windows, output_state_indices) and
the ring-buffer option (cache_seqlens) of tokenspeed causal_conv1d.py,
causal_conv1d_update.

None of these options has a printed example on the pages, so every check ties
the oracle to the varlen forward (itself pinned against the benchmark page's
Model.forward, exact brute force and closed forms) through what the options
mean:
  * the page's comment on rolling the state: after a verify pass of N drafts
    and the acceptance of a of them, continuing from the window at column
    a-1 must equal one unbroken run over history ++ accepted tokens;
  * an intermediate window after step t is the state an unbroken run over the
    first t+1 tokens leaves behind;
  * a ring buffer fed chunk by chunk must equal one unbroken run, and holds
    input n of the stream at column n mod state_len.
"""
import pytest
import torch

import oracle
import workloads as W

BF = torch.bfloat16


def fwd_single(x_dim_tok, weight, bias, hist, activation="silu"):
    """Unbroken run of one sequence (dim, T) from the given (dim, width-1)
    history through the varlen forward; returns (out, new width-1 state)."""
    dim, T = x_dim_tok.shape
    width = weight.shape[1]
    st = hist.reshape(1, dim, width - 1).clone()
    out = torch.empty(dim, T, dtype=BF)
    oracle.fwd_varlen(x_dim_tok.contiguous(), weight, bias, st,
                      torch.tensor([0, T], dtype=torch.int32), out,
                      has_initial_state=torch.ones(1, dtype=torch.bool),
                      activation=activation)
    return out, st[0]


def run_general(d, out_fill=7.0, activation="silu", **opts):
    out = torch.full(d["x"].shape, out_fill, dtype=BF)
    st = d["conv_state"].clone()
    inter = opts.pop("intermediate", None)
    oracle.update_general(d["x"], st, d["weight"], d["bias"], out,
                          cache_indices=d.get("cache_indices"), intermediate=inter,
                          activation=activation, **opts)
    return out, st


# ------------------------------------------------------------ plain mode --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("seqlen", [1, 3])
def test_no_options_is_the_plain_update(width, seqlen):
    d = W.decode_batch(batch=5, dim=7, width=width, seqlen=seqlen, seed=300 + width,
                       num_lines=8, n_pad=1)
    out, st = run_general(d)
    ref = torch.full(d["x"].shape, 7.0, dtype=BF)
    st_ref = d["conv_state"].clone()
    oracle.update_decode(d["x"], st_ref, d["weight"], d["bias"], ref,
                         cache_indices=d["cache_indices"], activation="silu")
    assert torch.equal(out, ref)
    assert torch.equal(st, st_ref)


def test_wider_state_keeps_extra_columns_in_plain_mode():
    d = W.decode_batch(batch=3, dim=5, width=4, seqlen=2, seed=311)
    wide = torch.randn(3, 5, 6).to(BF)
    wide[:, :, :3] = d["conv_state"]
    d2 = dict(d, conv_state=wide)
    out, st = run_general(d2)
    ref, st_ref = run_general(d)
    assert torch.equal(out, ref)
    assert torch.equal(st[:, :, :3], st_ref)
    assert torch.equal(st[:, :, 3:], wide[:, :, 3:])


# ------------------------------------------------------ speculative: roll --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("n1,n2", [(1, 1), (3, 2), (4, 4), (5, 1)])
def test_roll_then_accept_equals_unbroken_run(width, n1, n2):
    """Pass 1 verifies n1 tokens from window 0; pass 2 accepts a of them and
    verifies n2 more.  Pass 2 must see exactly history ++ x1[:a]."""
    dim, hist = 6, width - 1
    state_len = hist - 1 + max(n1, n2)
    g = torch.Generator().manual_seed(17 * width + n1)
    h0 = (torch.randn(dim, hist, generator=g) * 0.5).to(BF)
    x1 = (torch.randn(1, dim, n1, generator=g) * 0.5).to(BF)
    x2 = (torch.randn(1, dim, n2, generator=g) * 0.5).to(BF)
    w = (torch.randn(dim, width, generator=g) * 0.5).to(BF)
    b = (torch.randn(dim, generator=g) * 0.5).to(BF)
    line0 = torch.randn(1, dim, state_len, generator=g).to(BF)
    line0[0, :, :hist] = h0
    for a in range(1, n1 + 1):
        st = line0.clone()
        o1 = torch.empty_like(x1)
        oracle.update_general(x1, st, w, b, o1, activation="silu",
                              num_accepted_tokens=torch.tensor([1], dtype=torch.int32))
        ref1, _ = fwd_single(x1[0], w, b, h0)
        assert torch.equal(o1[0], ref1)
        # the rolled line: history minus its oldest input, then every draft
        assert torch.equal(st[0, :, :hist - 1], h0[:, 1:])
        assert torch.equal(st[0, :, hist - 1:hist - 1 + n1], x1[0])
        o2 = torch.empty_like(x2)
        oracle.update_general(x2, st, w, b, o2, activation="silu",
                              num_accepted_tokens=torch.tensor([a], dtype=torch.int32))
        ref2, _ = fwd_single(torch.cat([x1[0, :, :a], x2[0]], dim=1), w, b, h0)
        assert torch.equal(o2[0], ref2[:, a:])


@pytest.mark.parametrize("width", [2, 4, 5])
def test_roll_batch_matches_per_entry_runs(width):
    d = W.spec_decode_batch(batch=6, dim=5, width=width, seqlen=3, state_len=width + 3,
                            num_lines=9, n_pad=1, seed=320 + width, mode="roll")
    out, st = run_general(d, num_accepted_tokens=d["num_accepted_tokens"])
    hist = width - 1
    for b in range(6):
        line = int(d["cache_indices"][b])
        if line == -1:
            assert torch.all(out[b] == 7.0)
            continue
        off = int(d["num_accepted_tokens"][b]) - 1
        h = d["conv_state"][line, :, off:off + hist]
        ref, _ = fwd_single(d["x"][b], d["weight"], d["bias"], h)
        assert torch.equal(out[b], ref)
        u = torch.cat([h, d["x"][b]], dim=1)
        n = hist - 1 + 3
        assert torch.equal(st[line, :, :n], u[:, 1:])
        assert torch.equal(st[line, :, n:], d["conv_state"][line, :, n:])
    used = {int(v) for v in d["cache_indices"] if int(v) != -1}
    for line in range(9):
        if line not in used:
            assert torch.equal(st[line], d["conv_state"][line])


def test_roll_with_one_accepted_single_token_is_plain_decode():
    d = W.decode_batch(batch=4, dim=6, width=4, seqlen=1, seed=331, num_lines=6)
    out, st = run_general(d, num_accepted_tokens=torch.ones(4, dtype=torch.int32))
    ref, st_ref = run_general(d)
    assert torch.equal(out, ref)
    assert torch.equal(st, st_ref)


# --------------------------------------------------- speculative: scatter --

@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("state_len_extra", [0, 2])
def test_intermediate_windows_are_prefix_states(width, state_len_extra):
    seqlen = 4
    d = W.spec_decode_batch(batch=5, dim=6, width=width, seqlen=seqlen,
                            state_len=width - 1 + state_len_extra, num_lines=30,
                            n_pad=1, seed=340 + width, mode="scatter")
    inter = torch.full(d["intermediate"].shape, 5.0, dtype=BF)
    out, st = run_general(d, num_accepted_tokens=d["num_accepted_tokens"],
                          intermediate=inter)
    hist = width - 1
    for b in range(5):
        line = int(d["cache_indices"][b])
        if line == -1:
            assert torch.all(out[b] == 7.0) and torch.all(inter[b] == 5.0)
            continue
        off = int(d["num_accepted_tokens"][b]) - 1
        h = d["conv_state"][line, :, off:off + hist]
        ref, _ = fwd_single(d["x"][b], d["weight"], d["bias"], h)
        assert torch.equal(out[b], ref)
        for t in range(seqlen):
            _, s_t = fwd_single(d["x"][b, :, :t + 1], d["weight"], d["bias"], h)
            assert torch.equal(inter[b, t], s_t)
    # no in-place state update when windows are saved
    assert torch.equal(st, d["conv_state"])


@pytest.mark.parametrize("width", [2, 4, 5])
def test_output_state_indices_scatter_prefix_states(width):
    seqlen = 3
    d = W.spec_decode_batch(batch=4, dim=5, width=width, seqlen=seqlen,
                            state_len=width + 1, num_lines=24, n_pad=1,
                            seed=350 + width, mode="scatter")
    osi = d["output_state_indices"].clone()
    osi[0, 0] = 24          # out of range: no write
    out, st = run_general(d, num_accepted_tokens=d["num_accepted_tokens"],
                          output_state_indices=osi)
    hist = width - 1
    written = set()
    for b in range(4):
        line = int(d["cache_indices"][b])
        if line == -1:
            continue
        off = int(d["num_accepted_tokens"][b]) - 1
        h = d["conv_state"][line, :, off:off + hist]
        for t in range(seqlen):
            dst = int(osi[b, t])
            if 0 <= dst < 24:
                _, s_t = fwd_single(d["x"][b, :, :t + 1], d["weight"], d["bias"], h)
                assert torch.equal(st[dst, :, :hist], s_t)
                assert torch.equal(st[dst, :, hist:], d["conv_state"][dst, :, hist:])
                written.add(dst)
    for line in range(24):
        if line not in written:
            assert torch.equal(st[line], d["conv_state"][line])


def test_scatter_to_own_line_reads_before_writing():
    d = W.spec_decode_batch(batch=1, dim=4, width=4, seqlen=3, state_len=3,
                            num_lines=8, seed=361, mode="scatter")
    line = int(d["cache_indices"][0])
    osi = torch.tensor([[line, -1, line]], dtype=torch.int32)
    out, st = run_general(d, num_accepted_tokens=torch.ones(1, dtype=torch.int32),
                          output_state_indices=osi)
    ref, s_end = fwd_single(d["x"][0], d["weight"], d["bias"], d["conv_state"][line])
    assert torch.equal(out[0], ref)
    assert torch.equal(st[line], s_end)


# ------------------------------------------------------------------- ring --

def ring_from_stream(stream, state_len, seen):
    """A ring line holding the last inputs of `stream` (dim, n) with `seen`
    inputs so far: input m at column m mod state_len."""
    dim = stream.shape[0]
    line = torch.full((dim, state_len), 3.0, dtype=BF)
    for m in range(max(0, seen - state_len), seen):
        line[:, m % state_len] = stream[:, m]
    return line


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("state_len_extra", [0, 1, 4])
def test_ring_chunks_equal_unbroken_run(width, state_len_extra):
    hist = width - 1
    L = hist + state_len_extra
    dim = 5
    g = torch.Generator().manual_seed(370 + 10 * width + state_len_extra)
    n0 = hist + 2
    total = n0 + 12
    stream = (torch.randn(dim, total, generator=g) * 0.5).to(BF)
    w = (torch.randn(dim, width, generator=g) * 0.5).to(BF)
    b = (torch.randn(dim, generator=g) * 0.5).to(BF)
    line = ring_from_stream(stream, L, n0).reshape(1, dim, L)
    seen = n0
    ref, _ = fwd_single(stream[:, n0:], w, b, stream[:, n0 - hist:n0])
    for chunk in (1, 3, 1, 2, 5):
        x = stream[:, seen:seen + chunk].reshape(1, dim, chunk)
        o = torch.empty_like(x)
        oracle.update_general(x, line, w, b, o, activation="silu",
                              cache_seqlens=torch.tensor([seen], dtype=torch.int32))
        assert torch.equal(o[0], ref[:, seen - n0:seen - n0 + chunk])
        seen += chunk
        assert torch.equal(line[0], ring_from_stream(stream, L, seen))


def test_ring_chunk_longer_than_buffer_keeps_last_inputs():
    width, L, dim = 4, 4, 3
    g = torch.Generator().manual_seed(381)
    stream = (torch.randn(dim, 20, generator=g) * 0.5).to(BF)
    w = (torch.randn(dim, width, generator=g) * 0.5).to(BF)
    line = ring_from_stream(stream, L, 6).reshape(1, dim, L)
    x = stream[:, 6:17].reshape(1, dim, 11)
    o = torch.empty_like(x)
    oracle.update_general(x, line, w, None, o, activation=None,
                          cache_seqlens=torch.tensor([6], dtype=torch.int32))
    ref, _ = fwd_single(stream[:, 6:17], w, None, stream[:, 3:6], activation=None)
    assert torch.equal(o[0], ref)
    assert torch.equal(line[0], ring_from_stream(stream, L, 17))


def test_ring_at_zero_with_minimal_buffer_reads_columns_in_order():
    """state_len = width-1 and seen = a multiple of it: the window is the
    line read left to right, as in the plain layout."""
    d = W.ring_decode_batch(batch=3, dim=4, width=4, seqlen=1, state_len=3,
                            num_lines=3, seed=391)
    seen = torch.tensor([0, 3, 6], dtype=torch.int32)
    out, st = run_general(d, cache_seqlens=seen)
    ref, _ = run_general(d)
    assert torch.equal(out, ref)
    for b in range(3):
        line = int(d["cache_indices"][b])
        assert torch.equal(st[line, :, 0], d["x"][b, :, 0])
        assert torch.equal(st[line, :, 1:], d["conv_state"][line, :, 1:])


# ------------------------------------------------------------ skip rules --

def test_invalid_entries_are_skipped():
    d = W.spec_decode_batch(batch=4, dim=3, width=4, seqlen=2, state_len=5,
                            num_lines=6, seed=401, mode="roll")
    nacc = torch.tensor([0, 4, 3, -2], dtype=torch.int32)   # valid: 1..3
    out, st = run_general(d, num_accepted_tokens=nacc)
    for b in (0, 1, 3):
        assert torch.all(out[b] == 7.0)
        line = int(d["cache_indices"][b])
        assert torch.equal(st[line], d["conv_state"][line])
    assert not torch.all(out[2] == 7.0)
    r = W.ring_decode_batch(batch=2, dim=3, width=3, seqlen=1, state_len=4,
                            num_lines=2, seed=402)
    out, st = run_general(r, cache_seqlens=torch.tensor([-1, 5], dtype=torch.int32))
    assert torch.all(out[0] == 7.0)
    line0 = int(r["cache_indices"][0])
    assert torch.equal(st[line0], r["conv_state"][line0])
    assert not torch.all(out[1] == 7.0)


def test_rejected_option_combinations():
    r = W.ring_decode_batch(batch=1, dim=2, width=3, seqlen=1, state_len=4,
                            num_lines=1, seed=403)
    with pytest.raises(RuntimeError):
        run_general(r, cache_seqlens=torch.zeros(1, dtype=torch.int32),
                    num_accepted_tokens=torch.ones(1, dtype=torch.int32))
    d = W.spec_decode_batch(batch=1, dim=2, width=4, seqlen=3, state_len=3,
                            num_lines=4, seed=404, mode="roll")
    with pytest.raises(RuntimeError):       # roll needs width-2+seqlen columns
        run_general(d, num_accepted_tokens=torch.ones(1, dtype=torch.int32))
