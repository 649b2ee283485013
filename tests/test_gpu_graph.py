"""GPU parity for sconv_seq_metadata, and HIP-graph capture of every entry
point: the library allocates nothing, never synchronises and enqueues on the
caller's stream, so a captured step must replay exactly like the eager one
(the paged page's requirement that its kernels replay under full graphs)."""
import pytest
import torch

import causal_depthwise_short_conv1d_amd as S
import oracle
import workloads as W
from tests.parity import assert_bits, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16


# --------------------------------------------------------------- metadata --

@pytest.mark.parametrize("n_req,max_len,extra", [(1, 50, 0), (30, 6, 7), (41, 600, 300),
                                                (3000, 5, 1)])
def test_seq_metadata_matches_oracle(n_req, max_len, extra):
    g = torch.Generator().manual_seed(n_req + max_len)
    lengths = torch.randint(0, max_len + 1, (n_req,), generator=g)
    qsl = W.qsl_from_lengths(lengths)
    actual = int(qsl[-1])
    padded = actual + extra
    si_ref, qs_ref = oracle.seq_metadata(qsl, actual, padded)
    si = torch.full((padded + 5,), -9, dtype=torch.int32, device=DEV)
    qs = torch.full((padded + 5,), -9, dtype=torch.int32, device=DEV)
    S.sconv_seq_metadata(qsl.to(DEV), n_req, actual, si, qs, num_padded_tokens=padded)
    torch.cuda.synchronize()
    assert torch.equal(si[:padded].cpu(), si_ref)
    assert torch.equal(qs[:padded].cpu(), qs_ref)
    assert torch.all(si[padded:].cpu() == -9) and torch.all(qs[padded:].cpu() == -9)


def test_seq_metadata_rejects_short_buffers():
    qsl = W.qsl_from_lengths([3, 2]).to(DEV)
    si = torch.empty(4, dtype=torch.int32, device=DEV)
    qs = torch.empty(8, dtype=torch.int32, device=DEV)
    with pytest.raises(S.SconvError):
        S.sconv_seq_metadata(qsl, 2, 5, si, qs)
    with pytest.raises(S.SconvError):
        S.sconv_seq_metadata(qsl, 2, 5, qs, qs[:6], num_padded_tokens=4)


# ---------------------------------------------------------- graph capture --

class Step:
    """Every entry point once, on preallocated device buffers, with state and
    caches restored from pristine copies by reset()."""

    def __init__(self):
        v = W.varlen_batch(lengths=[5, 0, 37, 300, 1], dim=520, width=4, seed=700,
                           num_lines=8, n_pad=1)
        self.v = {k: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for k, t in v.items()}
        self.v_out = torch.empty_like(self.v["x"])
        d = W.decode_batch(batch=6, dim=300, width=3, seqlen=1, seed=701, num_lines=8, n_pad=1)
        self.d = {k: (t.to(DEV) if t is not None else None) for k, t in d.items()}
        self.d_out = torch.empty_like(self.d["x"])
        s = W.spec_decode_batch(batch=5, dim=260, width=4, seqlen=3, state_len=6, num_lines=40,
                                n_pad=1, seed=702, mode="scatter")
        self.s = {k: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for k, t in s.items()}
        self.s_out = torch.empty_like(self.s["x"])
        p = W.paged_batch(H=4, ws=16, N=4, D=48, off_s=16, num_blocks=96, n_decode=5,
                          n_prefill=3, chunk=37, max_pos=60, width=4, pad_frac=0.1, seed=703)
        self.p = {k: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for k, t in p.items()}
        self.p_out = torch.empty_like(self.p["x"])
        m = W.paged_multi_batch(offsets=(16, 0), H=3, ws=16, N=4, D=40, num_blocks=96,
                                n_decode=4, n_prefill=2, chunk=23, max_pos=60, width=3,
                                pad_frac=0.1, seed=704, with_bias=True)
        self.m = {k: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for k, t in m.items()}
        for k in ("xs", "weights", "biases"):
            self.m[k] = [t.to(DEV) for t in m[k]]
        self.m_outs = [torch.empty_like(x) for x in self.m["xs"]]
        r = W.ring_decode_batch(batch=5, dim=200, width=4, seqlen=2, state_len=6, num_lines=8,
                                n_pad=1, seed=705)
        self.r = {k: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for k, t in r.items()}
        self.r_out = torch.empty_like(self.r["x"])
        c = W.varlen_batch(lengths=[40, 3, 0, 129], dim=264, width=5, seed=706, num_lines=6,
                           n_pad=1, layout="tok_dim")
        self.c = {k: (t.to(DEV) if isinstance(t, torch.Tensor) else t) for k, t in c.items()}
        self.c_out = S.new_output(self.c["x"])
        # token-contiguous batch with rows of at least 2048 tokens: the call
        # enqueues two kernels (the stream, then the head lanes)
        t = W.varlen_batch(lengths=[900, 0, 1400, 3], dim=72, width=4, seed=707, num_lines=6,
                           n_pad=1, layout="dim_tok")
        self.t = {k: (x.to(DEV) if isinstance(x, torch.Tensor) else x) for k, x in t.items()}
        self.t_out = S.new_output(self.t["x"])
        qsl = self.p["query_start_loc"]
        self.n_req = qsl.numel() - 1
        self.n_tok = self.p["x"].shape[0]
        self.si = torch.empty(self.n_tok + 4, dtype=torch.int32, device=DEV)
        self.qs = torch.empty(self.n_tok + 4, dtype=torch.int32, device=DEV)
        self.pristine = [t.clone() for t in self.mutable()]

    def mutable(self):
        return [self.v["conv_states"], self.d["conv_state"], self.s["conv_state"],
                self.s["intermediate"], self.p["cache"], self.m["cache"], self.r["conv_state"],
                self.c["conv_states"], self.t["conv_states"]]

    def bf_outputs(self):
        return [self.v_out, self.d_out, self.s_out, self.p_out, self.r_out, self.c_out,
                self.t_out] + self.m_outs

    def outputs(self):
        return self.bf_outputs() + [self.si, self.qs] + self.mutable()

    def reset(self):
        for t, p in zip(self.mutable(), self.pristine):
            t.copy_(p)
        for t in self.bf_outputs():
            t.fill_(-5.0)
        self.si.fill_(-1)
        self.qs.fill_(-1)

    def run(self):
        v, d, s, p = self.v, self.d, self.s, self.p
        S.conv1d_fwd_varlen(v["x"], v["weight"], v["bias"], v["conv_states"],
                            v["query_start_loc"], cache_indices=v["cache_indices"],
                            has_initial_state=v["has_initial_state"], activation="silu",
                            out=self.v_out)
        S.conv1d_update_decode(d["x"], d["conv_state"], d["weight"], d["bias"],
                               activation="silu", cache_indices=d["cache_indices"],
                               out=self.d_out)
        S.conv1d_update(s["x"], s["conv_state"], s["weight"], s["bias"], activation="silu",
                        cache_indices=s["cache_indices"],
                        num_accepted_tokens=s["num_accepted_tokens"],
                        intermediate=s["intermediate"],
                        output_state_indices=s["output_state_indices"], out=self.s_out)
        S.sconv_paged_fused(p["x"], p["weight"], p["cache"], p["positions"], p["slot_mapping"],
                            p["query_start_loc"], p["block_table"], p["off_s"], p["ws"],
                            activation="silu", use_residual=True, out=self.p_out)
        S.sconv_seq_metadata(p["query_start_loc"], self.n_req, self.n_tok, self.si, self.qs,
                             num_padded_tokens=self.n_tok + 2)
        m, r, c = self.m, self.r, self.c
        S.sconv_paged_fused_multi(m["xs"], m["weights"], m["cache"], m["positions"],
                                  m["slot_mapping"], m["query_start_loc"], m["block_table"],
                                  m["offs"], m["ws"], activation="silu", use_residual=True,
                                  biases=m["biases"], outs=self.m_outs)
        S.conv1d_update(r["x"], r["conv_state"], r["weight"], r["bias"], activation="silu",
                        cache_indices=r["cache_indices"], cache_seqlens=r["cache_seqlens"],
                        out=self.r_out)
        S.conv1d_fwd_varlen(c["x"], c["weight"], c["bias"], c["conv_states"],
                            c["query_start_loc"], cache_indices=c["cache_indices"],
                            has_initial_state=c["has_initial_state"], activation="silu",
                            out=self.c_out)
        t = self.t
        S.conv1d_fwd_varlen(t["x"], t["weight"], t["bias"], t["conv_states"],
                            t["query_start_loc"], cache_indices=t["cache_indices"],
                            has_initial_state=t["has_initial_state"], activation="silu",
                            out=self.t_out)


def test_graph_capture_replays_every_entry_point():
    st = Step()
    st.reset()
    st.run()
    torch.cuda.synchronize()
    eager = [t.clone() for t in st.outputs()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        st.reset()
        st.run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st.run()
    torch.cuda.synchronize()

    noise = torch.empty(1 << 20, device=DEV)
    for rep in range(4):
        say(f"[graph] replay {rep}")
        st.reset()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, want) in enumerate(zip(st.outputs(), eager)):
            if got.dtype == torch.int32:
                assert torch.equal(got, want), f"replay {rep}, buffer {i}"
            else:
                assert_bits(got, want, f"replay {rep}, buffer {i}")
        noise.normal_()                       # eager work between replays
        float(noise.sum())
