"""GPU parity for sconv_paged_fused (through the C ABI) against the oracle."""
import pytest
import torch

import causal_depthwise_short_conv1d_amd as S
import oracle
import workloads as W
from tests.parity import assert_bits, assert_close, say

pytestmark = pytest.mark.gpu
DEV = "cuda"
BF = torch.bfloat16
SMALL = dict(H=4, ws=16, N=4, D=48, off_s=16, num_blocks=96, n_decode=5,
             n_prefill=3, chunk=37, max_pos=60)
SMALL_NO_OFF = {k: v for k, v in SMALL.items() if k != "off_s"}


def run_both(d, activation="silu", residual=True, exact=False, cache_dev=None, label=""):
    """d: CPU tensors except (optionally) the cache, given on the GPU."""
    say(f"[paged] {label} T={d['x'].shape[0]} C={d['x'].shape[1]}")
    cache_gpu = cache_dev if cache_dev is not None else d["cache"].to(DEV)
    cache_ref = cache_gpu.cpu()
    out_ref = torch.full(d["x"].shape, float("nan"), dtype=BF)
    oracle.paged(d["x"], d["weight"], d["bias"], cache_ref, d["positions"], d["slot_mapping"],
                 d["query_start_loc"], d["block_table"], d["off_s"], d["ws"], out_ref,
                 activation=activation, use_residual=residual)
    dv = lambda t: None if t is None else t.to(DEV)
    out = S.sconv_paged_fused(dv(d["x"]), dv(d["weight"]), cache_gpu, dv(d["positions"]),
                              dv(d["slot_mapping"]), dv(d["query_start_loc"]),
                              dv(d["block_table"]), d["off_s"], d["ws"],
                              activation=activation, use_residual=residual, bias=dv(d["bias"]))
    torch.cuda.synchronize()
    if exact:
        assert_bits(out, out_ref, f"{label} out")
    else:
        assert_close(out, out_ref, f"{label} out")
    assert_bits(cache_gpu, cache_ref, f"{label} cache")
    return out, cache_gpu


def test_paged_mixed_batch_full_size():
    """32 decode tokens + 8 prefill chunks of 512, H 32, ws 128, cache
    [4096, 32, 16, 512], 5% pad rows, residual + SiLU."""
    cfg = W.PAGED_MIXED
    # the 2 GiB cache (and x, weight) are drawn on the GPU
    d2 = W.paged_batch(H=cfg["H"], ws=cfg["ws"], N=cfg["N"], D=cfg["D"], off_s=cfg["off_s"],
                       num_blocks=cfg["num_blocks"], width=cfg["width"],
                       n_decode=cfg["n_decode"], n_prefill=cfg["n_prefill"], chunk=cfg["chunk"],
                       max_pos=cfg["max_pos"], pad_frac=cfg["pad_frac"], seed=W.seed_for(5),
                       device=DEV)
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) and k != "cache" else v)
            for k, v in d2.items()}
    run_both(host, cache_dev=d2["cache"], label="mixed full size")


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("residual", [True, False])
def test_paged_small(width, residual):
    d = W.paged_batch(**SMALL, width=width, pad_frac=0.1, trailing_pad=3,
                      seed=100 + width, with_bias=(width % 2 == 0), min_pos=0)
    run_both(d, residual=residual, label=f"small W{width}")


@pytest.mark.parametrize("width", [2, 4, 5])
def test_paged_exact_values(width):
    d = W.paged_batch(**SMALL, width=width, pad_frac=0.2, trailing_pad=2,
                      seed=200 + width, values="exact", with_bias=True, min_pos=0)
    run_both(d, activation=None, residual=True, exact=True, label=f"exact W{width}")


@pytest.mark.parametrize("width", [3, 4])
def test_paged_sixteen_token_tiles_exact(width):
    """A step large enough (8232 tokens x 16 slabs) for the 16-token tiles
    (smaller steps take 8-token tiles): decode tokens, prefill chunks with
    cached taps, interior and trailing pads, exact values, bit-exact against
    the oracle."""
    cfg = dict(H=32, ws=128, N=16, D=256, off_s=64, num_blocks=1024, n_decode=40,
               n_prefill=16, chunk=512, max_pos=4000)
    d2 = W.paged_batch(**cfg, width=width, pad_frac=0.05, trailing_pad=5, seed=450 + width,
                       values="exact", with_bias=True, device=DEV)
    assert d2["x"].shape[0] // 16 * (cfg["H"] * cfg["ws"] // 256) >= 8192
    host = {k: (v.cpu() if isinstance(v, torch.Tensor) and k != "cache" else v)
            for k, v in d2.items()}
    run_both(host, activation=None, residual=True, exact=True, cache_dev=d2["cache"],
             label=f"16-token tiles W{width}")


def test_paged_idempotent_on_gpu():
    d = W.paged_batch(**SMALL, width=4, pad_frac=0.1, seed=300)
    out1, cache1 = run_both(d, label="first")
    before = cache1.clone()
    dv = lambda t: t.to(DEV)
    out2 = S.sconv_paged_fused(dv(d["x"]), dv(d["weight"]), cache1, dv(d["positions"]),
                               dv(d["slot_mapping"]), dv(d["query_start_loc"]),
                               dv(d["block_table"]), d["off_s"], d["ws"], activation="silu")
    torch.cuda.synchronize()
    assert_bits(out2, out1, "second step out")
    assert_bits(cache1, before, "second step cache")


def test_paged_partial_slab_and_many_heads():
    # C = 20 heads * 24 = 480 channels: one partial 512-wide slab
    cfg = dict(H=20, ws=24, N=8, D=64, off_s=32, num_blocks=200, n_decode=7, n_prefill=2,
               chunk=45, max_pos=200)
    d = W.paged_batch(**cfg, width=4, pad_frac=0.05, seed=400)
    run_both(d, label="partial slab")


def test_paged_only_decode_tokens():
    d = W.paged_batch(**dict(SMALL, n_decode=40, n_prefill=0), width=4, pad_frac=0.1, seed=500)
    run_both(d, label="decode only")


# ---------------------------------------------------------- multi-stream --

def run_multi(d, activation="silu", residual=True, exact=False, label=""):
    """All streams of d in one sconv_paged_fused_multi launch against the
    oracle run stream by stream on one cache (the D sub-ranges are disjoint,
    so the order of the streams does not matter)."""
    say(f"[paged multi] {label} streams={len(d['xs'])} T={d['x'].shape[0]}")
    cache_gpu = d["cache"].to(DEV)
    cache_ref = d["cache"].clone()
    refs = []
    for x, w, b, off in zip(d["xs"], d["weights"], d["biases"], d["offs"]):
        o = torch.full(x.shape, float("nan"), dtype=BF)
        oracle.paged(x, w, b, cache_ref, d["positions"], d["slot_mapping"],
                     d["query_start_loc"], d["block_table"], off, d["ws"], o,
                     activation=activation, use_residual=residual)
        refs.append(o)
    dv = lambda t: None if t is None else t.to(DEV)
    outs = S.sconv_paged_fused_multi([dv(x) for x in d["xs"]], [dv(w) for w in d["weights"]],
                                     cache_gpu, dv(d["positions"]), dv(d["slot_mapping"]),
                                     dv(d["query_start_loc"]), dv(d["block_table"]), d["offs"],
                                     d["ws"], activation=activation, use_residual=residual,
                                     biases=[dv(b) for b in d["biases"]])
    torch.cuda.synchronize()
    for i, (o, r) in enumerate(zip(outs, refs)):
        if exact:
            assert_bits(o, r, f"{label} stream {i} out")
        else:
            assert_close(o, r, f"{label} stream {i} out")
    assert_bits(cache_gpu, cache_ref, f"{label} cache")
    return outs, cache_gpu


def test_paged_multi_four_streams_full_size():
    """The mixed step with the page's four streams filling D = 512."""
    cfg = {k: v for k, v in W.PAGED_MIXED.items() if k != "off_s"}
    d = W.paged_multi_batch(seed=W.seed_for(5, 1), **cfg)
    run_multi(d, label="four streams")


@pytest.mark.parametrize("width", [2, 3, 4, 5])
@pytest.mark.parametrize("residual", [True, False])
def test_paged_multi_small(width, residual):
    d = W.paged_multi_batch(offsets=(32, 0, 16), width=width, pad_frac=0.1, trailing_pad=2,
                            seed=600 + width, with_bias=(width % 2 == 1), min_pos=0, **SMALL_NO_OFF)
    run_multi(d, residual=residual, label=f"small W{width}")


def test_paged_multi_exact_bit_exact():
    d = W.paged_multi_batch(offsets=(0, 24), width=4, pad_frac=0.2, seed=610, values="exact",
                            with_bias=True, min_pos=0, **dict(SMALL_NO_OFF, ws=8, D=40))
    run_multi(d, activation=None, exact=True, label="exact")


def test_paged_multi_equals_single_stream_calls():
    d = W.paged_multi_batch(offsets=(16, 0), width=4, pad_frac=0.1, seed=620, **SMALL_NO_OFF)
    outs, cache_multi = run_multi(d, label="vs singles")
    cache = d["cache"].to(DEV)
    dv = lambda t: None if t is None else t.to(DEV)
    for i, (x, w, off) in enumerate(zip(d["xs"], d["weights"], d["offs"])):
        o = S.sconv_paged_fused(dv(x), dv(w), cache, dv(d["positions"]), dv(d["slot_mapping"]),
                                dv(d["query_start_loc"]), dv(d["block_table"]), off, d["ws"],
                                activation="silu", use_residual=True)
        torch.cuda.synchronize()
        assert_bits(o, outs[i], f"single stream {i}")
    assert_bits(cache, cache_multi, "cache after singles")


def test_paged_multi_rejects_overlapping_streams():
    d = W.paged_multi_batch(offsets=(0, 8), width=4, seed=630, **SMALL_NO_OFF)
    dv = lambda t: t.to(DEV)
    with pytest.raises(S.SconvError):
        S.sconv_paged_fused_multi([dv(x) for x in d["xs"]], [dv(w) for w in d["weights"]],
                                  dv(d["cache"]), dv(d["positions"]), dv(d["slot_mapping"]),
                                  dv(d["query_start_loc"]), dv(d["block_table"]), d["offs"],
                                  d["ws"])
