"""libsconv: causal depthwise short convolution on MI355X (gfx950).

Thin Python binding over the C ABI declared in include/sconv.h.  It only
marshals torch tensors into device pointers, element strides and the current
HIP stream; every step of the computation runs in the library's HIP kernels.
There is no fallback: if libsconv.so is missing or a call is rejected, the
binding raises.

Entry points (same names as the C ABI):
  conv1d_fwd_varlen    -- varlen prefill with per-sequence conv state
  conv1d_update_decode -- decode update (state shift), in place allowed
  conv1d_update        -- decode update with speculative-decoding and
                          ring-buffer options
  sconv_paged_fused    -- paged sliding-window cache insert + conv
  sconv_paged_fused_multi -- several conv streams sharing one paged cache
  sconv_seq_metadata   -- per-token (request, first row) buffers
bind_fwd_varlen and bind_update_decode marshal a forward or a decode step
once for repeated launches.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = ["conv1d_fwd_varlen", "conv1d_update_decode", "conv1d_update", "sconv_paged_fused",
           "sconv_paged_fused_multi", "sconv_seq_metadata", "new_output", "bind_fwd_varlen",
           "bind_update_decode",
           "SconvError", "library_path", "load_library", "exported_symbols",
           "version", "status_string"]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libsconv.so")
_lib = None

ACT_NONE, ACT_SILU = 0, 1


class SconvError(RuntimeError):
    """A libsconv call returned a non-zero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load libsconv.so (built by causal_depthwise_short_conv1d_amd.build).
    Raises FileNotFoundError when it has not been built."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise FileNotFoundError(
            f"libsconv not built: {p} is missing "
            "(run python -m causal_depthwise_short_conv1d_amd.build)")
    lib = ctypes.CDLL(p)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.sconv_status_string.argtypes = [ctypes.c_int]
    lib.sconv_status_string.restype = ctypes.c_char_p
    lib.sconv_version.argtypes = []
    lib.sconv_version.restype = ctypes.c_int
    lib.conv1d_fwd_varlen.argtypes = [
        P, I64, I64, P, I64, P, P, I64, I64, I64, I64, P, P, P,
        I32, I64, I32, I32, I32, I32, P, I64, I64, P]
    lib.conv1d_update_decode.argtypes = [
        P, I64, I64, I64, P, I64, P, P, I64, I64, I64, I64, P,
        I32, I32, I32, I32, I32, I32, P, I64, I64, I64, P]
    lib.conv1d_update.argtypes = [
        P, I64, I64, I64, P, I64, P, P, I64, I64, I64, I64, I32, P, P, P,
        P, I64, I64, I64, I64, P, I64, I64,
        I32, I32, I32, I32, I32, I32, P, I64, I64, I64, P]
    lib.sconv_paged_fused.argtypes = [
        P, I64, P, I64, P, P, I64, I64, I64, I64, I32, I32, I32, I32, I32,
        P, P, P, I32, P, I64, I32, I64, I32, I32, I32, P, I64, P]
    lib.sconv_seq_metadata.argtypes = [P, I32, I64, I64, P, I64, P, I64, P]
    lib.sconv_paged_fused_multi.argtypes = [
        I32, P, P, P, P, P, P, P, P, P, P, I64, I64, I64, I64, I32, I32, I32,
        P, P, P, I32, P, I64, I32, I64, I32, I32, I32, P]
    for f in (lib.conv1d_fwd_varlen, lib.conv1d_update_decode, lib.conv1d_update,
              lib.sconv_paged_fused, lib.sconv_paged_fused_multi, lib.sconv_seq_metadata):
        f.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def exported_symbols() -> list[str]:
    return ["sconv_status_string", "sconv_version", "conv1d_fwd_varlen",
            "conv1d_update_decode", "conv1d_update", "sconv_paged_fused",
            "sconv_paged_fused_multi", "sconv_seq_metadata"]


def version() -> tuple[int, int]:
    v = load_library().sconv_version()
    return v >> 16, v & 0xFFFF


def status_string(status: int) -> str:
    try:
        return load_library().sconv_status_string(int(status)).decode()
    except FileNotFoundError:
        return "unknown"


# ------------------------------------------------------------ marshalling --

def _dev(t: torch.Tensor | None, dtype: torch.dtype, name: str, device=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    return ctypes.c_void_p(t.data_ptr()) if t.numel() else None


def _index(t, dtype, name, device, n=None):
    p = _dev(t, dtype, name, device)
    if t is not None:
        if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous 1-D tensor")
        if n is not None and t.numel() < n:
            raise ValueError(f"{name} needs at least {n} entries")
    return p


def _act(activation) -> int:
    if activation is True or activation in ("silu", "swish"):
        return ACT_SILU
    if activation in (None, False):
        return ACT_NONE
    raise ValueError(f"unsupported activation {activation!r}")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(device) -> ctypes.c_void_p:
    """The current stream of `device` as a raw handle (torch's accessor when
    it has one: no Stream object per call)."""
    if _raw_stream is not None:
        return ctypes.c_void_p(_raw_stream(device.index if device.index is not None
                                           else torch.cuda.current_device()))
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _call(fn: str, *args) -> None:
    rc = getattr(load_library(), fn)(*args)
    if rc != 0:
        raise SconvError(fn, rc)


def _launch(fn: str, dev, args) -> None:
    """Call `fn` with the current stream of `dev` appended, with `dev` made
    the current device for the call (the library launches on the current
    device) unless it already is."""
    if dev.index is None or dev.index == torch.cuda.current_device():
        _call(fn, *args, _stream(dev))
    else:
        with torch.cuda.device(dev):
            _call(fn, *args, _stream(dev))


def new_output(x: torch.Tensor) -> torch.Tensor:
    """An uninitialised output in the storage class of x's smaller stride: a
    compact (dim, T) array when tokens are x's closer axis, else (T, pitch)
    storage viewed as (dim, T) with a row pitch rounded up to 8 elements
    (16-byte aligned rows).  Both are layouts the vector kernels take."""
    dim, total = x.shape
    if dim == 1 or (total > 1 and x.stride(1) < x.stride(0)):
        return torch.empty((dim, total), dtype=x.dtype, device=x.device)
    pitch = (dim + 7) // 8 * 8
    return torch.empty((total, pitch), dtype=x.dtype, device=x.device)[:, :dim].t()


def _fwd_varlen_args(x, weight, bias, conv_states, query_start_loc, cache_indices,
                     has_initial_state, activation, pad_slot_id, out):
    """Checked and marshalled arguments of conv1d_fwd_varlen (all but the
    stream), and the output tensor."""
    dev = x.device
    dim, total = x.shape
    width = weight.shape[1]
    batch = query_start_loc.numel() - 1
    if weight.dim() != 2 or weight.shape[0] != dim or weight.stride(1) != 1:
        raise ValueError("weight must be (dim, width) with unit width stride")
    if out is None:
        out = new_output(x)
    if out.shape != x.shape:
        raise ValueError("out must have x's shape")
    if bias is not None and (bias.shape != (dim,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous (dim,) tensor")
    cs = conv_states
    if cs is not None and (cs.dim() != 3 or cs.shape[1] != dim or cs.shape[2] != width - 1):
        raise ValueError("conv_states must be (lines, dim, width-1)")
    bf = torch.bfloat16
    args = (
        _dev(x, bf, "x", dev), x.stride(0), x.stride(1),
        _dev(weight, bf, "weight", dev), weight.stride(0),
        _dev(bias, bf, "bias", dev),
        _dev(cs, bf, "conv_states", dev),
        *(cs.stride() if cs is not None else (0, 0, 0)),
        cs.shape[0] if cs is not None else 0,
        _index(cache_indices, torch.int32, "cache_indices", dev, batch),
        _index(has_initial_state, torch.bool, "has_initial_state", dev, batch),
        _index(query_start_loc, torch.int32, "query_start_loc", dev),
        batch, total, dim, width, _act(activation), pad_slot_id,
        _dev(out, bf, "out", dev), out.stride(0), out.stride(1),
    )
    return args, out


def conv1d_fwd_varlen(x, weight, bias, conv_states, query_start_loc,
                      cache_indices=None, has_initial_state=None,
                      activation="silu", pad_slot_id: int = -1, out=None):
    """Varlen prefill.  x: logical (dim, total_T) bf16 with any strides
    (compact (dim, T) and 16-byte aligned (T, dim) rows take the vector
    kernels); weight (dim, width); bias (dim,) or None; conv_states
    (lines, dim, width-1) or None, updated in place; query_start_loc int32
    (batch+1,); cache_indices int32 (batch,) or None; has_initial_state bool
    (batch,) or None.  Returns out (a new tensor with x's strides unless
    given; see new_output)."""
    args, out = _fwd_varlen_args(x, weight, bias, conv_states, query_start_loc, cache_indices,
                                 has_initial_state, activation, pad_slot_id, out)
    _launch("conv1d_fwd_varlen", x.device, args)
    return out


def bind_fwd_varlen(x, weight, bias, conv_states, query_start_loc, cache_indices=None,
                    has_initial_state=None, activation="silu", pad_slot_id: int = -1,
                    out=None, stream=None):
    """A pre-bound conv1d_fwd_varlen for a caller that runs the same forward
    over and over on fixed buffers (a prefill loop over preallocated
    batches): the tensors are checked and marshalled once, here, and the
    returned function only enqueues the launch on `stream` (default: the
    current stream of x's device now) and raises on a non-zero status.  Its
    `out` attribute is the output tensor.  The tensors must stay alive and
    in place while the function is used."""
    args, out = _fwd_varlen_args(x, weight, bias, conv_states, query_start_loc, cache_indices,
                                 has_initial_state, activation, pad_slot_id, out)
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(x.device)
    f = load_library().conv1d_fwd_varlen
    full = (*args, st)

    def launch():
        rc = f(*full)
        if rc != 0:
            raise SconvError("conv1d_fwd_varlen", rc)
    launch.out = out
    return launch


def conv1d_update_decode(x, conv_state, weight, bias=None, activation=None,
                         cache_indices=None, pad_slot_id: int = -1, out=None):
    """Decode update.  x: (batch, dim) or (batch, dim, seqlen) bf16;
    conv_state (lines, dim, width-1) updated in place; returns out, which
    may be x itself (pass out=x to compute in place)."""
    dev = x.device
    squeeze = x.dim() == 2
    xv = x.unsqueeze(-1) if squeeze else x
    ov = None
    if out is not None:
        ov = out.unsqueeze(-1) if out.dim() == 2 else out
    else:
        ov = torch.empty_like(xv)
    batch, dim, seqlen = xv.shape
    width = weight.shape[1]
    if weight.dim() != 2 or weight.shape[0] != dim or weight.stride(1) != 1:
        raise ValueError("weight must be (dim, width) with unit width stride")
    if conv_state.dim() != 3 or conv_state.shape[1] != dim or conv_state.shape[2] != width - 1:
        raise ValueError("conv_state must be (lines, dim, width-1)")
    if bias is not None and (bias.shape != (dim,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous (dim,) tensor")
    if ov.shape != xv.shape:
        raise ValueError("out must have x's shape")
    bf = torch.bfloat16
    args = (
        _dev(xv, bf, "x", dev), *xv.stride(),
        _dev(weight, bf, "weight", dev), weight.stride(0),
        _dev(bias, bf, "bias", dev),
        _dev(conv_state, bf, "conv_state", dev), *conv_state.stride(), conv_state.shape[0],
        _index(cache_indices, torch.int32, "cache_indices", dev, batch),
        batch, dim, seqlen, width, _act(activation), pad_slot_id,
        _dev(ov, bf, "out", dev), *ov.stride(),
    )
    _launch("conv1d_update_decode", dev, args)
    if out is not None:
        return out
    return ov.squeeze(-1) if squeeze else ov


def bind_update_decode(x, conv_state, weight, bias=None, activation=None, cache_indices=None,
                       pad_slot_id: int = -1, out=None, stream=None):
    """A pre-bound conv1d_update_decode for a caller that launches the same
    decode step over and over on fixed buffers (a serving loop): the tensors
    are checked and marshalled once, here, and the returned function only
    enqueues the launch on `stream` (default: the current stream of x's
    device now) and raises on a non-zero status.  out=None computes in
    place (x is overwritten, as the page's update does).  The tensors must
    stay alive and in place while the function is used."""
    dev = x.device
    squeeze = x.dim() == 2
    xv = x.unsqueeze(-1) if squeeze else x
    ov = xv if out is None else (out.unsqueeze(-1) if out.dim() == 2 else out)
    batch, dim, seqlen = xv.shape
    width = weight.shape[1]
    if weight.dim() != 2 or weight.shape[0] != dim or weight.stride(1) != 1:
        raise ValueError("weight must be (dim, width) with unit width stride")
    if conv_state.dim() != 3 or conv_state.shape[1] != dim or conv_state.shape[2] != width - 1:
        raise ValueError("conv_state must be (lines, dim, width-1)")
    if bias is not None and (bias.shape != (dim,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous (dim,) tensor")
    if ov.shape != xv.shape:
        raise ValueError("out must have x's shape")
    bf = torch.bfloat16
    st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(dev)
    args = (
        _dev(xv, bf, "x", dev), *xv.stride(),
        _dev(weight, bf, "weight", dev), weight.stride(0),
        _dev(bias, bf, "bias", dev),
        _dev(conv_state, bf, "conv_state", dev), *conv_state.stride(), conv_state.shape[0],
        _index(cache_indices, torch.int32, "cache_indices", dev, batch),
        batch, dim, seqlen, width, _act(activation), pad_slot_id,
        _dev(ov, bf, "out", dev), *ov.stride(), st,
    )
    f = load_library().conv1d_update_decode

    def launch():
        rc = f(*args)
        if rc != 0:
            raise SconvError("conv1d_update_decode", rc)
    return launch


def conv1d_update(x, conv_state, weight, bias=None, activation=None, cache_indices=None,
                  cache_seqlens=None, num_accepted_tokens=None, intermediate=None,
                  output_state_indices=None, pad_slot_id: int = -1, out=None):
    """Decode update with the speculative-decoding options
    (num_accepted_tokens (batch,) int32; intermediate (batch, steps, dim,
    width-1) bf16; output_state_indices (batch, seqlen) int32) or ring-buffer
    states (cache_seqlens (batch,) int32).  x: (batch, dim) or
    (batch, dim, seqlen) bf16; conv_state (lines, dim, state_len) bf16,
    state_len >= width-1.  Returns out, which may be x itself."""
    dev = x.device
    squeeze = x.dim() == 2
    xv = x.unsqueeze(-1) if squeeze else x
    if out is not None:
        ov = out.unsqueeze(-1) if out.dim() == 2 else out
    else:
        ov = torch.empty_like(xv)
    batch, dim, seqlen = xv.shape
    width = weight.shape[1]
    if weight.dim() != 2 or weight.shape[0] != dim or weight.stride(1) != 1:
        raise ValueError("weight must be (dim, width) with unit width stride")
    if conv_state.dim() != 3 or conv_state.shape[1] != dim:
        raise ValueError("conv_state must be (lines, dim, state_len)")
    if bias is not None and (bias.shape != (dim,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous (dim,) tensor")
    if ov.shape != xv.shape:
        raise ValueError("out must have x's shape")
    inter = intermediate
    if inter is not None and (inter.dim() != 4 or inter.shape[0] < batch or
                              inter.shape[1] < seqlen or inter.shape[2] != dim or
                              inter.shape[3] != width - 1):
        raise ValueError("intermediate must be (batch, >= seqlen, dim, width-1)")
    osi = output_state_indices
    if osi is not None:
        if osi.dim() != 2 or osi.shape[0] < batch or osi.shape[1] < seqlen:
            raise ValueError("output_state_indices must be (batch, >= seqlen)")
        _dev(osi, torch.int32, "output_state_indices", dev)
    bf = torch.bfloat16
    args = (
        _dev(xv, bf, "x", dev), *xv.stride(),
        _dev(weight, bf, "weight", dev), weight.stride(0),
        _dev(bias, bf, "bias", dev),
        _dev(conv_state, bf, "conv_state", dev), *conv_state.stride(), conv_state.shape[0],
        conv_state.shape[2],
        _index(cache_indices, torch.int32, "cache_indices", dev, batch),
        _index(cache_seqlens, torch.int32, "cache_seqlens", dev, batch),
        _index(num_accepted_tokens, torch.int32, "num_accepted_tokens", dev, batch),
        _dev(inter, bf, "intermediate", dev), *(inter.stride() if inter is not None else (0,) * 4),
        _dev(osi, torch.int32, "output_state_indices", dev),
        *(osi.stride() if osi is not None else (0, 0)),
        batch, dim, seqlen, width, _act(activation), pad_slot_id,
        _dev(ov, bf, "out", dev), *ov.stride(),
    )
    _launch("conv1d_update", dev, args)
    if out is not None:
        return out
    return ov.squeeze(-1) if squeeze else ov


def sconv_paged_fused(x, weight, cache, positions, slot_mapping, query_start_loc,
                      block_table, off_s: int, ws: int, activation=None,
                      use_residual: bool = True, bias=None, out=None):
    """Paged insert + conv.  x (T, H*ws) bf16; weight (H*ws, width); cache
    (num_blocks, H, N, D) bf16 with unit D stride, updated in place;
    positions / slot_mapping int64 (T,); query_start_loc int32 (R+1,);
    block_table int32 (R, max_blocks).  Returns out (T, H*ws)."""
    dev = x.device
    T, C = x.shape
    num_blocks, H, N, D = cache.shape
    width = weight.shape[1]
    num_reqs = query_start_loc.numel() - 1
    if C != H * ws:
        raise ValueError("x's channel count must be cache heads * ws")
    if x.stride(1) != 1 or cache.stride(3) != 1:
        raise ValueError("x channels and cache D must have unit stride")
    if weight.dim() != 2 or weight.shape[0] != C or weight.stride(1) != 1:
        raise ValueError("weight must be (C, width) with unit width stride")
    if bias is not None and (bias.shape != (C,) or bias.stride(0) != 1):
        raise ValueError("bias must be a contiguous (C,) tensor")
    if block_table.dim() != 2 or (block_table.numel() and block_table.stride(1) != 1):
        raise ValueError("block_table must be 2-D with unit column stride")
    if out is None:
        out = torch.empty_like(x)
    if out.shape != x.shape or out.stride(1) != 1:
        raise ValueError("out must be (T, C) with unit channel stride")
    bf = torch.bfloat16
    args = (
        _dev(x, bf, "x", dev), x.stride(0),
        _dev(weight, bf, "weight", dev), weight.stride(0),
        _dev(bias, bf, "bias", dev),
        _dev(cache, bf, "cache", dev), cache.stride(0), cache.stride(1), cache.stride(2),
        num_blocks, H, N, D, off_s, ws,
        _index(positions, torch.int64, "positions", dev, T),
        _index(slot_mapping, torch.int64, "slot_mapping", dev, T),
        _index(query_start_loc, torch.int32, "query_start_loc", dev),
        num_reqs,
        _dev(block_table, torch.int32, "block_table", dev), block_table.stride(0),
        block_table.shape[1],
        T, width, _act(activation), int(bool(use_residual)),
        _dev(out, bf, "out", dev), out.stride(0),
    )
    _launch("sconv_paged_fused", dev, args)
    return out


def sconv_seq_metadata(query_start_loc, num_reqs: int, num_actual_tokens: int,
                       seq_idx_out, query_start_out, num_padded_tokens: int | None = None):
    """Fill seq_idx_out / query_start_out (int32 device tensors) for the
    first num_padded_tokens rows (default num_actual_tokens): owning request
    and its first row for actual rows, 0 / 0 for padded ones."""
    dev = seq_idx_out.device
    for name, t in (("seq_idx_out", seq_idx_out), ("query_start_out", query_start_out)):
        if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
            raise ValueError(f"{name} must be a contiguous 1-D tensor")
    padded = -1 if num_padded_tokens is None else int(num_padded_tokens)
    args = (
        _index(query_start_loc, torch.int32, "query_start_loc", dev, int(num_reqs) + 1),
        int(num_reqs), int(num_actual_tokens), padded,
        _dev(seq_idx_out, torch.int32, "seq_idx_out", dev), seq_idx_out.numel(),
        _dev(query_start_out, torch.int32, "query_start_out", dev), query_start_out.numel(),
    )
    _launch("sconv_seq_metadata", dev, args)


def sconv_paged_fused_multi(xs, weights, cache, positions, slot_mapping, query_start_loc,
                            block_table, offs, ws: int, activation=None,
                            use_residual: bool = True, biases=None, outs=None):
    """Several conv streams sharing one paged cache, in one launch.  xs,
    weights, offs (and biases / outs when given) are lists with one entry per
    stream; every stream has H * ws channels (ws may also be a list).
    Returns the list of outputs."""
    n = len(xs)
    if not (len(weights) == len(offs) == n) or n < 1:
        raise ValueError("xs, weights and offs need one entry per stream")
    wss = list(ws) if isinstance(ws, (list, tuple)) else [int(ws)] * n
    dev = xs[0].device
    num_blocks, H, N, D = cache.shape
    width = weights[0].shape[1]
    num_reqs = query_start_loc.numel() - 1
    T = xs[0].shape[0]
    if outs is None:
        outs = [torch.empty_like(x) for x in xs]
    if biases is None:
        biases = [None] * n
    bf = torch.bfloat16
    for i in range(n):
        x, w, b, o = xs[i], weights[i], biases[i], outs[i]
        if x.dim() != 2 or x.shape != (T, H * wss[i]) or x.stride(1) != 1:
            raise ValueError(f"stream {i}: x must be (T, H*ws) with unit channel stride")
        if o.shape != x.shape or o.stride(1) != 1:
            raise ValueError(f"stream {i}: out must match x")
        if w.dim() != 2 or w.shape != (H * wss[i], width) or w.stride(1) != 1:
            raise ValueError(f"stream {i}: weight must be (C, width) with unit width stride")
        if b is not None and (b.shape != (H * wss[i],) or b.stride(0) != 1):
            raise ValueError(f"stream {i}: bias must be a contiguous (C,) tensor")
    if cache.stride(3) != 1:
        raise ValueError("cache D must have unit stride")
    if block_table.dim() != 2 or (block_table.numel() and block_table.stride(1) != 1):
        raise ValueError("block_table must be (num_reqs, max_blocks) with unit inner stride")
    VP = ctypes.c_void_p * n
    I64A = ctypes.c_int64 * n
    I32A = ctypes.c_int32 * n
    xp = VP(*[_dev(x, bf, f"xs[{i}]", dev) for i, x in enumerate(xs)])
    wp = VP(*[_dev(w, bf, f"weights[{i}]", dev) for i, w in enumerate(weights)])
    bp = VP(*[_dev(b, bf, f"biases[{i}]", dev) for i, b in enumerate(biases)])
    op = VP(*[_dev(o, bf, f"outs[{i}]", dev) for i, o in enumerate(outs)])
    args = (
        n, xp, I64A(*[x.stride(0) for x in xs]), wp, I64A(*[w.stride(0) for w in weights]),
        bp if any(b is not None for b in biases) else None,
        I32A(*[int(o) for o in offs]), I32A(*wss), op, I64A(*[o.stride(0) for o in outs]),
        _dev(cache, bf, "cache", dev), cache.stride(0), cache.stride(1), cache.stride(2),
        num_blocks, H, N, D,
        _index(positions, torch.int64, "positions", dev, T),
        _index(slot_mapping, torch.int64, "slot_mapping", dev, T),
        _index(query_start_loc, torch.int32, "query_start_loc", dev, num_reqs + 1), num_reqs,
        _dev(block_table, torch.int32, "block_table", dev),
        block_table.stride(0) if block_table.dim() == 2 else 0,
        block_table.shape[1] if block_table.dim() == 2 else 0,
        T, width, _act(activation), int(bool(use_residual)),
    )
    _launch("sconv_paged_fused_multi", dev, args)
    return outs
