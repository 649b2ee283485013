"""CPU oracle for the causal depthwise short convolution.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the library itself never does and
must not.  It shares no code with the HIP implementation: the arithmetic lives
in ``sconv_oracle.c`` (plain C, fp64), compiled with gcc into
``liboracle.so``; this file only marshals torch CPU tensors into pointers and
element strides.

Every function works IN PLACE on the tensors it is given, like the library:
``out`` receives outputs, ``conv_states`` / ``cache`` receive the new state.
Callers clone first when they need the old contents.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sconv_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

__all__ = ["build", "fwd_varlen", "update_decode", "update_general", "paged", "seq_metadata",
           "bf16_from_f64", "f64_from_bf16", "silu"]


def build() -> str:
    """Compile the oracle with gcc (IEEE double arithmetic: no fast-math, no
    FMA contraction)."""
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    subprocess.run(["gcc", "-O2", "-std=c11", "-fPIC", "-shared",
                    "-ffp-contract=off", "-fno-fast-math", _SRC, "-o", tmp, "-lm"],
                   check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if (not os.path.exists(_LIB_PATH)
            or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_silu.argtypes = [ctypes.c_double]
    lib.oracle_silu.restype = ctypes.c_double
    lib.oracle_fwd_varlen.argtypes = [
        P, I64, I64, P, I64, I64, P, P, I64, I64, I64, I64, P, P, P,
        I32, I32, I32, I32, I32, P, I64, I64]
    lib.oracle_update_decode.argtypes = [
        P, I64, I64, I64, P, I64, I64, P, P, I64, I64, I64, I64, P,
        I32, I32, I32, I32, I32, I32, P, I64, I64, I64]
    lib.oracle_update_general.argtypes = [
        P, I64, I64, I64, P, I64, I64, P, P, I64, I64, I64, I64, I32, P, P, P,
        P, I64, I64, I64, I64, P, I64, I64, I32, I32, I32, I32, I32, I32,
        P, I64, I64, I64]
    lib.oracle_paged.argtypes = [
        P, I64, P, I64, I64, P, P, I64, I64, I64, I64, I32, I32, I32, I32,
        P, P, P, I32, P, I64, I32, I64, I32, I32, I32, P, I64]
    lib.oracle_seq_metadata.argtypes = [P, I32, I64, I64, P, P]
    for f in (lib.oracle_fwd_varlen, lib.oracle_update_decode, lib.oracle_update_general,
              lib.oracle_paged,
              lib.oracle_seq_metadata):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(t, dtype=None):
    if t is None:
        return None
    if t.device.type != "cpu":
        raise ValueError("the oracle takes CPU tensors")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _ptr1d(t, dtype):
    """A 1-D index array: the oracle reads it with unit stride."""
    if t is None:
        return None
    if t.dim() != 1 or (t.numel() > 1 and t.stride(0) != 1):
        raise ValueError("1-D contiguous index array expected")
    return _ptr(t, dtype)


def _check(rc, name):
    if rc != 0:
        raise RuntimeError(f"oracle {name} rejected its arguments ({rc})")


def _act(activation) -> int:
    if activation is True or activation in ("silu", "swish"):
        return 1
    if activation in (None, False, "none"):
        return 0
    raise ValueError(f"unsupported activation {activation!r}")


def bf16_from_f64(v: float) -> int:
    """Round one double to bf16 bits (nearest, ties to even)."""
    return int(_load().oracle_f64_to_bf16(float(v)))


def f64_from_bf16(bits: int) -> float:
    return float(_load().oracle_bf16_to_f64(int(bits) & 0xFFFF))


def silu(v: float) -> float:
    return float(_load().oracle_silu(float(v)))


def fwd_varlen(x, weight, bias, conv_states, query_start_loc, out,
               cache_indices=None, has_initial_state=None, activation="silu",
               pad_slot_id: int = -1) -> None:
    """Varlen prefill.  x / out: logical (dim, total_T) bf16, any strides;
    conv_states: (lines, dim, width-1) bf16 or None; updated in place."""
    lib = _load()
    dim, _ = x.shape
    width = weight.shape[1]
    batch = query_start_loc.numel() - 1
    bf = torch.bfloat16
    cs = conv_states
    rc = lib.oracle_fwd_varlen(
        _ptr(x, bf), x.stride(0), x.stride(1),
        _ptr(weight, bf), weight.stride(0), weight.stride(1),
        _ptr(bias, bf),
        _ptr(cs, bf), *(cs.stride() if cs is not None else (0, 0, 0)),
        cs.shape[0] if cs is not None else 0,
        _ptr1d(cache_indices, torch.int32), _ptr1d(has_initial_state, torch.bool),
        _ptr1d(query_start_loc, torch.int32), batch, dim, width,
        _act(activation), pad_slot_id,
        _ptr(out, bf), out.stride(0), out.stride(1))
    _check(rc, "fwd_varlen")


def update_decode(x, conv_state, weight, bias, out, cache_indices=None,
                  activation=None, pad_slot_id: int = -1) -> None:
    """Decode update.  x / out: (batch, dim, seqlen) bf16 (out may be x);
    conv_state: (lines, dim, width-1) bf16, updated in place."""
    lib = _load()
    batch, dim, seqlen = x.shape
    width = weight.shape[1]
    bf = torch.bfloat16
    rc = lib.oracle_update_decode(
        _ptr(x, bf), *x.stride(),
        _ptr(weight, bf), weight.stride(0), weight.stride(1),
        _ptr(bias, bf),
        _ptr(conv_state, bf), *conv_state.stride(), conv_state.shape[0],
        _ptr1d(cache_indices, torch.int32), batch, dim, seqlen, width,
        _act(activation), pad_slot_id,
        _ptr(out, bf), *out.stride())
    _check(rc, "update_decode")


def update_general(x, conv_state, weight, bias, out, cache_indices=None,
                   cache_seqlens=None, num_accepted_tokens=None,
                   intermediate=None, output_state_indices=None,
                   activation=None, pad_slot_id: int = -1) -> None:
    """Decode update with the speculative (num_accepted_tokens,
    intermediate, output_state_indices) or ring-buffer (cache_seqlens)
    options.  x / out: (batch, dim, seqlen) bf16 (out may be x);
    conv_state: (lines, dim, state_len) bf16; intermediate:
    (batch, steps, dim, width-1) bf16; output_state_indices: (batch, seqlen)
    int32.  Everything is updated in place."""
    lib = _load()
    batch, dim, seqlen = x.shape
    width = weight.shape[1]
    bf = torch.bfloat16
    inter = intermediate
    osi = output_state_indices
    if osi is not None and (osi.dtype != torch.int32 or osi.dim() != 2):
        raise TypeError("output_state_indices must be a 2-D int32 tensor")
    rc = lib.oracle_update_general(
        _ptr(x, bf), *x.stride(),
        _ptr(weight, bf), weight.stride(0), weight.stride(1),
        _ptr(bias, bf),
        _ptr(conv_state, bf), *conv_state.stride(), conv_state.shape[0],
        conv_state.shape[2],
        _ptr1d(cache_indices, torch.int32), _ptr1d(cache_seqlens, torch.int32),
        _ptr1d(num_accepted_tokens, torch.int32),
        _ptr(inter, bf), *(inter.stride() if inter is not None else (0, 0, 0, 0)),
        _ptr(osi, torch.int32), *(osi.stride() if osi is not None else (0, 0)),
        batch, dim, seqlen, width, _act(activation), pad_slot_id,
        _ptr(out, bf), *out.stride())
    _check(rc, "update_general")


def paged(x, weight, bias, cache, positions, slot_mapping, query_start_loc,
          block_table, off_s: int, ws: int, out, activation="silu",
          use_residual: bool = True) -> None:
    """Paged insert + conv.  x / out: (T, C) bf16 with unit channel stride;
    cache: (num_blocks, H, N, D) bf16 with unit D stride, updated in place."""
    lib = _load()
    T = x.shape[0]
    width = weight.shape[1]
    num_blocks, H, N, D = cache.shape
    if (x.stride(1) != 1 or out.stride(1) != 1 or cache.stride(3) != 1
            or block_table.stride(1) != 1):
        raise ValueError("unit innermost strides expected")
    num_reqs = query_start_loc.numel() - 1
    bf = torch.bfloat16
    rc = lib.oracle_paged(
        _ptr(x, bf), x.stride(0),
        _ptr(weight, bf), weight.stride(0), weight.stride(1), _ptr(bias, bf),
        _ptr(cache, bf), cache.stride(0), cache.stride(1), cache.stride(2),
        num_blocks, H, N, off_s, ws,
        _ptr1d(positions, torch.int64), _ptr1d(slot_mapping, torch.int64),
        _ptr1d(query_start_loc, torch.int32), num_reqs,
        _ptr(block_table, torch.int32), block_table.stride(0), block_table.shape[1],
        T, width, _act(activation), int(bool(use_residual)),
        _ptr(out, bf), out.stride(0))
    _check(rc, "paged")


def seq_metadata(query_start_loc, num_actual: int, num_padded: int | None = None):
    """Per-token (request, first row) for rows below num_actual, 0/0 for
    padded rows up to num_padded."""
    lib = _load()
    num_padded = num_actual if num_padded is None else num_padded
    num_reqs = query_start_loc.numel() - 1
    seq_idx = torch.empty(max(num_padded, 0), dtype=torch.int32)
    qstart = torch.empty(max(num_padded, 0), dtype=torch.int32)
    rc = lib.oracle_seq_metadata(_ptr1d(query_start_loc, torch.int32), num_reqs,
                                 num_actual, num_padded, _ptr(seq_idx), _ptr(qstart))
    _check(rc, "seq_metadata")
    return seq_idx, qstart
