"""CPU oracle for the packed varlen causal depthwise width-4 convolution.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU
baseline leg of ``bench.py`` may import this package. The product path (the HIP
library and its Python binding) never does, and shares no code with it.

The arithmetic lives in ``kdaconv_oracle.c`` (plain single-threaded C, built by
:func:`build` with gcc, no fast-math, no FP contraction). This module only
marshals numpy arrays into it. What it computes, and the readings taken where
the page "vllm.models.kimi_k3.nvidia.ops.kda_conv" is silent, are stated in the
C file's header.

Pins (tests/test_oracle_*.py): exhaustive bf16 rounding against torch's CPU
conversion; fp16 rounding and widening against numpy's float16; the correctly rounded exp against mpmath; the SiLU map against exact
rational arithmetic; the conv against exact-rational brute force, hand-derived
golden cases, invariants, and PyTorch's float64 conv1d within its error bound; the
decode step with a bf16 state against exact-rational brute force with the weight and
the state re-indexed by hand (tests/test_oracle_decode_bf16_state.py).
"""

from __future__ import annotations

import ctypes
import os
import pathlib
import subprocess
from typing import Optional

import numpy as np

_HERE = pathlib.Path(__file__).resolve().parent
SOURCE = _HERE / "kdaconv_oracle.c"
LIBRARY = _HERE / "libkdaconv_oracle.so"

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra"]


def build(output: Optional[pathlib.Path] = None, extra_flags: tuple = ()) -> pathlib.Path:
    """Compile the oracle with gcc into a shared library and return its path."""
    out = pathlib.Path(output) if output is not None else LIBRARY
    tmp = out.with_name(out.name + f".tmp{os.getpid()}")
    cmd = ["gcc", *_CFLAGS, *extra_flags, "-o", str(tmp), str(SOURCE), "-lquadmath", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


_lib = None


def _bind(lib: ctypes.CDLL) -> ctypes.CDLL:
    i64, i32, f32 = ctypes.c_int64, ctypes.c_int, ctypes.c_float
    vp = ctypes.c_void_p
    lib.oracle_bf16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f32.restype = f32
    lib.oracle_f32_to_bf16.argtypes = [f32]
    lib.oracle_f32_to_bf16.restype = ctypes.c_uint16
    lib.oracle_crexpf.argtypes = [f32]
    lib.oracle_crexpf.restype = f32
    lib.oracle_crexpf_escalates.argtypes = [f32]
    lib.oracle_crexpf_escalates.restype = i32
    lib.oracle_act_bf16.argtypes = [f32, i32]
    lib.oracle_act_bf16.restype = ctypes.c_uint16
    lib.oracle_act_bf16_range.argtypes = [ctypes.c_uint32, ctypes.c_uint64, i32, vp]
    lib.oracle_act_bf16_range.restype = None
    lib.oracle_act_bf16_list.argtypes = [vp, ctypes.c_uint64, i32, vp]
    lib.oracle_act_bf16_list.restype = None
    lib.oracle_f16_to_f32.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32.restype = f32
    lib.oracle_f16_to_f32_bits.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f32_bits.restype = ctypes.c_uint32
    lib.oracle_f32_to_f16.argtypes = [f32]
    lib.oracle_f32_to_f16.restype = ctypes.c_uint16
    lib.oracle_f32_word.argtypes = [f32]
    lib.oracle_f32_word.restype = ctypes.c_uint32
    lib.oracle_act_word.argtypes = [f32, i32, i32]
    lib.oracle_act_word.restype = ctypes.c_uint32
    lib.oracle_act_word_range.argtypes = [ctypes.c_uint32, ctypes.c_uint64, i32, i32, vp]
    lib.oracle_act_word_range.restype = None
    lib.oracle_act_word_list.argtypes = [vp, ctypes.c_uint64, i32, i32, vp]
    lib.oracle_act_word_list.restype = None
    lib.oracle_crexpf_scan.argtypes = [ctypes.c_uint32, ctypes.c_uint64, vp, ctypes.c_uint64,
                                       ctypes.POINTER(ctypes.c_double)]
    lib.oracle_crexpf_scan.restype = ctypes.c_uint64
    lib.oracle_packed_causal_conv1d.argtypes = [
        vp, i32, i64, i64, i64,  # x, format, num_tokens, dim, x_row_stride
        vp, i64, i64, vp,  # weight, w_stride0, w_stride1, bias
        vp, i64, i64, i64, i64,  # conv_states, lines, strides
        vp, i64,  # query_start_loc, num_seqs
        vp, i64, vp,  # cache_indices, ci_stride, has_initial_state
        i64, i32, i32, i64,  # part_dim, silu, has_null_block, null_block_id
        vp,  # out
    ]
    lib.oracle_packed_causal_conv1d.restype = i32
    lib.oracle_packed_causal_conv1d_update_bf16_state.argtypes = [
        vp, i64, i64, i64,  # x, batch, dim, x_row_stride
        vp, i64, i64, i64, vp,  # weight, part stride, channel stride, width stride, bias
        vp, i64, i64, i64, i64,  # conv_states (bf16 words), lines, strides
        vp, i64,  # cache_indices, ci_stride
        i64, i32, i32, i64,  # part_dim, silu, has_null_block, null_block_id
        vp,  # out
    ]
    lib.oracle_packed_causal_conv1d_update_bf16_state.restype = i32
    return lib


def load(path: Optional[pathlib.Path] = None) -> ctypes.CDLL:
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _bind(ctypes.CDLL(str(path)))
    if _lib is None:
        if not LIBRARY.exists():
            build()
        _lib = _bind(ctypes.CDLL(str(LIBRARY)))
    return _lib


#: Element formats of x and the output, as the C file numbers them, with the
#: numpy dtype that carries their raw words.
FORMATS = {"bf16": 0, "f16": 1, "f32": 2}
WORD_DTYPE = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}


def is_silu(activation) -> bool:
    """The page's activation rule: "silu", "swish" or True select SiLU, anything else none."""
    return activation in ("silu", "swish", True)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def crexpf(x, lib=None) -> np.ndarray:
    lib = lib or load()
    xs = np.asarray(x, dtype=np.float32).ravel()
    return np.array([lib.oracle_crexpf(float(v)) for v in xs], dtype=np.float32)


def act_bf16(a, silu: bool, lib=None) -> np.ndarray:
    """Stored bf16 word for each FP32 accumulator value in ``a``."""
    lib = lib or load()
    bits = np.ascontiguousarray(np.asarray(a, dtype=np.float32).ravel()).view(np.uint32)
    out = np.empty(bits.size, dtype=np.uint16)
    lib.oracle_act_bf16_list(bits.ctypes.data, bits.size, int(silu), out.ctypes.data)
    return out


def act_words(a, silu: bool, fmt: str = "bf16", lib=None) -> np.ndarray:
    """Stored word (format ``fmt``) for each FP32 accumulator value in ``a``."""
    lib = lib or load()
    bits = np.ascontiguousarray(np.asarray(a, dtype=np.float32).ravel()).view(np.uint32)
    out = np.empty(bits.size, dtype=WORD_DTYPE[fmt])
    lib.oracle_act_word_list(bits.ctypes.data, bits.size, int(silu), FORMATS[fmt], out.ctypes.data)
    return out


def act_words_range(first: int, count: int, silu: bool, fmt: str = "bf16", lib=None,
                    out: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored words (format ``fmt``) for the FP32 bit patterns first .. first+count-1."""
    lib = lib or load()
    if out is None:
        out = np.empty(count, dtype=WORD_DTYPE[fmt])
    assert out.dtype == WORD_DTYPE[fmt] and out.flags.c_contiguous and out.size >= count
    lib.oracle_act_word_range(first & 0xFFFFFFFF, count, int(silu), FORMATS[fmt], out.ctypes.data)
    return out


def act_bf16_range(first: int, count: int, silu: bool, lib=None,
                   out: Optional[np.ndarray] = None) -> np.ndarray:
    """Stored bf16 word for the FP32 bit patterns first, first+1, ..., first+count-1."""
    lib = lib or load()
    if out is None:
        out = np.empty(count, dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous and out.size >= count
    lib.oracle_act_bf16_range(first & 0xFFFFFFFF, count, int(silu), out.ctypes.data)
    return out


def packed_causal_conv1d(x: np.ndarray, dim: int, weight: np.ndarray, bias: Optional[np.ndarray],
                         conv_states: np.ndarray, query_start_loc: np.ndarray,
                         cache_indices: np.ndarray, has_initial_state: Optional[np.ndarray],
                         part_dim: int, activation="silu", null_block_id: Optional[int] = None,
                         out: Optional[np.ndarray] = None, lib=None,
                         x_dtype: str = "bf16") -> np.ndarray:
    """Run the oracle. ``conv_states`` is updated in place; returns ``out``.

    x: raw words of format ``x_dtype`` ("bf16" or "f16": uint16, "f32": uint32),
    shape (num_tokens, row_stride) with unit column stride; the op reads columns
    [0, dim). Returns words of the same format, (dim // part_dim, num_tokens,
    part_dim); rows that no sequence owns keep what ``out`` held (zeros when
    allocated here).
    """
    lib = lib or load()
    wd = WORD_DTYPE[x_dtype]
    esize = np.dtype(wd).itemsize
    # unit column stride (numpy gives an empty array zero strides: no rows, nothing read)
    assert x.dtype == wd and x.ndim == 2 and (x.strides[1] == esize or x.shape[0] == 0)
    assert weight.dtype == np.float32 and weight.ndim == 2 and weight.shape == (dim, 4)
    assert conv_states.dtype == np.float32 and conv_states.ndim == 3
    # The state is entries 0..2 of the last axis; wider states keep the rest untouched.
    assert conv_states.shape[1] == dim and conv_states.shape[2] >= 3
    assert query_start_loc.dtype == np.int32 and cache_indices.dtype == np.int32
    if bias is not None:
        assert bias.dtype == np.float32 and bias.shape == (dim,) and bias.flags.c_contiguous
    qsl = np.ascontiguousarray(query_start_loc)
    init = None
    if has_initial_state is not None:
        init = np.ascontiguousarray(has_initial_state.astype(np.uint8))
    T = x.shape[0]
    if out is None:
        out = np.zeros((dim // part_dim, T, part_dim), dtype=wd)
    assert out.dtype == wd and out.flags.c_contiguous
    assert out.shape == (dim // part_dim, T, part_dim)
    S = qsl.shape[0] - 1
    row_stride = x.strides[0] // esize if T else x.shape[1]  # no rows: the pitch is unused
    rc = lib.oracle_packed_causal_conv1d(
        x.ctypes.data, FORMATS[x_dtype], T, dim, row_stride,
        weight.ctypes.data, weight.strides[0] // 4, weight.strides[1] // 4, _ptr(bias),
        conv_states.ctypes.data, conv_states.shape[0], conv_states.strides[0] // 4,
        conv_states.strides[1] // 4, conv_states.strides[2] // 4,
        qsl.ctypes.data, S, cache_indices.ctypes.data, cache_indices.strides[0] // 4,
        _ptr(init), part_dim, int(is_silu(activation)), int(null_block_id is not None),
        0 if null_block_id is None else int(null_block_id), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the call (bad shapes or metadata)")
    return out


def packed_causal_conv1d_update(x: np.ndarray, dim: int, weight: np.ndarray,
                                bias: Optional[np.ndarray], conv_states: np.ndarray,
                                cache_indices: np.ndarray, part_dim: int, activation="silu",
                                null_block_id: Optional[int] = None,
                                out: Optional[np.ndarray] = None, lib=None,
                                x_dtype: str = "bf16") -> np.ndarray:
    """The decode step: row b of x is the one token of sequence b, whose history is
    its stored line. With the FP32 state this is the operation itself at one token
    per sequence with every initial-state flag set (page vllm.models.kimi_k3.amd.ops.
    kda_decode names the packed causal conv1d update as the decode step; the
    arithmetic is the prefill page's), so it runs the same C routine.
    ``conv_states`` is updated in place; returns (dim // part_dim, batch, part_dim)."""
    batch = x.shape[0]
    qsl = np.arange(batch + 1, dtype=np.int32)
    init = np.ones(batch, dtype=bool)
    return packed_causal_conv1d(x, dim, weight, bias, conv_states, qsl, cache_indices, init,
                                part_dim, activation, null_block_id, out=out, lib=lib,
                                x_dtype=x_dtype)


def weight_strides(weight: np.ndarray, part_dim: int):
    """(part stride, channel stride, width stride) in elements of an FP32 weight given
    either as the prefill page's (dim, 4) [channel, width] array or as the decode page's
    width-major (parts, 4, part_dim) [part, width, channel] array (any strides)."""
    assert weight.dtype == np.float32
    e = weight.itemsize
    if weight.ndim == 2:
        assert weight.shape[1] == 4
        return part_dim * weight.strides[0] // e, weight.strides[0] // e, weight.strides[1] // e
    assert weight.ndim == 3 and weight.shape[1:] == (4, part_dim)
    return weight.strides[0] // e, weight.strides[2] // e, weight.strides[1] // e


def packed_causal_conv1d_update_bf16_state(x: np.ndarray, dim: int, weight: np.ndarray,
                                           bias: Optional[np.ndarray], conv_states: np.ndarray,
                                           cache_indices: np.ndarray, part_dim: int,
                                           activation="silu",
                                           null_block_id: Optional[int] = None,
                                           out: Optional[np.ndarray] = None,
                                           lib=None) -> np.ndarray:
    """The decode step with a bf16 conv state (page vllm.models.kimi_k3.amd.ops.kda_decode:
    the fused decode kernel's bf16 input and bf16 state, and its width-major FP32 weight).

    x: bf16 words (batch, row_stride), unit column stride; row b is sequence b's token.
    weight: (dim, 4) [channel, width] or (dim // part_dim, 4, part_dim) width-major.
    conv_states: bf16 words (uint16), logical (lines, dim, >= 3), any strides; updated in
    place. Returns bf16 words (dim // part_dim, batch, part_dim)."""
    lib = lib or load()
    assert x.dtype == np.uint16 and x.ndim == 2 and x.strides[1] == 2
    assert conv_states.dtype == np.uint16 and conv_states.ndim == 3
    assert conv_states.shape[1] == dim and conv_states.shape[2] >= 3
    assert cache_indices.dtype == np.int32
    if bias is not None:
        assert bias.dtype == np.float32 and bias.shape == (dim,) and bias.flags.c_contiguous
    ps, s0, s1 = weight_strides(weight, part_dim)
    assert weight.shape[0] * (part_dim if weight.ndim == 3 else 1) == dim
    batch = x.shape[0]
    if out is None:
        out = np.zeros((dim // part_dim, batch, part_dim), dtype=np.uint16)
    assert out.dtype == np.uint16 and out.flags.c_contiguous
    assert out.shape == (dim // part_dim, batch, part_dim)
    rc = lib.oracle_packed_causal_conv1d_update_bf16_state(
        x.ctypes.data, batch, dim, x.strides[0] // 2,
        weight.ctypes.data, ps, s0, s1, _ptr(bias),
        conv_states.ctypes.data, conv_states.shape[0], conv_states.strides[0] // 2,
        conv_states.strides[1] // 2, conv_states.strides[2] // 2,
        cache_indices.ctypes.data, cache_indices.strides[0] // 4,
        part_dim, int(is_silu(activation)), int(null_block_id is not None),
        0 if null_block_id is None else int(null_block_id), out.ctypes.data)
    if rc != 0:
        raise ValueError("oracle rejected the call (bad shapes)")
    return out


def run_workload(wl, out: Optional[np.ndarray] = None, lib=None):
    """Run the oracle on a ``workloads.Workload``; returns (out, updated conv_states copy)."""
    st = wl.conv_states.copy()
    o = packed_causal_conv1d(wl.x, wl.dim, wl.weight, wl.bias, st, wl.query_start_loc,
                             wl.cache_indices, wl.has_initial_state, wl.part_dim,
                             wl.activation, wl.null_block_id, out=out, lib=lib,
                             x_dtype=wl.x_dtype)
    return o, st
