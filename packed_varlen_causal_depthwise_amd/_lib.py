"""ctypes binding of libkdaconv (include/kdaconv.h). Argument marshalling only."""

from __future__ import annotations

import ctypes
import pathlib

LIBRARY = pathlib.Path(__file__).resolve().parent / "libkdaconv.so"

OK, EINVAL, EUNSUPPORTED, ELAUNCH = 0, 1, 2, 3
ACT_NONE, ACT_SILU = 0, 1
BF16, F16, F32 = 0, 1, 2

# Every entry point include/kdaconv.h declares.
EXPORTS = (
    "kdaconv_packed_causal_conv1d",
    "kdaconv_packed_causal_conv1d_update",
    "kdaconv_packed_causal_conv1d_update_bf16_state",
    "kdaconv_validate",
    "kdaconv_activation_map",
    "kdaconv_status_string",
    "kdaconv_version",
)

_lib = None


class LibraryMissing(ImportError):
    pass


def load() -> ctypes.CDLL:
    """Load libkdaconv.so from the package directory; raise if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIBRARY.exists():
        raise LibraryMissing(
            f"{LIBRARY} is missing: build it with `python -m packed_varlen_causal_depthwise_amd.build`"
            " (or __graft_entry__.build()); there is no fallback implementation")
    lib = ctypes.CDLL(str(LIBRARY))
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    conv_args = [
        vp, i32, i64, i64, i64,  # x, dtype, num_tokens, dim, x_row_stride
        vp, i64, i64, vp,  # weight, weight strides, bias
        vp, i64, i64, i64, i64,  # conv_states, num_cache_lines, strides
        vp, i64,  # query_start_loc, num_seqs
        vp, i64, vp,  # cache_indices, stride, has_initial_state
        i64, i32, i32, i64,  # part_dim, activation, has_null_block, null_block_id
        vp,  # out
    ]
    lib.kdaconv_packed_causal_conv1d.argtypes = conv_args + [vp]
    lib.kdaconv_packed_causal_conv1d.restype = i32
    lib.kdaconv_packed_causal_conv1d_update.argtypes = [
        vp, i32, i64, i64, i64,  # x, dtype, batch, dim, x_row_stride
        vp, i64, i64, vp,  # weight, weight strides, bias
        vp, i64, i64, i64, i64,  # conv_states, num_cache_lines, strides
        vp, i64,  # cache_indices, stride
        i64, i32, i32, i64,  # part_dim, activation, has_null_block, null_block_id
        vp, vp,  # out, stream
    ]
    lib.kdaconv_packed_causal_conv1d_update.restype = i32
    lib.kdaconv_packed_causal_conv1d_update_bf16_state.argtypes = [
        vp, i32, i64, i64, i64,  # x, dtype, batch, dim, x_row_stride
        vp, i64, i64, i64, vp,  # weight, part stride, channel stride, width stride, bias
        vp, i64, i64, i64, i64,  # conv_states (bf16), num_cache_lines, strides
        vp, i64,  # cache_indices, stride
        i64, i32, i32, i64,  # part_dim, activation, has_null_block, null_block_id
        vp, vp,  # out, stream
    ]
    lib.kdaconv_packed_causal_conv1d_update_bf16_state.restype = i32
    lib.kdaconv_validate.argtypes = conv_args
    lib.kdaconv_validate.restype = i32
    lib.kdaconv_activation_map.argtypes = [ctypes.c_uint32, i64, i32, i32, vp, vp]
    lib.kdaconv_activation_map.restype = i32
    lib.kdaconv_status_string.argtypes = [i32]
    lib.kdaconv_status_string.restype = ctypes.c_char_p
    lib.kdaconv_version.argtypes = []
    lib.kdaconv_version.restype = i32
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().kdaconv_status_string(code).decode()


def check(code: int, what: str) -> None:
    if code == OK:
        return
    msg = f"{what}: {status_string(code)} (status {code})"
    if code in (EINVAL, EUNSUPPORTED):
        raise ValueError(msg)
    raise RuntimeError(msg)
