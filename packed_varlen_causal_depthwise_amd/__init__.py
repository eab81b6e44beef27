"""Packed varlen causal depthwise width-4 convolution (KDA prefill short conv) on MI355X.

Python face of libkdaconv (include/kdaconv.h): the two functions of the page
"vllm.models.kimi_k3.nvidia.ops.kda_conv", ``packed_causal_conv1d_fn`` and
``packed_causal_conv1d_supported``, with the same arguments. PyTorch supplies the
device memory and the current stream; every step of the computation runs in the
HIP kernels of libkdaconv. There is no CPU path: if the library is not built,
importing the functions still works but calling them raises.
"""

from __future__ import annotations

from typing import Optional

import torch

from . import _lib

__all__ = [
    "NULL_BLOCK_ID",
    "packed_causal_conv1d_fn",
    "packed_causal_conv1d_update",
    "packed_causal_conv1d_supported",
    "activation_map",
    "library_path",
]

#: Default null block id. The page names the default (NULL_BLOCK_ID) without
#: printing its value; 0, the block the paged cache reserves as its null block,
#: is taken here. Pass the id explicitly (or None) to be independent of this.
NULL_BLOCK_ID = 0


def library_path() -> str:
    return str(_lib.LIBRARY)


def _activation_code(activation) -> int:
    # The page selects SiLU for "silu", "swish" or True; identity for None or False.
    if activation in ("silu", "swish", True):
        return _lib.ACT_SILU
    if activation is None or activation is False:
        return _lib.ACT_NONE
    raise ValueError(f"unknown activation {activation!r}: use 'silu', 'swish', True, None or False")


# x formats the library takes, with their interface codes (the output takes x's dtype).
_DTYPE_CODES = {torch.bfloat16: _lib.BF16, torch.float16: _lib.F16, torch.float32: _lib.F32}
_FORMAT_NAMES = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


def _dtype_code(dtype: torch.dtype) -> int:
    if dtype not in _DTYPE_CODES:
        raise ValueError(f"x must be bfloat16, float16 or float32 (got {dtype})")
    return _DTYPE_CODES[dtype]


# The current stream's raw handle: torch's direct query where it has one (0.1 us against
# about 2 us for building a Stream object per call), else the public route.
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
# The current device, likewise by the direct query where torch has one (a plain call,
# without the initialisation checks of torch.cuda.current_device()).
_get_device = getattr(torch._C, "_cuda_getDevice", None)


def _current_device() -> int:
    return _get_device() if _get_device is not None else torch.cuda.current_device()


def _stream_handle(device: torch.device) -> int:
    if _raw_stream is not None:
        idx = device.index if device.index is not None else _current_device()
        return _raw_stream(idx)
    return torch.cuda.current_stream(device).cuda_stream


class _NoGuard:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


_NO_GUARD = _NoGuard()


def _on(device: torch.device):
    """The device context for a call on `device`: none when it is already current (the
    context manager costs more than the launch's own host work)."""
    if device.index is None or device.index == _current_device():
        return _NO_GUARD
    return torch.cuda.device(device)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


# Shapes and strides are read as whole tuples, once per tensor: torch's t.stride(i) and
# t.size(i) each cost two to three times t.stride() or t.shape.
def _conv_args(x, weight, bias, conv_states, query_start_loc, cache_indices, has_initial_state,
               part_dim, activation, null_block_id, out):
    num_tokens, dim = x.shape
    num_seqs = query_start_loc.numel() - 1
    ws = weight.stride()
    cs = conv_states.stride()
    return [
        _ptr(x), _dtype_code(x.dtype), num_tokens, dim, x.stride()[0],
        _ptr(weight), ws[0], ws[1], _ptr(bias),
        _ptr(conv_states), conv_states.shape[0], cs[0], cs[1], cs[2],
        _ptr(query_start_loc), num_seqs,
        _ptr(cache_indices), cache_indices.stride()[0] if cache_indices.dim() == 1 else 0,
        _ptr(has_initial_state),
        int(part_dim), _activation_code(activation),
        int(null_block_id is not None), 0 if null_block_id is None else int(null_block_id),
        _ptr(out),
    ]


def _check_common(x, weight, bias, conv_states, cache_indices, num_seqs):
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    _dtype_code(x.dtype)
    if x.dim() != 2 or x.stride()[1] != 1:
        raise ValueError("x must be 2-D (tokens, dim) with unit column stride")
    dim = x.shape[1]
    if weight.dtype != torch.float32 or weight.dim() != 2 or weight.shape != (dim, 4):
        raise ValueError("weight must be float32 of shape (dim, 4)")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (dim,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 (dim,) tensor or None")
    cshape = conv_states.shape
    if conv_states.dtype != torch.float32 or len(cshape) != 3 or cshape[1] != dim:
        raise ValueError("conv_states must be float32 of shape (cache lines, dim, >= 3)")
    if cshape[2] < 3:
        raise ValueError("conv_states needs at least 3 history entries per channel")
    if cache_indices.dtype != torch.int32 or cache_indices.dim() != 1 or cache_indices.numel() < num_seqs:
        raise ValueError("cache_indices must be a 1-D int32 tensor with one entry per sequence")
    xi = x.get_device()
    for t in (weight, bias, conv_states, cache_indices):
        if t is not None and t.get_device() != xi:
            raise ValueError("all tensors must be on the device of x")


def _check_tensors(x, weight, bias, conv_states, query_start_loc, cache_indices, has_initial_state):
    if query_start_loc.dtype != torch.int32 or query_start_loc.dim() != 1:
        raise ValueError("query_start_loc must be a 1-D int32 tensor")
    if not query_start_loc.is_contiguous():
        raise ValueError("query_start_loc must be contiguous")
    num_seqs = query_start_loc.numel() - 1
    _check_common(x, weight, bias, conv_states, cache_indices, num_seqs)
    if has_initial_state is not None:
        if has_initial_state.dtype not in (torch.bool, torch.uint8) or not has_initial_state.is_contiguous():
            raise ValueError("has_initial_state must be a contiguous bool tensor or None")
        if has_initial_state.numel() < num_seqs:
            raise ValueError("has_initial_state needs one entry per sequence")
    xi = x.get_device()
    for t in (query_start_loc, has_initial_state):
        if t is not None and t.get_device() != xi:
            raise ValueError("all tensors must be on the device of x")


def packed_causal_conv1d_fn(
    x: torch.Tensor,
    weight: torch.Tensor,
    bias: Optional[torch.Tensor],
    conv_states: torch.Tensor,
    query_start_loc: torch.Tensor,
    cache_indices: torch.Tensor,
    has_initial_state: Optional[torch.Tensor],
    part_dim: int,
    activation="silu",
    null_block_id: Optional[int] = NULL_BLOCK_ID,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Varlen causal depthwise width-4 conv of x (tokens, dim), dim = parts x part_dim.

    Semantics of page vllm.models.kimi_k3.nvidia.ops.kda_conv,
    packed_causal_conv1d_fn: causal_conv1d_fn(x.T, weight, bias, conv_states, ...).T
    with conv_states (cache lines, dim, 3) updated in place. x is bfloat16,
    float16 or float32 (page: packed_causal_conv1d_supported); the arithmetic is
    FP32 and the result has x's dtype, (dim // part_dim, tokens, part_dim); plane i
    holds channels [i * part_dim, (i + 1) * part_dim). ``out``, when given, must be
    a contiguous tensor of x's dtype and that shape and receives the result (rows
    no sequence owns are left as they were). Queued on the current stream; no
    synchronisation.
    """
    if x.dim() != 2:
        raise ValueError("x must be 2-D (tokens, dim)")
    num_tokens, dim = x.shape
    if part_dim <= 0 or dim % part_dim != 0:
        raise ValueError(f"dim {dim} is not a multiple of part_dim {part_dim}")
    shape = (dim // part_dim, num_tokens, part_dim)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif (out.shape != shape or out.dtype != x.dtype or not out.is_contiguous()
          or out.get_device() != x.get_device()):
        raise ValueError(f"out must be a contiguous {x.dtype} tensor of shape {shape} on {x.device}")
    # Nothing to convolve: return before touching anything (page: early return).
    if num_tokens == 0 or query_start_loc.numel() <= 1:
        return out
    _check_tensors(x, weight, bias, conv_states, query_start_loc, cache_indices, has_initial_state)
    lib = _lib.load()
    args = _conv_args(x, weight, bias, conv_states, query_start_loc, cache_indices,
                      has_initial_state, part_dim, activation, null_block_id, out)
    with _on(x.device):
        rc = lib.kdaconv_packed_causal_conv1d(*args, _stream_handle(x.device))
    _lib.check(rc, "packed_causal_conv1d_fn")
    return out


def _check_bf16_state(x, weight, bias, conv_states, cache_indices, batch, part_dim):
    if x.dtype != torch.bfloat16:
        raise ValueError("a bf16 conv state takes bf16 x (page: is_fused_kda_decode_supported)")
    if x.dim() != 2 or x.stride()[1] != 1:
        raise ValueError("x must be 2-D (batch, dim) with unit column stride")
    dim = x.shape[1]
    parts = dim // part_dim
    if weight.dtype != torch.float32 or not (
            (weight.dim() == 2 and weight.shape == (dim, 4))
            or (weight.dim() == 3 and weight.shape == (parts, 4, part_dim))):
        raise ValueError("weight must be float32 (dim, 4) or width-major "
                         "(dim // part_dim, 4, part_dim)")
    if bias is not None and (bias.dtype != torch.float32 or bias.shape != (dim,)
                             or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous float32 (dim,) tensor or None")
    cshape = conv_states.shape
    if len(cshape) != 3 or cshape[1] != dim or cshape[2] < 3:
        raise ValueError("conv_states must be bf16 of shape (cache lines, dim, >= 3)")
    if cache_indices.dtype != torch.int32 or cache_indices.dim() != 1 or cache_indices.numel() < batch:
        raise ValueError("cache_indices must be a 1-D int32 tensor with one entry per sequence")
    if not x.is_cuda:
        raise ValueError("x must be a GPU tensor")
    xi = x.get_device()
    for t in (weight, bias, conv_states, cache_indices):
        if t is not None and t.get_device() != xi:
            raise ValueError("all tensors must be on the device of x")


def _weight_strides(weight: torch.Tensor, part_dim: int):
    """(part stride, channel stride, width stride) of a (dim, 4) or a width-major
    (dim // part_dim, 4, part_dim) weight, in elements."""
    ws = weight.stride()
    if len(ws) == 2:
        return part_dim * ws[0], ws[0], ws[1]
    return ws[0], ws[2], ws[1]


def packed_causal_conv1d_update(
    x: torch.Tensor,
    weight: torch.Tensor,
    bias: Optional[torch.Tensor],
    conv_states: torch.Tensor,
    cache_indices: torch.Tensor,
    part_dim: int,
    activation="silu",
    null_block_id: Optional[int] = NULL_BLOCK_ID,
    out: Optional[torch.Tensor] = None,
) -> torch.Tensor:
    """Decode step: one token per sequence, row b of x (batch, dim) for sequence b.

    The packed causal conv1d update of page vllm.models.kimi_k3.amd.ops.kda_decode.
    With a float32 conv_states (the state of packed_causal_conv1d_fn) the result equals
    that function with query_start_loc = [0, 1, ..., batch] and every has_initial_state
    true, for bf16, fp16 or float32 x. With a bfloat16 conv_states (the decode page's
    fused kernel state) x must be bf16 and the weight may also be that page's
    width-major (dim // part_dim, 4, part_dim) float32 copy; the arithmetic is the same
    FP32 chain on the exactly widened state, and the line keeps the words of its
    entries 1, 2 and the token. The state lines named by cache_indices shift by one
    token in place (the null block's line is neither read nor written). Returns
    (dim // part_dim, batch, part_dim) in x's dtype. Queued on the current stream; no
    synchronisation.
    """
    if x.dim() != 2:
        raise ValueError("x must be 2-D (batch, dim)")
    batch, dim = x.shape
    if part_dim <= 0 or dim % part_dim != 0:
        raise ValueError(f"dim {dim} is not a multiple of part_dim {part_dim}")
    shape = (dim // part_dim, batch, part_dim)
    if out is None:
        out = torch.empty(shape, dtype=x.dtype, device=x.device)
    elif (out.shape != shape or out.dtype != x.dtype or not out.is_contiguous()
          or out.get_device() != x.get_device()):
        raise ValueError(f"out must be a contiguous {x.dtype} tensor of shape {shape} on {x.device}")
    if batch == 0:
        return out
    bf16_state = conv_states.dtype == torch.bfloat16
    if bf16_state:
        _check_bf16_state(x, weight, bias, conv_states, cache_indices, batch, part_dim)
    else:
        _check_common(x, weight, bias, conv_states, cache_indices, batch)
    lib = _lib.load()
    tail = (_ptr(cache_indices), cache_indices.stride()[0],
            int(part_dim), _activation_code(activation),
            int(null_block_id is not None), 0 if null_block_id is None else int(null_block_id),
            _ptr(out), _stream_handle(x.device))
    cs = conv_states.stride()
    states = (_ptr(conv_states), conv_states.shape[0], cs[0], cs[1], cs[2])
    x_row_stride = x.stride()[0]
    with _on(x.device):
        if bf16_state:
            rc = lib.kdaconv_packed_causal_conv1d_update_bf16_state(
                _ptr(x), _dtype_code(x.dtype), batch, dim, x_row_stride,
                _ptr(weight), *_weight_strides(weight, part_dim), _ptr(bias), *states, *tail)
        else:
            ws = weight.stride()
            rc = lib.kdaconv_packed_causal_conv1d_update(
                _ptr(x), _dtype_code(x.dtype), batch, dim, x_row_stride,
                _ptr(weight), ws[0], ws[1], _ptr(bias), *states, *tail)
    _lib.check(rc, "packed_causal_conv1d_update")
    return out


def packed_causal_conv1d_supported(x: torch.Tensor, weight: torch.Tensor,
                                   conv_states: torch.Tensor, part_dim: int) -> bool:
    """Whether packed_causal_conv1d_fn serves these tensors (page:
    packed_causal_conv1d_supported). The library takes bf16, fp16 or FP32 x with
    unit column stride and any row stride (aligned to the element size), FP32 weight
    (dim, 4), FP32 conv_states (lines, dim, >= 3) in any strided layout (entries 0..2
    of the last axis are the history), and part_dim a multiple of 8 dividing dim."""
    try:
        if not (x.is_cuda and x.dim() == 2 and x.stride(1) == 1 and x.dtype in _DTYPE_CODES):
            return False
        if not (weight.dtype == torch.float32 and weight.dim() == 2
                and tuple(weight.shape) == (x.size(1), 4)):
            return False
        if not (conv_states.dtype == torch.float32 and conv_states.dim() == 3
                and conv_states.size(1) == x.size(1) and conv_states.size(2) >= 3):
            return False
        if part_dim <= 0 or x.size(1) % part_dim != 0:
            return False
        lib = _lib.load()
    except _lib.LibraryMissing:
        return False
    num_tokens, dim = x.shape
    # The output buffer would be a fresh 256-byte-aligned allocation.
    rc = lib.kdaconv_validate(
        _ptr(x), _DTYPE_CODES[x.dtype], num_tokens, dim, x.stride(0), _ptr(weight), weight.stride(0), weight.stride(1),
        None, _ptr(conv_states), conv_states.size(0), conv_states.stride(0),
        conv_states.stride(1), conv_states.stride(2), 256, 1, 256, 1, None, int(part_dim),
        _lib.ACT_SILU, 0, 0, 256)
    return rc == _lib.OK


def activation_map(first: int, count: int, activation, out: Optional[torch.Tensor] = None,
                   fmt: str = "bf16") -> torch.Tensor:
    """The kernel's FP32 -> stored-word map (output format ``fmt``: "bf16", "f16" or
    "f32") on ``count`` consecutive FP32 bit patterns from ``first``; returns the
    words as an int16 (bf16, f16) or int32 (f32) tensor on the current device."""
    code = _DTYPE_CODES[_FORMAT_NAMES[fmt]]
    wdt = torch.int32 if code == _lib.F32 else torch.int16
    if out is None:
        out = torch.empty(count, dtype=wdt, device="cuda")
    if out.dtype != wdt or not out.is_contiguous() or out.numel() < count:
        raise ValueError(f"out must be a contiguous {wdt} tensor of at least {count} elements")
    lib = _lib.load()
    with torch.cuda.device(out.device):
        rc = lib.kdaconv_activation_map(first & 0xFFFFFFFF, count, _activation_code(activation),
                                        code, out.data_ptr(), _stream_handle(out.device))
    _lib.check(rc, "activation_map")
    return out
