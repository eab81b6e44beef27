"""Helpers for the GPU tests: move a Workload to the device, run the HIP path."""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

import packed_varlen_causal_depthwise_amd as kd

CANARY = 0xABCD
#: Canary for FP32 output words.
CANARY32 = 0xABCD1234

TORCH_DTYPE = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}
_SIGNED = {np.uint16: np.int16, np.uint32: np.int32}


def canary_for(x_dtype: str) -> int:
    return CANARY32 if x_dtype == "f32" else CANARY


def words_to_torch(words: np.ndarray, dtype: torch.dtype, device="cuda") -> torch.Tensor:
    """Raw uint16 / uint32 words as a device tensor of ``dtype`` (same bits)."""
    signed = np.ascontiguousarray(words).view(_SIGNED[words.dtype.type])
    return torch.from_numpy(signed).to(device).view(dtype)


def torch_to_words(t: torch.Tensor) -> np.ndarray:
    """A device tensor's raw words: uint16 for 2-byte dtypes, uint32 for 4-byte ones."""
    if t.element_size() == 4:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def to_device(wl, device="cuda"):
    """Device tensors for a Workload: x is the row-strided view of the whole buffer."""
    xb = words_to_torch(wl.x, TORCH_DTYPE[wl.x_dtype], device)
    return dict(
        x=xb[:, : wl.dim],
        weight=torch.from_numpy(wl.weight).to(device),
        bias=None if wl.bias is None else torch.from_numpy(wl.bias).to(device),
        conv_states=torch.from_numpy(wl.conv_states.copy()).to(device),
        query_start_loc=torch.from_numpy(wl.query_start_loc).to(device),
        cache_indices=torch.from_numpy(wl.cache_indices).to(device),
        has_initial_state=torch.from_numpy(wl.has_initial_state).to(device),
    )


def run_hip(wl, device="cuda", out_fill: Optional[int] = -1, dev=None):
    """Run the HIP path on a Workload; returns (out words (P, T, pd) uint16 or uint32,
    states float32).

    The output buffer is pre-filled with ``out_fill`` (default: the format's
    canary) so rows the op must not write can be checked."""
    d = dev or to_device(wl, device)
    P = wl.dim // wl.part_dim
    dt = TORCH_DTYPE[wl.x_dtype]
    out = torch.empty((P, wl.num_tokens, wl.part_dim), dtype=dt, device=device)
    if out_fill == -1:
        out_fill = canary_for(wl.x_dtype)
    if out_fill is not None:
        if out.element_size() == 4:
            out.view(torch.int32).fill_(int(np.uint32(out_fill).view(np.int32)))
        else:
            out.view(torch.int16).fill_(int(np.uint16(out_fill).view(np.int16)))
    kd.packed_causal_conv1d_fn(d["x"], d["weight"], d["bias"], d["conv_states"],
                               d["query_start_loc"], d["cache_indices"], d["has_initial_state"],
                               wl.part_dim, wl.activation, wl.null_block_id, out=out)
    torch.cuda.synchronize()
    o = torch_to_words(out)
    st = d["conv_states"].cpu().numpy()
    return o, st


def oracle_with_canary(wl, out_fill: Optional[int] = None):
    import oracle

    fill = canary_for(wl.x_dtype) if out_fill is None else out_fill
    out = np.full((wl.dim // wl.part_dim, wl.num_tokens, wl.part_dim), fill,
                  dtype=oracle.WORD_DTYPE[wl.x_dtype])
    return oracle.run_workload(wl, out=out)


def first_mismatches(a: np.ndarray, b: np.ndarray, k: int = 5):
    idx = np.argwhere(a != b)[:k]
    return [(tuple(int(v) for v in i), int(a[tuple(i)]), int(b[tuple(i)])) for i in idx]
