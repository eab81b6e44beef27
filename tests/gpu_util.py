"""Helpers for the GPU tests: move a Workload to the device, run the HIP path."""

from __future__ import annotations

from typing import Optional

import numpy as np
import torch

import packed_varlen_causal_depthwise_amd as kd

CANARY = 0xABCD


def to_device(wl, device="cuda"):
    """Device tensors for a Workload: x is the row-strided view of the whole buffer."""
    xb = torch.from_numpy(np.ascontiguousarray(wl.x).view(np.int16)).to(device).view(torch.bfloat16)
    return dict(
        x=xb[:, : wl.dim],
        weight=torch.from_numpy(wl.weight).to(device),
        bias=None if wl.bias is None else torch.from_numpy(wl.bias).to(device),
        conv_states=torch.from_numpy(wl.conv_states.copy()).to(device),
        query_start_loc=torch.from_numpy(wl.query_start_loc).to(device),
        cache_indices=torch.from_numpy(wl.cache_indices).to(device),
        has_initial_state=torch.from_numpy(wl.has_initial_state).to(device),
    )


def run_hip(wl, device="cuda", out_fill: Optional[int] = CANARY, dev=None):
    """Run the HIP path on a Workload; returns (out words (P, T, pd) uint16, states float32).

    The output buffer is pre-filled with ``out_fill`` so rows the op must not
    write can be checked."""
    d = dev or to_device(wl, device)
    P = wl.dim // wl.part_dim
    out = torch.empty((P, wl.num_tokens, wl.part_dim), dtype=torch.bfloat16, device=device)
    if out_fill is not None:
        out.view(torch.int16).fill_(np.int16(np.uint16(out_fill).view(np.int16)))
    kd.packed_causal_conv1d_fn(d["x"], d["weight"], d["bias"], d["conv_states"],
                               d["query_start_loc"], d["cache_indices"], d["has_initial_state"],
                               wl.part_dim, wl.activation, wl.null_block_id, out=out)
    torch.cuda.synchronize()
    o = out.view(torch.int16).cpu().numpy().view(np.uint16)
    st = d["conv_states"].cpu().numpy()
    return o, st


def oracle_with_canary(wl, out_fill: int = CANARY):
    import oracle

    out = np.full((wl.dim // wl.part_dim, wl.num_tokens, wl.part_dim), out_fill, dtype=np.uint16)
    return oracle.run_workload(wl, out=out)


def first_mismatches(a: np.ndarray, b: np.ndarray, k: int = 5):
    idx = np.argwhere(a != b)[:k]
    return [(tuple(int(v) for v in i), int(a[tuple(i)]), int(b[tuple(i)])) for i in idx]
