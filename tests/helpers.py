"""Test helpers: small hand-built workloads, exact brute force, plane reshaping."""

from __future__ import annotations

import math
from typing import Optional

import numpy as np

import exact
from workloads import (CANARIES, WORD_DTYPE, Workload, bf16_bits_to_f32, f32_to_bf16_bits,
                       f32_to_words, words_to_f32)


def make_workload(lengths, dim: int, part_dim: int, *, seed: int = 0, row_stride: Optional[int] = None,
                  lines: Optional[int] = None, init=None, bias: bool = True, activation="silu",
                  null_block_id: Optional[int] = None, cache_indices=None, x_scale: float = 1.0,
                  pad_tokens: int = 0, state_scale: float = 1.0, x_dtype: str = "bf16") -> Workload:
    rng = np.random.default_rng(seed)
    lengths = np.asarray(lengths, dtype=np.int64)
    S = len(lengths)
    T = int(lengths.sum()) + pad_tokens
    rs = row_stride or dim
    x = np.full((T, rs), CANARIES[x_dtype], dtype=WORD_DTYPE[x_dtype])
    x[:, :dim] = f32_to_words(rng.standard_normal((T, dim)).astype(np.float32) * np.float32(x_scale),
                              x_dtype)
    w = (rng.standard_normal((dim, 4)) * 0.5).astype(np.float32)
    b = (rng.standard_normal(dim) * 0.1).astype(np.float32) if bias else None
    lines = lines or S + 2
    st = (rng.standard_normal((lines, dim, 3)) * state_scale).astype(np.float32)
    if cache_indices is None:
        cache_indices = rng.permutation(lines)[:S]
    ci = np.asarray(cache_indices, dtype=np.int32)
    if init is None:
        init = rng.random(S) < 0.5
    init = np.asarray(init, dtype=bool)
    qsl = np.zeros(S + 1, dtype=np.int32)
    qsl[1:] = np.cumsum(lengths)
    return Workload("hand", x, dim, w, b, st, qsl, ci, init, part_dim, activation, null_block_id,
                    x_dtype)


def planes_to_rows(out: np.ndarray) -> np.ndarray:
    """(dim // part_dim, T, part_dim) -> (T, dim)."""
    P, T, pd = out.shape
    return np.ascontiguousarray(out.transpose(1, 0, 2).reshape(T, P * pd))


def brute_force(wl: Workload):
    """The operation in exact rational arithmetic with explicit binary32 rounding.

    Returns (out words as (T, dim) in x's format, updated conv_states copy). Rows
    no sequence owns are 0. Finite x only (the widening is numpy's).
    """
    T, dim = wl.num_tokens, wl.dim
    xf = words_to_f32(wl.x[:, :dim], wl.x_dtype)
    out = np.zeros((T, dim), dtype=WORD_DTYPE[wl.x_dtype])
    word = exact.WORDS[wl.x_dtype]
    st = wl.conv_states.copy()
    silu = wl.activation in ("silu", "swish", True)
    for s in range(wl.num_seqs):
        start, end = int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1])
        if end == start:
            continue
        line = int(wl.cache_indices[s])
        # a line outside the state array names no line: like the null block
        live = (not (wl.null_block_id is not None and line == wl.null_block_id)
                and 0 <= line < wl.num_cache_lines)
        init = live and wl.has_initial_state is not None and bool(wl.has_initial_state[s])
        for c in range(dim):
            e = [float(v) for v in st[line, c]] if init else [0.0, 0.0, 0.0]
            e += [float(v) for v in xf[start:end, c]]
            for i in range(end - start):
                acc = float(wl.bias[c]) if wl.bias is not None else 0.0
                for k in range(4):
                    acc = exact.fma32(float(wl.weight[c, k]), e[i + k], acc)
                out[start + i, c] = word(exact.silu32(acc) if silu else acc)
            if live:
                st[line, c] = np.array(e[-3:], dtype=np.float32)
    return out, st


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (normal range)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return np.exp2(np.floor(np.log2(a)) - 7)
