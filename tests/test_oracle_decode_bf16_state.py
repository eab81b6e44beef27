"""Pins for the oracle's decode step with a bf16 conv state and the width-major weight.

Page vllm.models.kimi_k3.amd.ops.kda_decode: is_fused_kda_decode_supported admits a
bf16 input with a bf16 conv state (not dim-first), and make_decode_conv1d_weight_loader
mirrors the FP32 conv weight width-major, [qkv, width, channel]. The page prints no
arithmetic; the reading taken is the prefill page's FP32 chain on the exactly widened
history and token, with the line then holding the bf16 words of entries 1, 2 and the
token unchanged.

Pins: exact-rational brute force with the weight re-indexed by hand from the
width-major array and the state widened and shifted here; NaN words kept in the state
with their payloads; strided views of the weight and the state; a chain of decode
steps after a prefill equals one prefill over all tokens; the null block and lines
outside the state array.
"""

import numpy as np
import pytest

import oracle
import workloads
from helpers import brute_force, planes_to_rows
from workloads import Workload


def _case(batch=9, parts=3, pd=4, seed=91, lines=12, row_stride=None, ci=None, null=None):
    d = workloads.decode_batch_bf16_state(batch, seed=seed, dim=parts * pd, part_dim=pd,
                                          row_stride=row_stride or parts * pd + 3, lines=lines,
                                          null_block_id=null)
    if ci is not None:
        d.cache_indices = np.asarray(ci, dtype=np.int32)
    return d


def _channel_major(wm: np.ndarray) -> np.ndarray:
    """(parts, 4, pd) -> (dim, 4) by explicit loops."""
    parts, _, pd = wm.shape
    w = np.empty((parts * pd, 4), dtype=np.float32)
    for c in range(parts * pd):
        for k in range(4):
            w[c, k] = wm[c // pd, k, c % pd]
    return w


def _widen(words: np.ndarray) -> np.ndarray:
    return (words.astype(np.uint32) << 16).view(np.float32)


def _expected_state(d) -> np.ndarray:
    """The line after one step: entries 1, 2 of the old words, then the token's word."""
    st = d.conv_states.copy()
    for b, line in enumerate(d.cache_indices):
        line = int(line)
        if (d.null_block_id is not None and line == d.null_block_id) or not 0 <= line < len(st):
            continue
        for c in range(d.dim):
            st[line, c] = [d.conv_states[line, c, 1], d.conv_states[line, c, 2], d.x[b, c]]
    return st


def _run(d, olib, weight=None, states=None):
    st = d.conv_states.copy() if states is None else states
    o = oracle.packed_causal_conv1d_update_bf16_state(
        d.x, d.dim, d.weight if weight is None else weight, d.bias, st, d.cache_indices,
        d.part_dim, d.activation, d.null_block_id, lib=olib)
    return o, st


@pytest.mark.parametrize("seed", range(3))
def test_brute_force_exact(olib, seed):
    """9 sequences over 12 lines, null block 7 among them, dim 12 in 3 planes of 4."""
    d = _case(seed=91 + seed, ci=[3, 0, 7, 1, 11, 5, 2, 9, 4], null=7)
    o, st = _run(d, olib)
    B = d.batch
    wl = Workload("bf16 state", d.x, d.dim, _channel_major(d.weight), d.bias,
                  _widen(d.conv_states), np.arange(B + 1, dtype=np.int32), d.cache_indices,
                  np.ones(B, dtype=bool), d.part_dim, d.activation, d.null_block_id)
    want, _ = brute_force(wl)
    assert np.array_equal(planes_to_rows(o), want)
    assert np.array_equal(st, _expected_state(d))
    assert np.array_equal(st[7], d.conv_states[7])


def test_width_major_taps_land_on_their_channels(olib):
    """Tap k of channel c is the only nonzero weight of a distinct (c, k): with x = 1 and
    a zero state, out[c] = w[c][3] exactly (activation none), and with the token 0 and
    state entry j = 1 it is w[c][j]. Any mix-up of part, width and channel strides
    moves a value to another channel."""
    d = _case(batch=1, parts=3, pd=8, lines=2, ci=[1])
    d.activation = None
    d.bias = None
    dim, pd = d.dim, d.part_dim
    w = np.zeros((dim, 4), dtype=np.float32)
    for c in range(dim):
        for k in range(4):
            w[c, k] = float(4 * c + k + 1)  # exact in bf16 up to 256
    d.weight = workloads.width_major(w, pd)
    one = 0x3F80
    for j in range(4):
        d.x[0, :dim] = one if j == 3 else 0
        d.conv_states[1] = 0
        if j < 3:
            d.conv_states[1, :, j] = one
        o, _ = _run(d, olib)
        assert np.array_equal(_widen(planes_to_rows(o)[0]), w[:, j]), j


def test_nan_words_keep_their_payloads(olib):
    """A token or state word that is a NaN is copied into the line unchanged; the output
    of its channel is the canonical quiet NaN."""
    d = _case(batch=2, parts=1, pd=8, lines=3, ci=[2, 0])
    d.x[0, 1] = 0x7F81  # signalling NaN payload
    d.x[1, 5] = 0xFFA5
    d.conv_states[2, 3, 1] = 0x7F82
    d.conv_states[0, 6, 2] = 0xFF83
    o, st = _run(d, olib)
    assert np.array_equal(st, _expected_state(d))
    assert st[2, 1, 2] == 0x7F81 and st[2, 3, 0] == 0x7F82 and st[0, 6, 1] == 0xFF83
    rows = planes_to_rows(o)
    assert rows[0, 1] == 0x7FC0 and rows[1, 5] == 0x7FC0


@pytest.mark.parametrize("form", ["weight_padded", "weight_channel_major", "state_padded",
                                  "state_dim_first"])
def test_strided_views_equal_contiguous(olib, form):
    """The same values through other strides give the same words."""
    d = _case(batch=7, parts=3, pd=8, lines=9, seed=95)
    want, want_st = _run(d, olib)
    if form == "weight_padded":
        buf = np.full((3, 4, d.part_dim + 5), np.float32(1e30), dtype=np.float32)
        buf[:, :, 2:2 + d.part_dim] = d.weight
        o, st = _run(d, olib, weight=buf[:, :, 2:2 + d.part_dim])
    elif form == "weight_channel_major":
        o, st = _run(d, olib, weight=_channel_major(d.weight))
    elif form == "state_padded":
        buf = np.full((d.num_cache_lines, d.dim, 5), 0x1234, dtype=np.uint16)
        buf[:, :, :3] = d.conv_states
        o, st = _run(d, olib, states=buf[:, :, :3])
        assert np.all(buf[:, :, 3:] == 0x1234)
        st = np.ascontiguousarray(st)
    else:
        buf = np.ascontiguousarray(d.conv_states.transpose(0, 2, 1))
        o, st = _run(d, olib, states=buf.transpose(0, 2, 1))
        st = np.ascontiguousarray(st)
    assert np.array_equal(o, want)
    assert np.array_equal(st, want_st)


@pytest.mark.parametrize("bad", [-1, 12, 2 ** 31 - 1])
def test_null_block_and_lines_outside(olib, bad):
    """A null-block sequence and one whose line lies outside the array run from zero
    history, and no line changes for them."""
    d = _case(ci=[3, 0, 7, 1, bad, 5, 2, 9, 4], null=7)
    o, st = _run(d, olib)
    # The brute force with the null block's line zeroed and one more zero line for the
    # sequence whose line lies outside: both run from zero history.
    zeroed = np.concatenate([d.conv_states, np.zeros((1, d.dim, 3), dtype=np.uint16)])
    zeroed[7] = 0
    ci = d.cache_indices.copy()
    ci[4] = d.num_cache_lines
    B = d.batch
    wl = Workload("bf16 state", d.x, d.dim, _channel_major(d.weight), d.bias, _widen(zeroed),
                  np.arange(B + 1, dtype=np.int32), ci, np.ones(B, dtype=bool), d.part_dim,
                  d.activation, None)
    want, _ = brute_force(wl)
    assert np.array_equal(planes_to_rows(o), want)
    assert np.array_equal(st, _expected_state(d))


def test_decode_chain_continues_a_prefill(olib):
    """Sequences of lengths 7, 3, 5 with bf16-representable initial lines: the FP32-state
    prefill of their first 2 tokens, its lines narrowed to bf16 (exact: they hold bf16
    values), then bf16-state decode steps for the rest, equal one FP32-state prefill over
    every token, outputs and final lines."""
    lens = [7, 3, 5]
    dim, pd = 16, 8
    rng = np.random.default_rng(97)
    T = sum(lens)
    x = workloads.f32_to_bf16_bits(rng.standard_normal((T, dim)).astype(np.float32))
    w = (rng.standard_normal((dim, 4)) * 0.5).astype(np.float32)
    b = (rng.standard_normal(dim) * 0.1).astype(np.float32)
    st_words = workloads.f32_to_bf16_bits(rng.standard_normal((4, dim, 3)).astype(np.float32))
    ci = np.array([3, 0, 2], dtype=np.int32)
    qsl = np.array([0, 7, 10, 15], dtype=np.int32)
    full = Workload("full", x, dim, w, b, _widen(st_words), qsl, ci, np.ones(3, dtype=bool), pd,
                    "silu", None)
    o_full, st_full = oracle.run_workload(full, lib=olib)
    rows_full = planes_to_rows(o_full)
    prefix = 2
    pre_rows = np.concatenate([np.arange(qsl[s], qsl[s] + prefix) for s in range(3)])
    pre = Workload("pre", x[pre_rows].copy(), dim, w, b, _widen(st_words),
                   np.arange(0, 3 * prefix + 1, prefix, dtype=np.int32), ci,
                   np.ones(3, dtype=bool), pd, "silu", None)
    o_pre, st32 = oracle.run_workload(pre, lib=olib)
    st16 = (st32.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(_widen(st16), st32)  # the narrowing is exact
    got = np.zeros_like(rows_full)
    got[pre_rows] = planes_to_rows(o_pre)
    wm = workloads.width_major(w, pd)
    for step in range(prefix, max(lens)):
        running = [s for s in range(3) if step < lens[s]]
        rows = np.array([qsl[s] + step for s in running])
        o = oracle.packed_causal_conv1d_update_bf16_state(
            x[rows].copy(), dim, wm, b, st16, ci[running].copy(), pd, "silu", None, lib=olib)
        got[rows] = planes_to_rows(o)
    assert np.array_equal(got, rows_full)
    assert np.array_equal(_widen(st16).view(np.uint32), st_full.view(np.uint32))
