"""Pins for the oracle's decode step (one token per sequence, history from the
stored FP32 line).

Page vllm.models.kimi_k3.amd.ops.kda_decode names the packed causal conv1d update
as the first step of a decode batch; with the FP32 state the arithmetic is that of
page vllm.models.kimi_k3.nvidia.ops.kda_conv. Pins: exact-rational brute force of
the step on its own; the defining property of an update, that feeding a sequence
one token at a time through decode steps after a prefill gives the outputs and
final state of one prefill over all its tokens; the null block.
"""

import numpy as np
import pytest

import oracle
from helpers import brute_force, make_workload, planes_to_rows
from workloads import Workload


def _decode_as_workload(x, dim, weight, bias, states, ci, pd, act, null, fmt):
    B = x.shape[0]
    return Workload("decode", x, dim, weight, bias, states, np.arange(B + 1, dtype=np.int32),
                    ci, np.ones(B, dtype=bool), pd, act, null, fmt)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_decode_step_brute_force(olib, fmt):
    base = make_workload([1] * 9, dim=12, part_dim=4, seed=81, lines=12, x_dtype=fmt,
                         cache_indices=[3, 0, 7, 1, 11, 5, 2, 9, 4])
    st = base.conv_states.copy()
    o = oracle.packed_causal_conv1d_update(base.x, 12, base.weight, base.bias, st,
                                           base.cache_indices, 4, "silu", 7, lib=olib,
                                           x_dtype=fmt)
    want, want_st = brute_force(_decode_as_workload(base.x, 12, base.weight, base.bias,
                                                    base.conv_states, base.cache_indices, 4,
                                                    "silu", 7, fmt))
    assert np.array_equal(planes_to_rows(o), want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))
    # the null block's line (7) is untouched
    assert np.array_equal(st[7], base.conv_states[7])


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_decode_steps_continue_a_prefill(olib, fmt):
    """Sequences of lengths 9, 4, 6: prefill their first 3 tokens, then decode the rest
    one step at a time (a batch of the sequences still running at each step). The
    outputs and final lines equal one prefill over every token."""
    lens = [9, 4, 6]
    full = make_workload(lens, dim=16, part_dim=8, seed=82, lines=5, x_dtype=fmt,
                         cache_indices=[4, 1, 2], init=[True, False, True])
    o_full, st_full = oracle.run_workload(full, lib=olib)
    rows_full = planes_to_rows(o_full)
    qsl = full.query_start_loc
    prefix = 3
    # prefill of the first `prefix` tokens of each sequence
    pre_rows = np.concatenate([np.arange(qsl[s], qsl[s] + prefix) for s in range(3)])
    pre = Workload("pre", full.x[pre_rows].copy(), 16, full.weight, full.bias,
                   full.conv_states.copy(), np.arange(0, 3 * prefix + 1, prefix, dtype=np.int32),
                   full.cache_indices, full.has_initial_state, 8, full.activation, None, fmt)
    o_pre, st = oracle.run_workload(pre, lib=olib)
    got = np.zeros_like(rows_full)
    got[pre_rows] = planes_to_rows(o_pre)
    for step in range(prefix, max(lens)):
        running = [s for s in range(3) if step < lens[s]]
        rows = np.array([qsl[s] + step for s in running])
        o = oracle.packed_causal_conv1d_update(
            full.x[rows].copy(), 16, full.weight, full.bias, st,
            full.cache_indices[running].copy(), 8, full.activation, None, lib=olib, x_dtype=fmt)
        got[rows] = planes_to_rows(o)
    assert np.array_equal(got, rows_full)
    assert np.array_equal(st.view(np.uint32), st_full.view(np.uint32))
