"""Pins for the oracle's convolution, state protocol and output layout.

Page: vllm.models.kimi_k3.nvidia.ops.kda_conv.
  - packed_causal_conv1d_fn docstring: causal_conv1d_fn semantics on x.T, width-4
    taps, conv_states (cache lines, dim, 3) updated in place, output planes
    (dim // part_dim, tokens, part_dim) with plane i = channels [i*pd, (i+1)*pd);
  - module docstring, third paragraph: the state is read at a sequence's start
    and the updated state written once;
  - packed_causal_conv1d_fn source: the null block id switches a sequence's state off.

Pins that do not restate the oracle: exact-rational brute force (tests/exact.py),
closed forms derived by hand (unit taps shift the input, all-ones taps sum four
integers), invariants (split calls, permutations, slicing, layouts), and
PyTorch's float64 conv1d (the library form of a causal depthwise conv) within
the FP32 chain's error bound.
"""

import numpy as np
import pytest
import torch

import exact
import oracle
from helpers import bf16_ulp, brute_force, make_workload, planes_to_rows
from workloads import bf16_bits_to_f32, f32_to_bf16_bits


def _run(wl, olib, out=None):
    o, st = oracle.run_workload(wl, out=out, lib=olib)
    return planes_to_rows(o), st


# ---------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
def test_brute_force_exact(olib, seed):
    act = "silu" if seed % 3 else None
    null = 1 if seed % 2 else None
    wl = make_workload([5, 0, 3, 9, 1, 2], dim=12, part_dim=4, seed=seed, activation=act,
                       null_block_id=null, cache_indices=[0, 2, 1, 3, 4, 5], lines=7,
                       bias=seed != 4, x_scale=1.0 + 10 * (seed == 5))
    got, st = _run(wl, olib)
    want, want_st = brute_force(wl)
    assert np.array_equal(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


def test_brute_force_near_bf16_midpoints(olib):
    """Biases chosen so that the first accumulator of every channel lies within a few
    FP32 ulps of a bf16 midpoint: there the order of the roundings (bias first, taps
    oldest to newest, each fused) decides the stored word."""
    for act in (None, "silu"):
        wl = make_workload([4, 3], dim=512, part_dim=128, seed=70, init=[True, True],
                           activation=act, cache_indices=[1, 0], lines=2)
        xf = bf16_bits_to_f32(wl.x[:, :wl.dim]).astype(np.float64)
        line = int(wl.cache_indices[0])  # first token of sequence 0: history is line 1
        taps = (wl.weight[:, :3].astype(np.float64) * wl.conv_states[line].astype(np.float64)).sum(1)
        taps += wl.weight[:, 3] * xf[0]
        target = taps + wl.bias
        u = (target.astype(np.float32).view(np.uint32) & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
        wl.bias[:] = (u.view(np.float32).astype(np.float64) - taps).astype(np.float32)
        got, st = _run(wl, olib)
        want, want_st = brute_force(wl)
        assert np.array_equal(got, want)
        assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


def _single_token(olib, w, hist, x0, bias):
    """One channel, one token, initial state hist, no activation; returns the stored word."""
    wl = make_workload([1], dim=8, part_dim=8, seed=0, init=[True], activation=None, lines=1,
                       cache_indices=[0])
    wl.weight[:] = np.array(w, dtype=np.float32)
    wl.conv_states[0] = np.array(hist, dtype=np.float32)
    wl.x[0, :8] = f32_to_bf16_bits(np.full(8, x0, dtype=np.float32))
    wl.bias[:] = np.float32(bias)
    got, _ = _run(wl, olib)
    return int(got[0, 0])


def test_bias_enters_first(olib):
    """bias = 1 + 2^-8 (a bf16 midpoint), two products of 2^-24 (half an FP32 ulp at 1).
    Bias first: each add is a tie kept at the even 1 + 2^-8, which bf16 rounds to 1.0.
    Bias last would give 2^-23 + 1 + 2^-8, which bf16 rounds up to 0x3F81."""
    word = _single_token(olib, [2.0 ** -12, 2.0 ** -12, 0.0, 0.0], [2.0 ** -12, 2.0 ** -12, 0.0],
                         1.0, 1.0 + 2.0 ** -8)
    assert word == 0x3F80


def test_taps_enter_oldest_first(olib):
    """bias = 1 + 2^-8, oldest product -2^-24, newest product 2^-23. Oldest first: the
    tie keeps 1 + 2^-8, then + 2^-23 gives 0x3F808001, which bf16 rounds up to 0x3F81.
    Newest first would end on the tie 0x3F808000 and round to 0x3F80."""
    word = _single_token(olib, [-(2.0 ** -12), 0.0, 0.0, 2.0 ** -11], [2.0 ** -12, 0.0, 0.0],
                         2.0 ** -12, 1.0 + 2.0 ** -8)
    assert word == 0x3F81


# ---------------------------------------------------------------- closed forms

@pytest.mark.parametrize("tap", range(4))
def test_unit_taps_shift_the_input(olib, tap):
    """w[c] = e_tap, no bias, no activation: out[t] is e[t - 3 + tap] of (history ++ x)."""
    wl = make_workload([7, 2, 1], dim=16, part_dim=8, seed=10 + tap, bias=False, activation=None,
                       init=[True, False, True], cache_indices=[2, 0, 1], lines=3)
    wl.weight[:] = 0.0
    wl.weight[:, tap] = 1.0
    # history values that bf16 holds exactly, so every output is an exact copy
    wl.conv_states[:] = bf16_bits_to_f32(f32_to_bf16_bits(wl.conv_states))
    got, _ = _run(wl, olib)
    xw = wl.x[:, :wl.dim]
    for s in range(wl.num_seqs):
        a, b = int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1])
        line = int(wl.cache_indices[s])
        hist = (f32_to_bf16_bits(wl.conv_states[line].T) if wl.has_initial_state[s]
                else np.zeros((3, wl.dim), dtype=np.uint16))
        ext = np.concatenate([hist, xw[a:b]])
        for i in range(b - a):
            assert np.array_equal(got[a + i], ext[i + tap]), (s, i)


@pytest.mark.parametrize("silu", [False, True])
def test_all_ones_taps_sum_integers(olib, silu):
    """w = [1, 1, 1, 1], bias 0.5, integer x in [-4, 4], zero history: acc = 0.5 + sum of 4."""
    rng = np.random.default_rng(40)
    wl = make_workload([9, 4], dim=8, part_dim=8, seed=40, activation="silu" if silu else None,
                       init=[False, False])
    ints = rng.integers(-4, 5, size=(wl.num_tokens, wl.dim)).astype(np.float32)
    wl.x[:, :wl.dim] = f32_to_bf16_bits(ints)
    wl.weight[:] = 1.0
    wl.bias[:] = 0.5
    got, st = _run(wl, olib)
    for s in range(2):
        a, b = int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1])
        ext = np.concatenate([np.zeros((3, wl.dim), np.float32), ints[a:b]])
        for i in range(b - a):
            acc = 0.5 + ext[i:i + 4].sum(axis=0)  # exact small integers plus a half
            for c in range(wl.dim):
                w = exact.silu_bf16_word(float(acc[c])) if silu else exact.bf16_word(float(acc[c]))
                assert got[a + i, c] == w
        assert np.array_equal(st[wl.cache_indices[s]].T, ext[-3:])


def test_plane_layout(olib):
    """Channel c lands at out[c // part_dim][t][c % part_dim]."""
    wl = make_workload([3, 2], dim=24, part_dim=8, seed=41, bias=False, activation=None)
    wl.weight[:] = 0.0
    wl.weight[:, 3] = 1.0
    vals = np.tile(np.arange(1, 25, dtype=np.float32), (wl.num_tokens, 1))
    vals *= np.where(np.arange(wl.num_tokens) % 2 == 0, 1.0, -1.0)[:, None].astype(np.float32)
    wl.x[:, :24] = f32_to_bf16_bits(vals)
    o, _ = oracle.run_workload(wl, lib=olib)
    assert o.shape == (3, wl.num_tokens, 8)
    for c in range(24):
        for t in range(wl.num_tokens):
            assert o[c // 8, t, c % 8] == wl.x[t, c]


@pytest.mark.parametrize("init", [False, True])
def test_state_is_last_three_inputs(olib, init):
    """Updated line = last three values of (history ++ x); history fills in when L < 3."""
    wl = make_workload([1, 2, 3, 7], dim=8, part_dim=8, seed=42, init=[init] * 4, lines=4,
                       cache_indices=[3, 1, 0, 2])
    old = wl.conv_states.copy()
    _, st = _run(wl, olib)
    xf = bf16_bits_to_f32(wl.x[:, :8])
    for s in range(4):
        a, b = int(wl.query_start_loc[s]), int(wl.query_start_loc[s + 1])
        line = int(wl.cache_indices[s])
        hist = old[line].T if init else np.zeros((3, 8), np.float32)
        ext = np.concatenate([hist, xf[a:b]])
        assert np.array_equal(st[line].T.view(np.uint32), ext[-3:].view(np.uint32))


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("k", [1, 2, 3, 17, 39])
def test_split_call_equals_one_call(olib, k):
    """A sequence cut at k into two calls, with the carried state and has_initial_state
    set on the second call, gives the same outputs and final state as one call."""
    wl = make_workload([40], dim=16, part_dim=8, seed=43, init=[True], lines=2, cache_indices=[1])
    full, st_full = _run(wl, olib)
    a = make_workload([k], dim=16, part_dim=8, seed=43, init=[True], lines=2, cache_indices=[1])
    a.x, a.weight, a.bias, a.conv_states = wl.x[:k].copy(), wl.weight, wl.bias, wl.conv_states.copy()
    out_a, st_a = _run(a, olib)
    b = make_workload([40 - k], dim=16, part_dim=8, seed=43, init=[True], lines=2, cache_indices=[1])
    b.x, b.weight, b.bias, b.conv_states = wl.x[k:].copy(), wl.weight, wl.bias, st_a
    out_b, st_b = _run(b, olib)
    assert np.array_equal(np.concatenate([out_a, out_b]), full)
    assert np.array_equal(st_b.view(np.uint32), st_full.view(np.uint32))


def test_permuting_sequences_permutes_outputs(olib):
    lens = [4, 1, 6, 3]
    wl = make_workload(lens, dim=16, part_dim=16, seed=44, init=[True, False, True, True],
                       cache_indices=[0, 1, 2, 3], lines=4)
    out, st = _run(wl, olib)
    perm = [2, 0, 3, 1]
    q = wl.query_start_loc
    rows = np.concatenate([np.arange(q[s], q[s + 1]) for s in perm])
    p = make_workload([lens[s] for s in perm], dim=16, part_dim=16, seed=44,
                      init=wl.has_initial_state[perm], cache_indices=wl.cache_indices[perm], lines=4)
    p.x, p.weight, p.bias, p.conv_states = wl.x[rows], wl.weight, wl.bias, wl.conv_states.copy()
    out_p, st_p = _run(p, olib)
    assert np.array_equal(out_p, out[rows])
    assert np.array_equal(st_p.view(np.uint32), st.view(np.uint32))


def test_channel_slice(olib):
    """Channel c's output and state depend only on channel c."""
    wl = make_workload([5, 9], dim=24, part_dim=8, seed=45)
    out, st = _run(wl, olib)
    sub = make_workload([5, 9], dim=8, part_dim=8, seed=45, init=wl.has_initial_state,
                        cache_indices=wl.cache_indices, lines=wl.num_cache_lines)
    sub.x = np.ascontiguousarray(wl.x[:, 8:16])
    sub.weight = np.ascontiguousarray(wl.weight[8:16])
    sub.bias = np.ascontiguousarray(wl.bias[8:16])
    sub.conv_states = np.ascontiguousarray(wl.conv_states[:, 8:16])
    out_s, st_s = _run(sub, olib)
    assert np.array_equal(out_s, out[:, 8:16])
    assert np.array_equal(st_s, st[:, 8:16])


def test_part_dim_only_reshapes(olib):
    wl = make_workload([6, 3], dim=24, part_dim=8, seed=46)
    a, _ = _run(wl, olib)
    wl.part_dim = 24
    b, _ = _run(wl, olib)
    wl.part_dim = 4
    c, _ = _run(wl, olib)
    assert np.array_equal(a, b) and np.array_equal(a, c)


def test_strided_x_equals_contiguous(olib):
    wl = make_workload([6, 3, 8], dim=16, part_dim=8, seed=47, row_stride=16 + 40)
    a, sa = _run(wl, olib)
    wl.x = np.ascontiguousarray(wl.x[:, :16])
    b, sb = _run(wl, olib)
    assert np.array_equal(a, b) and np.array_equal(sa, sb)


def test_no_initial_state_equals_zero_line(olib):
    wl = make_workload([7, 2], dim=16, part_dim=8, seed=48, init=[False, False])
    a, sa = _run(wl, olib)
    wl.has_initial_state[:] = True
    wl.conv_states[wl.cache_indices] = 0.0
    b, sb = _run(wl, olib)
    assert np.array_equal(a, b) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32))


def test_null_block_runs_from_zero_and_leaves_its_line(olib):
    wl = make_workload([5, 4, 2], dim=16, part_dim=8, seed=49, init=[True, True, True],
                       cache_indices=[1, 0, 2], lines=3, null_block_id=0)
    before = wl.conv_states.copy()
    a, sa = _run(wl, olib)
    assert np.array_equal(sa[0], before[0])
    wl.null_block_id = None
    wl.has_initial_state[1] = False
    b, _ = _run(wl, olib)
    assert np.array_equal(a, b)


def test_untouched_rows_lines_and_empty_sequences(olib):
    wl = make_workload([3, 0, 4], dim=16, part_dim=8, seed=50, init=[True, True, True],
                       cache_indices=[0, 3, 1], lines=5, pad_tokens=5)
    before = wl.conv_states.copy()
    out = np.full((2, wl.num_tokens, 8), 0xABCD, dtype=np.uint16)
    o, st = oracle.run_workload(wl, out=out, lib=olib)
    assert np.all(o[:, 7:, :] == 0xABCD)  # rows past the last sequence
    for line in (2, 3, 4):  # unreferenced lines and the empty sequence's line
        assert np.array_equal(st[line], before[line])


def test_no_tokens_at_all(olib):
    """Page vllm.models.kimi_k3.nvidia.ops.kda_conv, packed_causal_conv1d_fn: with no tokens
    the call returns at once. Every sequence empty, x with no rows (numpy gives such an
    array zero strides): the output has no rows and every state word is as it was, also
    for sequences with an initial state."""
    wl = make_workload([0, 0, 0], dim=24, part_dim=8, seed=52, init=[True, False, True],
                       cache_indices=[2, 0, 3], lines=5)
    assert wl.num_tokens == 0 and wl.x.shape[0] == 0
    before = wl.conv_states.copy()
    o, st = oracle.run_workload(wl, lib=olib)
    assert o.shape == (3, 0, 8)
    assert np.array_equal(st.view(np.uint32), before.view(np.uint32))


def test_rejects_bad_metadata(olib):
    wl = make_workload([3, 4], dim=16, part_dim=8, seed=51)
    bad = wl.query_start_loc.copy()
    bad[1] = 5
    bad[2] = 4
    with pytest.raises(ValueError):
        oracle.packed_causal_conv1d(wl.x, 16, wl.weight, wl.bias, wl.conv_states.copy(), bad,
                                    wl.cache_indices, wl.has_initial_state, 8, lib=olib)


@pytest.mark.parametrize("bad_line", [-1, -2 ** 31, 3, 2 ** 31 - 1])
def test_out_of_range_line_acts_as_null_block(olib, bad_line):
    """A cache line outside [0, lines) names no line: the sequence runs from zero history,
    reads and writes no state, and its outputs are still written (the reading shared with
    the null block). Checked against the exact brute force and against the same call with
    that sequence on the null block."""
    wl = make_workload([4, 6, 2], dim=16, part_dim=8, seed=52, init=[True, True, True],
                       cache_indices=[1, bad_line, 0], lines=3)
    before = wl.conv_states.copy()
    got, st = _run(wl, olib)
    want, want_st = brute_force(wl)
    assert np.array_equal(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))
    assert np.array_equal(st[2], before[2])  # the line no sequence names stays as it was
    nul = make_workload([4, 6, 2], dim=16, part_dim=8, seed=52, init=[True, True, True],
                        cache_indices=[1, 2, 0], lines=3, null_block_id=2)
    got_n, st_n = _run(nul, olib)
    assert np.array_equal(got, got_n)
    assert np.array_equal(st.view(np.uint32), st_n.view(np.uint32))


# ---------------------------------------------------------------- argument strides

def _replaced(wl, **kw):
    import dataclasses

    return dataclasses.replace(wl, conv_states=wl.conv_states.copy(), **kw)


@pytest.mark.parametrize("layout", ["transposed", "padded"])
def test_weight_strides_against_brute_force(olib, layout):
    """Tap k of channel c is read at weight[c * ws0 + k * ws1] for any two strides (page:
    the launch passes both weight strides). A (dim, 4) view of a (4, dim) array (strides
    1 and dim) and a view with a row pitch of 7 give the brute-force result, which reads
    the same values without strides."""
    wl = make_workload([5, 3, 8], dim=12, part_dim=4, seed=80, init=[True, False, True], lines=4)
    want, want_st = brute_force(wl)
    if layout == "transposed":
        view = np.ascontiguousarray(wl.weight.T).T
        assert view.strides == (4, 4 * 12)
    else:
        pad = np.full((12, 7), np.float32(1e30))
        pad[:, 2:6] = wl.weight
        view = pad[:, 2:6]
        assert view.strides == (28, 4)
    got, st = _run(_replaced(wl, weight=view), olib)
    assert np.array_equal(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


def test_cache_index_stride_against_brute_force(olib):
    """The line of sequence s is read at cache_indices[s * stride]: every other entry of an
    array whose other entries name different, valid lines."""
    wl = make_workload([5, 3, 8, 2], dim=8, part_dim=8, seed=81, init=[True, True, False, True],
                       cache_indices=[3, 0, 5, 1], lines=7)
    want, want_st = brute_force(wl)
    inter = np.array([3, 6, 0, 2, 5, 4, 1, 6], dtype=np.int32)
    view = inter[::2]
    assert view.strides == (8,) and np.array_equal(view, wl.cache_indices)
    got, st = _run(_replaced(wl, cache_indices=view), olib)
    assert np.array_equal(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


def test_no_initial_state_array_means_none_set(olib):
    """has_initial_state = None (a NULL pointer in the C call): every sequence starts from
    zeros and still writes its line, as with an all-false array."""
    wl = make_workload([5, 3, 8], dim=8, part_dim=8, seed=82, init=[True, True, True], lines=4)
    got, st = _run(_replaced(wl, has_initial_state=None), olib)
    wl.has_initial_state[:] = False
    want, want_st = brute_force(wl)
    assert np.array_equal(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


# ---------------------------------------------------------------- library form

@pytest.mark.parametrize("seed", range(3))
@pytest.mark.parametrize("silu", [False, True])
def test_against_torch_conv1d_float64(olib, seed, silu):
    """One sequence, no initial state: F.conv1d(x.T, w, b, padding=3, groups=dim)[..., :T]
    in float64, then SiLU in float64, agrees within the FP32 chain's error bound plus
    one bf16 rounding."""
    T, dim = 300, 64
    wl = make_workload([T], dim=dim, part_dim=32, seed=60 + seed, init=[False],
                       activation="silu" if silu else None)
    got, _ = _run(wl, olib)
    xs = torch.from_numpy(bf16_bits_to_f32(wl.x[:, :dim])).double().T[None]
    w = torch.from_numpy(wl.weight).double()[:, None, :]
    b = torch.from_numpy(wl.bias).double()
    ref = torch.nn.functional.conv1d(xs, w, b, padding=3, groups=dim)[0, :, :T].T
    mag = torch.nn.functional.conv1d(xs.abs(), w.abs(), b.abs(), padding=3, groups=dim)[0, :, :T].T
    if silu:
        ref = torch.nn.functional.silu(ref)
    ref, mag = ref.numpy(), mag.numpy()
    g = bf16_bits_to_f32(got).astype(np.float64)
    # four fused roundings of the chain, SiLU's own rounding (slope <= 1.1), one bf16 rounding
    tol = 8 * 2.0 ** -24 * mag + 4 * 2.0 ** -24 * np.abs(ref) + bf16_ulp(ref) * 0.5 + 1e-30
    assert np.all(np.abs(g - ref) <= tol)


# ------------------------------------------------------- conv-state layouts

def test_wide_state_uses_entries_zero_to_two(olib):
    """A state wider than 3 (the page's check admits size(2) >= 3 and its launch
    passes the three strides, not the size): entries 0..2 are the history and the
    rest stay as they were."""
    wl = make_workload([5, 2, 9, 1], dim=16, part_dim=8, seed=48, init=[True, True, False, True])
    o_ref, st_ref = oracle.run_workload(wl, lib=olib)
    lines = wl.conv_states.shape[0]
    wide = np.random.default_rng(48).standard_normal((lines, 16, 6)).astype(np.float32)
    wide[:, :, :3] = wl.conv_states
    extra = wide[:, :, 3:].copy()
    o = oracle.packed_causal_conv1d(wl.x, wl.dim, wl.weight, wl.bias, wide, wl.query_start_loc,
                                    wl.cache_indices, wl.has_initial_state, wl.part_dim,
                                    wl.activation, wl.null_block_id, lib=olib)
    assert np.array_equal(o, o_ref)
    assert np.array_equal(wide[:, :, :3].view(np.uint32), st_ref.view(np.uint32))
    assert np.array_equal(wide[:, :, 3:], extra)


def test_dim_first_state_equals_contiguous(olib):
    """The state stored as (lines, 3, dim) and passed through its strides gives the
    same outputs and the same updated values as the (lines, dim, 3) layout."""
    wl = make_workload([5, 2, 9, 1], dim=16, part_dim=8, seed=49, init=[True, False, True, True])
    o_ref, st_ref = oracle.run_workload(wl, lib=olib)
    first = np.ascontiguousarray(wl.conv_states.transpose(0, 2, 1))  # (lines, 3, dim)
    view = first.transpose(0, 2, 1)  # logical (lines, dim, 3), strides (3 dim, 1, dim)
    o = oracle.packed_causal_conv1d(wl.x, wl.dim, wl.weight, wl.bias, view, wl.query_start_loc,
                                    wl.cache_indices, wl.has_initial_state, wl.part_dim,
                                    wl.activation, wl.null_block_id, lib=olib)
    assert np.array_equal(o, o_ref)
    assert np.array_equal(first.transpose(0, 2, 1).view(np.uint32), st_ref.view(np.uint32))
