"""Pins for the oracle's fp16 and FP32 x formats.

Page: vllm.models.kimi_k3.nvidia.ops.kda_conv. packed_causal_conv1d_supported
admits bf16, fp16 and FP32 x with an FP32 state and FP32 weights; the
packed_causal_conv1d_fn docstring gives the output x's dtype; the note after the
module docstring fixes FP32 arithmetic for every input dtype. Readings: the FP32
result rounds to fp16 to nearest even (subnormals kept, overflow to infinity),
an FP32 output is the result itself, NaN results are stored as the format's
canonical quiet NaN, and fp16 -> FP32 widening is the IEEE 754 conversion
(a NaN becomes quiet, keeping sign and payload).

Pins that do not restate the oracle: numpy's float16 conversions (an
independent implementation of IEEE binary16 rounding) over every FP32 exponent
with the rounding-critical low bits and over an exhaustive block across the
fp16 subnormal range; exact rational rounding to 11 significant bits
(tests/exact.py) for closed forms and for the SiLU chain; exact-rational brute
force of the whole convolution on fp16 and FP32 inputs.
"""

import math

import numpy as np
import pytest

import exact
import oracle
from helpers import brute_force, make_workload, planes_to_rows


def _numpy_f16(u32: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return np.ascontiguousarray(u32).view(np.float32).astype(np.float16).view(np.uint16)


def _dropped_bits(expo_field: int) -> int:
    """FP32 fraction bits below the fp16 quantum for an FP32 exponent field
    (13 for fp16 normals, one more per binade below 2^-14)."""
    return 13 + max(0, 113 - expo_field)


def test_f16_round_every_binade_critical_bits(olib):
    """Every FP32 binade (both signs) with the low bits that decide the rounding
    (zero, one, just below, at and above the midpoint, all ones) under every
    combination of the kept bits (sampled where there are more than 1024)."""
    rng = np.random.default_rng(21)
    parts = []
    for e in range(255):
        k = _dropped_bits(e)
        if k >= 23:
            frac = np.concatenate([np.arange(0, 64, dtype=np.uint32),
                                   np.uint32(1 << 22) + np.arange(-32, 32, dtype=np.int64).astype(np.uint32),
                                   rng.integers(0, 1 << 23, 256).astype(np.uint32),
                                   np.array([(1 << 23) - 1], dtype=np.uint32)])
        else:
            half = 1 << (k - 1)
            lows = np.array([0, 1, half - 1, half, half + 1, 2 * half - 1], dtype=np.uint32)
            kept = 23 - k
            if kept <= 10:
                highs = np.arange(1 << kept, dtype=np.uint32)
            else:
                highs = rng.integers(0, 1 << kept, 1024).astype(np.uint32)
            frac = (highs[:, None] << np.uint32(k) | lows[None, :]).ravel()
        base = np.uint32(e << 23)
        parts.append(base | frac)
        parts.append(np.uint32(0x80000000) | base | frac)
    u = np.concatenate(parts)
    got = oracle.act_words(u.view(np.float32), False, "f16", lib=olib)
    assert np.array_equal(got, _numpy_f16(u))


def test_f16_round_exhaustive_block(olib):
    """2^26 consecutive patterns from 2^-18 up to 2^-10: the fp16 subnormal binades
    and the first normal ones, every pattern."""
    first = 0x36800000
    n = 1 << 26
    u = np.arange(n, dtype=np.uint32) + np.uint32(first)
    got = oracle.act_words_range(first, n, False, "f16", lib=olib)
    assert np.array_equal(got, _numpy_f16(u))


@pytest.mark.parametrize("y", [65504.0, 65519.99609375, 65520.0, 65536.0, -65520.0, 2.0 ** -24,
                               2.0 ** -25, exact.from_bits32(0x33000001), 3 * 2.0 ** -26,
                               2.0 ** -14, exact.from_bits32(0x387FFFFF), 1.0 + 2.0 ** -11,
                               1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -23, 1e-30, -0.0])
def test_f16_round_closed_forms(olib, y):
    """Against exact rational rounding to 11 significant bits, binary16 range."""
    assert olib.oracle_f32_to_f16(y) == exact.f16_word(y)


def test_f16_nan_reading(olib):
    for u in (0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF, 0xFF812345):
        assert olib.oracle_f32_to_f16(exact.from_bits32(u)) == 0x7E00


def test_f16_widen_every_pattern(olib):
    """All 65536 fp16 words: numbers against numpy's widening (exact); a NaN keeps
    sign and payload and has the quiet bit set."""
    h = np.arange(1 << 16, dtype=np.uint32)
    got = np.array([olib.oracle_f16_to_f32_bits(int(v)) for v in h], dtype=np.uint32)
    ref = h.astype(np.uint16).view(np.float16).astype(np.float32).view(np.uint32)
    nan = np.isnan(ref.view(np.float32))
    assert np.array_equal(got[~nan], ref[~nan])
    assert nan.sum() == 2 * 1023
    assert np.array_equal(got[nan], ref[nan] | np.uint32(0x00400000))


def test_f32_word_reading(olib):
    for y in (0.0, -0.0, 1.5, -3e-45, math.inf, -math.inf):
        assert olib.oracle_f32_word(y) == exact.bits32(y)
    for u in (0x7FC00000, 0xFFC00001, 0x7F800001):
        assert olib.oracle_f32_word(exact.from_bits32(u)) == 0x7FC00000


@pytest.mark.parametrize("fmt", ["f16", "f32"])
def test_silu_random_against_exact(olib, fmt):
    rng = np.random.default_rng(41)
    xs = np.concatenate([
        rng.standard_normal(2500),
        rng.standard_normal(800) * 12.0,
        rng.uniform(-90.0, 20.0, 800),
        rng.uniform(-1e-4, 1e-4, 300),  # fp16 subnormal results
        rng.uniform(6e4, 7e4, 100),  # around the fp16 overflow
    ]).astype(np.float32)
    got = oracle.act_words(xs, True, fmt, lib=olib)
    want = np.array([exact.silu_word(float(a), fmt) for a in xs], dtype=got.dtype)
    assert np.array_equal(got, want)


def test_silu_f32_where_exp_is_hard(olib):
    """The FP32 SiLU value itself on every accumulator whose exp(-a) needed the
    quad-precision branch (the escalation list of the exp certificate)."""
    import test_oracle_act

    rows = [ln.split()[0] for ln in test_oracle_act.GOLDEN.read_text().splitlines()
            if ln and ln[0] != "#"]
    a = np.array([int(u, 16) ^ 0x80000000 for u in rows], dtype=np.uint32).view(np.float32)
    got = oracle.act_words(a, True, "f32", lib=olib)
    want = np.array([exact.silu_word(float(v), "f32") for v in a], dtype=np.uint32)
    assert np.array_equal(got, want)


def _near_f16_midpoints(n: int, seed: int) -> np.ndarray:
    """Accumulators whose SiLU lies within a few FP32 ulps of an fp16 midpoint (low
    13 fraction bits 0x1000), by Newton's method in double on SiLU(a) = midpoint."""
    rng = np.random.default_rng(seed)
    out = []
    for a0 in rng.standard_normal(n) * 3.0:
        a = float(a0)
        y = a / (1.0 + math.exp(-a))
        if abs(y) < 2.0 ** -13:
            continue
        u = exact.bits32(exact.f32(y))
        mid = exact.from_bits32((u & 0xFFFFE000) | 0x1000)
        for _ in range(30):
            s = 1.0 / (1.0 + math.exp(-a))
            d = s + a * s * (1.0 - s)
            if d == 0.0:
                break
            a -= (a * s - mid) / d
        base = exact.bits32(exact.f32(a))
        out.extend(exact.from_bits32(base + k) for k in range(-3, 4))
    return np.array(out, dtype=np.float32)


def test_silu_near_f16_midpoints(olib):
    a = _near_f16_midpoints(250, 42)
    got = oracle.act_words(a, True, "f16", lib=olib)
    want = np.array([exact.silu_word(float(v), "f16") for v in a], dtype=np.uint16)
    assert np.array_equal(got, want)
    near = 0
    for v in a[::7]:
        y = float(v) / (1.0 + math.exp(-float(v)))
        near += abs((exact.bits32(exact.f32(y)) & 0x1FFF) - 0x1000) <= 3
    assert near > 80


@pytest.mark.parametrize("fmt", ["f16", "f32"])
@pytest.mark.parametrize("seed", range(3))
def test_brute_force_exact(olib, fmt, seed):
    act = "silu" if seed != 1 else None
    wl = make_workload([5, 0, 3, 9, 1, 2], dim=12, part_dim=4, seed=100 + seed, activation=act,
                       null_block_id=1 if seed == 2 else None, cache_indices=[0, 2, 1, 3, 4, 5],
                       lines=7, x_scale=1.0 + 10 * (seed == 2), x_dtype=fmt, row_stride=16)
    o, st = oracle.run_workload(wl, lib=olib)
    want, want_st = brute_force(wl)
    assert np.array_equal(planes_to_rows(o), want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


@pytest.mark.parametrize("fmt", ["f16", "f32"])
def test_state_holds_widened_inputs(olib, fmt):
    """With an identity tap the output is the input rounded back to its format and
    the state holds the last three widened inputs, so both are the input words."""
    wl = make_workload([7], dim=8, part_dim=8, seed=3, activation=None, bias=False,
                       init=[False], x_dtype=fmt)
    wl.weight[:] = 0.0
    wl.weight[:, 3] = 1.0
    o, st = oracle.run_workload(wl, lib=olib)
    x = wl.x[:, : wl.dim]
    assert np.array_equal(planes_to_rows(o), x)
    line = int(wl.cache_indices[0])
    from workloads import words_to_f32

    assert np.array_equal(st[line].T.view(np.uint32), words_to_f32(x[-3:], fmt).view(np.uint32))


def test_same_values_same_result_in_every_format(olib):
    """x values that are exact in bf16 give the same FP32 accumulators in every
    format, so the FP32 output rounded to bf16 and the bf16 output agree word for
    word, and so do the states."""
    wl = make_workload([9, 4], dim=16, part_dim=8, seed=5, x_dtype="bf16", init=[True, False])
    o_bf, st_bf = oracle.run_workload(wl, lib=olib)
    from workloads import bf16_bits_to_f32

    wl32 = make_workload([9, 4], dim=16, part_dim=8, seed=5, x_dtype="f32", init=[True, False])
    wl32.x[:, :16] = bf16_bits_to_f32(wl.x[:, :16]).view(np.uint32)
    o32, st32 = oracle.run_workload(wl32, lib=olib)
    assert np.array_equal(st_bf.view(np.uint32), st32.view(np.uint32))
    rounded = np.array([exact.bf16_word(float(v)) for v in o32.ravel().view(np.float32)],
                       dtype=np.uint16).reshape(o_bf.shape)
    assert np.array_equal(rounded, o_bf)


def test_unknown_format_rejected(olib):
    wl = make_workload([3], dim=8, part_dim=8, seed=1)
    rc = olib.oracle_packed_causal_conv1d(
        wl.x.ctypes.data, 7, 3, 8, 8, wl.weight.ctypes.data, 4, 1, None,
        wl.conv_states.ctypes.data, wl.conv_states.shape[0], 24, 3, 1,
        wl.query_start_loc.ctypes.data, 1, wl.cache_indices.ctypes.data, 1, None, 8, 1, 0, 0,
        np.zeros(24, dtype=np.uint16).ctypes.data)
    assert rc == 1


def test_workload_formats_share_draws():
    """The x format changes no draw: the FP32 inputs of a fuzz case round to its bf16
    and fp16 inputs, and the other arrays are identical."""
    import workloads

    for seed in (3, 2001):
        b = workloads.random_case(seed, x_dtype="bf16")
        h = workloads.random_case(seed, x_dtype="f16")
        f = workloads.random_case(seed, x_dtype="f32")
        vals = f.x[:, : f.dim].view(np.float32)
        assert np.array_equal(workloads.f32_to_bf16_bits(vals), b.x[:, : b.dim])
        assert np.array_equal(vals.astype(np.float16).view(np.uint16), h.x[:, : h.dim])
        assert np.all(f.x[:, f.dim:] == workloads.CANARIES["f32"])
        for name in ("weight", "conv_states", "query_start_loc", "cache_indices"):
            assert np.array_equal(getattr(b, name), getattr(f, name))
