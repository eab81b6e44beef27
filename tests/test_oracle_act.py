"""Pins for the oracle's activation-and-rounding map (FP32 accumulator -> stored bf16).

Page: vllm.models.kimi_k3.nvidia.ops.kda_conv, module docstring (second
paragraph: SiLU in FP32, FP32 -> bf16 round to nearest even) and the
``packed_causal_conv1d_fn`` source (activation "silu", "swish" or True selects
SiLU). Reading: y = a / (1 + exp(-a)) with exp correctly rounded and the add and
divide rounded to binary32. The pin is the same chain in exact rational
arithmetic with mpmath's exp (tests/exact.py), plus closed forms.
"""

import math
import pathlib

import numpy as np
import pytest

import exact
import oracle

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden" / "expf_escalations.txt"


def _silu_word(olib, a: float) -> int:
    return olib.oracle_act_bf16(a, 1)


def test_silu_random_against_exact(olib):
    rng = np.random.default_rng(31)
    xs = np.concatenate([
        rng.standard_normal(4000),
        rng.standard_normal(1500) * 12.0,
        rng.uniform(-90.0, 20.0, 1500),
        rng.uniform(-1e-30, 1e-30, 200),
    ]).astype(np.float32)
    got = oracle.act_bf16(xs, True, lib=olib)
    want = np.array([exact.silu_bf16_word(float(a)) for a in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_silu_where_exp_is_hard(olib):
    """Every accumulator a whose exp(-a) is one of the certificate's escalations."""
    rows = [ln.split()[0] for ln in GOLDEN.read_text().splitlines() if ln and ln[0] != "#"]
    a = np.array([int(u, 16) ^ 0x80000000 for u in rows], dtype=np.uint32).view(np.float32)
    got = oracle.act_bf16(a, True, lib=olib)
    want = np.array([exact.silu_bf16_word(float(v)) for v in a], dtype=np.uint16)
    assert np.array_equal(got, want)


def _near_midpoint_inputs(n: int, seed: int) -> np.ndarray:
    """FP32 accumulators whose SiLU lies within a few FP32 ulps of a bf16 midpoint:
    pick a, take the bf16 midpoint nearest SiLU(a), Newton-solve SiLU(a) = midpoint
    in double, keep the FP32 neighbours of the root."""
    rng = np.random.default_rng(seed)
    out = []
    for a0 in rng.standard_normal(n) * 3.0:
        a = float(a0)
        y = a / (1.0 + math.exp(-a))
        u = exact.bits32(exact.f32(y))
        mid = exact.from_bits32((u & 0xFFFF0000) | 0x8000)
        for _ in range(30):
            s = 1.0 / (1.0 + math.exp(-a))
            f = a * s - mid
            d = s + a * s * (1.0 - s)
            if d == 0.0:
                break
            a -= f / d
        base = exact.bits32(exact.f32(a))
        out.extend(exact.from_bits32(base + k) for k in range(-3, 4))
    return np.array(out, dtype=np.float32)


def test_silu_near_bf16_midpoints(olib):
    """Accumulators whose SiLU lands near a bf16 rounding boundary (the hard rounding cases)."""
    a = _near_midpoint_inputs(300, 32)
    got = oracle.act_bf16(a, True, lib=olib)
    want = np.array([exact.silu_bf16_word(float(v)) for v in a], dtype=np.uint16)
    assert np.array_equal(got, want)
    # the construction does hit the boundary region: many SiLU values sit within 3 FP32 ulps
    near = 0
    for v in a[::7]:
        y = float(v) / (1.0 + math.exp(-float(v)))
        near += abs((exact.bits32(exact.f32(y)) & 0xFFFF) - 0x8000) <= 3
    assert near > 100


@pytest.mark.parametrize("a,word", [
    (0.0, 0x0000),       # 0 / 2
    (-0.0, 0x8000),      # -0 / 2
    (math.inf, 0x7F80),  # inf / (1 + 0)
    (-math.inf, 0x7FC0), # -inf / inf is NaN
    (math.nan, 0x7FC0),
    (-89.0, 0x8000),     # exp(89) overflows binary32: a / inf = -0
    (-1e30, 0x8000),
    (17.0, 0x4188),      # 1 + exp(-17) rounds to 1, so y = a = 17
    (1e30, None),        # y = a
    (100.0, None),
])
def test_silu_closed_forms(olib, a, word):
    if word is None:
        word = exact.bf16_word(exact.f32(a))
    assert _silu_word(olib, a) == word


def test_silu_large_positive_is_identity(olib):
    """For a >= 17, exp(-a) < 2^-24 so 1 + exp(-a) rounds to 1 and y = a exactly."""
    rng = np.random.default_rng(33)
    a = rng.uniform(17.0, 1e6, 2000).astype(np.float32)
    assert np.array_equal(oracle.act_bf16(a, True, lib=olib), oracle.act_bf16(a, False, lib=olib))


def test_silu_large_negative_is_negative_zero(olib):
    rng = np.random.default_rng(34)
    a = -rng.uniform(89.0, 1e30, 2000).astype(np.float32)
    assert np.all(oracle.act_bf16(a, True, lib=olib) == 0x8000)


def test_activation_rule():
    assert oracle.is_silu("silu") and oracle.is_silu("swish") and oracle.is_silu(True)
    assert not oracle.is_silu(None) and not oracle.is_silu(False) and not oracle.is_silu("gelu")
