"""Pins for the oracle's correctly rounded binary32 exp.

The SiLU of the page (vllm.models.kimi_k3.nvidia.ops.kda_conv, module docstring,
second paragraph: the stock arithmetic in FP32, SiLU) needs an exp whose result
does not depend on a library: the reading is exp correctly rounded to binary32.
The pin is mpmath at 200 bits rounded by exact rational arithmetic (tests/exact.py),
on random inputs, on the range edges, and on every input of a scanned slice where
the oracle's double evaluation sits near a binary32 midpoint (the cases where a
plain ``(float)exp((double)x)`` could round the wrong way).
"""

import math
import pathlib

import numpy as np
import pytest

import exact
import oracle

GOLDEN = pathlib.Path(__file__).resolve().parent / "golden" / "expf_escalations.txt"


def _check(olib, xs):
    bad = []
    for x in xs:
        x = float(x)
        got = olib.oracle_crexpf(x)
        ref = exact.exp32(x)
        if not (got == ref or (math.isnan(got) and math.isnan(ref))):
            bad.append((x, got, ref))
    assert not bad, bad[:5]


def test_expf_random_against_mpmath(olib):
    rng = np.random.default_rng(21)
    xs = np.concatenate([
        rng.uniform(-104.0, 89.0, 3000),
        rng.standard_normal(2000) * 4.0,
        rng.uniform(-1e-3, 1e-3, 500),
    ]).astype(np.float32)
    _check(olib, xs)


def test_expf_edges(olib):
    """Overflow edge (about 88.7228), the subnormal range and the underflow to 0."""
    edges = []
    for centre in (88.72283, -87.33654, -103.27893, -103.97208, 0.0, 16.635532, -16.635532):
        c = np.float32(centre)
        u = int(np.array([c]).view(np.uint32)[0])
        edges.extend(exact.from_bits32(u + d) for d in range(-40, 41) if 0 <= u + d < 1 << 32)
    edges.extend([math.inf, -math.inf, 1e-45, -1e-45, 3.0e38, -3.0e38])
    _check(olib, edges)
    assert math.isnan(olib.oracle_crexpf(math.nan))


def test_expf_escalated_inputs_of_a_slice(olib):
    """Every input in a slice of 2^22 patterns that takes the quad branch, against mpmath."""
    import ctypes

    first, count = 0x41800000, 1 << 22  # 16.0 .. 32.0 subrange, and its negative below
    for base in (first, first | 0x80000000, 0x3F800000, 0xBF800000):
        cand = np.zeros(4096, dtype=np.uint32)
        gap = ctypes.c_double()
        n = olib.oracle_crexpf_scan(base, count, cand.ctypes.data, cand.size, ctypes.byref(gap))
        assert n < cand.size
        _check(olib, [exact.from_bits32(int(u)) for u in cand[:n]])
        if n:
            # The 113-bit value's own error is below 2^-110; the rounding decision is
            # certain while its distance to the midpoint stays far above that.
            assert gap.value > -100


def test_expf_certificate_file(olib):
    """The committed certificate (oracle/certify_expf.py, all 2^32 inputs): every listed
    escalation's result equals mpmath's correctly rounded value, and the smallest
    distance of a 113-bit value to its midpoint is far above that format's error."""
    assert GOLDEN.exists(), "run python -m oracle.certify_expf"
    text = GOLDEN.read_text().splitlines()
    head = {ln.split()[1]: ln for ln in text if ln.startswith("# count")}
    count = int(head["count"].split()[2])
    worst = float([ln for ln in text if ln.startswith("# smallest")][0].rsplit(":", 1)[1])
    rows = [ln.split() for ln in text if ln and not ln.startswith("#")]
    assert len(rows) == count > 1000
    assert -100 < worst < -40
    bad = []
    for u_hex, r_hex in rows:
        x = exact.from_bits32(int(u_hex, 16))
        if exact.bits32(exact.exp32(x)) != int(r_hex, 16):
            bad.append(u_hex)
    assert not bad, bad[:5]
    rng = np.random.default_rng(5)
    for i in rng.choice(len(rows), size=200, replace=False):
        x = exact.from_bits32(int(rows[i][0], 16))
        assert exact.bits32(olib.oracle_crexpf(x)) == int(rows[i][1], 16)
