"""The prefill kernel's program map, checked as arithmetic on the CPU.

Programs [0, S) are the first tiles of the sequences; program S + q is the later
tile (tile index j >= 1) whose first row lies in [(q + 1) R, (q + 2) R), found
through the sequence that contains row (q + 1) R. The kernel's describe_tile
evaluates the same formulas; these tests check that the map, over a grid of
S + cdiv(T, R) programs, names every tile of every sequence exactly once
(empty sequences, padding rows, every tile size the kernel uses). The GPU parity
tests check the kernel itself.
"""

import numpy as np
import pytest


def _tiles_by_map(qsl, T, R):
    S = len(qsl) - 1
    got = []
    for p in range(S + (T + R - 1) // R):
        if p < S:
            start = min(max(qsl[p], 0), T)
            end = min(max(qsl[p + 1], start), T)
            if end > start:
                got.append((p, 0))
            continue
        r0 = (p - S + 1) * R
        if r0 >= T:
            continue
        cand = [s for s in range(S) if qsl[s] <= r0]
        if not cand:
            continue
        s = max(cand)
        start = min(max(qsl[s], 0), T)
        end = min(max(qsl[s + 1], start), T)
        if r0 < start or r0 >= end:
            continue
        j = (r0 - start + R - 1) // R
        t0 = start + j * R
        if j < 1 or t0 >= end:
            continue
        got.append((s, j))
    return got


@pytest.mark.parametrize("R", [4, 8, 16])
def test_every_tile_exactly_once(R):
    rng = np.random.default_rng(R)
    for _ in range(600):
        S = int(rng.integers(1, 40))
        lens = rng.integers(0, 60, size=S)
        lens[rng.random(S) < 0.3] = 0
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(int)
        T = int(qsl[-1]) + int(rng.integers(0, 20))
        if T == 0:
            continue
        want = sorted((s, j) for s in range(S) for j in range(-(-int(lens[s]) // R)))
        got = _tiles_by_map(qsl, T, R)
        assert len(got) == len(set(got))
        assert sorted(got) == want


def test_one_long_sequence():
    qsl = np.array([0, 16384])
    got = _tiles_by_map(qsl, 16384, 16)
    assert got == [(0, j) for j in range(1024)]
