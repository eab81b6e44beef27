"""The prefill kernel's program map, checked as arithmetic on the CPU.

Programs [0, S) are the first tiles of the sequences. The later programs go to row
blocks q: block q owns the later tile (tile index j >= 1) whose first row lies in
[(q + 1) R, (q + 2) R), found through the sequence that contains row (q + 1) R.
Blocks below split_half take one program each, blocks in [split_half,
split_quarter) two (one half of the tile's rows each) and the rest four (one
quarter each); the host picks the split points so that a fixed number of waves
compute half and quarter tiles at the end of the launch, and splits nothing when
the sequences average under two tiles. The kernel's
describe_tile and launch evaluate the same formulas; these tests check that the
map, over the grid the host launches, computes every row of every sequence exactly
once, with the 3 rows before each later part inside the same sequence (empty
sequences, padding rows, every tile size and column-block count the kernel uses).
The GPU parity tests check the kernel itself.
"""

import numpy as np
import pytest

HALF_TILE_WAVES = 2304
QUARTER_TILE_WAVES = 1152


def _split(T, S, R, col_blocks):
    blocks = max(0, -(-T // R) - 1)
    split = T >= 2 * R * S
    quarter = min(blocks, -(-QUARTER_TILE_WAVES // (4 * col_blocks))) if split else 0
    half = min(blocks - quarter, -(-HALF_TILE_WAVES // (2 * col_blocks))) if split else 0
    return blocks - quarter - half, blocks - quarter, half, quarter


def _parts_by_map(qsl, T, R, col_blocks):
    """(sequence, first row, rows, halo) for every program that has work."""
    S = len(qsl) - 1
    split_half, split_quarter, half, quarter = _split(T, S, R, col_blocks)
    programs = S + split_half + 2 * half + 4 * quarter
    got = []
    for p in range(programs):
        if p < S:
            start = min(max(qsl[p], 0), T)
            end = min(max(qsl[p + 1], start), T)
            if end > start:
                got.append((p, start, min(R, end - start), 0))
            continue
        pl = p - S
        if pl < split_half:
            q, parts, h = pl, 1, 0
        else:
            ph = pl - split_half
            nh = 2 * (split_quarter - split_half)
            if ph < nh:
                q, parts, h = split_half + ph // 2, 2, ph % 2
            else:
                q, parts, h = split_quarter + (ph - nh) // 4, 4, (ph - nh) % 4
        r0 = (q + 1) * R
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
        ts = t0 + h * (R // parts)
        n = min(R // parts, min(t0 + R, end) - ts)
        if n <= 0:
            continue
        got.append((s, ts, n, 3))
    return got


def _check_cover(qsl, T, R, col_blocks):
    S = len(qsl) - 1
    got = _parts_by_map(qsl, T, R, col_blocks)
    seen = np.zeros(T, dtype=int)
    for s, ts, n, halo in got:
        start, end = qsl[s], qsl[s + 1]
        assert start <= ts and ts + n <= end
        assert ts - halo >= start  # history rows belong to the sequence
        assert halo == 0 or ts - start >= R  # later parts never touch the state
        seen[ts:ts + n] += 1
    want = np.zeros(T, dtype=int)
    for s in range(S):
        want[qsl[s]:qsl[s + 1]] = 1
    assert np.array_equal(seen, want)
    firsts = [g for g in got if g[3] == 0]
    assert sorted(g[0] for g in firsts) == [s for s in range(S) if qsl[s + 1] > qsl[s]]


@pytest.mark.parametrize("R", [8, 16])
@pytest.mark.parametrize("col_blocks", [1, 3, 18, 200])
def test_every_row_exactly_once(R, col_blocks):
    rng = np.random.default_rng(R * 1000 + col_blocks)
    for _ in range(300):
        S = int(rng.integers(1, 40))
        lens = rng.integers(0, 60 if _ % 2 else 400, size=S)
        lens[rng.random(S) < 0.3] = 0
        qsl = np.concatenate([[0], np.cumsum(lens)]).astype(int)
        T = int(qsl[-1]) + int(rng.integers(0, 20))
        if T == 0:
            continue
        _check_cover(qsl, T, R, col_blocks)


def test_one_long_sequence():
    """16384 tokens over 18 column blocks: 943 whole tiles, 64 tiles in halves and 16
    in quarters after the first tile, i.e. rows 15104-16127 in 8-row parts and the last
    256 rows in 4-row parts."""
    qsl = np.array([0, 16384])
    got = _parts_by_map(qsl, 16384, 16, 18)
    assert got[0] == (0, 0, 16, 0)
    sizes = [n for _, _, n, _ in got[1:]]
    assert sizes == [16] * 943 + [8] * 128 + [4] * 64
    _check_cover(qsl, 16384, 16, 18)


def test_workgroup_division_by_multiplication():
    """The launcher's multiplier and shift (l = ceil(log2 d), m = floor(2^32 (2^l - d)/d)
    + 1) divide every workgroup index below 2^31 exactly, for every divisor up to 2^22
    that a launch can have (sampled)."""
    rng = np.random.default_rng(5)
    divisors = list(range(1, 1100)) + [int(v) for v in rng.integers(1, 1 << 22, size=400)]
    for d in divisors:
        l = (d - 1).bit_length()
        m = ((1 << 32) * ((1 << l) - d)) // d + 1
        assert 0 < m < (1 << 32)
        ns = np.concatenate([[0, 1, d - 1, d, d + 1, (1 << 31) - 1],
                             rng.integers(0, 1 << 31, size=300)]).astype(object)
        for n in ns:
            assert ((((n * m) >> 32) + n) >> l) == n // d


def _division(d):
    l = (d - 1).bit_length()
    return ((1 << 32) * ((1 << l) - d)) // d + 1, l


def _wave_slot(n, groups, programs, xcd_chunks):
    """(program, column group) of workgroup n, as the kernels' wave_slot computes it."""
    gm, gl = _division(groups)
    cm, cl = _division(8 * groups)
    full = programs // 8 if xcd_chunks else 0
    c = (((n * cm) >> 32) + n) >> cl
    if c < full:
        k = n - c * 8 * groups
        x, i, whole = k & 7, k >> 3, groups >> 3
        if i < 8 * whole:
            g, pi = 8 * (i >> 3) + x, i & 7
        else:
            L = x * (groups & 7) + (i - 8 * whole)
            g, pi = 8 * whole + (L >> 3), L & 7
        return 8 * c + pi, g
    b = n - full * 8 * groups
    p = (((b * gm) >> 32) + b) >> gl
    return 8 * full + p, b - p * groups


@pytest.mark.parametrize("xcd_chunks", [False, True])
def test_workgroup_order_is_a_bijection(xcd_chunks):
    for groups in [1, 2, 3, 5, 7, 8, 9, 12, 16, 17, 40]:
        for programs in [1, 7, 8, 9, 23, 64, 200]:
            seen = set()
            for n in range(programs * groups):
                p, g = _wave_slot(n, groups, programs, xcd_chunks)
                assert 0 <= p < programs and 0 <= g < groups
                seen.add((p, g))
            assert len(seen) == programs * groups


def test_prefill_order_keeps_column_groups_on_one_xcd():
    """16384 tokens x 4608 channels: 9 column groups of 2 waves; the tile below a tile
    in the same column group runs on the same XCD (workgroup index mod 8) for 8 of
    every 9 groups, and the rows are still visited chunk by chunk in order."""
    groups, programs = 9, 1 + 943 + 128 + 64
    xcd = {}
    order = []
    for n in range(programs * groups):
        p, g = _wave_slot(n, groups, programs, True)
        xcd[(p, g)] = n % 8
        order.append(p)
    pairs = [(p, g) for (p, g) in xcd if (p + 1, g) in xcd]
    local = sum(xcd[(p, g)] == xcd[(p + 1, g)] for p, g in pairs)
    assert local / len(pairs) > 0.88
    # Every workgroup of chunk c is dispatched before any of chunk c + 1.
    assert all(order[n] // 8 <= order[m] // 8 for n, m in zip(range(len(order) - 1), range(1, len(order))))
