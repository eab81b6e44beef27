"""The staged state-line writes of the decode step and of a prefill sequence's first
tile, checked as arithmetic on the CPU.

A wave owns channels [cfirst, cfirst + n) of a launch, n = min(64 V, col_end - cfirst);
in a contiguous (dim, 3) line those channels are 12 n consecutive bytes, and lane l's
V channels (3 V floats) are bytes [12 V l, 12 V (l + 1)) of that part. Lanes past the
launch's last channel take the last active lane's channels. The kernel writes a line
part through the wave's LDS slice of 64 * 3 V floats (3 KB for V = 4): lane l writes
its 3 V floats at slot (cl - cfirst) / V, i.e. bytes [12 V slot, 12 V (slot + 1));
then piece q of lane l (q < 3 V / 4) is read back from bytes [16 (l + 64 q), +16) and
stored at the same byte offset of the line part, through a buffer descriptor whose
range is the part's 12 n bytes (pieces at or past it are dropped by the hardware).

These tests replay those formulas for every wave and lane of the decode launches the
bench and the GPU tests make (including partial last column blocks and the split of
large outputs into plane groups), and check that every LDS and memory byte offset
stays inside the slice and the line part, that lanes sharing a slot write the same
values, and that the bytes stored are exactly the part's bytes with the right values.
The GPU parity tests check the kernel itself.
"""

import pytest

WAVE = 64
V = 4  # channels per lane
PIECES = 3 * V // 4  # 16-byte pieces per lane
SLICE = 12 * V * WAVE  # bytes of one wave's LDS slice
INT32_MAX = 2 ** 31 - 1


def _plane_groups(tokens, dim, part_dim, eb):
    """(col_begin, col_end) of each launch, as the host splits large outputs."""
    plane_bytes = tokens * part_dim * eb
    planes = dim // part_dim
    per = max(1, INT32_MAX // plane_bytes) if plane_bytes > 0 else planes
    return [(pl * part_dim, min(planes, pl + per) * part_dim) for pl in range(0, planes, per)]


def _lanes(col_begin, col_end, cb):
    cfirst = col_begin + cb * WAVE * V
    n = min(WAVE * V, col_end - cfirst)
    out = []
    for lane in range(WAVE):
        c0 = col_begin + (cb * WAVE + lane) * V
        cl = c0 if c0 < col_end else col_end - V
        out.append((lane, cl, (cl - cfirst) // V))
    return cfirst, n, out


def _check_wave(col_begin, col_end, cb):
    cfirst, n, lanes = _lanes(col_begin, col_end, cb)
    part = 12 * n
    assert 0 < n <= WAVE * V and n % V == 0 and part <= SLICE
    # lanes write their floats, tagged (channel, entry), at their slot
    lds = {}
    for lane, cl, slot in lanes:
        assert 0 <= slot < WAVE
        for k in range(V):
            for j in range(3):
                b = 12 * V * slot + 4 * (3 * k + j)
                assert 0 <= b and b + 4 <= SLICE
                tag = (cl + k, j)
                assert lds.get(b, tag) == tag  # lanes sharing a slot write the same values
                lds[b] = tag
    stored = {}
    for lane, _, _ in lanes:
        for q in range(PIECES):
            off = 16 * (lane + WAVE * q)
            assert 0 <= off and off + 16 <= SLICE
            if off + 16 > part:  # outside the descriptor's range: dropped
                continue
            for w in range(4):
                b = off + 4 * w
                assert b not in stored
                stored[b] = lds[b]
    assert sorted(stored) == list(range(0, part, 4))  # the whole part, once
    for b, (c, j) in stored.items():
        assert c == cfirst + b // 12 and j == (b % 12) // 4  # the right value at each byte
        assert cfirst <= c < cfirst + n


def _check_launch(tokens, dim, part_dim, eb):
    for col_begin, col_end in _plane_groups(tokens, dim, part_dim, eb):
        cols = col_end - col_begin
        col_blocks = -(-(cols // V) // WAVE)
        for cb in range(col_blocks):
            _check_wave(col_begin, col_end, cb)


@pytest.mark.parametrize("batch", [64, 256, 1024, 4096])
def test_bench_decode_batches(batch):
    """The bench's decode steps: dim 4608 = 3 x 1536."""
    _check_launch(batch, 4608, 1536, 2)


@pytest.mark.parametrize("dim,part_dim", [(3 * 256, 256), (3 * 200, 200), (3 * 1536, 1536),
                                          (3 * 192, 192), (3 * 40, 40), (5 * 40, 40),
                                          (4 * 112, 112), (24, 8), (3 * 520, 520)])
@pytest.mark.parametrize("eb", [2, 4])
def test_test_shapes(dim, part_dim, eb):
    """Every channel count the decode tests use, with partial last column blocks."""
    _check_launch(37, dim, part_dim, eb)


def test_plane_groups_of_a_large_batch():
    """A batch whose output is split into several launches (col_begin > 0)."""
    tokens, dim, part_dim = 262144, 4608, 1536
    groups = _plane_groups(tokens, dim, part_dim, 2)
    assert len(groups) == 2 and groups[1][0] == 3072
    _check_launch(tokens, dim, part_dim, 2)
    many = _plane_groups(300000, 4608, 8, 4)
    assert len(many) == 1 or all(b % 8 == 0 for b, _ in many)
    _check_launch(300000, 4608, 8, 4)


# ----------------------------------------------------------------- bf16 lines

PIECES16 = 3 * V // 4  # 8-byte pieces per lane
SLICE_READ16 = 8 * WAVE * PIECES16  # bytes of the slice the store instructions read


def _check_wave_bf16(col_begin, col_end, cb):
    """The bf16 staged write: lane l writes its 6 V bytes (3 V words) at bytes
    [6 V slot, 6 V (slot + 1)) of the slice; piece q of lane l is bytes [8 (l + 64 q), +8),
    stored at the same offset of the line part through a descriptor whose range is the
    part's 6 n bytes."""
    cfirst, n, lanes = _lanes(col_begin, col_end, cb)
    part = 6 * n
    assert part % 8 == 0 and SLICE_READ16 <= SLICE  # no straddling piece; reads in the slice
    lds = {}
    for lane, cl, slot in lanes:
        for k in range(V):
            for j in range(3):
                b = 6 * V * slot + 2 * (3 * k + j)
                assert 0 <= b and b + 2 <= SLICE
                tag = (cl + k, j)
                assert lds.get(b, tag) == tag
                lds[b] = tag
    stored = {}
    for lane, _, _ in lanes:
        for q in range(PIECES16):
            off = 8 * (lane + WAVE * q)
            assert 0 <= off and off + 8 <= SLICE_READ16
            if off + 8 > part:  # at or past the range (part % 8 == 0): dropped
                assert off >= part
                continue
            for w in range(4):
                b = off + 2 * w
                assert b not in stored
                stored[b] = lds[b]
    assert sorted(stored) == list(range(0, part, 2))
    for b, (c, j) in stored.items():
        assert c == cfirst + b // 6 and j == (b % 6) // 2
        assert cfirst <= c < cfirst + n


def _check_launch_bf16(tokens, dim, part_dim):
    for col_begin, col_end in _plane_groups(tokens, dim, part_dim, 2):
        cols = col_end - col_begin
        for cb in range(-(-(cols // V) // WAVE)):
            _check_wave_bf16(col_begin, col_end, cb)


@pytest.mark.parametrize("batch", [64, 256, 1024, 4096])
def test_bf16_state_bench_batches(batch):
    _check_launch_bf16(batch, 4608, 1536)


@pytest.mark.parametrize("dim,part_dim", [(3 * 256, 256), (3 * 200, 200), (3 * 40, 40),
                                          (24, 8), (3 * 520, 520), (3 * 1536, 1536)])
def test_bf16_state_test_shapes(dim, part_dim):
    _check_launch_bf16(37, dim, part_dim)
