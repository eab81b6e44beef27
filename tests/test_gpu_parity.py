"""GPU parity: the HIP path against the CPU oracle, bit for bit.

Output planes (bf16 words) and the updated FP32 conv state must be identical to
the oracle on the five named workloads at full size, on seeded fuzz cases
(zero-length sequences, null blocks, padding rows, strided x, several part_dim
values, wide accumulator ranges) and on edge cases. Rows no sequence owns must
keep the canary the output buffer was filled with; unread x columns hold bf16
NaN, so an over-read would show.
"""

import sys

import numpy as np
import pytest
import torch

import workloads
from gpu_util import CANARY, first_mismatches, oracle_with_canary, run_hip, to_device

pytestmark = pytest.mark.gpu


def _compare(wl):
    print(f"case: {wl.name}", flush=True)
    got, st = run_hip(wl)
    want, want_st = oracle_with_canary(wl)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32)), \
        first_mismatches(st.view(np.uint32), want_st.view(np.uint32))


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_named_workloads_bit_exact(cfg):
    _compare(workloads.CONFIGS[cfg]())


@pytest.mark.parametrize("seed", range(24))
def test_fuzz_bit_exact(seed):
    wl = workloads.random_case(1000 + seed, max_seqs=12, max_len=300,
                               x_scale=[1.0, 8.0, 40.0][seed % 3], pad_tokens=seed % 4)
    _compare(wl)


# One sequence of at most 2048 tokens (or sequences averaging 256 or more) takes 8-row
# tiles, other calls 16-row tiles: single lengths cover the 8-row edges, the same
# lengths beside a one-token sequence the 16-row edges, and 2048 / 2049 the switch.
@pytest.mark.parametrize("lengths", [[1], [2], [3], [4], [7], [8], [9], [15], [16], [17], [63],
                                     [64], [65], [127], [128], [129], [2048], [2049],
                                     [15, 1], [16, 1], [17, 1], [31, 1], [32, 1], [33, 1],
                                     [63, 1], [64, 1], [65, 1], [127, 1], [128, 1], [129, 1],
                                     [300, 700], [0, 5, 0], [1, 1, 1, 1, 1, 1, 1, 1, 1, 1],
                                     [200, 1, 64, 3]])
def test_chunk_edges(lengths):
    from helpers import make_workload

    wl = make_workload(lengths, dim=768, part_dim=256, seed=sum(lengths) + len(lengths),
                       row_stride=768 + 16, init=[i % 2 == 0 for i in range(len(lengths))])
    _compare(wl)


def test_many_sequences_three_search_levels():
    """More than 64^2 sequences: the program search takes three radix-64 levels."""
    from helpers import make_workload

    rng = np.random.default_rng(9)
    lens = rng.integers(0, 4, size=4200)
    wl = make_workload(lens, dim=64, part_dim=64, seed=9, lines=4300, activation=None, bias=False)
    _compare(wl)


@pytest.mark.parametrize("dim,part_dim", [(2304, 768), (4096, 1024), (6656, 1664), (8704, 4352)])
def test_xcd_chunk_order_and_split_tail(dim, part_dim):
    """Launches with at least 8 column groups take the XCD-chunked workgroup order; these
    dims give 9 groups of one wave, and 8, 13 and 17 groups of two waves (no remainder,
    remainders of 5 and 1), with a partial last chunk of programs and the launch's last
    row blocks split into half and quarter tiles. Padding rows follow the sequences."""
    from helpers import make_workload

    wl = make_workload([1500, 17, 250, 3], dim=dim, part_dim=part_dim, seed=dim, row_stride=dim + 64,
                       init=[True, False, True, True], pad_tokens=5)
    _compare(wl)


def test_dim_not_a_multiple_of_the_wave_width():
    from helpers import make_workload

    wl = make_workload([70, 5], dim=3 * 40, part_dim=40, seed=12, row_stride=128)
    _compare(wl)


@pytest.mark.parametrize("parts,part_dim", [(3, 200), (5, 40), (3, 192), (4, 112)])
def test_partial_last_column_block_with_states(parts, part_dim):
    """Several column blocks, the last one partial, every sequence starting from its
    stored state: lanes past the last channel must not disturb other lanes' outputs."""
    from helpers import make_workload

    wl = make_workload([1, 2, 3, 4, 70, 2], dim=parts * part_dim, part_dim=part_dim, seed=parts,
                       init=[True] * 6, lines=8, activation=None, bias=False)
    _compare(wl)


@pytest.mark.parametrize("activation", ["silu", None])
def test_tiles_full_of_non_finite_inputs(activation):
    """Rows of NaN and infinity make every element of their tiles need the exact
    path, far more than a wave's fixup list holds: those tiles recompute their words
    themselves. Outputs and states must still match the oracle word for word."""
    from helpers import make_workload

    wl = make_workload([40, 17, 70], dim=3 * 256, part_dim=256, seed=41, row_stride=768 + 64,
                       init=[True, False, True], activation=activation)
    specials = np.array([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x7F81], dtype=np.uint16)
    rng = np.random.default_rng(41)
    for r0, r1 in ((4, 30), (45, 50), (90, 127)):
        block = wl.x[r0:r1, : wl.dim]
        block[...] = specials[rng.integers(0, len(specials), size=block.shape)]
    _compare(wl)


def test_empty_calls_touch_nothing():
    import packed_varlen_causal_depthwise_amd as kd
    from helpers import make_workload

    wl = make_workload([0, 0], dim=64, part_dim=64, seed=13)
    got, st = run_hip(wl)
    assert np.all(got == CANARY)
    assert np.array_equal(st, wl.conv_states)
    d = to_device(wl)
    empty_q = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = kd.packed_causal_conv1d_fn(d["x"], d["weight"], d["bias"], d["conv_states"], empty_q,
                                     d["cache_indices"], d["has_initial_state"], 64, "silu", None)
    assert out.shape == (1, wl.num_tokens, 64)


def test_graph_replay_with_new_device_data():
    """Capture one call in a graph, then replay it on new token splits, lines and values
    of the same shapes; every replay matches the oracle for its data."""
    import packed_varlen_causal_depthwise_amd as kd
    from helpers import make_workload

    shape_wl = make_workload([100, 50, 30, 20], dim=512, part_dim=128, seed=20, lines=8)
    d = to_device(shape_wl)
    out = torch.empty((4, shape_wl.num_tokens, 128), dtype=torch.bfloat16, device="cuda")
    args = lambda: (d["x"], d["weight"], d["bias"], d["conv_states"], d["query_start_loc"],
                    d["cache_indices"], d["has_initial_state"], 128, "silu", None)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kd.packed_causal_conv1d_fn(*args(), out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kd.packed_causal_conv1d_fn(*args(), out=out)
    for trial, lens in enumerate([[150, 10, 30, 10], [1, 2, 3, 194], [200, 0, 0, 0]]):
        wl = make_workload(lens, dim=512, part_dim=128, seed=30 + trial, lines=8)
        nd = to_device(wl)
        for k in ("x", "weight", "bias", "conv_states", "query_start_loc", "cache_indices",
                  "has_initial_state"):
            d[k].copy_(nd[k])
        out.view(torch.int16).fill_(np.int16(np.uint16(CANARY).view(np.int16)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.view(torch.int16).cpu().numpy().view(np.uint16)
        want, want_st = oracle_with_canary(wl)
        assert np.array_equal(got, want), (trial, first_mismatches(got, want))
        assert np.array_equal(d["conv_states"].cpu().numpy(), want_st), trial
