"""GPU parity for fp16 and FP32 x: the HIP path against the CPU oracle, bit for bit.

Page: vllm.models.kimi_k3.nvidia.ops.kda_conv. packed_causal_conv1d_supported
admits bf16, fp16 and FP32 x; the output takes x's dtype and the arithmetic is
FP32 for every input dtype. Output words (fp16 or FP32) and the updated FP32
state must equal the oracle's on the named workloads at full size, fuzz cases,
tile edges and tiles of non-finite inputs; for FP32 with SiLU also on
accumulators whose exp lies closest to a binary32 rounding boundary (the exp
certificate's list), where the kernel takes its double-double path. The
activation-and-rounding map of each format is compared on all 2^32 inputs.
"""

import os
import pathlib
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
import workloads
from gpu_util import first_mismatches, oracle_with_canary, run_hip

pytestmark = pytest.mark.gpu

FORMATS = ["f16", "f32"]
GOLDEN = pathlib.Path(__file__).resolve().parent / "golden" / "expf_escalations.txt"


def _compare(wl):
    print(f"case: {wl.name} x {wl.x_dtype}", flush=True)
    got, st = run_hip(wl)
    want, want_st = oracle_with_canary(wl)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32)), \
        first_mismatches(st.view(np.uint32), want_st.view(np.uint32))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_named_workloads_bit_exact(cfg, fmt):
    _compare(workloads.CONFIGS[cfg](x_dtype=fmt))


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("seed", range(10))
def test_fuzz_bit_exact(seed, fmt):
    # fp16 inputs of scale 40 keep |x| far below the fp16 range; the FP32 output
    # of such accumulators still spans every SiLU regime.
    wl = workloads.random_case(2000 + seed, max_seqs=12, max_len=300,
                               x_scale=[1.0, 8.0, 40.0][seed % 3], pad_tokens=seed % 4,
                               x_dtype=fmt)
    _compare(wl)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("lengths", [[1], [3], [7], [8], [9], [15], [16], [17], [33],
                                     [0, 5, 0], [1, 1, 1, 1, 1, 1, 1, 1, 1, 1], [200, 1, 64, 3]])
def test_tile_edges(lengths, fmt):
    from helpers import make_workload

    wl = make_workload(lengths, dim=768, part_dim=256, seed=sum(lengths) + len(lengths),
                       row_stride=768 + 16, init=[i % 2 == 0 for i in range(len(lengths))],
                       x_dtype=fmt)
    _compare(wl)


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("parts,part_dim", [(3, 200), (5, 40)])
def test_partial_last_column_block_with_states(parts, part_dim, fmt):
    from helpers import make_workload

    wl = make_workload([1, 2, 3, 4, 70, 2], dim=parts * part_dim, part_dim=part_dim, seed=parts,
                       init=[True] * 6, lines=8, activation=None, bias=False, x_dtype=fmt,
                       row_stride=parts * part_dim + 8)
    _compare(wl)


SPECIALS = {
    # quiet NaN, negative NaN with payload, +-inf, signalling NaN
    "f16": np.array([0x7E00, 0xFE01, 0x7C00, 0xFC00, 0x7C01], dtype=np.uint16),
    "f32": np.array([0x7FC00000, 0xFFC00001, 0x7F800000, 0xFF800000, 0x7F800001], dtype=np.uint32),
}


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("activation", ["silu", None])
def test_tiles_full_of_non_finite_inputs(activation, fmt):
    """Every element of these tiles needs the exact path (NaN and infinite
    accumulators); the state must hold the widened specials (fp16: quieted)."""
    from helpers import make_workload

    wl = make_workload([40, 17, 70], dim=3 * 256, part_dim=256, seed=41, row_stride=768 + 64,
                       init=[True, False, True], activation=activation, x_dtype=fmt)
    rng = np.random.default_rng(41)
    for r0, r1 in ((4, 30), (45, 50), (90, 127)):
        block = wl.x[r0:r1, : wl.dim]
        block[...] = SPECIALS[fmt][rng.integers(0, len(SPECIALS[fmt]), size=block.shape)]
    _compare(wl)


@pytest.mark.parametrize("fmt", FORMATS)
def test_fp16_range_edges(fmt):
    """Accumulators around the fp16 overflow (65504, the 65520 tie) and in the fp16
    subnormal range, for both activations: unit current tap, no bias."""
    from helpers import make_workload

    vals = np.array([65504.0, 65519.0, 65520.0, 65536.0, -65520.0, 1e-5, -3e-6, 6.0e-8,
                     2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, 1e-3, -7.4, -7.6, 17.0, 88.0],
                    dtype=np.float32)
    for act in ("silu", None):
        wl = make_workload([64], dim=256, part_dim=256, seed=5, activation=act, bias=False,
                           init=[False], x_dtype="f32")
        wl.weight[:] = 0.0
        wl.weight[:, 3] = 1.0
        rng = np.random.default_rng(5)
        xv = vals[rng.integers(0, len(vals), size=(64, 256))]
        if fmt == "f16":
            # fp16 x cannot hold these; scale through the tap instead
            wl.x_dtype = "f16"
            wl.x = np.full((64, 256), 0x3C00, dtype=np.uint16)  # 1.0
            wl.weight[:, 3] = xv[0]
        else:
            wl.x = xv.view(np.uint32).copy()
        _compare(wl)


def test_f32_silu_on_hard_exp_arguments():
    """Accumulators a whose exp(-a) sits closest to a binary32 rounding boundary:
    the kernel's double exp is not trusted there and its double-double path must
    give the correctly rounded exp. Whole tiles of them also overflow the wave's
    fixup list."""
    from helpers import make_workload

    rows = [ln.split()[0] for ln in GOLDEN.read_text().splitlines() if ln and ln[0] != "#"]
    hard = np.array([int(u, 16) ^ 0x80000000 for u in rows], dtype=np.uint32)
    hard = hard[np.abs(hard.view(np.float32)) < 104.0]
    T, dim = 64, 768
    wl = make_workload([T], dim=dim, part_dim=256, seed=6, activation="silu", bias=False,
                       init=[False], x_dtype="f32")
    wl.weight[:] = 0.0
    wl.weight[:, 3] = 1.0
    reps = np.resize(hard, T * dim).reshape(T, dim)
    wl.x = reps.copy()
    _compare(wl)


CHUNK = 1 << 27


@pytest.mark.parametrize("fmt", FORMATS)
@pytest.mark.parametrize("act", ["silu", None])
def test_activation_map_all_fp32_inputs(act, fmt):
    lib = oracle.load()
    silu = act == "silu"
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    sub = CHUNK // threads
    wdt = torch.int32 if fmt == "f32" else torch.int16
    buf = torch.empty(CHUNK, dtype=wdt, device="cuda")
    ref = np.empty(CHUNK, dtype=oracle.WORD_DTYPE[fmt])
    bad = []
    nbad = 0
    with ThreadPoolExecutor(threads) as ex:
        for first in range(0, 1 << 32, CHUNK):
            kd.activation_map(first, CHUNK, act, out=buf, fmt=fmt)
            futs = [ex.submit(oracle.act_words_range, first + i * sub, sub, silu, fmt, lib,
                              ref[i * sub:(i + 1) * sub]) for i in range(threads)]
            got = buf.cpu().numpy().view(ref.dtype)
            for f in futs:
                f.result()
            diff = np.nonzero(got != ref)[0]
            nbad += diff.size
            for i in diff[: max(0, 8 - len(bad))]:
                bad.append((hex(first + int(i)), hex(int(got[i])), hex(int(ref[i]))))
    print(f"activation {act} {fmt}: {nbad} mismatches", flush=True)
    assert nbad == 0, bad
