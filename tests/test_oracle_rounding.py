"""Pins for the oracle's bf16 <-> FP32 conversions.

Page: vllm.models.kimi_k3.nvidia.ops.kda_conv, module docstring (second
paragraph): bf16 -> FP32 is exact and FP32 -> bf16 rounds to nearest even, as
torch's ``.to(bfloat16)`` does. The library routine that statement names is the
pin: torch's CPU conversion, over every high half-word with a spread of low
half-words, and over one exhaustive block of 2^26 consecutive patterns. NaN is the
one place torch's own paths disagree (its scalar routine gives 0x7FC0, its vector
routine 0xFFFF); the oracle's reading is 0x7FC0, checked on its own.
"""

import numpy as np
import pytest
import torch

import exact
import oracle


def _torch_bf16(u32: np.ndarray) -> np.ndarray:
    f = torch.from_numpy(np.ascontiguousarray(u32).view(np.float32))
    return f.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _oracle_identity(u32: np.ndarray, olib) -> np.ndarray:
    return oracle.act_bf16(u32.view(np.float32), False, lib=olib)


def test_bf16_round_every_high_half(olib):
    rng = np.random.default_rng(11)
    lows = np.concatenate([np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32),
                           rng.integers(0, 1 << 16, size=10).astype(np.uint32)])
    highs = np.arange(1 << 16, dtype=np.uint32)
    u = (highs[:, None] << np.uint32(16) | lows[None, :]).ravel()
    got = _oracle_identity(u, olib)
    ref = _torch_bf16(u)
    isnan = np.isnan(u.view(np.float32))
    assert np.array_equal(got[~isnan], ref[~isnan])
    assert np.all(got[isnan] == 0x7FC0)


def test_bf16_round_exhaustive_block(olib):
    first = 0x3F000000  # eight whole binades, from 0.5 up to 128
    n = 1 << 26
    u = np.arange(n, dtype=np.uint32) + np.uint32(first)
    got = oracle.act_bf16_range(first, n, False, lib=olib)
    assert np.array_equal(got, _torch_bf16(u))


@pytest.mark.parametrize("u", [0x00000000, 0x80000000, 0x00000001, 0x00008000, 0x00018000,
                               0x007FFFFF, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0xFF7F8000,
                               0x7F800000, 0xFF800000, 0x3F808000, 0x3F818000, 0xBF808001])
def test_bf16_round_closed_forms(olib, u):
    """Each pattern against exact rational rounding to 8 significant bits."""
    y = exact.from_bits32(u)
    assert olib.oracle_f32_to_bf16(y) == exact.bf16_word(y)


def test_bf16_nan_reading(olib):
    for u in (0x7FC00000, 0xFFC00000, 0x7F800001, 0x7FFFFFFF, 0xFF812345):
        assert olib.oracle_f32_to_bf16(exact.from_bits32(u)) == 0x7FC0


def test_bf16_widen_is_exact(olib):
    h = np.arange(1 << 16, dtype=np.uint32)
    ref = torch.from_numpy((h.astype(np.uint16)).view(np.int16)).view(torch.bfloat16).float()
    ref = ref.numpy().view(np.uint32)
    got = np.array([exact.bits32(olib.oracle_bf16_to_f32(int(v))) for v in h[::257]],
                   dtype=np.uint32)
    assert np.array_equal(got, ref[::257])
    assert np.array_equal(ref[~np.isnan(ref.view(np.float32))] >> 16,
                          h[~np.isnan(ref.view(np.float32))])
