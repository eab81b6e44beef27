"""Seeded synthetic inputs for the packed varlen causal depthwise convolution.

This module only draws inputs. It holds none of the convolution's arithmetic and
is shared by the tests, the bench and the smoke check, which hand the same arrays
both to the CPU oracle and to the HIP path.

Every array comes from ``numpy.random.Generator(PCG64(seed))`` in a fixed order
of draws, so a (config, seed) pair gives the same bytes on every host. Float
inputs are drawn as float32 and rounded to x's format (bfloat16 by the helper
below, float16 by numpy's conversion, both to nearest even; float32 as drawn),
which is input preparation, not the method. The x format changes no draw.

Shapes follow the workloads the kda_conv page talks about (vllm.models.kimi_k3.
nvidia.ops.kda_conv, the ``_config`` comment: 2K-16K tokens x 3 x 1536 packed
Q|K|V channels read in place from the in_proj output) and the five named
configurations listed in ``CONFIGS``.
"""

from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

#: bf16 quiet NaN written into the x columns the op must never read (canary).
BF16_CANARY = 0x7FC0
#: The same canary for the other x formats (a quiet NaN of each).
CANARIES = {"bf16": 0x7FC0, "f16": 0x7E00, "f32": 0x7FC00000}
#: numpy dtype of the raw words of each x format, and bytes per element.
WORD_DTYPE = {"bf16": np.uint16, "f16": np.uint16, "f32": np.uint32}
ELEMENT_BYTES = {"bf16": 2, "f16": 2, "f32": 4}

#: Row stride (elements) of the in_proj output the Q|K|V columns live in.
IN_PROJ_ROW_STRIDE = 9728


@dataclasses.dataclass
class Workload:
    """One call's worth of host inputs.

    ``x`` is the whole row-strided buffer, shape ``(num_tokens, row_stride)``,
    stored as raw words of format ``x_dtype`` (uint16 bit patterns for "bf16" and
    "f16", uint32 for "f32"); the op reads its first ``dim`` columns. The output
    has the same format.
    """

    name: str
    x: np.ndarray  # raw words (T, row_stride)
    dim: int
    weight: np.ndarray  # float32 (dim, 4) [channel, tap]
    bias: Optional[np.ndarray]  # float32 (dim,) or None
    conv_states: np.ndarray  # float32 (lines, dim, 3)
    query_start_loc: np.ndarray  # int32 (S + 1,)
    cache_indices: np.ndarray  # int32 (S,)
    has_initial_state: np.ndarray  # bool (S,)
    part_dim: int
    activation: Optional[str]  # "silu" or None
    null_block_id: Optional[int]
    x_dtype: str = "bf16"  # "bf16", "f16" or "f32"

    @property
    def num_tokens(self) -> int:
        return int(self.x.shape[0])

    @property
    def num_seqs(self) -> int:
        return int(self.query_start_loc.shape[0]) - 1

    @property
    def row_stride(self) -> int:
        return int(self.x.shape[1])

    @property
    def num_cache_lines(self) -> int:
        return int(self.conv_states.shape[0])

    def algorithmic_bytes(self) -> int:
        """Bytes the operation must move (no halo re-reads, no slack work).

        x read and out written once (2 B each per element for bf16 and fp16,
        4 B for FP32), 12 B of state per
        channel read for every sequence that starts from its stored state and
        written for every live non-empty sequence, the weight (16 B per channel),
        the bias (4 B per channel) and the per-sequence metadata.
        """
        qsl = self.query_start_loc.astype(np.int64)
        lens = qsl[1:] - qsl[:-1]
        live = np.ones(self.num_seqs, dtype=bool)
        if self.null_block_id is not None:
            live &= self.cache_indices != self.null_block_id
        reads_state = live & self.has_initial_state
        writes_state = live & (lens > 0)
        tokens = int(qsl[-1]) if self.num_seqs > 0 else 0
        b = tokens * self.dim * ELEMENT_BYTES[self.x_dtype] * 2
        b += 12 * self.dim * int(reads_state.sum())
        b += 12 * self.dim * int(writes_state.sum())
        b += 16 * self.dim
        if self.bias is not None:
            b += 4 * self.dim
        b += 4 * (self.num_seqs + 1) + 4 * self.num_seqs + self.num_seqs
        return b


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round finite float32 values to bfloat16 bit patterns (nearest, ties to even)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + r) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_words(a: np.ndarray, x_dtype: str) -> np.ndarray:
    """Finite float32 values as raw words of ``x_dtype`` (nearest, ties to even)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if x_dtype == "bf16":
        return f32_to_bf16_bits(a)
    if x_dtype == "f16":
        return a.astype(np.float16).view(np.uint16)
    if x_dtype == "f32":
        return a.view(np.uint32).copy()
    raise ValueError(f"unknown x format {x_dtype!r}")


def words_to_f32(h: np.ndarray, x_dtype: str) -> np.ndarray:
    """Raw words of ``x_dtype`` widened to float32 (exact for numbers)."""
    if x_dtype == "bf16":
        return bf16_bits_to_f32(h)
    if x_dtype == "f16":
        return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float32)
    if x_dtype == "f32":
        return np.asarray(h, dtype=np.uint32).view(np.float32).copy()
    raise ValueError(f"unknown x format {x_dtype!r}")


def _x_buffer(rng: np.random.Generator, tokens: int, dim: int, row_stride: int,
              scale: float = 1.0, x_dtype: str = "bf16") -> np.ndarray:
    vals = rng.standard_normal((tokens, dim), dtype=np.float32)
    if scale != 1.0:
        vals *= np.float32(scale)
    x = np.full((tokens, row_stride), CANARIES[x_dtype], dtype=WORD_DTYPE[x_dtype])
    x[:, :dim] = f32_to_words(vals, x_dtype)
    return x


def _normal(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    return (rng.standard_normal(shape, dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def _qsl(lengths: np.ndarray) -> np.ndarray:
    q = np.zeros(len(lengths) + 1, dtype=np.int64)
    np.cumsum(lengths, out=q[1:])
    return q.astype(np.int32)


def config1(seed: int = 1, x_dtype: str = "bf16") -> Workload:
    """1 sequence of 64 tokens, dim 384 as 3 planes of 128, contiguous x, zero state, no init."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, dim = 64, 384
    x = _x_buffer(rng, T, dim, dim, x_dtype=x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = np.zeros((1, dim, 3), dtype=np.float32)
    return Workload("config1: 1 x 64 tokens, dim 384, part_dim 128", x, dim, w, b, st,
                    _qsl(np.array([T])), np.array([0], dtype=np.int32),
                    np.array([False]), 128, "silu", None, x_dtype)


def config2(seed: int = 2, x_dtype: str = "bf16") -> Workload:
    """8 sequences of 1-300 tokens, dim 4608 (3 x 1536) in rows of 9728, 4 with initial state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dim, S, lines = 4608, 8, 64
    lens = rng.integers(1, 300, size=S, endpoint=True)
    T = int(lens.sum())
    x = _x_buffer(rng, T, dim, IN_PROJ_ROW_STRIDE, x_dtype=x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = _normal(rng, (lines, dim, 3), 1.0)
    ci = rng.permutation(lines)[:S].astype(np.int32)
    init = np.zeros(S, dtype=bool)
    init[rng.choice(S, size=4, replace=False)] = True
    return Workload("config2: 8 seqs of 1-300 tokens, dim 4608, part_dim 1536, stride 9728",
                    x, dim, w, b, st, _qsl(lens), ci, init, 1536, "silu", None, x_dtype)


def config3(seed: int = 3, x_dtype: str = "bf16") -> Workload:
    """1 sequence of 16384 tokens, dim 4608 (3 x 1536) in rows of 9728, initial state."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, dim, lines = 16384, 4608, 8
    x = _x_buffer(rng, T, dim, IN_PROJ_ROW_STRIDE, x_dtype=x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = _normal(rng, (lines, dim, 3), 1.0)
    ci = np.array([rng.integers(lines)], dtype=np.int32)
    return Workload("config3: 1 x 16384 tokens, dim 4608, part_dim 1536, stride 9728",
                    x, dim, w, b, st, _qsl(np.array([T])), ci, np.array([True]), 1536,
                    "silu", None, x_dtype)


def lognormal_lengths(rng: np.random.Generator, count: int, total: int,
                      sigma: float = 1.0) -> np.ndarray:
    """``count`` lengths >= 1 summing to ``total``: log-normal shares, largest remainder."""
    raw = rng.lognormal(mean=0.0, sigma=sigma, size=count)
    spare = total - count
    share = raw / raw.sum() * spare
    base = np.floor(share).astype(np.int64)
    rem = spare - int(base.sum())
    order = np.argsort(-(share - base), kind="stable")
    base[order[:rem]] += 1
    return base + 1


def config4(seed: int = 4, x_dtype: str = "bf16") -> Workload:
    """64 sequences, log-normal lengths plus 1, 2, 3 (16384 tokens), a null-block sequence."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dim, S, lines, T = 4608, 64, 256, 16384
    lens = np.concatenate([lognormal_lengths(rng, S - 3, T - 6), np.array([1, 2, 3])])
    lens = lens[rng.permutation(S)]
    x = _x_buffer(rng, T, dim, IN_PROJ_ROW_STRIDE, x_dtype=x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = _normal(rng, (lines, dim, 3), 1.0)
    null_seq = int(rng.integers(S))
    others = (rng.permutation(lines - 1)[: S - 1] + 1).astype(np.int32)
    ci = np.empty(S, dtype=np.int32)
    ci[null_seq] = 0
    ci[np.arange(S) != null_seq] = others
    init = np.zeros(S, dtype=bool)
    init[rng.choice(S, size=48, replace=False)] = True
    return Workload("config4: 64 log-normal seqs (16384 tokens), null block 0, stride 9728",
                    x, dim, w, b, st, _qsl(lens), ci, init, 1536, "silu", 0, x_dtype)


def config5(seed: int = 5, x_dtype: str = "bf16") -> Workload:
    """4096 sequences of 1-4 tokens, dim 576 as 3 planes of 192, no bias, no activation."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dim, S, lines = 576, 4096, 8192
    lens = rng.integers(1, 4, size=S, endpoint=True)
    T = int(lens.sum())
    x = _x_buffer(rng, T, dim, dim, x_dtype=x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    st = _normal(rng, (lines, dim, 3), 1.0)
    ci = rng.permutation(lines)[:S].astype(np.int32)
    init = np.ones(S, dtype=bool)
    return Workload("config5: 4096 seqs of 1-4 tokens, dim 576, part_dim 192, no bias, no act",
                    x, dim, w, None, st, _qsl(lens), ci, init, 192, None, None, x_dtype)


def decode_batch(batch: int = 256, seed: int = 6, x_dtype: str = "bf16") -> Workload:
    """A decode step: ``batch`` sequences of one token each, dim 4608 (3 x 1536) in rows
    of 9728, every sequence continuing from its own stored line (max(1024, batch)
    lines), bias, SiLU.
    As a Workload its offsets are 0, 1, ..., batch and every initial-state flag is set,
    which is what the decode entry point computes."""
    rng = np.random.Generator(np.random.PCG64(seed))
    dim, lines = 4608, max(1024, batch)  # one distinct line per sequence
    x = _x_buffer(rng, batch, dim, IN_PROJ_ROW_STRIDE, x_dtype=x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = _normal(rng, (lines, dim, 3), 1.0)
    ci = rng.permutation(lines)[:batch].astype(np.int32)
    return Workload(f"decode: {batch} sequences x 1 token, dim 4608, part_dim 1536, stride 9728",
                    x, dim, w, b, st, _qsl(np.ones(batch, dtype=np.int64)), ci,
                    np.ones(batch, dtype=bool), 1536, "silu", None, x_dtype)


@dataclasses.dataclass
class Bf16StateDecode:
    """One decode step with the operands of the fused decode kernel on page
    vllm.models.kimi_k3.amd.ops.kda_decode: bf16 x, a bf16 conv state and the FP32
    weight mirrored width-major, ``(dim // part_dim, 4, part_dim)`` [part, width,
    channel]. Row b of ``x`` (raw bf16 words, ``(batch, row_stride)``) is the one token
    of sequence b; ``conv_states`` holds raw bf16 words ``(lines, dim, 3)``."""

    name: str
    x: np.ndarray
    dim: int
    weight: np.ndarray  # float32 (parts, 4, part_dim)
    bias: Optional[np.ndarray]
    conv_states: np.ndarray  # uint16 (lines, dim, 3)
    cache_indices: np.ndarray  # int32 (batch,)
    part_dim: int
    activation: Optional[str]
    null_block_id: Optional[int]

    @property
    def batch(self) -> int:
        return int(self.x.shape[0])

    @property
    def num_cache_lines(self) -> int:
        return int(self.conv_states.shape[0])

    def algorithmic_bytes(self) -> int:
        """x read and out written (2 B per element each), 6 B of state per channel read
        and written for every live sequence, the weight (16 B per channel), the bias
        (4 B per channel) and the cache indices."""
        ci = self.cache_indices.astype(np.int64)
        live = (ci >= 0) & (ci < self.num_cache_lines)
        if self.null_block_id is not None:
            live &= ci != self.null_block_id
        b = 4 * self.batch * self.dim + 12 * self.dim * int(live.sum()) + 16 * self.dim
        if self.bias is not None:
            b += 4 * self.dim
        return b + 4 * self.batch


def width_major(weight: np.ndarray, part_dim: int) -> np.ndarray:
    """A (dim, 4) [channel, width] weight rearranged as (dim // part_dim, 4, part_dim)
    [part, width, channel] (page vllm.models.kimi_k3.amd.ops.kda_decode,
    make_decode_conv1d_weight_loader: the decode kernel's copy of the weight)."""
    dim = weight.shape[0]
    return np.ascontiguousarray(weight.reshape(dim // part_dim, part_dim, 4).transpose(0, 2, 1))


def decode_batch_bf16_state(batch: int = 256, seed: int = 8, dim: int = 4608,
                            part_dim: int = 1536, row_stride: int = IN_PROJ_ROW_STRIDE,
                            lines: Optional[int] = None,
                            null_block_id: Optional[int] = None) -> Bf16StateDecode:
    """A decode step of ``batch`` sequences with the decode kernel's operands: dim 4608
    = 3 x 1536 bf16 x in rows of 9728, bias, SiLU, a bf16 state of max(1024, batch)
    lines drawn N(0, 1) and rounded to bf16, distinct random lines."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lines = lines or max(1024, batch)
    x = _x_buffer(rng, batch, dim, row_stride)
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = f32_to_bf16_bits(_normal(rng, (lines, dim, 3), 1.0))
    ci = rng.permutation(lines)[:batch].astype(np.int32)
    return Bf16StateDecode(f"decode, bf16 state: {batch} sequences x 1 token, dim {dim}, "
                           f"part_dim {part_dim}, stride {row_stride}",
                           x, dim, width_major(w, part_dim), b, st, ci, part_dim, "silu",
                           null_block_id)


def large_output_case(seed: int = 7) -> Workload:
    """An output of 2.4 GB, beyond the 2 GiB a single launch addresses: 262144 tokens,
    dim 4608 = 3 x 1536 contiguous (x is 2.4 GB as well), six sequences including lengths
    1, 2 and 3, eight lines, mixed initial-state flags, bias, SiLU.

    x is drawn as raw bf16 words (uniform random sign, exponent in [120, 127], mantissa
    bits), i.e. magnitudes in [2^-7, 2), which is far cheaper than 1.2e9 normal draws;
    every row differs, so a misplaced row offset shows."""
    rng = np.random.Generator(np.random.PCG64(seed))
    T, dim, lines = 262144, 4608, 8
    raw = rng.integers(0, 1 << 16, size=(T, dim), dtype=np.uint16)
    np.bitwise_and(raw, np.uint16(0x83FF), out=raw)
    np.bitwise_xor(raw, np.uint16(0x3C00), out=raw)
    lens = np.array([100003, 1, 2, 3, 62135, 100000])
    assert int(lens.sum()) == T
    w = _normal(rng, (dim, 4), 0.5)
    b = _normal(rng, (dim,), 0.1)
    st = _normal(rng, (lines, dim, 3), 1.0)
    ci = rng.permutation(lines)[: len(lens)].astype(np.int32)
    init = np.array([True, False, True, True, False, True])
    return Workload("large output: 262144 tokens x 4608 channels, 6 seqs, contiguous",
                    raw, dim, w, b, st, _qsl(lens), ci, init, 1536, "silu", None)


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


def random_case(seed: int, *, max_seqs: int = 12, max_len: int = 200, parts: int = 3,
                part_dim: Optional[int] = None, x_scale: float = 1.0,
                allow_empty: bool = True, pad_tokens: int = 0,
                row_pad: Optional[int] = None, x_dtype: str = "bf16") -> Workload:
    """Random fuzz case: zero-length sequences, null block, strides, padding rows.

    ``x_scale`` widens the accumulator range so that large negative and positive
    SiLU arguments appear; ``pad_tokens`` appends rows after the last sequence
    that no sequence owns.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    S = int(rng.integers(1, max_seqs, endpoint=True))
    lo = 0 if allow_empty else 1
    lens = rng.integers(lo, max_len, size=S, endpoint=True)
    if allow_empty and S > 1:
        lens[rng.random(S) < 0.2] = 0
    if part_dim is None:
        part_dim = int(rng.choice([8, 16, 64, 72, 128, 192, 256, 520]))
    dim = parts * part_dim
    if row_pad is None:
        row_pad = int(rng.choice([0, 8, 64, 5136]))
    row_stride = dim + row_pad
    T = int(lens.sum()) + pad_tokens
    x = _x_buffer(rng, T, dim, row_stride, x_scale, x_dtype)
    w = _normal(rng, (dim, 4), 0.5)
    has_bias = bool(rng.integers(2))
    b = _normal(rng, (dim,), 0.1) if has_bias else None
    lines = S + int(rng.integers(1, 5))
    st = _normal(rng, (lines, dim, 3), float(x_scale))
    ci = rng.permutation(lines)[:S].astype(np.int32)
    init = rng.random(S) < 0.6
    null_id = None
    if bool(rng.integers(2)):
        null_id = int(ci[int(rng.integers(S))])
    act = "silu" if bool(rng.integers(4)) else None
    fmt = "" if x_dtype == "bf16" else f" x {x_dtype}"
    return Workload(f"random seed {seed}: S={S} dim={dim} pd={part_dim} stride={row_stride}{fmt}",
                    x, dim, w, b, st, _qsl(lens), ci, init, part_dim, act,
                    null_id, x_dtype)
