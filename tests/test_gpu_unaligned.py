"""GPU parity for x and out that are not 16-byte aligned.

Page vllm.models.kimi_k3.nvidia.ops.kda_conv, packed_causal_conv1d_supported: x needs a
unit column stride and may have any row stride, so a Q|K|V slice may start at any
column of the in_proj output. Such x (and an out at any element offset) move through
the same 8- and 16-byte lane vectors as aligned ones, at addresses that are not
multiples of the vector size. Each case compares outputs and states with the
oracle word for word: ragged sequences over several tiles, every format, odd row
strides, the exact-SiLU path, the decode step with either state, and the 16384-token
workload read from a slice at column 1.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
import workloads
from gpu_util import (TORCH_DTYPE, canary_for, first_mismatches, oracle_with_canary, to_device,
                      torch_to_words, words_to_torch)
from helpers import make_workload

pytestmark = pytest.mark.gpu

_SIGNED = {np.uint16: np.int16, np.uint32: np.int32}


def _x_at_offset(wl, off: int) -> torch.Tensor:
    """wl.x's values in a device buffer whose columns start `off` elements in: the
    returned (T, dim) view is aligned to its element size only."""
    T, rs = wl.x.shape
    buf = np.zeros((T, rs + off), dtype=wl.x.dtype)
    buf[:, off:off + rs] = wl.x
    dev = torch.from_numpy(buf.view(_SIGNED[wl.x.dtype.type])).cuda().view(TORCH_DTYPE[wl.x_dtype])
    v = dev[:, off:off + wl.dim]
    assert v.data_ptr() % 16 != 0 or (v.stride(0) * v.element_size()) % 16 != 0
    return v


def _out_at_offset(shape, dtype, off: int) -> torch.Tensor:
    n = int(np.prod(shape))
    buf = torch.empty(n + off + 8, dtype=dtype, device="cuda")
    out = buf[off:off + n].view(shape)
    assert out.data_ptr() % 16 != 0 and out.is_contiguous()
    return out


def _run(wl, x, out=None):
    d = to_device(wl)
    P = wl.dim // wl.part_dim
    if out is None:
        out = torch.empty((P, wl.num_tokens, wl.part_dim), dtype=TORCH_DTYPE[wl.x_dtype],
                          device="cuda")
    fill = canary_for(wl.x_dtype)
    if out.element_size() == 4:
        out.view(torch.int32).fill_(int(np.uint32(fill).view(np.int32)))
    else:
        out.view(torch.int16).fill_(int(np.uint16(fill).view(np.int16)))
    kd.packed_causal_conv1d_fn(x, d["weight"], d["bias"], d["conv_states"], d["query_start_loc"],
                               d["cache_indices"], d["has_initial_state"], wl.part_dim,
                               wl.activation, wl.null_block_id, out=out)
    torch.cuda.synchronize()
    return torch_to_words(out), d["conv_states"].cpu().numpy()


def _check(wl, got, st):
    want, want_st = oracle_with_canary(wl)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


def _case(fmt, seed, x_scale=1.0, act="silu", row_stride=3 * 200 + 9):
    return make_workload([1, 2, 3, 40, 17, 0, 90, 300], dim=3 * 200, part_dim=200, seed=seed,
                         lines=12, x_dtype=fmt, row_stride=row_stride, x_scale=x_scale,
                         activation=act, init=[True, False, True, True, False, True, True, True],
                         null_block_id=None)


# Offsets that are a multiple of 4 elements keep 2-byte formats' 8-byte vectors aligned;
# the others, and every FP32 offset that is not a multiple of 4, make them unaligned.
@pytest.mark.parametrize("fmt,off", [("bf16", 1), ("bf16", 3), ("bf16", 4), ("bf16", 5),
                                     ("f16", 1), ("f16", 4), ("f16", 7), ("f32", 1), ("f32", 2),
                                     ("f32", 3)])
def test_x_at_a_column_offset(fmt, off):
    # the buffer's row pitch is row_stride + off: a multiple of 4 for offsets 4
    wl = _case(fmt, 200 + off, row_stride=604 if off % 4 == 0 else 609)
    print(f"case: x at column {off}, {fmt}", flush=True)
    got, st = _run(wl, _x_at_offset(wl, off))
    _check(wl, got, st)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_out_at_an_element_offset(fmt):
    wl = _case(fmt, 210)
    print(f"case: out at element 1, {fmt}", flush=True)
    d = to_device(wl)
    P = wl.dim // wl.part_dim
    out = _out_at_offset((P, wl.num_tokens, wl.part_dim), TORCH_DTYPE[fmt], 1)
    got, st = _run(wl, d["x"], out=out)
    _check(wl, got, st)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_both_unaligned_with_the_exact_path(fmt):
    """Accumulators scaled up so that many elements take the exact SiLU path (the list
    and, for whole tiles of them, the tile rewrite)."""
    wl = _case(fmt, 220, x_scale=40.0)
    print(f"case: x and out unaligned, exact path, {fmt}", flush=True)
    P = wl.dim // wl.part_dim
    out = _out_at_offset((P, wl.num_tokens, wl.part_dim), TORCH_DTYPE[fmt], 3)
    got, st = _run(wl, _x_at_offset(wl, 1), out=out)
    _check(wl, got, st)


def test_headline_workload_from_column_one():
    """16384 tokens x 4608 channels (rows of 9728) read from a slice starting at column 1."""
    wl = workloads.config3()
    print("case: 16384 x 4608 from column 1", flush=True)
    got, st = _run(wl, _x_at_offset(wl, 1))
    want, want_st = oracle.run_workload(wl)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_decode_unaligned(fmt):
    dim, pd, batch = 3 * 256, 256, 37
    wl = make_workload([1] * batch, dim=dim, part_dim=pd, seed=230, lines=batch + 6,
                       x_dtype=fmt, row_stride=dim + 5)
    print(f"case: decode, x at column 1 and out at element 1, {fmt}", flush=True)
    x = _x_at_offset(wl, 1)
    out = _out_at_offset((3, batch, pd), TORCH_DTYPE[fmt], 1)
    st_dev = torch.from_numpy(wl.conv_states.copy()).cuda()
    kd.packed_causal_conv1d_update(x, torch.from_numpy(wl.weight).cuda(),
                                   torch.from_numpy(wl.bias).cuda(), st_dev,
                                   torch.from_numpy(wl.cache_indices).cuda(), pd, "silu", None,
                                   out=out)
    torch.cuda.synchronize()
    got = torch_to_words(out)
    st = wl.conv_states.copy()
    want = oracle.packed_causal_conv1d_update(wl.x, dim, wl.weight, wl.bias, st, wl.cache_indices,
                                              pd, "silu", None, x_dtype=fmt)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st_dev.cpu().numpy().view(np.uint32), st.view(np.uint32))


def test_bf16_state_decode_unaligned():
    d = workloads.decode_batch_bf16_state(37, seed=231, dim=3 * 256, part_dim=256,
                                          row_stride=3 * 256 + 3, lines=43)
    print("case: bf16-state decode, x at column 1 and out at element 1", flush=True)
    T, rs = d.x.shape
    buf = np.zeros((T, rs + 1), dtype=np.uint16)
    buf[:, 1:] = d.x
    x = words_to_torch(buf, torch.bfloat16)[:, 1:1 + d.dim]
    out = _out_at_offset((3, 37, 256), torch.bfloat16, 1)
    st_dev = torch.from_numpy(d.conv_states.view(np.int16).copy()).cuda().view(torch.bfloat16)
    kd.packed_causal_conv1d_update(x, torch.from_numpy(d.weight).cuda(),
                                   torch.from_numpy(d.bias).cuda(), st_dev,
                                   torch.from_numpy(d.cache_indices).cuda(), 256, "silu", None,
                                   out=out)
    torch.cuda.synchronize()
    got = torch_to_words(out)
    st = d.conv_states.copy()
    want = oracle.packed_causal_conv1d_update_bf16_state(d.x, d.dim, d.weight, d.bias, st,
                                                         d.cache_indices, 256, "silu", None)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(torch_to_words(st_dev), st)


@pytest.mark.parametrize("seed", range(12))
def test_fuzz_unaligned(seed):
    """Seeded fuzz cases (zero-length sequences, null blocks, padding rows, several
    part_dim values, wide accumulator ranges) with x at a random column offset of its
    buffer and out at a random element offset, in every format."""
    fmt = ["bf16", "f16", "f32"][seed % 3]
    wl = workloads.random_case(3000 + seed, max_seqs=10, max_len=150, x_dtype=fmt,
                               x_scale=[1.0, 8.0, 40.0][(seed // 3) % 3], pad_tokens=seed % 3)
    rng = np.random.default_rng(seed)
    off_x, off_o = int(rng.integers(1, 8)), int(rng.integers(1, 8))
    print(f"case: {wl.name}, x at column {off_x}, out at element {off_o}", flush=True)
    P = wl.dim // wl.part_dim
    out = _out_at_offset((P, wl.num_tokens, wl.part_dim), TORCH_DTYPE[fmt], off_o)
    got, st = _run(wl, _x_at_offset(wl, off_x), out=out)
    _check(wl, got, st)


@pytest.mark.parametrize("batch", [300, 600])
@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_decode_unaligned_several_per_wave(fmt, batch):
    """Batches that give two (300) and four (600) sequences per wave at dim 4608 (18 column
    blocks, two waves per workgroup), x at column 3 of rows 9731 elements apart and out at
    element 1."""
    wl = workloads.decode_batch(batch, seed=240 + batch, x_dtype=fmt)
    print(f"case: decode, {batch} sequences, x at column 3, out at element 1, {fmt}", flush=True)
    x = _x_at_offset(wl, 3)
    out = _out_at_offset((3, batch, 1536), TORCH_DTYPE[fmt], 1)
    st_dev = torch.from_numpy(wl.conv_states.copy()).cuda()
    kd.packed_causal_conv1d_update(x, torch.from_numpy(wl.weight).cuda(),
                                   torch.from_numpy(wl.bias).cuda(), st_dev,
                                   torch.from_numpy(wl.cache_indices).cuda(), 1536, "silu", None,
                                   out=out)
    torch.cuda.synchronize()
    got = torch_to_words(out)
    st = wl.conv_states.copy()
    want = oracle.packed_causal_conv1d_update(wl.x, wl.dim, wl.weight, wl.bias, st,
                                              wl.cache_indices, 1536, "silu", None, x_dtype=fmt)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st_dev.cpu().numpy().view(np.uint32), st.view(np.uint32))


@pytest.mark.parametrize("batch", [300, 600])
def test_bf16_state_decode_unaligned_several_per_wave(batch):
    d = workloads.decode_batch_bf16_state(batch, seed=250 + batch)
    print(f"case: bf16-state decode, {batch} sequences, x at column 1, out at element 3",
          flush=True)
    T, rs = d.x.shape
    buf = np.zeros((T, rs + 1), dtype=np.uint16)
    buf[:, 1:] = d.x
    x = words_to_torch(buf, torch.bfloat16)[:, 1:1 + d.dim]
    out = _out_at_offset((3, batch, 1536), torch.bfloat16, 3)
    st_dev = torch.from_numpy(d.conv_states.view(np.int16).copy()).cuda().view(torch.bfloat16)
    kd.packed_causal_conv1d_update(x, torch.from_numpy(d.weight).cuda(),
                                   torch.from_numpy(d.bias).cuda(), st_dev,
                                   torch.from_numpy(d.cache_indices).cuda(), 1536, "silu", None,
                                   out=out)
    torch.cuda.synchronize()
    got = torch_to_words(out)
    st = d.conv_states.copy()
    want = oracle.packed_causal_conv1d_update_bf16_state(d.x, d.dim, d.weight, d.bias, st,
                                                         d.cache_indices, 1536, "silu", None)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(torch_to_words(st_dev), st)
