"""Seeded fuzz over every argument form the ABI accepts, drawn together.

Page vllm.models.kimi_k3.nvidia.ops.kda_conv (packed_causal_conv1d_fn: the launch passes
both weight strides, the cache_indices stride and the three state strides, x at any row
stride with unit column stride; packed_causal_conv1d_supported: bf16, fp16 or FP32 x,
size(2) >= 3) and page vllm.models.kimi_k3.amd.ops.kda_decode (the decode step, the bf16
state and the width-major weight). The other GPU tests vary one form at a time; here each
seed draws all of them at once: the x format, sequence counts and lengths (zero-length
sequences, padding rows), accumulator range, x at a column offset of its buffer, out at an
element offset, the weight as a transposed or padded view, the bias at a 4-byte offset,
the state dim-first, padded or wider than 3, strided cache_indices, no initial-state
array, a null block and either activation; for the decode step also the batch size (one,
two or four sequences per wave), the state format and the weight form. Outputs, updated
state entries and every entry the call must leave alone are compared with the oracle
word for word. The oracle takes the same values in contiguous arrays.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
import workloads
from gpu_util import (TORCH_DTYPE, canary_for, first_mismatches, oracle_with_canary,
                      torch_to_words, words_to_torch)
from helpers import make_workload

pytestmark = pytest.mark.gpu

_SIGNED = {np.uint16: np.int16, np.uint32: np.int32}


def _pick(rng, options):
    return options[int(rng.integers(len(options)))]


def _x_view(words: np.ndarray, fmt: str, dim: int, off: int) -> torch.Tensor:
    """The (T, dim) view of x whose columns start `off` elements into a device buffer with
    rows of row_stride + off elements."""
    T, rs = words.shape
    buf = np.zeros((T, rs + off), dtype=words.dtype)
    buf[:, off:off + rs] = words
    dev = torch.from_numpy(buf.view(_SIGNED[words.dtype.type])).cuda().view(TORCH_DTYPE[fmt])
    return dev[:, off:off + dim]


def _out_view(shape, fmt: str, off: int) -> torch.Tensor:
    """A contiguous output at element offset `off` of its buffer, filled with the canary."""
    n = int(np.prod(shape))
    dt = TORCH_DTYPE[fmt]
    buf = torch.empty(n + off + 8, dtype=dt, device="cuda")
    fill = canary_for(fmt)
    if buf.element_size() == 4:
        buf.view(torch.int32).fill_(int(np.uint32(fill).view(np.int32)))
    else:
        buf.view(torch.int16).fill_(int(np.uint16(fill).view(np.int16)))
    return buf[off:off + n].view(shape)


def _weight_view(weight: np.ndarray, form: str) -> torch.Tensor:
    dim = weight.shape[0]
    if form == "transposed":
        return torch.from_numpy(np.ascontiguousarray(weight.T)).cuda().t()
    if form == "padded":
        buf = torch.full((dim, 7), 1e30, dtype=torch.float32, device="cuda")
        buf[:, 2:6] = torch.from_numpy(weight).cuda()
        return buf[:, 2:6]
    return torch.from_numpy(weight).cuda()


def _bias_view(bias, form: str):
    if bias is None:
        return None
    if form == "offset":
        buf = torch.empty(bias.shape[0] + 1, dtype=torch.float32, device="cuda")
        b = buf[1:]
        b.copy_(torch.from_numpy(bias))
        return b
    return torch.from_numpy(bias).cuda()


def _indices_view(ci: np.ndarray, lines: int, form: str) -> torch.Tensor:
    if form == "strided":
        inter = np.empty(2 * ci.shape[0], dtype=np.int32)
        inter[0::2] = ci
        inter[1::2] = (ci + 1) % lines
        return torch.from_numpy(inter).cuda()[::2]
    return torch.from_numpy(ci).cuda()


def _state_view(st: np.ndarray, form: str, rng):
    """(device buffer, (lines, dim, 3) view of it, reader of the logical entries, reader of
    the entries the call must not touch) for an FP32 state in layout `form`."""
    lines, dim, _ = st.shape
    if form == "dim_first":
        buf = torch.from_numpy(np.ascontiguousarray(st.transpose(0, 2, 1))).cuda()
        return buf, buf.transpose(1, 2), lambda a: a.transpose(0, 2, 1), lambda a: a[:, :, :0]
    if form == "dim_first_padded":
        host = rng.standard_normal((lines, 3, dim + 72)).astype(np.float32)
        host[:, :, :dim] = st.transpose(0, 2, 1)
        buf = torch.from_numpy(host).cuda()
        return (buf, buf[:, :, :dim].transpose(1, 2),
                lambda a: a[:, :, :dim].transpose(0, 2, 1), lambda a: a[:, :, dim:])
    if form == "wide5":
        host = rng.standard_normal((lines, dim, 5)).astype(np.float32)
        host[:, :, :3] = st
        buf = torch.from_numpy(host).cuda()
        return buf, buf, lambda a: a[:, :, :3], lambda a: a[:, :, 3:]
    buf = torch.from_numpy(st.copy()).cuda()
    return buf, buf, lambda a: a, lambda a: a[:, :, :0]


def _same_words(got: np.ndarray, want: np.ndarray, what: str):
    g = np.ascontiguousarray(got).view(np.uint32)
    w = np.ascontiguousarray(want).view(np.uint32)
    assert np.array_equal(g, w), (what, first_mismatches(g, w))


def prefill_case(seed: int) -> str:
    rng = np.random.default_rng(10_000 + seed)
    fmt = _pick(rng, ["bf16", "bf16", "f16", "f32"])
    # (most sequences, longest sequence): a few long ones up to many very short ones
    max_seqs, max_len = _pick(rng, [(4, 600), (12, 150), (40, 100), (64, 20), (300, 3)])
    wl = workloads.random_case(20_000 + seed, max_seqs=max_seqs, max_len=max_len,
                               x_scale=_pick(rng, [1.0, 1.0, 8.0, 40.0]),
                               pad_tokens=_pick(rng, [0, 0, 5]), x_dtype=fmt)
    off_x = _pick(rng, [0, 0, 0, 1, 2, 3, 5, 7])
    off_o = _pick(rng, [0, 0, 0, 1, 3])
    w_form = _pick(rng, ["contig", "contig", "transposed", "padded"])
    b_form = _pick(rng, ["aligned", "offset"])
    s_form = _pick(rng, ["contig", "contig", "dim_first", "dim_first_padded", "wide5"])
    ci_form = _pick(rng, ["contig", "strided"])
    init_form = _pick(rng, ["array", "array", "none"])
    desc = (f"{wl.name}; x at column {off_x}, out at element {off_o}, weight {w_form}, bias "
            f"{b_form}, state {s_form}, indices {ci_form}, initial states {init_form}, "
            f"activation {wl.activation}, null block {wl.null_block_id}")
    print(f"case: prefill fuzz {seed}: {desc}", flush=True)
    if init_form == "none":
        wl = dataclasses.replace(wl, has_initial_state=np.zeros_like(wl.has_initial_state))
    want, want_st = oracle_with_canary(wl)

    lines = wl.conv_states.shape[0]
    P = wl.dim // wl.part_dim
    out = _out_view((P, wl.num_tokens, wl.part_dim), fmt, off_o)
    buf, st, logical, untouched = _state_view(wl.conv_states, s_form, rng)
    before = untouched(buf.cpu().numpy()).copy()
    kd.packed_causal_conv1d_fn(
        _x_view(wl.x, fmt, wl.dim, off_x), _weight_view(wl.weight, w_form),
        _bias_view(wl.bias, b_form), st, torch.from_numpy(wl.query_start_loc).cuda(),
        _indices_view(wl.cache_indices, lines, ci_form),
        None if init_form == "none" else torch.from_numpy(wl.has_initial_state).cuda(),
        wl.part_dim, wl.activation, wl.null_block_id, out=out)
    torch.cuda.synchronize()
    got = torch_to_words(out)
    assert np.array_equal(got, want), (desc, first_mismatches(got, want))
    after = buf.cpu().numpy()
    _same_words(logical(after), want_st, desc)
    _same_words(untouched(after), before, desc + " (entries outside the history)")
    return desc


def decode_case(seed: int) -> str:
    rng = np.random.default_rng(30_000 + seed)
    bf16_state = rng.random() < 0.4
    pd = _pick(rng, [8, 64, 192, 256, 520, 1536])
    dim = 3 * pd
    B = _pick(rng, [1, 5, 37, 64, 300, 700])
    fmt = "bf16" if bf16_state else _pick(rng, ["bf16", "f16", "f32"])
    row_stride = dim + _pick(rng, [0, 8, 3, 64])
    lines = B + int(rng.integers(1, 6))
    off_x = _pick(rng, [0, 0, 1, 3])
    off_o = _pick(rng, [0, 0, 1, 2])
    use_null = rng.random() < 0.5
    P = dim // pd
    out = _out_view((P, B, pd), fmt, off_o)
    if bf16_state:
        d = workloads.decode_batch_bf16_state(B, seed=40_000 + seed, dim=dim, part_dim=pd,
                                              row_stride=row_stride, lines=lines)
        null = int(d.cache_indices[int(rng.integers(B))]) if use_null else None
        w_form = _pick(rng, ["width_major", "dim_by_4"])
        s_form = _pick(rng, ["contig", "contig", "wide4"])
        desc = (f"bf16-state decode {seed}: B={B} dim={dim} pd={pd} stride={row_stride}; x at "
                f"column {off_x}, out at element {off_o}, weight {w_form}, state {s_form}, "
                f"null block {null}")
        print(f"case: decode fuzz {seed}: {desc}", flush=True)
        w = torch.from_numpy(d.weight).cuda()
        if w_form == "dim_by_4":
            w = torch.from_numpy(np.ascontiguousarray(
                d.weight.transpose(0, 2, 1).reshape(dim, 4))).cuda()
        if s_form == "wide4":
            host = rng.integers(0, 1 << 16, size=(lines, dim, 4), dtype=np.uint16)
            host[:, :, :3] = d.conv_states
            buf = words_to_torch(host, torch.bfloat16)
            st = buf[:, :, :3]
        else:
            buf = words_to_torch(d.conv_states, torch.bfloat16)
            st = buf
        before = torch_to_words(buf).copy()
        kd.packed_causal_conv1d_update(_x_view(d.x, "bf16", dim, off_x), w,
                                       torch.from_numpy(d.bias).cuda(), st,
                                       torch.from_numpy(d.cache_indices).cuda(), pd, "silu",
                                       null, out=out)
        torch.cuda.synchronize()
        s = d.conv_states.copy()
        want = oracle.packed_causal_conv1d_update_bf16_state(d.x, dim, d.weight, d.bias, s,
                                                             d.cache_indices, pd, "silu", null)
        got = torch_to_words(out)
        assert np.array_equal(got, want), (desc, first_mismatches(got, want))
        after = torch_to_words(buf)
        assert np.array_equal(after[:, :, :3], s), desc
        if s_form == "wide4":
            assert np.array_equal(after[:, :, 3:], before[:, :, 3:]), desc
        return desc

    act = _pick(rng, ["silu", "silu", None])
    has_bias = rng.random() < 0.8
    wl = make_workload([1] * B, dim=dim, part_dim=pd, seed=40_000 + seed, lines=lines,
                       x_dtype=fmt, row_stride=row_stride, activation=act, bias=has_bias,
                       init=[True] * B, x_scale=_pick(rng, [1.0, 8.0, 40.0]))
    null = int(wl.cache_indices[int(rng.integers(B))]) if use_null else None
    w_form = _pick(rng, ["contig", "contig", "transposed", "padded"])
    s_form = _pick(rng, ["contig", "contig", "dim_first", "dim_first_padded", "wide5"])
    ci_form = _pick(rng, ["contig", "strided"])
    desc = (f"decode {seed}: B={B} dim={dim} pd={pd} stride={row_stride} x {fmt}; x at column "
            f"{off_x}, out at element {off_o}, weight {w_form}, state {s_form}, indices "
            f"{ci_form}, activation {act}, bias {has_bias}, null block {null}")
    print(f"case: decode fuzz {seed}: {desc}", flush=True)
    buf, st, logical, untouched = _state_view(wl.conv_states, s_form, rng)
    before = untouched(buf.cpu().numpy()).copy()
    kd.packed_causal_conv1d_update(_x_view(wl.x, fmt, dim, off_x), _weight_view(wl.weight, w_form),
                                   None if wl.bias is None else torch.from_numpy(wl.bias).cuda(),
                                   st, _indices_view(wl.cache_indices, lines, ci_form), pd, act,
                                   null, out=out)
    torch.cuda.synchronize()
    s = wl.conv_states.copy()
    want = oracle.packed_causal_conv1d_update(wl.x, dim, wl.weight, wl.bias, s, wl.cache_indices,
                                              pd, act, null, x_dtype=fmt)
    got = torch_to_words(out)
    assert np.array_equal(got, want), (desc, first_mismatches(got, want))
    after = buf.cpu().numpy()
    _same_words(logical(after), s, desc)
    _same_words(untouched(after), before, desc + " (entries outside the history)")
    return desc


@pytest.mark.parametrize("seed", range(40))
def test_prefill_fuzz_all_forms(seed):
    prefill_case(seed)


@pytest.mark.parametrize("seed", range(30))
def test_decode_fuzz_all_forms(seed):
    decode_case(seed)
