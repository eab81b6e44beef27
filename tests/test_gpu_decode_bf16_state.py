"""GPU parity of the decode step with a bf16 conv state and the width-major weight.

Page vllm.models.kimi_k3.amd.ops.kda_decode: the fused decode kernel takes a bf16
input with a bf16 conv state and the FP32 conv weight mirrored width-major,
[qkv, width, channel]. Outputs and state lines must equal the oracle's
(oracle.packed_causal_conv1d_update_bf16_state) word for word: over the batch sizes
that give waves of 1, 2 and 4 sequences, partial column blocks, the null block and
lines outside the array, every weight form (width-major and (dim, 4), contiguous and
strided) and state form (contiguous, padded, dim-first, a base off 8-byte alignment),
and NaN words, whose payloads the state keeps.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
import workloads
from gpu_util import first_mismatches, torch_to_words, words_to_torch

pytestmark = pytest.mark.gpu


def _case(batch, parts, pd, seed, lines=None, null=None):
    dim = parts * pd
    return workloads.decode_batch_bf16_state(batch, seed=seed, dim=dim, part_dim=pd,
                                             row_stride=dim + 8, lines=lines or batch + 5,
                                             null_block_id=null)


def _states16(words: np.ndarray, form: str):
    """A device view (lines, dim, 3) of bf16 words in the given layout, and its buffer."""
    L, D, _ = words.shape
    w16 = torch.from_numpy(words.view(np.int16)).cuda()
    if form == "contiguous":
        buf = w16.clone()
        return buf.view(torch.bfloat16), buf
    if form == "padded":  # (lines, dim, 5), entries 3..4 must stay untouched
        buf = torch.full((L, D, 5), 0x1234, dtype=torch.int16, device="cuda")
        buf[:, :, :3] = w16
        return buf.view(torch.bfloat16)[:, :, :3], buf
    if form == "dim_first":  # (lines, 3, dim) seen as (lines, dim, 3)
        buf = w16.transpose(1, 2).contiguous()
        return buf.view(torch.bfloat16).transpose(1, 2), buf
    # one element past a 16-byte boundary: 2-byte aligned only, scalar path
    flat = torch.zeros(L * D * 3 + 8, dtype=torch.int16, device="cuda")
    v = flat[1:1 + L * D * 3].view(L, D, 3)
    v.copy_(w16)
    assert v.data_ptr() % 8 == 2
    return v.view(torch.bfloat16), flat


def _weight(d, form: str) -> torch.Tensor:
    wm = torch.from_numpy(d.weight).cuda()  # (parts, 4, pd) contiguous
    if form == "width_major":
        return wm
    if form == "width_major_padded":  # channel runs of pd inside rows of pd + 6: scalar path
        parts, _, pd = d.weight.shape
        buf = torch.full((parts, 4, pd + 6), 1e30, dtype=torch.float32, device="cuda")
        buf[:, :, 3:3 + pd] = wm
        return buf[:, :, 3:3 + pd]
    cm = wm.permute(0, 2, 1).reshape(-1, 4).contiguous()  # (dim, 4) [channel, width]
    if form == "channel_major":
        return cm
    # (dim, 4) with strides (1, dim): part stride part_dim, channel stride 1, width stride
    # dim, which the width-major vector path takes when part_dim and dim are multiples of 4
    return cm.t().contiguous().t()


def _run(d, weight=None, states=None, x=None):
    xt = words_to_torch(d.x if x is None else x, torch.bfloat16)[:, :d.dim]
    st_view, st_buf = states if states is not None else _states16(d.conv_states, "contiguous")
    out = kd.packed_causal_conv1d_update(
        xt, _weight(d, "width_major") if weight is None else weight,
        None if d.bias is None else torch.from_numpy(d.bias).cuda(), st_view,
        torch.from_numpy(d.cache_indices).cuda(), d.part_dim, d.activation, d.null_block_id)
    torch.cuda.synchronize()
    return torch_to_words(out), st_view, st_buf


def _want(d):
    st = d.conv_states.copy()
    o = oracle.packed_causal_conv1d_update_bf16_state(d.x, d.dim, d.weight, d.bias, st,
                                                      d.cache_indices, d.part_dim, d.activation,
                                                      d.null_block_id)
    return o, st


def _state_words(st_view) -> np.ndarray:
    return st_view.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# 18 column blocks at dim 4608: 37 sequences -> 1 per wave, 300 -> 2, 500 -> 4.
@pytest.mark.parametrize("batch,parts,pd,act", [(1, 3, 256, "silu"), (37, 3, 1536, "silu"),
                                                (300, 3, 1536, None), (500, 3, 1536, "silu"),
                                                (7, 3, 200, "silu"), (61, 3, 40, None),
                                                (4093, 3, 192, "silu")])
def test_decode_bf16_state_bit_exact(batch, parts, pd, act):
    d = _case(batch, parts, pd, seed=batch + pd)
    d.activation = act
    if batch % 2:
        d.bias = None
    d.null_block_id = int(d.cache_indices[batch // 2])
    print(f"case: bf16-state decode batch {batch} dim {parts * pd} act {act}", flush=True)
    got, st_view, _ = _run(d)
    want, want_st = _want(d)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(_state_words(st_view), want_st), \
        first_mismatches(_state_words(st_view), want_st)


@pytest.mark.parametrize("wform", ["width_major", "width_major_padded", "channel_major",
                                   "channel_major_transposed"])
@pytest.mark.parametrize("sform", ["contiguous", "padded", "dim_first", "misaligned"])
def test_weight_and_state_forms(wform, sform):
    d = _case(37, 3, 200, seed=777)
    print(f"case: bf16-state decode weight {wform} state {sform}", flush=True)
    states = _states16(d.conv_states, sform)
    got, st_view, st_buf = _run(d, weight=_weight(d, wform), states=states)
    want, want_st = _want(d)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(_state_words(st_view), want_st)
    if sform == "padded":
        assert bool((st_buf[:, :, 3:] == 0x1234).all())


@pytest.mark.parametrize("bad", [-1, 42, 2 ** 31 - 1, -2 ** 31])
def test_null_block_and_lines_outside(bad):
    d = _case(37, 3, 256, seed=778, lines=42, null=None)
    d.null_block_id = int(d.cache_indices[3])
    d.cache_indices[10] = bad
    d.cache_indices[20] = bad
    print(f"case: bf16-state decode line {bad}", flush=True)
    got, st_view, _ = _run(d)
    want, want_st = _want(d)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(_state_words(st_view), want_st)


def test_nan_words_keep_their_payloads():
    d = _case(9, 3, 256, seed=779)
    d.x[0, 5] = 0x7F81
    d.x[4, 700] = 0xFFA5
    line = int(d.cache_indices[2])
    d.conv_states[line, 100, 1] = 0x7F82
    d.conv_states[line, 101, 2] = 0xFF83
    print("case: bf16-state decode NaN words", flush=True)
    got, st_view, _ = _run(d)
    want, want_st = _want(d)
    st = _state_words(st_view)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st, want_st)
    assert st[line, 100, 0] == 0x7F82 and st[line, 101, 1] == 0xFF83
    assert st[int(d.cache_indices[0]), 5, 2] == 0x7F81


def test_equals_fp32_state_decode_on_widened_lines():
    """The bf16-state step and the FP32-state step on the widened lines give the same
    output words, and the FP32 lines afterwards are the bf16 lines widened."""
    d = _case(500, 3, 1536, seed=780)
    print("case: bf16-state decode vs FP32-state decode", flush=True)
    got, st_view, _ = _run(d)
    wide = (d.conv_states.astype(np.uint32) << 16).view(np.float32)
    st32 = torch.from_numpy(wide.copy()).cuda()
    cm = _weight(d, "channel_major")
    out32 = kd.packed_causal_conv1d_update(
        words_to_torch(d.x, torch.bfloat16)[:, :d.dim], cm, torch.from_numpy(d.bias).cuda(), st32,
        torch.from_numpy(d.cache_indices).cuda(), d.part_dim, d.activation, d.null_block_id)
    torch.cuda.synchronize()
    assert np.array_equal(got, torch_to_words(out32))
    st16 = _state_words(st_view)
    assert np.array_equal((st16.astype(np.uint32) << 16), st32.cpu().numpy().view(np.uint32))


def test_graph_replay():
    """Captured once, replayed three times on new tokens with eager work and
    synchronisations between the replays; each replay equals the oracle's step."""
    d = _case(300, 3, 1536, seed=781)
    print("case: bf16-state decode graph replay", flush=True)
    xs = words_to_torch(d.x, torch.bfloat16)
    x_dev = xs.clone()
    w = _weight(d, "width_major")
    b = torch.from_numpy(d.bias).cuda()
    ci = torch.from_numpy(d.cache_indices).cuda()
    st_view, _ = _states16(d.conv_states, "contiguous")
    out = torch.empty((3, d.batch, d.part_dim), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kd.packed_causal_conv1d_update(x_dev[:, :d.dim], w, b, st_view, ci, d.part_dim,
                                       d.activation, None, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref_states = d.conv_states.copy()
    oracle.packed_causal_conv1d_update_bf16_state(d.x, d.dim, d.weight, d.bias, ref_states,
                                                  d.cache_indices, d.part_dim, d.activation, None)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kd.packed_causal_conv1d_update(x_dev[:, :d.dim], w, b, st_view, ci, d.part_dim,
                                       d.activation, None, out=out)
    rng = np.random.default_rng(782)
    for rep in range(3):
        xw = d.x.copy()
        xw[:, :d.dim] = workloads.f32_to_bf16_bits(
            rng.standard_normal((d.batch, d.dim)).astype(np.float32))
        x_dev.copy_(words_to_torch(xw, torch.bfloat16))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want = oracle.packed_causal_conv1d_update_bf16_state(
            xw, d.dim, d.weight, d.bias, ref_states, d.cache_indices, d.part_dim, d.activation, None)
        got = torch_to_words(out)
        assert np.array_equal(got, want), (rep, first_mismatches(got, want))
        assert np.array_equal(_state_words(st_view), ref_states), rep


@pytest.mark.parametrize("seed", range(10))
def test_fuzz(seed):
    """Random batch sizes, part widths (partial column blocks), row pitches, null blocks,
    lines outside the array, bias or none, SiLU or none, and weight and state forms."""
    rng = np.random.default_rng(900 + seed)
    pd = int(rng.choice([8, 16, 64, 72, 128, 192, 256, 520]))
    batch = int(rng.integers(1, 700))
    d = _case(batch, 3, pd, seed=910 + seed, lines=batch + int(rng.integers(1, 9)))
    if rng.integers(2):
        d.bias = None
    if rng.integers(4) == 0:
        d.activation = None
    if rng.integers(2):
        d.null_block_id = int(d.cache_indices[int(rng.integers(batch))])
    if batch > 2 and rng.integers(2):
        d.cache_indices[int(rng.integers(batch))] = -1
    wform = ["width_major", "width_major_padded", "channel_major", "channel_major_transposed"][seed % 4]
    sform = ["contiguous", "padded", "dim_first", "misaligned"][(seed // 2) % 4]
    print(f"case: bf16-state fuzz seed {seed}: batch {batch} pd {pd} weight {wform} state {sform}",
          flush=True)
    got, st_view, _ = _run(d, weight=_weight(d, wform), states=_states16(d.conv_states, sform))
    want, want_st = _want(d)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(_state_words(st_view), want_st)
