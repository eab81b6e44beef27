"""GPU parity for the argument forms the ABI accepts beyond the contiguous ones.

Page vllm.models.kimi_k3.nvidia.ops.kda_conv, packed_causal_conv1d_fn source: the
launch passes both weight strides, the cache_indices stride and the three state
strides, and has_initial_state may be absent. Each case below runs a kernel path
that the contiguous inputs never take (the scalar weight and bias loads, strided
line lookups, the missing initial-state array, lines outside the state array, and
the split of an output larger than one launch addresses) and compares outputs and
states with the oracle word for word. The oracle is given the same values in
contiguous arrays; its own handling of the strides is pinned separately
(tests/test_oracle_conv.py).
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
from gpu_util import (TORCH_DTYPE, first_mismatches, oracle_with_canary, run_hip, to_device,
                      torch_to_words, words_to_torch)
from helpers import make_workload

pytestmark = pytest.mark.gpu


def _weight_view(weight: np.ndarray, layout: str) -> torch.Tensor:
    """A (dim, 4) device view of the weight values with non-contiguous strides."""
    dim = weight.shape[0]
    if layout == "transposed":  # a (4, dim) array seen as (dim, 4): strides (1, dim)
        v = torch.from_numpy(np.ascontiguousarray(weight.T)).cuda().t()
        assert v.stride() == (1, dim)
    else:  # rows of 7 floats, taps at columns 2..5: strides (7, 1), base not 16-byte aligned
        buf = torch.full((dim, 7), 1e30, dtype=torch.float32, device="cuda")
        buf[:, 2:6] = torch.from_numpy(weight).cuda()
        v = buf[:, 2:6]
        assert v.stride() == (7, 1)
    return v


def _misaligned_bias(bias: np.ndarray) -> torch.Tensor:
    """The bias values at a 4-byte offset from a 256-byte aligned allocation."""
    buf = torch.empty(bias.shape[0] + 1, dtype=torch.float32, device="cuda")
    b = buf[1:]
    b.copy_(torch.from_numpy(bias))
    assert b.data_ptr() % 16 == 4 and b.is_contiguous()
    return b


def _strided_indices(ci: np.ndarray, lines: int) -> torch.Tensor:
    """cache_indices as every other entry of an array whose other entries name other,
    valid lines."""
    inter = np.empty(2 * ci.shape[0], dtype=np.int32)
    inter[0::2] = ci
    inter[1::2] = (ci + 1) % lines
    v = torch.from_numpy(inter).cuda()[::2]
    assert v.stride() == (2,)
    return v


def _check(wl, got, st):
    want, want_st = oracle_with_canary(wl)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st.view(np.uint32), want_st.view(np.uint32)), \
        first_mismatches(st.view(np.uint32), want_st.view(np.uint32))


def _case(seed, fmt="bf16", **kw):
    return make_workload([1, 2, 3, 40, 17, 0, 90], dim=3 * 256, part_dim=256, seed=seed, lines=10,
                         init=[True, False, True, True, False, True, True], x_dtype=fmt,
                         row_stride=3 * 256 + 8, **kw)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("layout", ["transposed", "padded"])
def test_weight_views(layout, fmt):
    wl = _case(100, fmt)
    print(f"case: weight {layout}, x {fmt}", flush=True)
    d = to_device(wl)
    d["weight"] = _weight_view(wl.weight, layout)
    got, st = run_hip(wl, dev=d)
    _check(wl, got, st)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_misaligned_bias(fmt):
    wl = _case(101, fmt)
    print(f"case: bias at a 4-byte offset, x {fmt}", flush=True)
    d = to_device(wl)
    d["bias"] = _misaligned_bias(wl.bias)
    got, st = run_hip(wl, dev=d)
    _check(wl, got, st)


def test_strided_cache_indices():
    wl = _case(102)
    print("case: cache_indices[::2]", flush=True)
    d = to_device(wl)
    d["cache_indices"] = _strided_indices(wl.cache_indices, wl.num_cache_lines)
    got, st = run_hip(wl, dev=d)
    _check(wl, got, st)


def test_no_initial_state_array():
    """has_initial_state=None: every sequence starts from zeros and writes its line."""
    wl = _case(103)
    print("case: has_initial_state None", flush=True)
    d = to_device(wl)
    d["has_initial_state"] = None
    got, st = run_hip(wl, dev=d)
    wl.has_initial_state = None
    _check(wl, got, st)


@pytest.mark.parametrize("bad", [-1, 10, 2 ** 31 - 1, -2 ** 31])
def test_out_of_range_line_acts_as_null_block(bad):
    """A line outside [0, lines) reads and writes no state and runs from zeros, the
    reading the oracle takes (two sequences, one of a single token, one of 40)."""
    wl = _case(104)
    wl.cache_indices[0] = bad
    wl.cache_indices[3] = bad
    print(f"case: line {bad}", flush=True)
    got, st = run_hip(wl)
    _check(wl, got, st)


def test_all_argument_forms_together():
    wl = _case(105)
    print("case: every argument form at once", flush=True)
    d = to_device(wl)
    d["weight"] = _weight_view(wl.weight, "transposed")
    d["bias"] = _misaligned_bias(wl.bias)
    d["cache_indices"] = _strided_indices(wl.cache_indices, wl.num_cache_lines)
    got, st = run_hip(wl, dev=d)
    _check(wl, got, st)


# ------------------------------------------------------------------ decode step

def _decode_case(seed, fmt):
    dim, pd, batch = 3 * 256, 256, 37
    return make_workload([1] * batch, dim=dim, part_dim=pd, seed=seed, lines=batch + 6,
                         x_dtype=fmt, row_stride=dim + 8)


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
@pytest.mark.parametrize("form", ["weight_transposed", "weight_padded", "bias", "indices", "lines"])
def test_decode_argument_forms(form, fmt):
    wl = _decode_case(110, fmt)
    print(f"case: decode {form}, x {fmt}", flush=True)
    if form == "lines":
        wl.cache_indices[5] = -1
        wl.cache_indices[9] = wl.num_cache_lines
    w = torch.from_numpy(wl.weight).cuda()
    b = torch.from_numpy(wl.bias).cuda()
    ci = torch.from_numpy(wl.cache_indices).cuda()
    if form.startswith("weight"):
        w = _weight_view(wl.weight, form.split("_")[1])
    elif form == "bias":
        b = _misaligned_bias(wl.bias)
    elif form == "indices":
        ci = _strided_indices(wl.cache_indices, wl.num_cache_lines)
    st_dev = torch.from_numpy(wl.conv_states.copy()).cuda()
    x = words_to_torch(wl.x, TORCH_DTYPE[fmt])[:, : wl.dim]
    out = kd.packed_causal_conv1d_update(x, w, b, st_dev, ci, wl.part_dim, "silu", None)
    torch.cuda.synchronize()
    got = torch_to_words(out)
    st = wl.conv_states.copy()
    want = oracle.packed_causal_conv1d_update(wl.x, wl.dim, wl.weight, wl.bias, st, wl.cache_indices,
                                              wl.part_dim, "silu", None, x_dtype=fmt)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st_dev.cpu().numpy().view(np.uint32), st.view(np.uint32))


# ------------------------------------------------------------ output above 2 GiB

def test_output_above_two_gib():
    """262144 tokens x 4608 channels: the 2.4 GB output is written by two launches (planes
    0-1, then plane 2 from channel 3072), each addressing under 2 GiB. The oracle runs on
    channel slices (a channel's output and state depend on that channel alone, a pinned
    invariant): the first and last 16 channels, the 16 around the launch boundary at
    channel 3072, and the 16 around the plane boundary at 1536; the states are compared
    on all lines for those channels."""
    import workloads

    wl = workloads.large_output_case()
    T, dim, pd = wl.num_tokens, wl.dim, wl.part_dim
    assert T * dim * 2 > 2 ** 31 and T * pd * 2 * 3 > 2 ** 31 - 1
    print(f"case: {wl.name}", flush=True)
    d = to_device(wl)
    out = torch.empty((dim // pd, T, pd), dtype=torch.bfloat16, device="cuda")
    out.view(torch.int16).fill_(np.int16(0x5555))
    kd.packed_causal_conv1d_fn(d["x"], d["weight"], d["bias"], d["conv_states"],
                               d["query_start_loc"], d["cache_indices"], d["has_initial_state"],
                               pd, "silu", None, out=out)
    torch.cuda.synchronize()
    st_gpu = d["conv_states"].cpu().numpy()
    for c0 in (0, 1528, 3064, dim - 16):
        c1 = c0 + 16
        sub = workloads.Workload(f"channels {c0}..{c1}", wl.x[:, c0:c1], 16,
                                 np.ascontiguousarray(wl.weight[c0:c1]),
                                 np.ascontiguousarray(wl.bias[c0:c1]),
                                 np.ascontiguousarray(wl.conv_states[:, c0:c1]),
                                 wl.query_start_loc, wl.cache_indices, wl.has_initial_state,
                                 16, wl.activation, wl.null_block_id)
        want, want_st = oracle.run_workload(sub)
        cols = np.arange(c0, c1)
        got = np.empty((T, 16), dtype=np.uint16)
        for p in np.unique(cols // pd):
            sel = cols // pd == p
            lo, hi = int(cols[sel][0] % pd), int(cols[sel][-1] % pd) + 1
            got[:, sel] = torch_to_words(out[p, :, lo:hi].contiguous())
        assert np.array_equal(got, want[0]), (c0, first_mismatches(got, want[0]))
        assert np.array_equal(st_gpu[:, c0:c1].view(np.uint32), want_st.view(np.uint32)), c0
    del d, out
    torch.cuda.empty_cache()
