"""GPU parity of the decode step (one token per sequence) against the oracle.

Page vllm.models.kimi_k3.amd.ops.kda_decode: the packed causal conv1d update is the
first step of a decode batch; with the FP32 state its arithmetic is that of page
vllm.models.kimi_k3.nvidia.ops.kda_conv, and the oracle's update is the prefill
routine at one token per sequence with the stored history. Outputs and state
lines must match word for word; a chain of GPU decode steps after a GPU prefill
must equal the oracle's single prefill over all tokens.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
from gpu_util import TORCH_DTYPE, first_mismatches, torch_to_words, words_to_torch
from helpers import make_workload, planes_to_rows

pytestmark = pytest.mark.gpu


def _run_update(x_words, fmt, dim, weight, bias, states_dev, ci, pd, act, null):
    x = words_to_torch(x_words, TORCH_DTYPE[fmt])[:, :dim]
    out = kd.packed_causal_conv1d_update(
        x, torch.from_numpy(weight).cuda(), None if bias is None else torch.from_numpy(bias).cuda(),
        states_dev, torch.from_numpy(ci).cuda(), pd, act, null)
    torch.cuda.synchronize()
    return torch_to_words(out)


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
# Waves take 1, 2, 4 or 8 sequences depending on the batch (at least 2048 waves per
# launch); the batches below cover each, with a last wave that is only partly used.
@pytest.mark.parametrize("batch,parts,pd,act", [(1, 3, 256, "silu"), (7, 3, 200, None),
                                                (64, 3, 1536, "silu"), (300, 3, 192, "silu"),
                                                (4096, 3, 192, None), (4093, 3, 192, "silu"),
                                                (250, 3, 1536, "silu"), (1021, 3, 1536, "silu")])
def test_decode_step_bit_exact(batch, parts, pd, act, fmt):
    dim = parts * pd
    lines = batch + 5
    wl = make_workload([1] * batch, dim=dim, part_dim=pd, seed=batch + pd, lines=lines,
                       activation=act, x_dtype=fmt, row_stride=dim + 8,
                       bias=batch % 2 == 1)
    null = int(wl.cache_indices[batch // 2])
    print(f"case: decode batch {batch} dim {dim} x {fmt} act {act}", flush=True)
    st_dev = torch.from_numpy(wl.conv_states.copy()).cuda()
    got = _run_update(wl.x, fmt, dim, wl.weight, wl.bias, st_dev, wl.cache_indices, pd, act, null)
    st = wl.conv_states.copy()
    want = oracle.packed_causal_conv1d_update(wl.x, dim, wl.weight, wl.bias, st, wl.cache_indices,
                                              pd, act, null, x_dtype=fmt)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st_dev.cpu().numpy().view(np.uint32), st.view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
def test_gpu_decode_chain_equals_one_prefill(fmt):
    """GPU prefill of the first 5 tokens of 6 sequences, then GPU decode steps for the
    rest: outputs and lines equal the oracle's prefill over all tokens."""
    lens = [20, 9, 5, 13, 30, 6]
    dim, pd = 3 * 256, 256
    full = make_workload(lens, dim=dim, part_dim=pd, seed=91, lines=8, x_dtype=fmt,
                         cache_indices=[7, 0, 3, 5, 1, 6], init=[True, False, True, True, False, True])
    o_full, st_full = oracle.run_workload(full)
    rows_full = planes_to_rows(o_full)
    qsl = full.query_start_loc
    prefix = 5
    pre_rows = np.concatenate([np.arange(qsl[s], qsl[s] + prefix) for s in range(len(lens))])
    st_dev = torch.from_numpy(full.conv_states.copy()).cuda()
    w = torch.from_numpy(full.weight).cuda()
    b = torch.from_numpy(full.bias).cuda()
    x_pre = words_to_torch(full.x[pre_rows], TORCH_DTYPE[fmt])[:, :dim]
    q = torch.arange(0, prefix * len(lens) + 1, prefix, dtype=torch.int32).cuda()
    ci = torch.from_numpy(full.cache_indices).cuda()
    init = torch.from_numpy(full.has_initial_state).cuda()
    o_pre = kd.packed_causal_conv1d_fn(x_pre, w, b, st_dev, q, ci, init, pd, "silu", None)
    got = np.zeros_like(rows_full)
    got[pre_rows] = planes_to_rows(torch_to_words(o_pre))
    for step in range(prefix, max(lens)):
        running = [s for s in range(len(lens)) if step < lens[s]]
        rows = np.array([qsl[s] + step for s in running])
        o = _run_update(full.x[rows], fmt, dim, full.weight, full.bias, st_dev,
                        full.cache_indices[running].copy(), pd, "silu", None)
        got[rows] = planes_to_rows(o)
    assert np.array_equal(got, rows_full), first_mismatches(got, rows_full)
    assert np.array_equal(st_dev.cpu().numpy().view(np.uint32), st_full.view(np.uint32))


def test_decode_dim_first_state():
    wl = make_workload([1] * 50, dim=768, part_dim=256, seed=93, lines=60)
    buf = torch.from_numpy(np.ascontiguousarray(wl.conv_states.transpose(0, 2, 1))).cuda()
    got = _run_update(wl.x, "bf16", 768, wl.weight, wl.bias, buf.transpose(1, 2),
                      wl.cache_indices, 256, "silu", None)
    st = wl.conv_states.copy()
    want = oracle.packed_causal_conv1d_update(wl.x, 768, wl.weight, wl.bias, st, wl.cache_indices,
                                              256, "silu", None)
    assert np.array_equal(got, want)
    assert np.array_equal(buf.cpu().numpy().transpose(0, 2, 1).view(np.uint32), st.view(np.uint32))


@pytest.mark.parametrize("fmt", ["bf16", "f16", "f32"])
def test_decode_bench_workload(fmt):
    """The decode batch the bench times (256 sequences, dim 4608 in rows of 9728)."""
    import workloads

    wl = workloads.decode_batch(256, x_dtype=fmt)
    st_dev = torch.from_numpy(wl.conv_states.copy()).cuda()
    got = _run_update(wl.x, fmt, wl.dim, wl.weight, wl.bias, st_dev, wl.cache_indices,
                      wl.part_dim, wl.activation, wl.null_block_id)
    want, want_st = oracle.run_workload(wl)
    assert np.array_equal(got, want), first_mismatches(got, want)
    assert np.array_equal(st_dev.cpu().numpy().view(np.uint32), want_st.view(np.uint32))


def test_decode_graph_replay_with_new_device_data():
    """One decode step captured in a HIP graph and replayed on new x, lines and line
    choices of the same shapes: every replay matches the oracle for its data."""
    B, dim, pd = 96, 768, 256
    base = make_workload([1] * B, dim=dim, part_dim=pd, seed=95, lines=B + 8)
    x = words_to_torch(base.x, torch.bfloat16)[:, :dim].contiguous()
    w = torch.from_numpy(base.weight).cuda()
    b = torch.from_numpy(base.bias).cuda()
    st = torch.from_numpy(base.conv_states.copy()).cuda()
    ci = torch.from_numpy(base.cache_indices).cuda()
    out = torch.empty((3, B, pd), dtype=torch.bfloat16, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        kd.packed_causal_conv1d_update(x, w, b, st, ci, pd, "silu", None, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kd.packed_causal_conv1d_update(x, w, b, st, ci, pd, "silu", None, out=out)
    for trial in range(3):
        wl = make_workload([1] * B, dim=dim, part_dim=pd, seed=96 + trial, lines=B + 8)
        x.copy_(words_to_torch(wl.x, torch.bfloat16)[:, :dim])
        w.copy_(torch.from_numpy(wl.weight))
        b.copy_(torch.from_numpy(wl.bias))
        st.copy_(torch.from_numpy(wl.conv_states))
        ci.copy_(torch.from_numpy(wl.cache_indices))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        want_st = wl.conv_states.copy()
        want = oracle.packed_causal_conv1d_update(wl.x, dim, wl.weight, wl.bias, want_st,
                                                  wl.cache_indices, pd, "silu", None)
        got = torch_to_words(out)
        assert np.array_equal(got, want), (trial, first_mismatches(got, want))
        assert np.array_equal(st.cpu().numpy().view(np.uint32), want_st.view(np.uint32)), trial
