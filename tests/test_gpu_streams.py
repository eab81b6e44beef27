"""Concurrent calls on different streams.

The library keeps no state between calls and allocates nothing, so calls that write
different memory may run at the same time on different streams (the header's
convention). Here a prefill of the 16384-token workload, a decode step with the FP32
state, a decode step with the bf16 state and a second prefill of a batch of short
sequences are queued on four streams without synchronising between them, each several
times on fresh buffers; every result must equal the oracle's word for word.
"""

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd
import workloads
from gpu_util import first_mismatches, to_device, torch_to_words, words_to_torch

pytestmark = pytest.mark.gpu


def _prefill_job(wl):
    d = to_device(wl)
    P = wl.dim // wl.part_dim
    out = torch.empty((P, wl.num_tokens, wl.part_dim), dtype=torch.bfloat16, device="cuda")

    def run():
        kd.packed_causal_conv1d_fn(d["x"], d["weight"], d["bias"], d["conv_states"],
                                   d["query_start_loc"], d["cache_indices"], d["has_initial_state"],
                                   wl.part_dim, wl.activation, wl.null_block_id, out=out)

    def check():
        want, want_st = oracle.run_workload(wl)
        got = torch_to_words(out)
        assert np.array_equal(got, want), first_mismatches(got, want)
        assert np.array_equal(d["conv_states"].cpu().numpy().view(np.uint32), want_st.view(np.uint32))

    return run, check


def _decode_job(wl):
    x = words_to_torch(wl.x, torch.bfloat16)[:, :wl.dim]
    w = torch.from_numpy(wl.weight).cuda()
    b = torch.from_numpy(wl.bias).cuda()
    st = torch.from_numpy(wl.conv_states.copy()).cuda()
    ci = torch.from_numpy(wl.cache_indices).cuda()
    out = torch.empty((wl.dim // wl.part_dim, wl.num_tokens, wl.part_dim), dtype=torch.bfloat16,
                      device="cuda")

    def run():
        kd.packed_causal_conv1d_update(x, w, b, st, ci, wl.part_dim, wl.activation,
                                       wl.null_block_id, out=out)

    def check():
        s = wl.conv_states.copy()
        want = oracle.packed_causal_conv1d_update(wl.x, wl.dim, wl.weight, wl.bias, s,
                                                  wl.cache_indices, wl.part_dim, wl.activation,
                                                  wl.null_block_id)
        got = torch_to_words(out)
        assert np.array_equal(got, want), first_mismatches(got, want)
        assert np.array_equal(st.cpu().numpy().view(np.uint32), s.view(np.uint32))

    return run, check


def _decode16_job(d):
    x = words_to_torch(d.x, torch.bfloat16)[:, :d.dim]
    w = torch.from_numpy(d.weight).cuda()
    b = torch.from_numpy(d.bias).cuda()
    st = torch.from_numpy(d.conv_states.view(np.int16).copy()).cuda().view(torch.bfloat16)
    ci = torch.from_numpy(d.cache_indices).cuda()
    out = torch.empty((d.dim // d.part_dim, d.batch, d.part_dim), dtype=torch.bfloat16,
                      device="cuda")

    def run():
        kd.packed_causal_conv1d_update(x, w, b, st, ci, d.part_dim, d.activation,
                                       d.null_block_id, out=out)

    def check():
        s = d.conv_states.copy()
        want = oracle.packed_causal_conv1d_update_bf16_state(d.x, d.dim, d.weight, d.bias, s,
                                                             d.cache_indices, d.part_dim,
                                                             d.activation, d.null_block_id)
        got = torch_to_words(out)
        assert np.array_equal(got, want), first_mismatches(got, want)
        assert np.array_equal(torch_to_words(st), s)

    return run, check


@pytest.mark.parametrize("round_", range(2))
def test_four_streams_at_once(round_):
    print(f"case: four streams, round {round_}", flush=True)
    jobs = [_prefill_job(workloads.config3()),
            _decode_job(workloads.decode_batch(1024, seed=40 + round_)),
            _decode16_job(workloads.decode_batch_bf16_state(512, seed=50 + round_)),
            _prefill_job(workloads.config5())]
    streams = [torch.cuda.Stream() for _ in jobs]
    torch.cuda.synchronize()
    for s, (run, _) in zip(streams, jobs):
        with torch.cuda.stream(s):
            run()
    torch.cuda.synchronize()
    for _, check in jobs:
        check()
