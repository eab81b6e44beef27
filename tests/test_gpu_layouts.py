"""GPU parity for conv-state layouts other than contiguous (lines, dim, 3).

Page: vllm.models.kimi_k3.nvidia.ops.kda_conv. The launch passes all three state
strides; packed_causal_conv1d_supported admits size(2) >= 3. Layouts: "dim
first" (lines, 3, dim), the same with padded rows, and a wider state (lines, dim,
5) whose entries 3 and 4 must stay untouched. Outputs and the updated entries
0..2 must equal the oracle's on the contiguous layout word for word.
"""

import numpy as np
import pytest
import torch

from gpu_util import first_mismatches, oracle_with_canary, run_hip, to_device
from helpers import make_workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("fmt", ["bf16", "f32"])
@pytest.mark.parametrize("layout", ["dim_first", "dim_first_padded", "wide5"])
def test_state_layouts(layout, fmt):
    wl = make_workload([1, 2, 3, 40, 17, 0, 5], dim=3 * 200, part_dim=200, seed=61, lines=9,
                       init=[True, False, True, True, False, True, True], x_dtype=fmt,
                       row_stride=3 * 200 + 8)
    print(f"case: state layout {layout}, x {fmt}", flush=True)
    want, want_st = oracle_with_canary(wl)
    d = to_device(wl)
    lines, dim = wl.conv_states.shape[0], wl.dim
    rng = np.random.default_rng(61)
    if layout == "dim_first":
        buf = torch.from_numpy(np.ascontiguousarray(wl.conv_states.transpose(0, 2, 1))).cuda()
        st = buf.transpose(1, 2)
    elif layout == "dim_first_padded":
        host = rng.standard_normal((lines, 3, dim + 72)).astype(np.float32)
        host[:, :, :dim] = wl.conv_states.transpose(0, 2, 1)
        buf = torch.from_numpy(host).cuda()
        st = buf[:, :, :dim].transpose(1, 2)
    else:
        host = rng.standard_normal((lines, dim, 5)).astype(np.float32)
        host[:, :, :3] = wl.conv_states
        buf = torch.from_numpy(host).cuda()
        st = buf
    before = buf.cpu().numpy().copy()
    d["conv_states"] = st
    got, _ = run_hip(wl, dev=d)
    assert np.array_equal(got, want), first_mismatches(got, want)
    after = buf.cpu().numpy()
    if layout == "wide5":
        hist, rest, rest0 = after[:, :, :3], after[:, :, 3:], before[:, :, 3:]
    else:
        hist = after[:, :, :dim].transpose(0, 2, 1)
        rest, rest0 = after[:, :, dim:], before[:, :, dim:]
    assert np.array_equal(np.ascontiguousarray(hist).view(np.uint32), want_st.view(np.uint32))
    assert np.array_equal(rest.view(np.uint32), rest0.view(np.uint32))
