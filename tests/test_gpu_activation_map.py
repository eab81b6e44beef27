"""The kernel's activation-and-rounding map against the oracle on every FP32 input.

Every stored word is bf16(act(acc)) for an FP32 accumulator acc (page
vllm.models.kimi_k3.nvidia.ops.kda_conv, module docstring), and the device
computes that map with one routine (fast SiLU plus an exact fallback near bf16
rounding boundaries) shared by the convolution and by kdaconv_activation_map.
Comparing the map on all 2^32 inputs with the oracle's proves the activation
step of the convolution exact for every accumulator value.
"""

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
import packed_varlen_causal_depthwise_amd as kd

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27


@pytest.mark.parametrize("act", ["silu", None])
def test_activation_map_all_fp32_inputs(act):
    lib = oracle.load()
    silu = act == "silu"
    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    sub = CHUNK // threads
    buf = torch.empty(CHUNK, dtype=torch.int16, device="cuda")
    ref = np.empty(CHUNK, dtype=np.uint16)
    bad = []
    nbad = 0
    with ThreadPoolExecutor(threads) as ex:
        for first in range(0, 1 << 32, CHUNK):
            kd.activation_map(first, CHUNK, act, out=buf)
            futs = [ex.submit(oracle.act_bf16_range, first + i * sub, sub, silu, lib,
                              ref[i * sub:(i + 1) * sub]) for i in range(threads)]
            got = buf.cpu().numpy().view(np.uint16)
            for f in futs:
                f.result()
            diff = np.nonzero(got != ref)[0]
            nbad += diff.size
            for i in diff[: max(0, 8 - len(bad))]:
                bad.append((hex(first + int(i)), hex(int(got[i])), hex(int(ref[i]))))
    print(f"activation {act}: {nbad} mismatches", flush=True)
    assert nbad == 0, bad
