"""The C-ABI boundary on the host: the library loads, exports every declared entry
point, and rejects bad arguments with the documented status codes (no GPU call:
kdaconv_validate only looks at sizes, strides and pointer values)."""

import ctypes
import pathlib
import re

import pytest
import torch

import packed_varlen_causal_depthwise_amd as kd
from packed_varlen_causal_depthwise_amd import _lib

HEADER = pathlib.Path(__file__).resolve().parent.parent / "include" / "kdaconv.h"


def _declared():
    text = re.sub(r"/\*.*?\*/", "", HEADER.read_text(), flags=re.S)
    return sorted(set(re.findall(r"\b(kdaconv_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.load()
    names = _declared()
    assert set(names) == set(_lib.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings_and_version():
    lib = _lib.load()
    for code in (0, 1, 2, 3, 99):
        assert lib.kdaconv_status_string(code)
    assert lib.kdaconv_version() >= 100


# Fake, 256-byte-aligned addresses: kdaconv_validate compares them with NULL and
# checks their alignment, nothing more.
A = 0x10000


def _args(**kw):
    a = dict(x=A, dt=_lib.BF16, T=64, dim=384, sx=384, w=A, ws0=4, ws1=1, b=A, st=A, lines=4,
             cs0=1152, cs1=3, cs2=1, qsl=A, S=2, ci=A, cis=1, init=A, pd=128, act=1, hn=0, nid=0,
             out=A)
    a.update(kw)
    return [a["x"], a["dt"], a["T"], a["dim"], a["sx"], a["w"], a["ws0"], a["ws1"], a["b"], a["st"],
            a["lines"], a["cs0"], a["cs1"], a["cs2"], a["qsl"], a["S"], a["ci"], a["cis"],
            a["init"], a["pd"], a["act"], a["hn"], a["nid"], a["out"]]


@pytest.mark.parametrize("kw,code", [
    ({}, _lib.OK),
    (dict(T=-1), _lib.EINVAL),
    (dict(dim=-8), _lib.EINVAL),
    (dict(S=-1), _lib.EINVAL),
    (dict(pd=0), _lib.EINVAL),
    (dict(pd=100), _lib.EINVAL),  # 384 % 100
    (dict(sx=376), _lib.EINVAL),  # row stride below dim
    (dict(act=2), _lib.EINVAL),
    (dict(x=0), _lib.EINVAL),
    (dict(w=0), _lib.EINVAL),
    (dict(st=0), _lib.EINVAL),
    (dict(qsl=0), _lib.EINVAL),
    (dict(ci=0), _lib.EINVAL),
    (dict(out=0), _lib.EINVAL),
    (dict(b=0), _lib.OK),  # no bias
    (dict(init=0), _lib.OK),  # no initial states
    (dict(dim=96, sx=96, pd=12), _lib.EUNSUPPORTED),  # part_dim not a multiple of 8
    (dict(sx=390), _lib.OK),  # rows not 16 bytes apart: unaligned vectors
    (dict(x=A + 2), _lib.OK),  # x at an odd column: unaligned vectors
    (dict(out=A + 8), _lib.OK),
    (dict(x=A + 1), _lib.EUNSUPPORTED),  # not aligned to the element size
    (dict(out=A + 1), _lib.EUNSUPPORTED),
    (dict(dt=_lib.F32, x=A + 2), _lib.EUNSUPPORTED),
    (dict(dt=_lib.F32, x=A + 4, sx=385), _lib.OK),
    (dict(cs1=-3), _lib.EUNSUPPORTED),
    (dict(T=0, x=0, out=0), _lib.OK),  # nothing to do: no launch, pointers unused
    (dict(S=0, qsl=0), _lib.OK),
    (dict(T=1 << 31), _lib.EUNSUPPORTED),
    (dict(dt=3), _lib.EINVAL),  # unknown format
    (dict(dt=-1), _lib.EINVAL),
    (dict(dt=_lib.F16), _lib.OK),
    (dict(dt=_lib.F32), _lib.OK),
    (dict(dt=_lib.F16, sx=388), _lib.OK),  # fp16 rows 776 bytes apart: unaligned vectors
    (dict(dt=_lib.F32, sx=388), _lib.OK),  # FP32 rows 1552 bytes apart
    (dict(dt=_lib.F32, sx=386), _lib.OK),
    (dict(dt=_lib.F32, T=1 << 25, pd=8, dim=8, sx=8), _lib.EUNSUPPORTED),  # plane of 2^30 bytes
    (dict(dt=_lib.BF16, T=1 << 25, pd=8, dim=8, sx=8), _lib.OK),
])
def test_validate_status_codes(kw, code):
    lib = _lib.load()
    assert lib.kdaconv_validate(*_args(**kw)) == code


def test_activation_map_argument_errors():
    lib = _lib.load()
    assert lib.kdaconv_activation_map(0, 7, 1, 0, A, None) == _lib.EINVAL  # not a multiple of 8
    assert lib.kdaconv_activation_map(0, 8, 5, 0, A, None) == _lib.EINVAL
    assert lib.kdaconv_activation_map(0, 8, 1, 3, A, None) == _lib.EINVAL  # unknown format
    assert lib.kdaconv_activation_map(0, 8, 1, 0, None, None) == _lib.EINVAL
    assert lib.kdaconv_activation_map(0, 8, 1, 2, A + 2, None) == _lib.EUNSUPPORTED
    assert lib.kdaconv_activation_map(0, 0, 1, 1, None, None) == _lib.OK


def test_python_checks_reject_host_tensors_and_bad_args():
    x = torch.zeros(4, 16, dtype=torch.bfloat16)
    w = torch.zeros(16, 4)
    st = torch.zeros(1, 16, 3)
    q = torch.tensor([0, 4], dtype=torch.int32)
    ci = torch.zeros(1, dtype=torch.int32)
    init = torch.zeros(1, dtype=torch.bool)
    with pytest.raises(ValueError):
        kd.packed_causal_conv1d_fn(x, w, None, st, q, ci, init, 8)
    assert not kd.packed_causal_conv1d_supported(x, w, st, 8)
    with pytest.raises(ValueError):
        kd._dtype_code(torch.float64)
    assert kd._dtype_code(torch.float16) == _lib.F16 and kd._dtype_code(torch.float32) == _lib.F32
    with pytest.raises(ValueError):
        kd._activation_code("gelu")
    assert kd._activation_code("swish") == _lib.ACT_SILU
    assert kd._activation_code(True) == _lib.ACT_SILU
    assert kd._activation_code(None) == _lib.ACT_NONE


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    monkeypatch.setattr(_lib, "LIBRARY", tmp_path / "absent.so")
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(_lib.LibraryMissing):
        _lib.load()


def _update_args(**kw):
    a = dict(x=A, dt=_lib.BF16, B=64, dim=384, sx=384, w=A, ws0=4, ws1=1, b=A, st=A, lines=4,
             cs0=1152, cs1=3, cs2=1, ci=A, cis=1, pd=128, act=1, hn=0, nid=0, out=A)
    a.update(kw)
    return [a["x"], a["dt"], a["B"], a["dim"], a["sx"], a["w"], a["ws0"], a["ws1"], a["b"],
            a["st"], a["lines"], a["cs0"], a["cs1"], a["cs2"], a["ci"], a["cis"], a["pd"],
            a["act"], a["hn"], a["nid"], a["out"], None]


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), _lib.EINVAL),
    (dict(dt=7), _lib.EINVAL),
    (dict(pd=100), _lib.EINVAL),
    (dict(sx=376), _lib.EINVAL),
    (dict(act=3), _lib.EINVAL),
    (dict(x=0), _lib.EINVAL),
    (dict(ci=0), _lib.EINVAL),
    (dict(out=0), _lib.EINVAL),
    (dict(dim=96, sx=96, pd=12), _lib.EUNSUPPORTED),
    (dict(x=A + 1), _lib.EUNSUPPORTED),
    (dict(out=A + 1), _lib.EUNSUPPORTED),
    (dict(dt=_lib.F32, x=A + 2), _lib.EUNSUPPORTED),
    (dict(cs2=-1), _lib.EUNSUPPORTED),
    (dict(B=0, x=0, out=0), _lib.OK),  # nothing to do: no launch
])
def test_update_status_codes(kw, code):
    """Argument checks of the decode entry point (they run before any HIP call)."""
    lib = _lib.load()
    assert lib.kdaconv_packed_causal_conv1d_update(*_update_args(**kw)) == code


def _update_bf16_args(**kw):
    a = dict(x=A, dt=_lib.BF16, B=64, dim=384, sx=384, w=A, wps=512, ws0=1, ws1=128, b=A, st=A,
             lines=4, cs0=1152, cs1=3, cs2=1, ci=A, cis=1, pd=128, act=1, hn=0, nid=0, out=A)
    a.update(kw)
    return [a["x"], a["dt"], a["B"], a["dim"], a["sx"], a["w"], a["wps"], a["ws0"], a["ws1"],
            a["b"], a["st"], a["lines"], a["cs0"], a["cs1"], a["cs2"], a["ci"], a["cis"],
            a["pd"], a["act"], a["hn"], a["nid"], a["out"], None]


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), _lib.EINVAL),
    (dict(dt=7), _lib.EINVAL),
    (dict(pd=100), _lib.EINVAL),
    (dict(act=3), _lib.EINVAL),
    (dict(x=0), _lib.EINVAL),
    (dict(w=0), _lib.EINVAL),
    (dict(st=0), _lib.EINVAL),
    (dict(ci=0), _lib.EINVAL),
    (dict(out=0), _lib.EINVAL),
    (dict(dt=_lib.F16), _lib.EUNSUPPORTED),  # the page's gate: bf16 input only
    (dict(dt=_lib.F32, sx=384), _lib.EUNSUPPORTED),
    (dict(wps=-1), _lib.EUNSUPPORTED),
    (dict(ws1=-128), _lib.EUNSUPPORTED),
    (dict(cs1=-3), _lib.EUNSUPPORTED),
    (dict(x=A + 1), _lib.EUNSUPPORTED),
    (dict(out=A + 3), _lib.EUNSUPPORTED),
    (dict(dim=96, sx=96, pd=12), _lib.EUNSUPPORTED),
    (dict(B=0, x=0, out=0), _lib.OK),  # nothing to do: no launch
    (dict(dim=0), _lib.OK),
])
def test_update_bf16_state_status_codes(kw, code):
    """Argument checks of the bf16-state decode entry point (before any HIP call)."""
    lib = _lib.load()
    assert lib.kdaconv_packed_causal_conv1d_update_bf16_state(*_update_bf16_args(**kw)) == code


def test_python_bf16_state_checks():
    """The binding's checks for a bf16 state run before the library is called."""
    x = torch.zeros((4, 384), dtype=torch.float16)
    st = torch.zeros((4, 384, 3), dtype=torch.bfloat16)
    w = torch.zeros((3, 4, 128), dtype=torch.float32)
    ci = torch.zeros(4, dtype=torch.int32)
    xb = torch.zeros((4, 384), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        kd.packed_causal_conv1d_update(xb, w, None, st, ci, 128)
    with pytest.raises(ValueError, match="bf16 x"):
        kd.packed_causal_conv1d_update(x, w, None, st, ci, 128)
    with pytest.raises(ValueError, match="width-major"):
        kd.packed_causal_conv1d_update(xb, torch.zeros((3, 128, 4)), None, st, ci, 128)
    assert kd._weight_strides(w, 128) == (512, 1, 128)
    assert kd._weight_strides(torch.zeros((384, 4)), 128) == (512, 4, 1)
