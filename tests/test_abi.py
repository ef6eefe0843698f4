"""The C-ABI library loads, exports every entry point include/beam_moe.h
declares, and rejects bad arguments on the host before any GPU work (these
calls return before touching HIP, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

import group_limited_routing_sigmoid_amd as gl
from synth import BEAM, TINY

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "beam_moe.h")


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\**\s+\**(beam_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert set(names) == set(gl.SYMBOLS), names
    L = ctypes.CDLL(gl.LIB_PATH)
    for n in names:
        assert getattr(L, n) is not None


def _desc(**kw):
    d = gl.make_desc(BEAM, gl.BF16, gl.BF16)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def test_validate_accepts_layer_shapes():
    assert gl.validate(_desc(), 16384) == gl.OK
    assert gl.validate(gl.make_desc(TINY, gl.F32, gl.F32), 16) == gl.OK
    assert gl.validate(_desc(weight_dtype=gl.FP8_E4M3), 8192) == gl.OK
    assert gl.validate(_desc(), 0) == gl.OK
    assert gl.validate(_desc(flags=gl.PATH_GROUPED | gl.TILE_128), 64) == gl.OK
    assert gl.validate(_desc(flags=gl.TILE_256), 64) == gl.OK
    assert gl.validate(_desc(flags=gl.TILE_64), 64) == gl.OK


@pytest.mark.parametrize("field,value,status", [
    ("n_experts", 0, gl.ERR_UNSUPPORTED),
    ("n_experts", 2048, gl.ERR_UNSUPPORTED),
    ("n_groups", 7, gl.ERR_UNSUPPORTED),            # 256 % 7
    ("n_groups", 2, gl.ERR_UNSUPPORTED),            # 128 experts per group
    ("topk_groups", 9, gl.ERR_UNSUPPORTED),
    ("topk_groups", 0, gl.ERR_UNSUPPORTED),
    ("top_k", 17, gl.ERR_UNSUPPORTED),
    ("top_k", 0, gl.ERR_UNSUPPORTED),
    ("group_score_topn", 3, gl.ERR_UNSUPPORTED),
    ("hidden", 5000, gl.ERR_UNSUPPORTED),
    ("intermediate", 2500, gl.ERR_UNSUPPORTED),
    ("routed_scale", 0.0, gl.ERR_INVALID_ARG),
    ("routed_scale", float("inf"), gl.ERR_INVALID_ARG),
    ("act_dtype", 7, gl.ERR_INVALID_ARG),
    ("act_dtype", gl.F32, gl.ERR_UNSUPPORTED),      # bf16 weights need bf16 x
    ("weight_dtype", 9, gl.ERR_INVALID_ARG),
    ("flags", 1 << 9, gl.ERR_INVALID_ARG),
    ("flags", gl.PATH_STREAM | gl.PATH_GROUPED, gl.ERR_INVALID_ARG),
    ("flags", gl.TILE_128 | gl.TILE_256, gl.ERR_INVALID_ARG),
    ("flags", gl.TILE_160 | gl.TILE_256, gl.ERR_INVALID_ARG),
    ("flags", gl.TILE_64 | gl.TILE_128, gl.ERR_INVALID_ARG),
])
def test_validate_rejects(field, value, status):
    assert gl.validate(_desc(**{field: value}), 64) == status


def test_validate_small_top_k_bound():
    # top_k larger than the experts the kept groups hold
    d = gl.make_desc(TINY, gl.F32, gl.F32)
    d.top_k = 9                     # 2 groups of 4 experts kept
    assert gl.validate(d, 4) == gl.ERR_UNSUPPORTED
    assert gl.validate(gl.make_desc(TINY, gl.F32, gl.F32), -1) == gl.ERR_INVALID_ARG


def test_validate_bounds_expert_weight_offsets():
    # one expert's gate/up matrix (2 I H values) is addressed with 32-bit
    # element and byte offsets
    assert gl.validate(_desc(hidden=32768, intermediate=16384), 1) == gl.OK
    assert gl.validate(_desc(hidden=32768, intermediate=32768), 1) == gl.ERR_UNSUPPORTED
    assert gl.validate(_desc(hidden=65536, intermediate=16384), 1) == gl.ERR_UNSUPPORTED
    for wdt in (gl.FP8_E4M3, gl.MXFP4):
        assert gl.validate(_desc(hidden=65536, intermediate=16384, weight_dtype=wdt),
                           1) == gl.ERR_UNSUPPORTED


def test_workspace_bytes():
    assert gl.workspace_bytes(_desc(), 0) == 0
    a, b = gl.workspace_bytes(_desc(), 64), gl.workspace_bytes(_desc(), 16384)
    assert 0 < a < b
    # the grouped path keeps h and y in bf16: at least S*(I+H)*2 bytes
    assert b >= 16384 * 8 * (2560 + 5120) * 2


def test_host_errors_before_launch():
    L = gl.lib()
    d = _desc()
    null = None
    # T == 0 is a no-op that succeeds without touching the device
    assert L.beam_moe_forward(ctypes.byref(d), 0, *([null] * 12), 0, null) == gl.OK
    # missing inputs
    assert L.beam_moe_route(ctypes.byref(d), 8, null, null, null, null, null,
                            null, null, 0, null) == gl.ERR_INVALID_ARG
    # misaligned pointer
    bad = ctypes.c_void_p(0x1001)
    good = ctypes.c_void_p(0x10000)
    assert L.beam_moe_route(ctypes.byref(d), 8, bad, good, null, null, good,
                            good, good, 1 << 30, null) == gl.ERR_INVALID_ARG
    # workspace too small
    assert L.beam_moe_route(ctypes.byref(d), 8, good, good, null, null, good,
                            good, good, 16, null) == gl.ERR_WORKSPACE
    assert L.beam_moe_forward(ctypes.byref(d), 8, good, good, null, good, null,
                              good, null, good, null, null, null, good, 16,
                              null) == gl.ERR_WORKSPACE
    # FP8 weights without their scales
    d8 = _desc(weight_dtype=gl.FP8_E4M3)
    assert L.beam_moe_forward(ctypes.byref(d8), 8, good, good, null, good, null,
                              good, null, good, null, null, null, good, 1 << 40,
                              null) == gl.ERR_INVALID_ARG
    # quantiser shape rule
    assert L.beam_moe_quant_e4m3(4, 100, gl.F32, good, good, good, null) == gl.ERR_UNSUPPORTED
    assert L.beam_moe_quant_e4m3(4, 128, 5, good, good, good, null) == gl.ERR_INVALID_ARG


def test_status_strings():
    for s in (gl.OK, gl.ERR_INVALID_ARG, gl.ERR_UNSUPPORTED, gl.ERR_WORKSPACE, gl.ERR_HIP):
        assert gl.status_string(s)
    assert gl.status_string(-99) == "unknown status"
