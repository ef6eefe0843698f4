"""Helpers shared by the GPU parity tests: inputs on the device, the oracle on
sampled tokens, error metrics.  The oracle only ever sees the inputs and the
router's fp32 logits, never the GPU's expert outputs."""
from __future__ import annotations

import dataclasses
import functools

import numpy as np
import pytest
import torch

import group_limited_routing_sigmoid_amd as gl
import oracle
from synth import WORKLOADS, Shape, make_inputs, small_shape, F32, BF16, FP8, MXFP4


def device():
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    gl.lib()   # raises if the HIP library is not built
    return torch.device("cuda:0")


@functools.lru_cache(maxsize=2)
def inputs(name: str, tokens=None, shape=None, bias=None, seed=None):
    w = WORKLOADS[name]
    return make_inputs(w, device=device(), tokens=tokens, shape=shape, bias=bias,
                       seed=seed)


def desc_for(w, shape, flags=0):
    act = gl.F32 if w.act_dtype == F32 else gl.BF16
    wd = {F32: gl.F32, BF16: gl.BF16, FP8: gl.FP8_E4M3, MXFP4: gl.MXFP4}[w.weight_dtype]
    return gl.make_desc(shape, act, wd, flags)


def max_rel_err(y, r) -> float:
    """max |y - r| / max |r| over the whole output."""
    y = np.asarray(y, np.float64)
    r = np.asarray(r, np.float64)
    return float(np.max(np.abs(y - r)) / np.max(np.abs(r)))


def oracle_forward(inp, shape, tokens, idx, w, act_quant=False):
    """Oracle block output for the listed tokens (binary64), given routing.
    Only the experts those tokens use are copied to the host."""
    tokens = np.asarray(tokens, np.int64)
    idx = np.asarray(idx)
    w = np.asarray(w, np.float32)
    sub = idx[tokens]
    need = np.unique(sub)
    remap = np.full(shape.n_experts, -1, np.int64)
    remap[need] = np.arange(need.size)
    sel = torch.as_tensor(need, device=inp.w_gate_up.device)
    wgu = inp.w_gate_up.index_select(0, sel).cpu()
    wd = inp.w_down.index_select(0, sel).cpu()
    sgu = sd = None
    if inp.s_gate_up is not None:
        sgu = inp.s_gate_up.index_select(0, sel).cpu()
        sd = inp.s_down.index_select(0, sel).cpu()
    x = inp.x[torch.as_tensor(tokens, device=inp.x.device)].cpu()
    return oracle.forward_tokens(shape, np.arange(tokens.size), x,
                                 remap[sub].astype(np.int32), w[tokens], wgu, wd,
                                 sgu, sd, act_quant=act_quant)


def logits_bound(inp, shape):
    """Rigorous bound on |fp32 logits - exact| for an accumulation of depth
    n <= H + 64 in binary32: n * 2^-24 * sum_k |x_k w_k| (per token, expert)."""
    ax = inp.x.double().abs()
    aw = inp.w_router.double().abs()
    s = (ax @ aw.T).cpu().numpy()
    n = shape.hidden + 64
    return n * 2.0 ** -24 * s
