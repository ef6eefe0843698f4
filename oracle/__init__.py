"""Python face of the CPU oracle for the Beam MoE block.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
benchmark's CPU-baseline leg.  The GPU library and its Python binding never
import it.

What each oracle function follows, and what pins it (tests/test_oracle_*.py):
  * sigmoid32      -- the sigmoid of the router scores ("Reflection Releases
                      Beam ...", section "Where Beam Saves and Where the
                      Memory Bill Comes In").  Pinned against a 60-digit
                      decimal evaluation rounded to binary32.
  * route          -- group-limited top-k of that section and of "Reflection
                      Beam", section "What Beam is"; bias for selection only
                      from the load-balancing paragraph of "Reflection AI
                      Introduces Beam ...".  Pinned by an exact-rational
                      brute force over all group and expert subsets
                      (oracle/bruteforce.py), by the special case where all
                      groups are kept (a stable argsort), and by invariants.
                      The group score (sum of the two largest biased scores)
                      is DeepSeek-V3's rule, which the pages invoke but do not
                      state: the brute force enumerates that same rule, so the
                      rule itself is "parity unpinned" against the pages.
  * logits         -- binary64 x W_r^T.  Pinned against torch float64 matmul.
  * forward_tokens -- SwiGLU experts and weighted combine.  Pinned by the
                      one-expert case (torch float64 dense SwiGLU), identical
                      experts (2.5 x one expert), experts differing only by a
                      down-projection factor (checks which weight goes with
                      which expert), and token-permutation invariance.
  * bias_update    -- aux-loss-free balancing step (load-balancing paragraph
                      of "Reflection AI Introduces Beam ..."; rule of
                      DeepSeek-V3).  Pinned by a closed form on crafted loads
                      and by repeated route/update rounds driving the expert
                      load towards balance (a flipped sign diverges).
  * residual_epilogue -- post-block RMSNorm (SandwichNorm's post-norm) and
                      the depth-scaled FP32 residual stream ("Reflection Beam",
                      section "Hybrid Attention and Unusual Residuals").
                      Pinned by the telescoped stream (after steps 1..K every
                      addend carries weight 1/sqrt(K)), the unit-scale
                      property (the two weights' squares sum to one), the
                      constant-row closed form of the norm and its scale
                      invariance.  The norm's eps and weights are not on the
                      pages: caller inputs.
  * MX codecs      -- OCP Microscaling v1.0: E2M1 elements pinned against
                      the specification's value table (tests/golden) and a
                      brute-force nearest-even encoder; E8M0 scales against
                      torch.float8_e8m0fnu; the OCP shared-exponent rule by
                      the block maximum landing in the element format's top
                      binade; the activation blocks' exponent (a reading:
                      the smallest power of two keeping the maximum within
                      448, no saturation) by its range (224, 448]; MXFP8
                      elements against torch e4m3fn of the exactly scaled
                      values.  MXFP4 weights with MXFP8
                      activations stand in for the pages' 4-bit (NVFP4)
                      checkpoint: parity with NVFP4 itself is not claimed.
  * e4m3 codec     -- pinned against torch.float8_e4m3fn on all 256 codes and
                      on random values.  The FP8 activation recipe (per-128
                      amax/448 scales) is a reading the pages do not fix:
                      "parity unpinned" beyond the codec and its definition.
"""
from __future__ import annotations

import contextlib
import ctypes
import os

import numpy as np

from . import build as _build

F32, BF16, E4M3, MXFP4 = 0, 1, 2, 3

_lib = None


class Shape(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("group_score_topn", ctypes.c_int32),
                ("routed_scale", ctypes.c_float)]


def shape_of(s) -> Shape:
    """Build the oracle's shape struct from any object with the same fields."""
    return Shape(s.hidden, s.intermediate, s.n_experts, s.n_groups,
                 s.topk_groups, s.top_k, getattr(s, "group_score_topn", 2),
                 getattr(s, "routed_scale", 2.5))


def lib():
    global _lib
    if _lib is None and os.environ.get("BEAM_ORACLE_LIB"):
        # another build of the oracle's source (the host-sanitizer runs)
        _lib = _bind(ctypes.CDLL(os.environ["BEAM_ORACLE_LIB"]))
    if _lib is None:
        if not os.path.exists(_build.LIB) or (
                os.path.getmtime(_build.LIB) < os.path.getmtime(_build.SRC)):
            _build.build()
        _lib = _bind(ctypes.CDLL(_build.LIB))
    return _lib


@contextlib.contextmanager
def library(path: str):
    """Run the wrapper's functions on another build of the oracle's source
    (the tests compile copies with planted mistakes to show that a pin
    catches them), restoring the regular build afterwards."""
    global _lib
    saved = lib()
    _lib = _bind(ctypes.CDLL(path))
    try:
        yield
    finally:
        _lib = saved


def _bind(L):
    """Declare the argument and result types of the oracle's exports."""
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.bo_sigmoid32.argtypes = [ctypes.c_float]
    L.bo_sigmoid32.restype = ctypes.c_float
    L.bo_sigmoid_f64.argtypes = [ctypes.c_float]
    L.bo_sigmoid_f64.restype = ctypes.c_double
    L.bo_e4m3_decode.argtypes = [ctypes.c_uint8]
    L.bo_e4m3_decode.restype = ctypes.c_double
    L.bo_e4m3_encode.argtypes = [ctypes.c_float]
    L.bo_e4m3_encode.restype = ctypes.c_uint8
    L.bo_route.argtypes = [ctypes.POINTER(Shape), i64, vp, vp, vp, vp, vp]
    L.bo_route.restype = i32
    L.bo_logits.argtypes = [ctypes.POINTER(Shape), i64, vp, i32, vp, vp, i32]
    L.bo_logits.restype = None
    L.bo_e2m1_decode.argtypes = [ctypes.c_uint8]
    L.bo_e2m1_decode.restype = ctypes.c_double
    L.bo_e2m1_encode.argtypes = [ctypes.c_double]
    L.bo_e2m1_encode.restype = ctypes.c_uint8
    L.bo_mx_scale.argtypes = [ctypes.c_double, i32]
    L.bo_mx_scale.restype = ctypes.c_uint8
    L.bo_quant_mx.argtypes = [vp, i64, i32, vp, vp]
    L.bo_mx8_act_scale.argtypes = [ctypes.c_double]
    L.bo_mx8_act_scale.restype = ctypes.c_uint8
    L.bo_quant_mx.restype = None
    L.bo_quant_e4m3.argtypes = [vp, i64, i32, vp, vp]
    L.bo_quant_e4m3.restype = None
    L.bo_forward_tokens.argtypes = [ctypes.POINTER(Shape), i64, vp, vp, i32,
                                    vp, vp, vp, vp, vp, vp, i32, i32, vp, i32]
    L.bo_forward_tokens.restype = i32
    L.bo_bias_update.argtypes = [i32, i64, i32, vp, ctypes.c_float, vp]
    L.bo_bias_update.restype = None
    L.bo_residual_epilogue.argtypes = [i64, i32, vp, vp, ctypes.c_double, i32, vp]
    L.bo_residual_epilogue.restype = None
    L.bo_bias_gamma.argtypes = [i64, i64, ctypes.c_float, ctypes.c_float]
    L.bo_bias_gamma.restype = ctypes.c_float
    L.bo_max_threads.argtypes = []
    L.bo_max_threads.restype = i32
    return L


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.c_void_p)


def _np(t):
    """torch tensor (any device) or ndarray -> contiguous host ndarray, with
    bf16 kept as its raw uint16 bits."""
    try:
        import torch
        if isinstance(t, torch.Tensor):
            t = t.detach()
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
                return np.ascontiguousarray(t.cpu().numpy().view(np.uint16))
            return np.ascontiguousarray(t.cpu().numpy())
    except ImportError:
        pass
    return np.ascontiguousarray(t)


def _dtype_code(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(a.dtype)


def max_threads() -> int:
    return lib().bo_max_threads()


def sigmoid32(v) -> np.ndarray:
    v = np.asarray(v, dtype=np.float32).ravel()
    f = lib().bo_sigmoid32
    return np.array([f(float(a)) for a in v], dtype=np.float32)


def sigmoid_f64(v) -> np.ndarray:
    """The binary64 sigmoid value before its rounding to binary32."""
    v = np.asarray(v, dtype=np.float32).ravel()
    f = lib().bo_sigmoid_f64
    return np.array([f(float(a)) for a in v], dtype=np.float64)


def e4m3_decode(codes) -> np.ndarray:
    f = lib().bo_e4m3_decode
    return np.array([f(int(c)) for c in np.asarray(codes).ravel()])


def e4m3_encode(v) -> np.ndarray:
    f = lib().bo_e4m3_encode
    return np.array([f(float(a)) for a in np.asarray(v, np.float32).ravel()],
                    dtype=np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    """OCP MX FP4 (E2M1) values of 4-bit codes."""
    f = lib().bo_e2m1_decode
    return np.array([f(int(c)) for c in np.asarray(codes).ravel()])


def e2m1_encode(v) -> np.ndarray:
    f = lib().bo_e2m1_encode
    return np.array([f(float(a)) for a in np.asarray(v, np.float64).ravel()], dtype=np.uint8)


def mx_scale(amax, emax_elem) -> int:
    """E8M0 code of an MX block's shared scale."""
    return int(lib().bo_mx_scale(float(amax), int(emax_elem)))


def mx8_act_scale(amax) -> int:
    """E8M0 code of the 4-bit variant's activation blocks (no saturation)."""
    return int(lib().bo_mx8_act_scale(float(amax)))


def quant_mx(v, fmt: int):
    """MX quantisation of each row of v [rows, n] (n a multiple of 32):
    fmt 4 -> (E2M1 codes packed [rows, n/2] uint8, E8M0 scales [rows, n/32]),
    OCP shared exponent; fmt 8 -> (E4M3 codes [rows, n] uint8, E8M0 scales),
    the activation recipe's exponent (block maximum within 448)."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    rows, n = v.reshape(-1, v.shape[-1]).shape
    q = np.zeros((rows, n // 2 if fmt == 4 else n), np.uint8)
    sc = np.empty((rows, n // 32), np.uint8)
    lib().bo_quant_mx(_ptr(v), rows * n, int(fmt), _ptr(q), _ptr(sc))
    return (q.reshape(v.shape[:-1] + (q.shape[-1],)),
            sc.reshape(v.shape[:-1] + (n // 32,)))


def quant_e4m3(v, block: int = 128):
    """Per-block dynamic e4m3 quantisation of each row of v [rows, n]."""
    v = np.ascontiguousarray(np.asarray(v, dtype=np.float32))
    rows, n = v.reshape(-1, v.shape[-1]).shape
    q = np.empty((rows, n), np.uint8)
    s = np.empty((rows, n // block), np.float32)
    lib().bo_quant_e4m3(_ptr(v), rows * n, block, _ptr(q), _ptr(s))
    return q.reshape(v.shape), s.reshape(v.shape[:-1] + (n // block,))


def route(shape, logits, bias=None):
    """Route every token from fp32 logits [T, E]: returns (idx [T,K] int32,
    w [T,K] float32, kept groups [T,TG] int32)."""
    sh = shape_of(shape)
    lg = np.ascontiguousarray(_np(logits), dtype=np.float32)
    T = lg.shape[0]
    b = None if bias is None else np.ascontiguousarray(_np(bias), np.float32)
    idx = np.empty((T, sh.top_k), np.int32)
    w = np.empty((T, sh.top_k), np.float32)
    kept = np.empty((T, sh.topk_groups), np.int32)
    rc = lib().bo_route(ctypes.byref(sh), T, _ptr(lg),
                        None if b is None else _ptr(b), _ptr(idx), _ptr(w),
                        _ptr(kept))
    if rc:
        raise ValueError("oracle route: shape cannot supply top_k experts")
    return idx, w, kept


def logits(shape, x, w_router, nthreads: int = 0) -> np.ndarray:
    """binary64 router logits [T, E]."""
    sh = shape_of(shape)
    xa = _np(x)
    wr = np.ascontiguousarray(_np(w_router), np.float32)
    T = xa.shape[0]
    out = np.empty((T, sh.n_experts), np.float64)
    lib().bo_logits(ctypes.byref(sh), T, _ptr(xa), _dtype_code(xa), _ptr(wr),
                    _ptr(out), nthreads)
    return out


def forward_tokens(shape, tokens, x, idx, w, w_gate_up, w_down,
                   s_gate_up=None, s_down=None, act_quant: bool = False,
                   nthreads: int = 0) -> np.ndarray:
    """binary64 block output for the listed tokens given their routing.
    Weights may be f32, bf16 (uint16 bits), e4m3 codes (uint8) with fp32
    per-128x128 scales, or MXFP4 (E2M1 codes packed two per byte, uint8)
    with E8M0 scales (uint8) per 32 values of a row."""
    sh = shape_of(shape)
    tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    xa = _np(x)
    idx = np.ascontiguousarray(_np(idx), np.int32)
    w = np.ascontiguousarray(_np(w), np.float32)
    wgu = _np(w_gate_up)
    wd = _np(w_down)
    dt = _dtype_code(wgu)
    assert _dtype_code(wd) == dt
    sgu = None if s_gate_up is None else np.ascontiguousarray(_np(s_gate_up))
    sdn = None if s_down is None else np.ascontiguousarray(_np(s_down))
    if dt == E4M3:
        assert sgu is not None and sdn is not None
        if sgu.dtype == np.uint8:        # E8M0 scales: packed MXFP4 weights
            assert sdn.dtype == np.uint8
            dt = MXFP4
        else:
            sgu, sdn = sgu.astype(np.float32), sdn.astype(np.float32)
    out = np.empty((tok.size, sh.hidden), np.float64)
    rc = lib().bo_forward_tokens(
        ctypes.byref(sh), tok.size, _ptr(tok), _ptr(xa), _dtype_code(xa),
        _ptr(idx), _ptr(w), _ptr(wgu), None if sgu is None else _ptr(sgu),
        _ptr(wd), None if sdn is None else _ptr(sdn), dt, int(act_quant),
        _ptr(out), nthreads)
    if rc:
        raise ValueError("oracle forward: unsupported shape")
    return out


def bias_update(n_experts, idx, gamma, bias):
    """Aux-loss-free balancing step: returns the updated fp32 bias."""
    idx = np.ascontiguousarray(_np(idx), np.int32)
    b = np.array(_np(bias), dtype=np.float32, copy=True)
    T, K = idx.shape
    lib().bo_bias_update(n_experts, T, K, _ptr(idx), float(gamma), _ptr(b))
    return b


def bias_gamma(t, n, g0, g1):
    """Cosine-decayed update speed for step t of n."""
    return lib().bo_bias_gamma(t, n, g0, g1)


def residual_epilogue(out, gamma, eps, k, residual):
    """Post-block RMSNorm and depth-scaled residual update (binary64):
    returns sqrt((k-1)/k) * residual + RMSNorm(out) * gamma / sqrt(k)."""
    o = np.ascontiguousarray(_np(out), np.float64)
    r = np.array(_np(residual), dtype=np.float64, copy=True)
    g = np.ascontiguousarray(_np(gamma), np.float32)
    T, H = o.shape
    assert r.shape == (T, H) and g.shape == (H,) and k >= 1
    lib().bo_residual_epilogue(T, H, _ptr(o), _ptr(g), float(eps), int(k), _ptr(r))
    return r
