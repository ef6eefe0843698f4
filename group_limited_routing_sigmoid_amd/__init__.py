"""Python binding of libbeam_moe.so, the MI355X (gfx950) Beam MoE block.

Argument marshalling only: every step of the block runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  The names
follow the C ABI in include/beam_moe.h (beam_moe_route, beam_moe_forward,
beam_moe_permute, beam_moe_quant_e4m3, beam_moe_workspace_bytes,
beam_moe_validate).  There is no CPU fallback: without the built library
every call raises.
"""
from __future__ import annotations

import contextlib
import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# another build of the same library (e.g. a host-sanitizer build) may be
# named in BEAM_MOE_LIB; there is no fallback when the file is missing
LIB_PATH = os.environ.get("BEAM_MOE_LIB") or os.path.join(_HERE, "libbeam_moe.so")

F32, BF16, FP8_E4M3, MXFP4 = 0, 1, 2, 3
ROUTE_LOGITS_IN, PATH_STREAM, PATH_GROUPED = 1 << 0, 1 << 1, 1 << 2
TILE_128, TILE_256, TILE_160, TILE_64 = 1 << 3, 1 << 4, 1 << 5, 1 << 6
OK, ERR_INVALID_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4

SYMBOLS = ("beam_status_string", "beam_moe_validate", "beam_moe_workspace_bytes",
           "beam_moe_route", "beam_moe_permute", "beam_moe_quant_e4m3",
           "beam_moe_forward", "beam_moe_timer_create", "beam_moe_timer_destroy",
           "beam_moe_timer_reset", "beam_moe_timer_count", "beam_moe_timer_read",
           "beam_moe_forward_timed", "beam_moe_bias_update", "beam_moe_bias_gamma",
           "beam_moe_forward_residual", "beam_moe_quant_mxfp8",
           "beam_moe_forward_noalloc")
NOALLOC_SCRATCH_BYTES = 64 << 20


class Desc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("topk_groups", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("group_score_topn", ctypes.c_int32),
                ("routed_scale", ctypes.c_float), ("act_dtype", ctypes.c_int32),
                ("weight_dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


class BeamError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} ({status})")


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m group_limited_routing_sigmoid_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        D = ctypes.POINTER(Desc)
        L.beam_status_string.argtypes = [ctypes.c_int]
        L.beam_status_string.restype = ctypes.c_char_p
        L.beam_moe_validate.argtypes = [D, i64]
        L.beam_moe_workspace_bytes.argtypes = [D, i64, ctypes.POINTER(sz)]
        L.beam_moe_route.argtypes = [D, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_permute.argtypes = [D, i64, vp, vp, vp, vp, vp, vp, sz, vp]
        L.beam_moe_quant_e4m3.argtypes = [i64, i64, i32, vp, vp, vp, vp]
        L.beam_moe_quant_mxfp8.argtypes = [i64, i64, i32, vp, vp, vp, vp]
        L.beam_moe_forward.argtypes = [D, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, vp, vp, vp, sz, vp]
        L.beam_moe_forward_timed.argtypes = L.beam_moe_forward.argtypes + [vp]
        L.beam_moe_forward_noalloc.argtypes = [D, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, vp, vp, vp]
        L.beam_moe_forward_residual.argtypes = [D, i64, vp, vp, vp, vp, vp, vp, vp, vp,
                                                ctypes.c_float, i32, vp, vp, vp, sz, vp]
        L.beam_moe_timer_create.argtypes = [i32, ctypes.POINTER(vp)]
        L.beam_moe_timer_destroy.argtypes = [vp]
        L.beam_moe_timer_destroy.restype = None
        L.beam_moe_timer_reset.argtypes = [vp]
        L.beam_moe_timer_reset.restype = None
        L.beam_moe_timer_count.argtypes = [vp]
        L.beam_moe_timer_read.argtypes = [vp, i32, ctypes.POINTER(ctypes.c_char_p),
                                          ctypes.POINTER(ctypes.c_float)]
        L.beam_moe_bias_update.argtypes = [D, i64, vp, ctypes.c_float, vp, vp]
        L.beam_moe_bias_gamma.argtypes = [i64, i64, ctypes.c_float, ctypes.c_float]
        L.beam_moe_bias_gamma.restype = ctypes.c_float
        for f in SYMBOLS[1:]:
            if getattr(L, f).restype is ctypes.c_int or f in (
                    "beam_moe_timer_destroy", "beam_moe_timer_reset",
                    "beam_moe_bias_gamma"):
                continue
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().beam_status_string(status).decode()


def _check(status: int, what: str):
    if status != OK:
        raise BeamError(status, what)


def make_desc(shape, act_dtype: int, weight_dtype: int, flags: int = 0) -> Desc:
    """Descriptor from any object with the layer-shape fields (hidden,
    intermediate, n_experts, n_groups, topk_groups, top_k, group_score_topn,
    routed_scale)."""
    return Desc(shape.hidden, shape.intermediate, shape.n_experts,
                shape.n_groups, shape.topk_groups, shape.top_k,
                getattr(shape, "group_score_topn", 2),
                getattr(shape, "routed_scale", 2.5), act_dtype, weight_dtype,
                flags)


def with_flags(desc: Desc, flags: int) -> Desc:
    d = Desc.from_buffer_copy(desc)
    d.flags = flags
    return d


def validate(desc: Desc, T: int) -> int:
    return lib().beam_moe_validate(ctypes.byref(desc), T)


def workspace_bytes(desc: Desc, T: int) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().beam_moe_workspace_bytes(ctypes.byref(desc), T, ctypes.byref(n)),
           "beam_moe_workspace_bytes")
    return n.value


def _p(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP library must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _torch_stream(stream, device):
    return stream if stream is not None else torch.cuda.current_stream(device)


def _stream(stream=None, device=None):
    return ctypes.c_void_p(_torch_stream(stream, device).cuda_stream)


class Workspace:
    """A growable device byte buffer reused across calls.

    Calls that may overlap (calls on different streams) need distinct
    workspaces.  The buffer is allocated on the stream of the call that
    grows it, and marked as used by any other stream a later call runs on,
    so torch's allocator never hands its memory out again while queued
    kernels may still use it."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = None
        self.streams = set()

    def get(self, nbytes: int, stream=None) -> Optional[torch.Tensor]:
        if nbytes == 0:
            return None
        s = _torch_stream(stream, self.device)
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = None
            with torch.cuda.stream(s):
                self.buf = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
            self.streams = {s.cuda_stream}
        elif s.cuda_stream not in self.streams:
            self.buf.record_stream(s)
            self.streams.add(s.cuda_stream)
        return self.buf


# one default workspace per (device, stream): calls on one stream are
# ordered, calls on different streams never share scratch memory
_default_ws = {}


def _ws(desc: Desc, T: int, workspace: Optional[Workspace], device, stream=None):
    n = workspace_bytes(desc, T)
    s = _torch_stream(stream, device)
    if workspace is None:
        key = (str(device), s.cuda_stream)
        workspace = _default_ws.setdefault(key, Workspace(device))
    return workspace.get(n, s), n


def _alloc_on(stream):
    """Context in which the binding allocates a call's outputs: the call's
    stream, so that torch's allocator orders their reuse after its kernels."""
    return torch.cuda.stream(stream) if stream is not None else contextlib.nullcontext()


def route(desc: Desc, x: Optional[torch.Tensor], w_router: Optional[torch.Tensor],
          bias: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
          workspace: Optional[Workspace] = None, stream=None):
    """beam_moe_route.  Returns (topk_idx [T,K] int32, topk_w [T,K] fp32,
    logits [T,E] fp32).  With ROUTE_LOGITS_IN in desc.flags, `logits` is the
    input and x / w_router may be None."""
    lin = bool(desc.flags & ROUTE_LOGITS_IN)
    ref = logits if lin else x
    T, dev = ref.shape[0], ref.device
    with _alloc_on(stream):
        idx = torch.empty(T, desc.top_k, dtype=torch.int32, device=dev)
        w = torch.empty(T, desc.top_k, dtype=torch.float32, device=dev)
        if logits is None:
            logits = torch.empty(T, desc.n_experts, dtype=torch.float32, device=dev)
    buf, n = _ws(desc, T, workspace, dev, stream)
    _check(lib().beam_moe_route(ctypes.byref(desc), T, _p(x), _p(w_router),
                                _p(bias), _p(logits), _p(idx), _p(w), _p(buf),
                                n, _stream(stream, dev)), "beam_moe_route")
    return idx, w, logits


def permute(desc: Desc, topk_idx: torch.Tensor,
            workspace: Optional[Workspace] = None, stream=None):
    """beam_moe_permute.  Returns dict(counts, offsets, slot_token, slot_of)."""
    T, dev = topk_idx.shape[0], topk_idx.device
    E, S = desc.n_experts, T * desc.top_k
    with _alloc_on(stream):
        out = dict(counts=torch.empty(E, dtype=torch.int32, device=dev),
                   offsets=torch.empty(E + 1, dtype=torch.int32, device=dev),
                   slot_token=torch.empty(max(S, 1), dtype=torch.int32, device=dev),
                   slot_of=torch.empty(max(S, 1), dtype=torch.int32, device=dev))
    buf, n = _ws(desc, T, workspace, dev, stream)
    _check(lib().beam_moe_permute(ctypes.byref(desc), T, _p(topk_idx),
                                  _p(out["counts"]), _p(out["offsets"]),
                                  _p(out["slot_token"]), _p(out["slot_of"]),
                                  _p(buf), n, _stream(stream, dev)), "beam_moe_permute")
    out["slot_token"] = out["slot_token"][:S]
    out["slot_of"] = out["slot_of"][:S].view(T, desc.top_k)
    return out


def forward_residual(desc: Desc, x: torch.Tensor, w_router: Optional[torch.Tensor],
                     bias: Optional[torch.Tensor], w_gate_up: torch.Tensor,
                     w_down: torch.Tensor, norm_weight: torch.Tensor, eps: float,
                     step: int, residual: torch.Tensor,
                     s_gate_up: Optional[torch.Tensor] = None,
                     s_down: Optional[torch.Tensor] = None,
                     out: Optional[torch.Tensor] = None,
                     workspace: Optional[Workspace] = None, stream=None):
    """beam_moe_forward_residual: the block, then residual (fp32 [T,H], in
    place) = sqrt((k-1)/k) residual + RMSNorm(block output) * norm_weight /
    sqrt(k).  Returns residual (and writes out when given)."""
    T, dev = x.shape[0], x.device
    buf, n = _ws(desc, T, workspace, dev, stream)
    _check(lib().beam_moe_forward_residual(
        ctypes.byref(desc), T, _p(x), _p(w_router), _p(bias), _p(w_gate_up),
        _p(s_gate_up), _p(w_down), _p(s_down), _p(norm_weight), float(eps),
        int(step), _p(residual), _p(out), _p(buf), n, _stream(stream, dev)),
        "beam_moe_forward_residual")
    return residual


def bias_update(desc: Desc, topk_idx: torch.Tensor, gamma: float,
                bias: torch.Tensor, stream=None):
    """beam_moe_bias_update: one balancing step on `bias` (in place)."""
    _check(lib().beam_moe_bias_update(ctypes.byref(desc), topk_idx.shape[0],
                                      _p(topk_idx), float(gamma), _p(bias),
                                      _stream(stream, bias.device)), "beam_moe_bias_update")
    return bias


def bias_gamma(t: int, n: int, g0: float, g1: float) -> float:
    """beam_moe_bias_gamma: cosine-decayed update speed (host only)."""
    return lib().beam_moe_bias_gamma(t, n, g0, g1)


def quant_e4m3(v: torch.Tensor, stream=None):
    """beam_moe_quant_e4m3 of a 2-D fp32/bf16 tensor: (codes uint8, scales)."""
    rows, cols = v.shape
    dt = BF16 if v.dtype == torch.bfloat16 else F32
    if v.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(v.dtype)
    with _alloc_on(stream):
        q = torch.empty(rows, cols, dtype=torch.uint8, device=v.device)
        s = torch.empty(rows, max(cols // 128, 1), dtype=torch.float32, device=v.device)
    _check(lib().beam_moe_quant_e4m3(rows, cols, dt, _p(v), _p(q), _p(s),
                                     _stream(stream, v.device)), "beam_moe_quant_e4m3")
    return q, s[:, :cols // 128]


def quant_mxfp8(v: torch.Tensor, stream=None):
    """beam_moe_quant_mxfp8 of a 2-D fp32/bf16 tensor: (codes uint8, E8M0
    scales uint8 [rows, cols/32])."""
    rows, cols = v.shape
    if v.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError(v.dtype)
    dt = BF16 if v.dtype == torch.bfloat16 else F32
    with _alloc_on(stream):
        q = torch.empty(rows, cols, dtype=torch.uint8, device=v.device)
        s = torch.empty(rows, max(cols // 32, 16), dtype=torch.uint8, device=v.device)
    _check(lib().beam_moe_quant_mxfp8(rows, cols, dt, _p(v), _p(q), _p(s),
                                      _stream(stream, v.device)), "beam_moe_quant_mxfp8")
    return q, s[:, :cols // 32]


class Timer:
    """beam_moe_timer: HIP event pairs around each kernel of a timed forward."""

    def __init__(self, capacity: int = 4096):
        h = ctypes.c_void_p()
        _check(lib().beam_moe_timer_create(capacity, ctypes.byref(h)),
               "beam_moe_timer_create")
        self.handle = h

    def reset(self):
        lib().beam_moe_timer_reset(self.handle)

    def records(self):
        """[(kernel name, ms)] in launch order; waits for the events."""
        L = lib()
        out = []
        for i in range(L.beam_moe_timer_count(self.handle)):
            name, ms = ctypes.c_char_p(), ctypes.c_float()
            _check(L.beam_moe_timer_read(self.handle, i, ctypes.byref(name),
                                         ctypes.byref(ms)), "beam_moe_timer_read")
            out.append((name.value.decode(), ms.value))
        return out

    def __del__(self):
        if getattr(self, "handle", None) and _lib is not None:
            _lib.beam_moe_timer_destroy(self.handle)
            self.handle = None


def forward(desc: Desc, x: torch.Tensor, w_router: Optional[torch.Tensor],
            bias: Optional[torch.Tensor], w_gate_up: torch.Tensor,
            w_down: torch.Tensor, s_gate_up: Optional[torch.Tensor] = None,
            s_down: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, logits: Optional[torch.Tensor] = None,
            return_routing: bool = False, workspace: Optional[Workspace] = None,
            stream=None, timer: Optional[Timer] = None):
    """beam_moe_forward (beam_moe_forward_timed with a timer).  Returns out
    [T,H] (act dtype), or (out, topk_idx, topk_w, logits) with
    return_routing."""
    T, dev = x.shape[0], x.device
    idx = w = None
    with _alloc_on(stream):
        if out is None:
            out = torch.empty(T, desc.hidden, dtype=x.dtype, device=dev)
        if return_routing:
            idx = torch.empty(T, desc.top_k, dtype=torch.int32, device=dev)
            w = torch.empty(T, desc.top_k, dtype=torch.float32, device=dev)
            if logits is None:
                logits = torch.empty(T, desc.n_experts, dtype=torch.float32, device=dev)
    buf, n = _ws(desc, T, workspace, dev, stream)
    args = [ctypes.byref(desc), T, _p(x), _p(w_router), _p(bias), _p(w_gate_up),
            _p(s_gate_up), _p(w_down), _p(s_down), _p(out), _p(idx), _p(w),
            _p(logits), _p(buf), n, _stream(stream, dev)]
    if timer is None:
        _check(lib().beam_moe_forward(*args), "beam_moe_forward")
    else:
        _check(lib().beam_moe_forward_timed(*args, timer.handle),
               "beam_moe_forward_timed")
    if return_routing:
        return out, idx, w, logits
    return out


def forward_noalloc(desc: Desc, x: torch.Tensor, w_router: Optional[torch.Tensor],
                    bias: Optional[torch.Tensor], w_gate_up: torch.Tensor,
                    w_down: torch.Tensor, out: torch.Tensor,
                    s_gate_up: Optional[torch.Tensor] = None,
                    s_down: Optional[torch.Tensor] = None,
                    topk_idx: Optional[torch.Tensor] = None,
                    topk_w: Optional[torch.Tensor] = None,
                    logits: Optional[torch.Tensor] = None, stream=None):
    """beam_moe_forward_noalloc: the block with the library's own per-device
    scratch array as workspace (at most NOALLOC_SCRATCH_BYTES).  Every output
    is the caller's; nothing is allocated.  Calls that may overlap on one GPU
    race on the shared array."""
    T, dev = x.shape[0], x.device
    _check(lib().beam_moe_forward_noalloc(
        ctypes.byref(desc), T, _p(x), _p(w_router), _p(bias), _p(w_gate_up),
        _p(s_gate_up), _p(w_down), _p(s_down), _p(out), _p(topk_idx), _p(topk_w),
        _p(logits), _stream(stream, dev)), "beam_moe_forward_noalloc")
    return out
