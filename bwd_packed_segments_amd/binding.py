"""ctypes binding of libbps_attn.so (declared in include/bps_attn.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the computation runs in the library's
HIP kernels.  There is no fallback: if the library is missing or a call
fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os
import threading
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))

ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_WORKSPACE, ATTN_E_DEVICE = range(5)
ATTN_BF16, ATTN_FP32 = 0, 1
ATTN_FORCE_GENERAL = 1 << 0
ATTN_REVERSE_SCHEDULE = 1 << 1
ATTN_FUSED_BWD = 1 << 2
ATTN_LOG_ROUTE = 1 << 3
ROUTE_NAMES = {0: "dense", 1: "fast", 2: "general"}

STATUS_NAMES = {
    ATTN_OK: "ATTN_OK", ATTN_E_INVALID: "ATTN_E_INVALID", ATTN_E_UNSUPPORTED: "ATTN_E_UNSUPPORTED",
    ATTN_E_WORKSPACE: "ATTN_E_WORKSPACE", ATTN_E_DEVICE: "ATTN_E_DEVICE",
}

# Every symbol the header declares (the CPU tests check the library exports them).
EXPORTS = ("attn_fwd_workspace_size", "attn_bwd_workspace_size", "attn_fwd", "attn_bwd", "attn_bwd_phase",
           "attn_debug_mask", "attn_ring_fwd_workspace_size", "attn_ring_bwd_workspace_size", "attn_ring_fwd",
           "attn_ring_bwd", "attn_fwd_ex_workspace_size", "attn_bwd_ex_workspace_size", "attn_fwd_ex",
           "attn_bwd_ex", "attn_bwd_ex_phase", "attn_route_rows", "attn_bwd_noalloc", "attn_last_error",
           "attn_version")
ATTN_BWD_PREPARE, ATTN_BWD_DKDV, ATTN_BWD_DQ, ATTN_BWD_ALL = 1, 2, 4, 7


class AttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class attn_strides(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("token", ctypes.c_int64), ("head", ctypes.c_int64)]


class attn_desc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("Sq", ctypes.c_int32), ("Skv", ctypes.c_int32),
        ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
        ("Dqk", ctypes.c_int32), ("Dv", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float), ("flags", ctypes.c_uint32),
        ("q", attn_strides), ("k", attn_strides), ("v", attn_strides), ("o", attn_strides),
    ]


class attn_segments(ctypes.Structure):
    _fields_ = [("ids_q", ctypes.c_void_p), ("pos_q", ctypes.c_void_p),
                ("ids_kv", ctypes.c_void_p), ("pos_kv", ctypes.c_void_p)]


class attn_variant(ctypes.Structure):
    _fields_ = [("bias", ctypes.c_void_p), ("bias_batch", ctypes.c_int32), ("softcap", ctypes.c_float),
                ("sink", ctypes.c_void_p), ("max_logit", ctypes.c_void_p), ("dbias", ctypes.c_void_p),
                ("dsink", ctypes.c_void_p)]


def library_path() -> str:
    return os.environ.get("BPS_ATTN_LIB", os.path.join(_HERE, "libbps_attn.so"))


_lib = None
_lock = threading.Lock()


def lib():
    """Load the library once; raise if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m bwd_packed_segments_amd.build` "
                               "(or __graft_entry__.build()); there is no fallback path")
        # torch first: it carries its own HIP runtime, and the library must
        # bind to that one.  Loaded before torch, the library would pull in
        # the system's HIP runtime and the process would hold two (kernel
        # launches then fail with misleading errors such as "no ROCm-capable
        # device").
        import torch  # noqa: F401
        L = ctypes.CDLL(path)
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        dp, sp = ctypes.POINTER(attn_desc), ctypes.POINTER(attn_segments)
        i32p = ctypes.POINTER(ctypes.c_int32)
        L.attn_fwd_workspace_size.argtypes = [dp, sp]
        L.attn_fwd_workspace_size.restype = sz
        L.attn_bwd_workspace_size.argtypes = [dp, sp]
        L.attn_bwd_workspace_size.restype = sz
        L.attn_fwd.argtypes = [dp, sp, vp, vp, vp, vp, vp, vp, sz, vp, i32p]
        L.attn_fwd.restype = ctypes.c_int
        L.attn_bwd.argtypes = [dp, sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i32p]
        L.attn_bwd.restype = ctypes.c_int
        L.attn_bwd_phase.argtypes = [ctypes.c_int32, dp, sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i32p]
        L.attn_bwd_phase.restype = ctypes.c_int
        L.attn_debug_mask.argtypes = [dp, sp, vp, vp, vp, sz, vp]
        L.attn_debug_mask.restype = ctypes.c_int
        L.attn_ring_fwd_workspace_size.argtypes = [dp, sp, ctypes.c_int32]
        L.attn_ring_fwd_workspace_size.restype = sz
        L.attn_ring_bwd_workspace_size.argtypes = [dp, sp, ctypes.c_int32]
        L.attn_ring_bwd_workspace_size.restype = sz
        L.attn_ring_fwd.argtypes = [dp, sp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_ring_fwd.restype = ctypes.c_int
        L.attn_ring_bwd.argtypes = [dp, sp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.attn_ring_bwd.restype = ctypes.c_int
        varp = ctypes.POINTER(attn_variant)
        L.attn_fwd_ex_workspace_size.argtypes = [dp, sp, varp]
        L.attn_fwd_ex_workspace_size.restype = sz
        L.attn_bwd_ex_workspace_size.argtypes = [dp, sp, varp]
        L.attn_bwd_ex_workspace_size.restype = sz
        L.attn_fwd_ex.argtypes = [dp, sp, varp, vp, vp, vp, vp, vp, vp, sz, vp, i32p]
        L.attn_fwd_ex.restype = ctypes.c_int
        L.attn_bwd_ex.argtypes = [dp, sp, varp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, i32p]
        L.attn_bwd_ex.restype = ctypes.c_int
        L.attn_bwd_ex_phase.argtypes = [ctypes.c_int32, dp, sp, varp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                        vp, i32p]
        L.attn_bwd_ex_phase.restype = ctypes.c_int
        L.attn_bwd_noalloc.argtypes = [dp, sp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32p]
        L.attn_bwd_noalloc.restype = ctypes.c_int
        L.attn_route_rows.argtypes = [dp, sp, vp, sz, vp, vp]
        L.attn_route_rows.restype = ctypes.c_int
        L.attn_last_error.argtypes = []
        L.attn_last_error.restype = ctypes.c_char_p
        L.attn_version.argtypes = []
        L.attn_version.restype = ctypes.c_char_p
        _lib = L
        return L


def _check(status: int):
    if status != ATTN_OK:
        msg = lib().attn_last_error().decode(errors="replace")
        raise AttnError(status, msg)


# ------------------------------------------------------------------ helpers

def make_desc(*, B, Sq, Skv, Hq, Hkv, Dqk, Dv, dtype=ATTN_BF16, causal=False, scale=0.0, flags=0,
              q=None, k=None, v=None, o=None) -> attn_desc:
    """Descriptor with contiguous BSHD strides unless strides are given as
    (batch, token, head) tuples."""
    def st(given, S, H, D):
        return attn_strides(*(given if given is not None else (S * H * D, H * D, D)))
    return attn_desc(B, Sq, Skv, Hq, Hkv, Dqk, Dv, dtype, int(bool(causal)), float(scale), int(flags),
                     st(q, Sq, Hq, Dqk), st(k, Skv, Hkv, Dqk), st(v, Skv, Hkv, Dv), st(o, Sq, Hq, Dv))


@dataclass
class Segments:
    """THD metadata as device int32 tensors [B, S] (pos and kv parts optional)."""
    ids_q: object
    pos_q: object = None
    ids_kv: object = None
    pos_kv: object = None

    def c(self) -> attn_segments:
        def p(t):
            if t is None:
                return None
            _require_device_int32(t)
            return t.data_ptr()
        return attn_segments(p(self.ids_q), p(self.pos_q), p(self.ids_kv), p(self.pos_kv))


def _require_device_int32(t):
    import torch
    if not (isinstance(t, torch.Tensor) and t.is_cuda and t.dtype == torch.int32 and t.is_contiguous()):
        raise TypeError("segment metadata must be contiguous int32 device tensors")


def _strides(t):
    s = t.stride()
    if s[3] != 1:
        raise ValueError("the head-dim axis must be contiguous")
    return (s[0], s[1], s[2])


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_FP32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _require_device(*ts):
    for t in ts:
        if not t.is_cuda:
            raise TypeError("tensors must live in GPU memory")


def _stream(device):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _desc_for(q, k, v, o_strides, causal, scale, flags):
    B, Sq, Hq, Dqk = q.shape
    Skv, Hkv, Dv = k.shape[1], k.shape[2], v.shape[3]
    if k.shape[0] != B or v.shape[:3] != (B, Skv, Hkv) or k.shape[3] != Dqk:
        raise ValueError("inconsistent q/k/v shapes")
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share a dtype")
    return make_desc(B=B, Sq=Sq, Skv=Skv, Hq=Hq, Hkv=Hkv, Dqk=Dqk, Dv=Dv, dtype=_dtype_code(q), causal=causal,
                     scale=0.0 if scale is None else scale, flags=flags, q=_strides(q), k=_strides(k),
                     v=_strides(v), o=o_strides)


def _seg_ptr(segments):
    if segments is None:
        return None, None
    cs = segments.c()
    return cs, ctypes.byref(cs)


def fwd_workspace_size(desc: attn_desc, segments: attn_segments | None = None) -> int:
    return lib().attn_fwd_workspace_size(ctypes.byref(desc), ctypes.byref(segments) if segments else None)


def bwd_workspace_size(desc: attn_desc, segments: attn_segments | None = None) -> int:
    return lib().attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(segments) if segments else None)


def _workspace(nbytes, device):
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def _route_rows(desc, csp, ws, device, stream):
    """Device int32 [B]: the route each batch row took in the last call that
    used workspace ws with this descriptor (attn_route_rows)."""
    import torch
    out = torch.empty((desc.B,), dtype=torch.int32, device=device)
    _check(lib().attn_route_rows(ctypes.byref(desc), csp, ws.data_ptr() if ws is not None else None,
                                 ws.numel() if ws is not None else 0, out.data_ptr(), stream))
    return out


def route_counts(rows) -> dict:
    """{route name: number of batch rows} of a route_rows tensor (synchronises)."""
    vals = rows.cpu().tolist()
    return {name: sum(1 for r in vals if r == code) for code, name in ROUTE_NAMES.items() if code in vals}


# ------------------------------------------------------------------ public API

def attn_fwd(q, k, v, *, causal=False, scale=None, segments: Segments | None = None, flags=0, out=None,
             return_route=False, return_route_rows=False):
    """O [B,Sq,Hq,Dv] and LSE [B,Hq,Sq] (fp32) of fused attention.  With
    return_route, also the route the host requested ("dense", "fast",
    "general"); with return_route_rows, also the device int32 [B] routes
    the batch rows took (a row may fall back from fast to general)."""
    import torch
    _require_device(q, k, v)
    B, Sq, Hq, _ = q.shape
    Dv = v.shape[3]
    o = out if out is not None else torch.empty((B, Sq, Hq, Dv), dtype=q.dtype, device=q.device)
    _require_device(o)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws_bytes = L.attn_fwd_workspace_size(ctypes.byref(desc), csp)
    ws = _workspace(ws_bytes, q.device)
    route = ctypes.c_int32(-1)
    _check(L.attn_fwd(ctypes.byref(desc), csp, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device), ctypes.byref(route)))
    res = (o, lse)
    if return_route:
        res += (ROUTE_NAMES[route.value],)
    if return_route_rows:
        res += (_route_rows(desc, csp, ws, q.device, _stream(q.device)),)
    return res


def attn_bwd(q, k, v, o, lse, do, *, causal=False, scale=None, segments: Segments | None = None, flags=0):
    """dQ, dK, dV of fused attention from the saved O and LSE."""
    import torch
    _require_device(q, k, v, o, lse, do)
    if do.stride() != o.stride() or do.shape != o.shape:
        raise ValueError("dO must have the shape and strides of O")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        dq, dk, dv = (torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device) for t in (q, k, v))
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws_bytes = L.attn_bwd_workspace_size(ctypes.byref(desc), csp)
    ws = _workspace(ws_bytes, q.device)
    _check(L.attn_bwd(ctypes.byref(desc), csp, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                      lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                      ws.data_ptr(), ws.numel(), _stream(q.device), None))
    return dq, dk, dv


def attn_bwd_noalloc(q, k, v, o, lse, do, *, causal=False, scale=None, segments: Segments | None = None, flags=0,
                     out=None):
    """dQ, dK, dV through attn_bwd_noalloc: the library takes no workspace
    and allocates nothing (its scratch is a per-GPU device array).  The
    outputs are allocated here unless given as out=(dq, dk, dv) with the
    strides of q, k, v."""
    import torch
    _require_device(q, k, v, o, lse, do)
    if do.stride() != o.stride() or do.shape != o.shape:
        raise ValueError("dO must have the shape and strides of O")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    if out is None:
        out = tuple(torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device) for t in (q, k, v))
    dq, dk, dv = out
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("dq, dk, dv must have the strides of q, k, v")
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    cs, csp = _seg_ptr(segments)
    _check(lib().attn_bwd_noalloc(ctypes.byref(desc), csp, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                                  _stream(q.device), None))
    return dq, dk, dv


def validate_bwd_noalloc(desc: attn_desc, segments: attn_segments | None = None, *, ptr=1 << 12):
    """attn_bwd_noalloc with placeholder addresses, for descriptors that must
    fail host validation (nothing may launch); returns (status, message)."""
    L = lib()
    st = L.attn_bwd_noalloc(ctypes.byref(desc), ctypes.byref(segments) if segments else None, ptr, ptr, ptr, ptr,
                            ptr, ptr, ptr, ptr, ptr, None, None)
    return st, L.attn_last_error().decode(errors="replace")


class FwdPlan:
    """A forward for fixed tensors with its outputs and workspace allocated
    once, so that repeated calls allocate nothing.  With any of bias,
    softcap, sink or max_logit it runs attn_fwd_ex (self.max_logit holds the
    per-head maxima when asked)."""

    def __init__(self, q, k, v, *, causal=False, scale=None, segments: Segments | None = None, flags=0, bias=None,
                 softcap=0.0, sink=None, max_logit=False):
        import torch
        _require_device(q, k, v)
        B, Sq, Hq, _ = q.shape
        self.t = (q, k, v)
        self.o = torch.empty((B, Sq, Hq, v.shape[3]), dtype=q.dtype, device=q.device)
        self.lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
        self.max_logit = torch.empty((Hq,), dtype=torch.float32, device=q.device) if max_logit else None
        self.desc = _desc_for(q, k, v, _strides(self.o), causal, scale, flags)
        self.cs, self.csp = _seg_ptr(segments)
        self.segments = segments
        self.ex = bias is not None or bool(softcap) or sink is not None or max_logit
        self.keep = (bias, sink)
        self.var = _variant(q, bias, softcap, sink, max_logit=self.max_logit) if self.ex else None
        L = lib()
        nbytes = (L.attn_fwd_ex_workspace_size(ctypes.byref(self.desc), self.csp, ctypes.byref(self.var))
                  if self.ex else L.attn_fwd_workspace_size(ctypes.byref(self.desc), self.csp))
        self.ws = _workspace(nbytes, q.device)
        self.route = None

    def run(self, stream=None):
        q, k, v = self.t
        st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(q.device)
        route = ctypes.c_int32(-1)
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), self.o.data_ptr(), self.lse.data_ptr(), self.ws.data_ptr(),
                self.ws.numel(), st, ctypes.byref(route))
        if self.ex:
            _check(lib().attn_fwd_ex(ctypes.byref(self.desc), self.csp, ctypes.byref(self.var), *args))
        else:
            _check(lib().attn_fwd(ctypes.byref(self.desc), self.csp, *args))
        self.route = ROUTE_NAMES[route.value]
        return self.o, self.lse

    def route_rows(self, stream=None):
        """Device int32 [B]: the route each batch row took in the last run()."""
        q = self.t[0]
        st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(q.device)
        return _route_rows(self.desc, self.csp, self.ws, q.device, st)


class BwdPlan:
    """A backward prepared once for fixed tensors, whose phases can be
    launched separately (prepare, then dK/dV and dQ in either order or on
    two streams).  Holds the outputs and the workspace.  With any of bias,
    softcap or sink it runs attn_bwd_ex_phase and also returns dbias and
    dsink (self.dbias, self.dsink)."""

    def __init__(self, q, k, v, o, lse, do, *, causal=False, scale=None, segments: Segments | None = None,
                 flags=0, bias=None, softcap=0.0, sink=None):
        import torch
        _require_device(q, k, v, o, lse, do)
        if do.stride() != o.stride() or do.shape != o.shape:
            raise ValueError("dO must have the shape and strides of O")
        self.t = (q, k, v, o, lse, do)
        self.dq = torch.empty_strided(q.shape, q.stride(), dtype=q.dtype, device=q.device)
        self.dk = torch.empty_strided(k.shape, k.stride(), dtype=k.dtype, device=k.device)
        self.dv = torch.empty_strided(v.shape, v.stride(), dtype=v.dtype, device=v.device)
        self.desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
        self.cs, self.csp = _seg_ptr(segments)
        self.segments = segments
        self.ex = bias is not None or bool(softcap) or sink is not None
        self.dbias = torch.empty_like(bias) if bias is not None else None
        self.dsink = torch.empty((q.shape[2],), dtype=torch.float32, device=q.device) if sink is not None else None
        self.keep = (bias, sink)
        self.var = _variant(q, bias, softcap, sink, dbias=self.dbias, dsink=self.dsink) if self.ex else None
        L = lib()
        nbytes = (L.attn_bwd_ex_workspace_size(ctypes.byref(self.desc), self.csp, ctypes.byref(self.var))
                  if self.ex else L.attn_bwd_workspace_size(ctypes.byref(self.desc), self.csp))
        self.ws = _workspace(nbytes, q.device)

    def run(self, phases=ATTN_BWD_ALL, stream=None):
        q, k, v, o, lse, do = self.t
        st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(q.device)
        args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), do.data_ptr(),
                self.dq.data_ptr(), self.dk.data_ptr(), self.dv.data_ptr(), self.ws.data_ptr(), self.ws.numel(), st,
                None)
        if self.ex:
            _check(lib().attn_bwd_ex_phase(phases, ctypes.byref(self.desc), self.csp, ctypes.byref(self.var), *args))
        else:
            _check(lib().attn_bwd_phase(phases, ctypes.byref(self.desc), self.csp, *args))
        return self.dq, self.dk, self.dv

    def route_rows(self, stream=None):
        """Device int32 [B]: the route each batch row took in the last run()
        that included the PREPARE phase."""
        q = self.t[0]
        st = ctypes.c_void_p(stream.cuda_stream) if stream is not None else _stream(q.device)
        return _route_rows(self.desc, self.csp, self.ws, q.device, st)


def attn_debug_mask(*, B, Sq, Skv, causal=False, segments: Segments | None = None, flags=0, device="cuda"):
    """The mask the kernels apply (uint8 [B,Sq,Skv]) and each row's route."""
    import torch
    desc = make_desc(B=B, Sq=Sq, Skv=Skv, Hq=1, Hkv=1, Dqk=64, Dv=64, causal=causal, flags=flags)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws = _workspace(L.attn_fwd_workspace_size(ctypes.byref(desc), csp), device)
    mask = torch.empty((B, Sq, Skv), dtype=torch.uint8, device=device)
    routes = torch.empty((B,), dtype=torch.int32, device=device)
    _check(L.attn_debug_mask(ctypes.byref(desc), csp, mask.data_ptr(), routes.data_ptr(), ws.data_ptr(),
                             ws.numel(), _stream(torch.device(device))))
    return mask, routes


def attn_ring_fwd(q, k, v, *, cp, causal=False, scale=None, segments: Segments | None = None, flags=0):
    """O and LSE of fused attention computed as a one-GPU ring of cp shards
    (attn_ring_fwd in the C ABI)."""
    import torch
    _require_device(q, k, v)
    B, Sq, Hq, _ = q.shape
    o = torch.empty((B, Sq, Hq, v.shape[3]), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws = _workspace(L.attn_ring_fwd_workspace_size(ctypes.byref(desc), csp, int(cp)), q.device)
    _check(L.attn_ring_fwd(ctypes.byref(desc), csp, int(cp), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device)))
    return o, lse


def attn_ring_bwd(q, k, v, o, lse, do, *, cp, causal=False, scale=None, segments: Segments | None = None, flags=0):
    """dQ, dK, dV computed as a one-GPU ring of cp shards (attn_ring_bwd)."""
    import torch
    _require_device(q, k, v, o, lse, do)
    if do.stride() != o.stride() or do.shape != o.shape:
        raise ValueError("dO must have the shape and strides of O")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    dq, dk, dv = (torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device) for t in (q, k, v))
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws = _workspace(L.attn_ring_bwd_workspace_size(ctypes.byref(desc), csp, int(cp)), q.device)
    _check(L.attn_ring_bwd(ctypes.byref(desc), csp, int(cp), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                           o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device)))
    return dq, dk, dv


def ring_workspace_sizes(desc: attn_desc, segments: attn_segments | None, cp: int):
    L = lib()
    sp = ctypes.byref(segments) if segments else None
    return (L.attn_ring_fwd_workspace_size(ctypes.byref(desc), sp, int(cp)),
            L.attn_ring_bwd_workspace_size(ctypes.byref(desc), sp, int(cp)))


def validate_ring_fwd(desc: attn_desc, segments: attn_segments | None, cp: int, *, ptr=1 << 12, ws=None,
                      ws_bytes=0):
    """attn_ring_fwd with placeholder addresses, for descriptors that must
    fail host validation (nothing may launch); returns (status, message)."""
    L = lib()
    st = L.attn_ring_fwd(ctypes.byref(desc), ctypes.byref(segments) if segments else None, int(cp), ptr, ptr, ptr,
                         ptr, ptr, ws, ws_bytes, None)
    return st, L.attn_last_error().decode(errors="replace")


def validate_fwd(desc: attn_desc, segments: attn_segments | None = None, *, q=1 << 12, k=1 << 12, v=1 << 12,
                 o=1 << 12, lse=1 << 12, ws=None, ws_bytes=0):
    """Call attn_fwd with placeholder addresses to exercise host validation.
    Only for descriptors that must fail validation (nothing may launch);
    returns (status, message)."""
    L = lib()
    st = L.attn_fwd(ctypes.byref(desc), ctypes.byref(segments) if segments else None, q, k, v, o, lse, ws,
                    ws_bytes, None, None)
    return st, L.attn_last_error().decode(errors="replace")


def validate_bwd(desc: attn_desc, segments: attn_segments | None = None, *, ptr=1 << 12, ws=None, ws_bytes=0,
                 dq=...):
    """attn_bwd counterpart of validate_fwd (same restriction)."""
    L = lib()
    dqp = ptr if dq is ... else dq
    st = L.attn_bwd(ctypes.byref(desc), ctypes.byref(segments) if segments else None, ptr, ptr, ptr, ptr, ptr,
                    ptr, dqp, ptr, ptr, ws, ws_bytes, None, None)
    return st, L.attn_last_error().decode(errors="replace")


# ------------------------------------------------------------------ variants

def _variant(q, bias, softcap, sink, max_logit=None, dbias=None, dsink=None):
    """attn_variant for device tensors (None fields stay NULL)."""
    import torch
    B, Sq, Hq, _ = q.shape
    bias_batch = 1
    if bias is not None:
        _require_device(bias)
        if bias.dtype != q.dtype or not bias.is_contiguous() or bias.dim() != 4 or bias.shape[1] != Hq \
                or bias.shape[2] != Sq or bias.shape[0] not in (1, B):
            raise ValueError("bias must be a contiguous [1 or B, Hq, Sq, Skv] tensor of q's dtype")
        bias_batch = bias.shape[0]
    if sink is not None:
        _require_device(sink)
        if sink.dtype != torch.float32 or not sink.is_contiguous() or tuple(sink.shape) != (Hq,):
            raise ValueError("sink must be a contiguous float32 [Hq] tensor")

    def ptr(t):
        return None if t is None else t.data_ptr()
    return attn_variant(ptr(bias), bias_batch, float(softcap or 0.0), ptr(sink), ptr(max_logit), ptr(dbias),
                        ptr(dsink))


def attn_fwd_ex(q, k, v, *, causal=False, scale=None, segments: Segments | None = None, flags=0, bias=None,
                softcap=0.0, sink=None, return_max_logit=False):
    """O, LSE (and the per-head max logit when asked) of fused attention with
    an additive bias [1 or B, Hq, Sq, Skv], soft-capping and sink logits
    [Hq] (attn_fwd_ex in the C ABI)."""
    import torch
    _require_device(q, k, v)
    B, Sq, Hq, _ = q.shape
    o = torch.empty((B, Sq, Hq, v.shape[3]), dtype=q.dtype, device=q.device)
    lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    ml = torch.empty((Hq,), dtype=torch.float32, device=q.device) if return_max_logit else None
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    var = _variant(q, bias, softcap, sink, max_logit=ml)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws = _workspace(L.attn_fwd_ex_workspace_size(ctypes.byref(desc), csp, ctypes.byref(var)), q.device)
    _check(L.attn_fwd_ex(ctypes.byref(desc), csp, ctypes.byref(var), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         o.data_ptr(), lse.data_ptr(), ws.data_ptr(), ws.numel(), _stream(q.device), None))
    return (o, lse, ml) if return_max_logit else (o, lse)


def attn_bwd_ex(q, k, v, o, lse, do, *, causal=False, scale=None, segments: Segments | None = None, flags=0,
                bias=None, softcap=0.0, sink=None, need_dbias=True, need_dsink=True):
    """dQ, dK, dV, dbias (None without bias or when not needed) and dsink
    (None without sink or when not needed) of fused attention with the
    variants of attn_fwd_ex (attn_bwd_ex in the C ABI)."""
    import torch
    _require_device(q, k, v, o, lse, do)
    if do.stride() != o.stride() or do.shape != o.shape:
        raise ValueError("dO must have the shape and strides of O")
    if lse.dtype != torch.float32 or not lse.is_contiguous():
        raise TypeError("lse must be a contiguous float32 tensor")
    dq, dk, dv = (torch.empty_strided(t.shape, t.stride(), dtype=t.dtype, device=t.device) for t in (q, k, v))
    dbias = torch.empty_like(bias) if (bias is not None and need_dbias) else None
    dsink = torch.empty((q.shape[2],), dtype=torch.float32, device=q.device) \
        if (sink is not None and need_dsink) else None
    desc = _desc_for(q, k, v, _strides(o), causal, scale, flags)
    var = _variant(q, bias, softcap, sink, dbias=dbias, dsink=dsink)
    cs, csp = _seg_ptr(segments)
    L = lib()
    ws = _workspace(L.attn_bwd_ex_workspace_size(ctypes.byref(desc), csp, ctypes.byref(var)), q.device)
    _check(L.attn_bwd_ex(ctypes.byref(desc), csp, ctypes.byref(var), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                         o.data_ptr(), lse.data_ptr(), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                         ws.data_ptr(), ws.numel(), _stream(q.device), None))
    return dq, dk, dv, dbias, dsink


def validate_ex(desc: attn_desc, var: attn_variant, segments: attn_segments | None = None, *, bwd=False,
                ptr=1 << 12, ws=None, ws_bytes=0):
    """attn_fwd_ex / attn_bwd_ex with placeholder addresses, for variants
    that must fail host validation (nothing may launch); returns (status,
    message)."""
    L = lib()
    sp = ctypes.byref(segments) if segments else None
    if bwd:
        st = L.attn_bwd_ex(ctypes.byref(desc), sp, ctypes.byref(var), ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr,
                           ws, ws_bytes, None, None)
    else:
        st = L.attn_fwd_ex(ctypes.byref(desc), sp, ctypes.byref(var), ptr, ptr, ptr, ptr, ptr, ws, ws_bytes, None,
                           None)
    return st, L.attn_last_error().decode(errors="replace")


def ex_workspace_sizes(desc: attn_desc, var: attn_variant | None, segments: attn_segments | None = None):
    L = lib()
    sp = ctypes.byref(segments) if segments else None
    vp = ctypes.byref(var) if var is not None else None
    return (L.attn_fwd_ex_workspace_size(ctypes.byref(desc), sp, vp),
            L.attn_bwd_ex_workspace_size(ctypes.byref(desc), sp, vp))
