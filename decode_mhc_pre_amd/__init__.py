"""decode_mhc_pre_amd -- the mHC seam block on MI355X (gfx950).

A thin ctypes binding over ``libmhc.so`` (C ABI in ``include/mhc.h``).  It only
marshals arguments: tensors become device pointers, the current HIP stream is
passed along, outputs are allocated with torch.  Every step of the seam runs in
the library's HIP kernels; there is no fallback path.  If the library is not
built, importing the ops raises.

Entry points (same names as the C ABI):
    mhc_pack_fn, mhc_pre, mhc_pre_delayed, mhc_post, mhc_post_pre_delayed,
    mhc_post_pre_delayed_noalloc, mhc_broadcast_entry, mhc_collapse, mhc_workspace_bytes, mhc_fn_packed_bytes,
    mhc_status_str, mhc_debug_force_wait_timeouts (test hook)
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

from . import build as _build

HC_MULT = 4
NUM_LOGITS = 24

STATUS = {
    0: "MHC_OK", 1: "MHC_ERR_NULL", 2: "MHC_ERR_SHAPE", 3: "MHC_ERR_UNSUPPORTED",
    4: "MHC_ERR_ALIGN", 5: "MHC_ERR_ALIAS", 6: "MHC_ERR_WORKSPACE", 7: "MHC_ERR_HIP",
}


class MhcError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__("%s: %s" % (what, mhc_status_str(status)))


class _Weights(ctypes.Structure):
    _fields_ = [("fn_packed", ctypes.c_void_p), ("bias", ctypes.c_void_p),
                ("alpha", ctypes.c_void_p)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmhc.so (built in-tree by __graft_entry__.build() / build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            raise ImportError("libmhc.so is not built (%s); run `python -m decode_mhc_pre_amd.build`"
                              % _build.LIB)
        L = ctypes.CDLL(_build.LIB)
        P, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.mhc_fn_packed_bytes.argtypes = [I]
        L.mhc_fn_packed_bytes.restype = Z
        L.mhc_pack_fn.argtypes = [P, I, P, P]
        L.mhc_workspace_bytes.argtypes = [I, I, I]
        L.mhc_workspace_bytes.restype = Z
        L.mhc_pre.argtypes = [P, I, I, I, _Weights, P, F, I, P, P, P, P, P, Z, P]
        L.mhc_pre_delayed.argtypes = [P, P, I, I, I, _Weights, P, F, I, P, P, P, P, P, Z, P]
        L.mhc_post.argtypes = [P, P, P, P, I, I, I, P, P]
        L.mhc_broadcast_entry.argtypes = [P, I, I, I, _Weights, P, F, I, P, P, P, P, P, P, Z, P]
        L.mhc_collapse.argtypes = [P, P, I, I, I, P, F, P, P]
        L.mhc_post_pre_delayed.argtypes = [P, P, P, P, P, I, I, I, _Weights, P, F, I, P, P, P, P, P, P, Z, P]
        L.mhc_post_pre_delayed_noalloc.argtypes = [P, P, P, P, P, I, I, I, _Weights, P, F, I, P, P, P, P,
                                                   P, P]
        for f in ("mhc_pack_fn", "mhc_pre", "mhc_pre_delayed", "mhc_post", "mhc_post_pre_delayed",
                  "mhc_post_pre_delayed_noalloc", "mhc_broadcast_entry",
                  "mhc_collapse"):
            getattr(L, f).restype = I
        L.mhc_debug_force_wait_timeouts.argtypes = [I]
        L.mhc_debug_force_wait_timeouts.restype = I
        L.mhc_status_str.argtypes = [I]
        L.mhc_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


EXPORTS = ("mhc_fn_packed_bytes", "mhc_pack_fn", "mhc_workspace_bytes", "mhc_pre",
           "mhc_pre_delayed", "mhc_post", "mhc_post_pre_delayed", "mhc_post_pre_delayed_noalloc",
           "mhc_broadcast_entry", "mhc_collapse",
           "mhc_status_str", "mhc_debug_force_wait_timeouts")

# Workspace byte offsets (include/mhc.h): the region calls leave zero, and the
# words a bounded wait that ran out sets.
WS_FLAG_BYTES = 192 * 1024
WS_WAIT_ERROR_PERSIST = 8
WS_WAIT_ERROR_SPLIT = 96 * 1024 + 1024
MAX_TOKENS = 1 << 22
MAX_SINKHORN_ITERS = 1024
NOALLOC_SCRATCH_BYTES = 8 << 20


def mhc_debug_force_wait_timeouts(sleeps: int) -> None:
    """Test hook: sleeps > 0 makes every later wait run out after that many sleeps; 0 restores."""
    _check(lib().mhc_debug_force_wait_timeouts(int(sleeps)), "mhc_debug_force_wait_timeouts")


def mhc_status_str(status: int) -> str:
    return lib().mhc_status_str(int(status)).decode()


def mhc_fn_packed_bytes(K: int) -> int:
    return int(lib().mhc_fn_packed_bytes(int(K)))


def mhc_workspace_bytes(T_max: int, n: int = HC_MULT, C: int = 5120) -> int:
    return int(lib().mhc_workspace_bytes(int(T_max), int(n), int(C)))


# ----------------------------------------------------------------------------- torch marshalling

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev):
    torch = _torch()
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _check(status: int, what: str):
    if status != 0:
        raise MhcError(status, what)


def _u16(t):
    """bf16 tensor -> same storage viewed as int16 (the ABI takes bit patterns)."""
    torch = _torch()
    if t is None:
        return None
    if t.dtype == torch.bfloat16:
        return t
    if t.dtype in (torch.int16, torch.uint16):
        return t
    raise TypeError("expected a bfloat16 tensor, got %s" % t.dtype)


def _arg(t, name, shape, kind, dev, optional=False):
    """Check one tensor argument before its pointer goes to the library, which sees
    only raw addresses: a CUDA tensor on `dev`, dense (contiguous), of the exact
    shape and element type ('bf16': bfloat16 or its int16 bit view; 'f32')."""
    torch = _torch()
    if t is None:
        if optional:
            return
        raise ValueError("%s is required" % name)
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda or (dev is not None and t.device != dev):
        raise ValueError("%s must be on %s, got %s" % (name, dev if dev is not None else "a GPU", t.device))
    if kind == "bf16":
        if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
            raise TypeError("%s must be bfloat16, got %s" % (name, t.dtype))
    elif kind == "f32":
        if t.dtype != torch.float32:
            raise TypeError("%s must be float32, got %s" % (name, t.dtype))
    elif kind == "u8":
        if t.dtype != torch.uint8:
            raise TypeError("%s must be uint8, got %s" % (name, t.dtype))
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _residual(x, name="x"):
    """Shape (T, n, C) of a residual argument (checked against the other arguments later)."""
    torch = _torch()
    if not isinstance(x, torch.Tensor) or x.dim() != 3:
        raise ValueError("%s must be a [T, 4, C] tensor" % name)
    T, n, C = x.shape
    if n != HC_MULT:
        raise ValueError("%s must have %d streams, got %d" % (name, HC_MULT, n))
    _arg(x, name, (T, n, C), "bf16", None)
    return int(T), int(n), int(C), x.device


def _weights_arg(w, K, dev):
    if not isinstance(w, Weights):
        raise TypeError("w must be a Weights (make_weights)")
    if w.K != K:
        raise ValueError("weights are for K = %d rows, this call needs K = %d" % (w.K, K))
    _arg(w.fn_packed, "w.fn_packed", (mhc_fn_packed_bytes(K),), "u8", dev)
    _arg(w.bias, "w.bias", (NUM_LOGITS,), "f32", dev)
    _arg(w.alpha, "w.alpha", (3,), "f32", dev)


def _ws_arg(ws, dev):
    torch = _torch()
    if not isinstance(ws, torch.Tensor) or ws.dim() != 1:
        raise ValueError("ws must be a 1-D uint8 tensor")
    _arg(ws, "ws", (ws.numel(),), "u8", dev)


def _scalars(eps, iters):
    if not (float(eps) >= 0.0) or float(eps) == float("inf"):
        raise ValueError("eps must be finite and >= 0")
    if not (1 <= int(iters) <= MAX_SINKHORN_ITERS):
        raise ValueError("iters must be in [1, %d]" % MAX_SINKHORN_ITERS)


@dataclass
class Weights:
    """Weights of one seam on the device: fn packed for the library, bias [24], alpha [3]."""
    fn_packed: object
    bias: object
    alpha: object
    K: int

    def as_c(self) -> _Weights:
        return _Weights(self.fn_packed.data_ptr(), self.bias.data_ptr(), self.alpha.data_ptr())


def mhc_pack_fn(fn, out=None):
    """Pack fn [K, 24] float32 (device) for the library; returns a uint8 device tensor."""
    torch = _torch()
    if not isinstance(fn, torch.Tensor) or fn.dim() != 2:
        raise ValueError("fn must be a [K, 24] tensor")
    K = int(fn.shape[0])
    _arg(fn, "fn", (K, NUM_LOGITS), "f32", None)
    if out is None:
        out = torch.empty(mhc_fn_packed_bytes(K), dtype=torch.uint8, device=fn.device)
    _arg(out, "out", (mhc_fn_packed_bytes(K),), "u8", fn.device)
    _check(lib().mhc_pack_fn(_ptr(fn), K, _ptr(out), _stream(fn.device)), "mhc_pack_fn")
    return out


def make_weights(fn, bias, alpha) -> Weights:
    """Device float32 fn [K,24], bias [24], alpha [3] -> packed Weights (packing runs once)."""
    return Weights(mhc_pack_fn(fn), bias.contiguous(), alpha.contiguous(), int(fn.shape[0]))


# Default workspaces, one per (device, stream, hidden size): calls on different
# streams may run concurrently and need workspaces of their own.  Each is
# allocated once at the size that serves every token count, zero-filled, and
# never replaced or freed, so a HIP graph that captured calls using it stays
# valid (a graph replays into the addresses it recorded).
_ws_cache = {}


def workspace(device, T: int, C: int, stream=None):
    """The default zero-filled workspace of (device, stream, C): large enough for any T."""
    torch = _torch()
    device = torch.device(device)
    if device.type == "cuda" and device.index is None:
        device = torch.device("cuda", torch.cuda.current_device())
    if stream is None:
        stream = torch.cuda.current_stream(device)
    key = (str(device), int(stream.cuda_stream), int(C))
    ws = _ws_cache.get(key)
    if ws is None:
        if torch.cuda.is_current_stream_capturing():
            raise RuntimeError("no default workspace exists yet for this stream: make one call outside "
                               "graph capture first, or pass ws= explicitly")
        need = max(mhc_workspace_bytes(MAX_TOKENS, HC_MULT, C), WS_FLAG_BYTES)
        ws = torch.zeros(need, dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


class MhcWaitRunOut(RuntimeError):
    """A bounded cross-workgroup wait of a call on this workspace ran out: the
    outputs of that call are unspecified and must be discarded."""


def check_workspace(ws, clear=True):
    """Read the two run-out words of `ws` (waits for the device).  If either is set,
    zero-fill the workspace (when `clear`) so that it can be used again, and raise
    MhcWaitRunOut.  No arithmetic: the words are the library's, at the offsets
    include/mhc.h documents."""
    torch = _torch()
    w = ws[:WS_FLAG_BYTES].view(torch.int32)
    persist = int(w[WS_WAIT_ERROR_PERSIST // 4])
    split = int(w[WS_WAIT_ERROR_SPLIT // 4])
    if persist or split:
        if clear:
            ws.zero_()
        raise MhcWaitRunOut("a bounded wait ran out (persistent word %d, split word %d): the outputs of "
                            "the calls since the last check must be discarded" % (persist, split))


def check_default_workspaces(clear=True):
    """check_workspace on every default workspace made so far."""
    for ws in list(_ws_cache.values()):
        check_workspace(ws, clear)


def _pre_outputs(T, C, dev, li=True):
    torch = _torch()
    pre = torch.empty((T, HC_MULT), dtype=torch.float32, device=dev)
    post = torch.empty((T, HC_MULT), dtype=torch.float32, device=dev)
    comb = torch.empty((T, HC_MULT, HC_MULT), dtype=torch.float32, device=dev)
    lo = torch.empty((T, C), dtype=torch.bfloat16, device=dev) if li else None
    return pre, post, comb, lo


def _check_pre_outs(outs, T, C, dev, li_optional=False):
    pre, post, comb, li = outs
    _arg(pre, "pre", (T, HC_MULT), "f32", dev)
    _arg(post, "post", (T, HC_MULT), "f32", dev)
    _arg(comb, "comb", (T, HC_MULT, HC_MULT), "f32", dev)
    _arg(li, "layer_input", (T, C), "bf16", dev, optional=li_optional)


def mhc_pre(x, w: Weights, norm_weight=None, eps=1e-6, iters=20, out=None, ws=None):
    """x [T,4,C] bf16 -> (pre [T,4], post [T,4], comb [T,4,4], layer_input [T,C] bf16)."""
    T, n, C, dev = _residual(x)
    _weights_arg(w, n * C, dev)
    _arg(norm_weight, "norm_weight", (C,), "bf16", dev, optional=True)
    _scalars(eps, iters)
    pre, post, comb, li = out if out is not None else _pre_outputs(T, C, dev)
    _check_pre_outs((pre, post, comb, li), T, C, dev)
    ws = workspace(dev, T, C) if ws is None else ws
    _ws_arg(ws, dev)
    st = lib().mhc_pre(_ptr(_u16(x)), T, n, C, w.as_c(), _ptr(_u16(norm_weight)), float(eps), int(iters),
                       _ptr(pre), _ptr(post), _ptr(comb), _ptr(li), _ptr(ws), ws.numel(),
                       _stream(dev))
    _check(st, "mhc_pre")
    return pre, post, comb, li


def mhc_pre_delayed(x, pre_in, w: Weights, norm_weight=None, eps=1e-6, iters=20, out=None, ws=None):
    """Delayed pre: collapse with pre_in [T,4] float32; returns (pre_out, post, comb, layer_input)."""
    T, n, C, dev = _residual(x)
    _arg(pre_in, "pre_in", (T, n), "f32", dev)
    _weights_arg(w, n * C, dev)
    _arg(norm_weight, "norm_weight", (C,), "bf16", dev, optional=True)
    _scalars(eps, iters)
    pre, post, comb, li = out if out is not None else _pre_outputs(T, C, dev)
    _check_pre_outs((pre, post, comb, li), T, C, dev)
    ws = workspace(dev, T, C) if ws is None else ws
    _ws_arg(ws, dev)
    st = lib().mhc_pre_delayed(_ptr(_u16(x)), _ptr(pre_in), T, n, C, w.as_c(), _ptr(_u16(norm_weight)),
                               float(eps), int(iters), _ptr(pre), _ptr(post), _ptr(comb), _ptr(li),
                               _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "mhc_pre_delayed")
    return pre, post, comb, li


def mhc_post(y, x, post, comb, out=None):
    """out [T,4,C] bf16 = post_i * y + sum_j comb_ij x_j; out may be x itself."""
    torch = _torch()
    T, n, C, dev = _residual(x)
    _arg(y, "y", (T, C), "bf16", dev)
    _arg(post, "post", (T, n), "f32", dev)
    _arg(comb, "comb", (T, n, n), "f32", dev)
    if out is None:
        out = torch.empty_like(x)
    _arg(out, "out", (T, n, C), "bf16", dev)
    st = lib().mhc_post(_ptr(_u16(y)), _ptr(_u16(x)), _ptr(post), _ptr(comb), T, n, C, _ptr(_u16(out)),
                        _stream(dev))
    _check(st, "mhc_post")
    return out


def mhc_post_pre_delayed(y, x, post_in, comb_in, pre_in, w: Weights, norm_weight=None, eps=1e-6,
                         iters=20, out=None, ws=None):
    """Post stage of seam k (y [T,C], x [T,4,C], post_in [T,4], comb_in [T,4,4]) fused with the
    delayed pre stage of seam k+1 (pre_in [T,4], weights w): returns (x_out [T,4,C], pre_out,
    post, comb, layer_input).  x_out must be a separate buffer (not x)."""
    torch = _torch()
    T, n, C, dev = _residual(x)
    _arg(y, "y", (T, C), "bf16", dev)
    _arg(post_in, "post_in", (T, n), "f32", dev)
    _arg(comb_in, "comb_in", (T, n, n), "f32", dev)
    _arg(pre_in, "pre_in", (T, n), "f32", dev)
    _weights_arg(w, n * C, dev)
    _arg(norm_weight, "norm_weight", (C,), "bf16", dev, optional=True)
    _scalars(eps, iters)
    if out is None:
        x_out = torch.empty_like(x)
        pre, post, comb, li = _pre_outputs(T, C, dev)
    else:
        x_out, pre, post, comb, li = out
    _arg(x_out, "x_out", (T, n, C), "bf16", dev)
    _check_pre_outs((pre, post, comb, li), T, C, dev)
    ws = workspace(dev, T, C) if ws is None else ws
    _ws_arg(ws, dev)
    st = lib().mhc_post_pre_delayed(_ptr(_u16(y)), _ptr(_u16(x)), _ptr(post_in), _ptr(comb_in), _ptr(pre_in),
                                    T, n, C, w.as_c(), _ptr(_u16(norm_weight)), float(eps), int(iters),
                                    _ptr(_u16(x_out)), _ptr(pre), _ptr(post), _ptr(comb), _ptr(li),
                                    _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "mhc_post_pre_delayed")
    return x_out, pre, post, comb, li


def mhc_post_pre_delayed_noalloc(y, x, post_in, comb_in, pre_in, w: Weights, norm_weight=None, eps=1e-6,
                                 iters=20, out=None):
    """mhc_post_pre_delayed with the library's own per-GPU scratch buffer instead of a workspace:
    the C call allocates nothing (pass `out` = (x_out, pre_out, post, comb, layer_input) to keep
    this wrapper from allocating them).  Calls that overlap on one GPU race."""
    torch = _torch()
    T, n, C, dev = _residual(x)
    _arg(y, "y", (T, C), "bf16", dev)
    _arg(post_in, "post_in", (T, n), "f32", dev)
    _arg(comb_in, "comb_in", (T, n, n), "f32", dev)
    _arg(pre_in, "pre_in", (T, n), "f32", dev)
    _weights_arg(w, n * C, dev)
    _arg(norm_weight, "norm_weight", (C,), "bf16", dev, optional=True)
    _scalars(eps, iters)
    if out is None:
        x_out = torch.empty_like(x)
        pre, post, comb, li = _pre_outputs(T, C, dev)
    else:
        x_out, pre, post, comb, li = out
    _arg(x_out, "x_out", (T, n, C), "bf16", dev)
    _check_pre_outs((pre, post, comb, li), T, C, dev)
    st = lib().mhc_post_pre_delayed_noalloc(_ptr(_u16(y)), _ptr(_u16(x)), _ptr(post_in), _ptr(comb_in),
                                            _ptr(pre_in), T, n, C, w.as_c(), _ptr(_u16(norm_weight)),
                                            float(eps), int(iters), _ptr(_u16(x_out)), _ptr(pre), _ptr(post),
                                            _ptr(comb), _ptr(li), _stream(dev))
    _check(st, "mhc_post_pre_delayed_noalloc")
    return x_out, pre, post, comb, li


def mhc_collapse(x, p, norm_weight=None, eps=1e-6, out=None):
    """out [T,C] bf16 = exact-order collapse of x [T,4,C] with p [T,4] float32 (optional folded norm)."""
    torch = _torch()
    T, n, C, dev = _residual(x)
    _arg(p, "p", (T, n), "f32", dev)
    _arg(norm_weight, "norm_weight", (C,), "bf16", dev, optional=True)
    if norm_weight is not None:
        _scalars(eps, 1)
    if out is None:
        out = torch.empty((T, C), dtype=torch.bfloat16, device=dev)
    _arg(out, "out", (T, C), "bf16", dev)
    st = lib().mhc_collapse(_ptr(_u16(x)), _ptr(p), T, n, C,
                            _ptr(_u16(norm_weight)) if norm_weight is not None else None, float(eps),
                            _ptr(_u16(out)), _stream(dev))
    _check(st, "mhc_collapse")
    return out


def mhc_broadcast_entry(h, w: Weights, norm_weight=None, eps=1e-6, iters=20, layer_input=True,
                        out=None, ws=None):
    """h [T,C] bf16 -> (x_out [T,4,C], pre, post, comb, layer_input or None)."""
    torch = _torch()
    if not isinstance(h, torch.Tensor) or h.dim() != 2:
        raise ValueError("h must be a [T, C] tensor")
    T, C = (int(v) for v in h.shape)
    dev = h.device
    _arg(h, "h", (T, C), "bf16", None)
    _weights_arg(w, C, dev)
    _arg(norm_weight, "norm_weight", (C,), "bf16", dev, optional=True)
    _scalars(eps, iters)
    if out is None:
        x_out = torch.empty((T, HC_MULT, C), dtype=torch.bfloat16, device=dev)
        pre, post, comb, li = _pre_outputs(T, C, dev, li=layer_input)
    else:
        x_out, pre, post, comb, li = out
    _arg(x_out, "x_out", (T, HC_MULT, C), "bf16", dev)
    _check_pre_outs((pre, post, comb, li), T, C, dev, li_optional=True)
    ws = workspace(dev, T, C) if ws is None else ws
    _ws_arg(ws, dev)
    st = lib().mhc_broadcast_entry(_ptr(_u16(h)), T, HC_MULT, C, w.as_c(), _ptr(_u16(norm_weight)),
                                   float(eps), int(iters), _ptr(x_out), _ptr(pre), _ptr(post), _ptr(comb),
                                   _ptr(li), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "mhc_broadcast_entry")
    return x_out, pre, post, comb, li
