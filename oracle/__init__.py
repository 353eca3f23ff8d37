"""CPU oracle for the mHC seam block -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (``decode_mhc_pre_amd``)
never imports, links or calls it, and it shares no code with the HIP library.

The arithmetic lives in ``mhc_oracle.c`` (plain loops, IEEE double, plus one
exact-order single-precision collapse); this module only builds that file with
gcc, loads it with ctypes and strings its steps together per operation:

* :func:`mhc_pre`            -- projection, RMS, gates, Sinkhorn, collapse with
                                the seam's own pre-mix, optional folded RMSNorm.
* :func:`mhc_pre_delayed`    -- the same gates, collapse with the carried pre-mix
                                (vLLM PR "[ROCm][DSV4.1][Perf] Use AITER mHC for
                                the delayed pre block", Purpose).
* :func:`mhc_post`           -- post * y + comb . x.
* :func:`mhc_broadcast_entry`-- one stream broadcast to four, projected with the
                                narrower entry weight (same PR, Summary/Approach).
* :func:`mhc_post_pre_delayed` -- the post stage of one seam feeding the delayed
                                pre stage of the next (cross-seam composition).

Each returns exact values in float64 together with their bf16 roundings and the
size of the summed terms (for error bounds).  Every function is pinned by tests
that do not reuse it (closed forms, invariants, brute force); see tests/test_oracle.py.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "mhc_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11"]

NS = 4
NLOG = 24


def build(force: bool = True) -> str:
    """Compile mhc_oracle.c into liboracle.so with gcc (no contraction, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        D = ctypes.c_double
        L.orc_bf16_rne.argtypes = [D]
        L.orc_bf16_rne.restype = ctypes.c_uint16
        L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
        L.orc_bf16_to_double.restype = D
        L.orc_bf16_rne_array.argtypes = [P, I64, P]
        L.orc_logits.argtypes = [P, I64, I64, P, P, P, D, P, P]
        L.orc_sinkhorn.argtypes = [P, ctypes.c_int, P]
        L.orc_gates.argtypes = [P, I64, ctypes.c_int, P, P, P]
        L.orc_collapse64.argtypes = [P, P, I64, I64, P, P]
        L.orc_collapse32.argtypes = [P, P, I64, I64, P]
        L.orc_norm.argtypes = [P, P, I64, I64, D, P, P]
        L.orc_post.argtypes = [P, P, P, P, I64, I64, P, P]
        L.orc_post32.argtypes = [P, P, P, P, I64, I64, P]
        for name in ("orc_bf16_rne_array", "orc_logits", "orc_sinkhorn", "orc_gates",
                     "orc_collapse64", "orc_collapse32", "orc_norm", "orc_post", "orc_post32"):
            getattr(L, name).restype = None
        _lib = L
    return _lib


def set_threads(n: int) -> None:
    """Set the OpenMP thread count used by the oracle (libgomp honours omp_set_num_threads)."""
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_set_num_threads(int(n))
    except OSError:
        os.environ["OMP_NUM_THREADS"] = str(int(n))


def max_threads() -> int:
    try:
        gomp = ctypes.CDLL("libgomp.so.1")
        gomp.omp_get_max_threads.restype = ctypes.c_int
        return int(gomp.omp_get_max_threads())
    except OSError:
        return 1


# ----------------------------------------------------------------------------- helpers

def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def bf16_to_f64(bits) -> np.ndarray:
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def bf16_rne(v) -> np.ndarray:
    """Round float64 values to bf16 bits, nearest-even, directly from double."""
    v = _c(v, np.float64)
    out = np.empty(v.shape, dtype=np.uint16)
    lib().orc_bf16_rne_array(_ptr(v), v.size, _ptr(out))
    return out


def sinkhorn(m, iters: int) -> np.ndarray:
    m = _c(m, np.float64).reshape(16)
    out = np.empty(16, dtype=np.float64)
    lib().orc_sinkhorn(_ptr(m), int(iters), _ptr(out))
    return out.reshape(4, 4)


def logits(x_bits, fn, bias, alpha, eps: float):
    """x_bits: [T, K] (or [T, 4, C]) bf16 bits; fn: [K, 24] fp32.  Returns (logits [T,24], r [T])."""
    x = _c(x_bits, np.uint16)
    T = x.shape[0]
    K = x.size // max(T, 1) if T else int(np.asarray(fn).shape[0])
    fn = _c(fn, np.float32)
    assert fn.shape == (K, NLOG), (fn.shape, K)
    bias = _c(bias, np.float32)
    alpha = _c(alpha, np.float32)
    lg = np.empty((T, NLOG), dtype=np.float64)
    r = np.empty(T, dtype=np.float64)
    lib().orc_logits(_ptr(x), T, K, _ptr(fn), _ptr(bias), _ptr(alpha), float(eps), _ptr(lg), _ptr(r))
    return lg, r


def gates(lg, iters: int):
    lg = _c(lg, np.float64)
    T = lg.shape[0]
    pre = np.empty((T, NS))
    post = np.empty((T, NS))
    comb = np.empty((T, NS, NS))
    lib().orc_gates(_ptr(lg), T, int(iters), _ptr(pre), _ptr(post), _ptr(comb))
    return pre, post, comb


def collapse64(x_bits, p):
    x = _c(x_bits, np.uint16)
    T, ns, C = x.shape
    assert ns == NS
    p = _c(p, np.float64)
    y = np.empty((T, C))
    mag = np.empty((T, C))
    lib().orc_collapse64(_ptr(x), _ptr(p), T, C, _ptr(y), _ptr(mag))
    return y, mag


def collapse32(x_bits, p32):
    """Exact-order single-precision collapse; returns float32 [T, C]."""
    x = _c(x_bits, np.uint16)
    T, ns, C = x.shape
    p = _c(p32, np.float32)
    y = np.empty((T, C), dtype=np.float32)
    lib().orc_collapse32(_ptr(x), _ptr(p), T, C, _ptr(y))
    return y


def norm(y, w_bits, eps: float):
    y = _c(y, np.float64)
    T, C = y.shape
    w = _c(w_bits, np.uint16)
    assert w.shape == (C,)
    out = np.empty((T, C))
    ry = np.empty(T)
    lib().orc_norm(_ptr(y), _ptr(w), T, C, float(eps), _ptr(out), _ptr(ry))
    return out, ry


# ----------------------------------------------------------------------------- operations

def _finish_layer_input(x_bits, p, norm_weight, eps, res):
    """Steps 7-8: collapse with p (float64 values) and optional folded RMSNorm."""
    y, mag = collapse64(x_bits, p)
    if norm_weight is None:
        val = y
    else:
        val, ry = norm(y, norm_weight, eps)
        w = bf16_to_f64(norm_weight)
        mag = mag * ry[:, None] * np.abs(w)[None, :]
        res["ry"] = ry
    res["y"] = y
    res["li_val"] = val
    res["li_mag"] = mag
    res["li"] = bf16_rne(val)
    return res


def mhc_pre(x_bits, fn, bias, alpha, eps=1e-6, iters=20, norm_weight=None):
    """Non-delayed pre: gates from x, collapse x with this seam's own pre-mix."""
    x = _c(x_bits, np.uint16)
    lg, r = logits(x.reshape(x.shape[0], -1), fn, bias, alpha, eps)
    pre, post, comb = gates(lg, iters)
    res = dict(logits=lg, r=r, pre=pre, post=post, comb=comb)
    return _finish_layer_input(x, pre, norm_weight, eps, res)


def mhc_pre_delayed(x_bits, pre_in, fn, bias, alpha, eps=1e-6, iters=20, norm_weight=None):
    """Delayed pre: identical gates; collapse with the carried fp32 pre-mix pre_in [T,4];
    this seam's pre-mix is returned as pre_out for the next seam."""
    x = _c(x_bits, np.uint16)
    lg, r = logits(x.reshape(x.shape[0], -1), fn, bias, alpha, eps)
    pre, post, comb = gates(lg, iters)
    res = dict(logits=lg, r=r, pre_out=pre, post=post, comb=comb)
    p = _c(pre_in, np.float32).astype(np.float64)
    return _finish_layer_input(x, p, norm_weight, eps, res)


def mhc_collapse(x_bits, p, norm_weight=None, eps=1e-6):
    """Standalone collapse (p1 Result: the collapse at its other call sites): steps 7-8
    with the given float32 mixing weights p [T,4]."""
    x = _c(x_bits, np.uint16)
    pp = _c(p, np.float32).astype(np.float64)
    return _finish_layer_input(x, pp, norm_weight, eps, {})


def mhc_post(y_bits, x_bits, post, comb):
    y = _c(y_bits, np.uint16)
    x = _c(x_bits, np.uint16)
    T, ns, C = x.shape
    post = _c(post, np.float32).reshape(T, NS)
    comb = _c(comb, np.float32).reshape(T, NS * NS)
    out = np.empty((T, NS, C))
    mag = np.empty((T, NS, C))
    lib().orc_post(_ptr(y), _ptr(x), _ptr(post), _ptr(comb), T, C, _ptr(out), _ptr(mag))
    return dict(out_val=out, out_mag=mag, out=bf16_rne(out))


def post32(y_bits, x_bits, post, comb):
    """Post stage evaluated in single precision in the fixed order fl(post*y), then one
    fused multiply-add per stream j = 0..3, rounded once to bf16: returns bits [T,4,C]."""
    y = _c(y_bits, np.uint16)
    x = _c(x_bits, np.uint16)
    T, ns, C = x.shape
    post = _c(post, np.float32).reshape(T, NS)
    comb = _c(comb, np.float32).reshape(T, NS * NS)
    out = np.empty((T, NS, C), dtype=np.uint16)
    lib().orc_post32(_ptr(y), _ptr(x), _ptr(post), _ptr(comb), T, C, _ptr(out))
    return out


def mhc_post_pre_delayed(y_bits, x_bits, post_in, comb_in, pre_in, fn, bias, alpha, eps=1e-6, iters=20,
                         norm_weight=None):
    """Cross-seam composition: the post stage of seam k (gates post_in, comb_in) writes the
    residual x_out, and the delayed pre stage of seam k+1 reads it, collapsing with
    pre_in (seam k's pre-mix).  x_out is the single-precision post rounded once
    (post32); everything after it is mhc_pre_delayed on those bits."""
    xo = post32(y_bits, x_bits, post_in, comb_in)
    res = mhc_pre_delayed(xo, pre_in, fn, bias, alpha, eps, iters, norm_weight=norm_weight)
    res["x_out"] = xo
    return res


def mhc_broadcast_entry(h_bits, fn_e, bias, alpha, eps=1e-6, iters=20, norm_weight=None):
    """Model-entry seam: x_out[t,i,:] = h[t,:]; logits from the narrower projection of h
    against fn_e [C,24] with the RMS over C; collapse with the seam's own pre-mix."""
    h = _c(h_bits, np.uint16)
    T, C = h.shape
    lg, r = logits(h, fn_e, bias, alpha, eps)
    pre, post, comb = gates(lg, iters)
    x_out = np.repeat(h[:, None, :], NS, axis=1)
    res = dict(logits=lg, r=r, pre=pre, post=post, comb=comb, x_out=x_out)
    return _finish_layer_input(x_out, pre, norm_weight, eps, res)
