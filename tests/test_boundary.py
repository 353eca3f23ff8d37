"""The C-ABI boundary on the CPU (no GPU): the library loads, exports every
entry point that include/mhc.h declares, and its host-side validation returns
the documented status before any kernel is enqueued.  Pointers here are fake
device addresses; validation never dereferences them."""
import ctypes
import os
import re

import pytest

import decode_mhc_pre_amd as m

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mhc.h")

OK, NULL, SHAPE, UNSUP, ALIGN, ALIAS, WS, HIP = range(8)
T, C = 8, 5120
MiB = 1 << 20


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mhc_[a-z_]+)\s*\(", src)))


def test_header_declares_the_exports():
    assert _declared() == sorted(m.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = m.lib()
    for name in _declared():
        assert hasattr(L, name), name


RUNTIME_ALLOWED = {"hipLaunchKernel", "hipGetLastError", "hipStreamGetDevice", "hipDeviceGetAttribute",
                   "hipStreamIsCapturing", "hipGetSymbolAddress", "hipGetDevice", "hipSetDevice",
                   "__hipPushCallConfiguration", "__hipRegisterVar", "__hipPopCallConfiguration", "__hipRegisterFatBinary",
                   "__hipRegisterFunction", "__hipUnregisterFatBinary"}


def test_library_imports_no_allocating_or_blocking_runtime_call():
    """Every call is capturable in a HIP graph: the library links no allocation, free,
    memset, copy, synchronisation, module load or run-time compilation."""
    import shutil
    import subprocess
    if shutil.which("nm") is None:
        pytest.skip("nm not available")
    so = m.lib()._name
    out = subprocess.run(["nm", "-D", "--undefined-only", so], capture_output=True, text=True,
                         check=True).stdout
    used = {ln.split()[-1].split("@")[0] for ln in out.splitlines() if ln.strip()}
    hip = {s for s in used if s.startswith(("hip", "__hip")) or "hiprtc" in s}
    assert hip and hip <= RUNTIME_ALLOWED, sorted(hip - RUNTIME_ALLOWED)
    # the persistent kernels' grid and the no-allocation buffer follow the launch
    # stream's device, not the calling thread's current device (which may be
    # another GPU); the current device is only switched to look the buffer up
    # and then restored
    assert "hipStreamGetDevice" in hip and "hipGetSymbolAddress" in hip


def test_sizes():
    assert m.mhc_fn_packed_bytes(4 * C) == 4 * C * 24 * 4
    assert m.mhc_fn_packed_bytes(0) == 0
    assert m.mhc_workspace_bytes(1, 4, C) > 0
    # up to 3072 tokens only split partials, bounded; beyond (the persistent
    # fused form, then the persistent delayed form): a fixed set of exchange
    # records, whatever the token count
    assert m.mhc_workspace_bytes(128, 4, C) < 2 * MiB
    assert m.mhc_workspace_bytes(3072, 4, C) < 2 * MiB
    assert m.mhc_workspace_bytes(3073, 4, C) == m.mhc_workspace_bytes(16384, 4, C)
    assert m.mhc_workspace_bytes(16384, 4, C) < 16 * MiB
    assert m.mhc_workspace_bytes(1 << 20, 4, C) == m.mhc_workspace_bytes(16384, 4, C)
    # hidden sizes with a persistent form (4096, 5120, 7168) need its records; others do not
    assert m.mhc_workspace_bytes(1 << 20, 4, 4096) == m.mhc_workspace_bytes(16384, 4, 4096) < 16 * MiB
    assert m.mhc_workspace_bytes(1 << 20, 4, 7168) == m.mhc_workspace_bytes(16384, 4, 7168) < 16 * MiB
    assert m.mhc_workspace_bytes(1 << 20, 4, 1024) < 2 * MiB
    assert m.mhc_workspace_bytes(1 << 20, 4, 6144) < 2 * MiB
    assert m.mhc_workspace_bytes(16, 3, C) == 0
    assert m.mhc_workspace_bytes(16, 4, 5000) == 0
    for s in range(8):
        assert m.mhc_status_str(s).startswith(m.STATUS[s])


class Ptrs:
    """Distinct, 16-byte aligned fake device addresses, far apart."""
    def __init__(self):
        self.next = 0x100000000

    def __call__(self, size=64 * MiB):
        p = self.next
        self.next += ((size + 0xFFFFF) // 0x100000) * 0x100000 + 0x100000
        return p


def _pre_args(**kw):
    P = Ptrs()
    a = dict(x=P(), pre_in=P(), T=T, n=4, C=C, w=m._Weights(P(), P(), P()), nw=P(), eps=1e-6, iters=20,
             pre=P(), post=P(), comb=P(), li=P(), ws=P(), ws_bytes=m.mhc_workspace_bytes(T, 4, C))
    a.update(kw)
    return a


def call_delayed(**kw):
    a = _pre_args(**kw)
    return m.lib().mhc_pre_delayed(a["x"], a["pre_in"], a["T"], a["n"], a["C"], a["w"], a["nw"], a["eps"],
                                   a["iters"], a["pre"], a["post"], a["comb"], a["li"], a["ws"],
                                   a["ws_bytes"], None)


def call_pre(**kw):
    a = _pre_args(**kw)
    return m.lib().mhc_pre(a["x"], a["T"], a["n"], a["C"], a["w"], a["nw"], a["eps"], a["iters"],
                           a["pre"], a["post"], a["comb"], a["li"], a["ws"], a["ws_bytes"], None)


def call_fused(**kw):
    a = _pre_args(**kw)
    P = Ptrs()
    P.next = 0x80000000000
    for k in ("y", "post_in", "comb_in", "xo"):
        a.setdefault(k, kw.get(k, P()))
    return m.lib().mhc_post_pre_delayed(a["y"], a["x"], a["post_in"], a["comb_in"], a["pre_in"], a["T"], a["n"],
                                        a["C"], a["w"], a["nw"], a["eps"], a["iters"], a["xo"], a["pre"], a["post"],
                                        a["comb"], a["li"], a["ws"], a["ws_bytes"], None)


def call_entry(**kw):
    a = _pre_args(**kw)
    xo = a.get("xo", Ptrs().__call__() + (1 << 40))
    return m.lib().mhc_broadcast_entry(a["x"], a["T"], a["n"], a["C"], a["w"], a["nw"], a["eps"], a["iters"],
                                       xo, a["pre"], a["post"], a["comb"], a["li"], a["ws"], a["ws_bytes"],
                                       None)


@pytest.mark.parametrize("call", [call_pre, call_delayed, call_entry, call_fused])
def test_pre_validation(call):
    assert call(n=3) == UNSUP
    assert call(C=5000) == UNSUP
    assert call(C=128) == UNSUP
    assert call(C=16384 + 256) == UNSUP
    assert call(T=-1) == SHAPE
    assert call(T=(1 << 22) + 1) == SHAPE
    assert call(eps=-1e-6) == SHAPE
    assert call(eps=float("nan")) == SHAPE
    assert call(eps=float("inf")) == SHAPE
    assert call(iters=0) == SHAPE
    assert call(iters=1025) == SHAPE     # above MHC_MAX_SINKHORN_ITERS: rejected before any launch
    assert call(iters=1 << 30) == SHAPE
    assert call(iters=1024) == HIP       # the cap itself is valid (then: no GPU here)
    assert call(x=None) == NULL
    assert call(pre=None) == NULL
    assert call(comb=None) == NULL
    assert call(w=m._Weights(None, 0x100, 0x200)) == NULL
    assert call(x=0x100000008) == ALIGN
    assert call(comb=0x7000000004) == ALIGN
    assert call(ws_bytes=16) == WS
    assert call(ws=None) == WS
    assert call(T=0) == OK              # no-op, nothing launched
    assert call(T=0, ws=None) == OK


def test_delayed_specific():
    assert call_delayed(pre_in=None) == NULL
    assert call_delayed(li=None) == NULL
    # layer_input overlapping x
    P = Ptrs()
    x = P()
    assert call_delayed(x=x, li=x + T * 4 * C * 2 - 16) == ALIAS
    assert call_delayed(x=x, li=x + T * 4 * C * 2) != ALIAS   # adjacent is fine (then: no GPU)
    # outputs overlapping each other or the workspace
    pre = P()
    assert call_delayed(pre=pre, post=pre + 16) == ALIAS
    assert call_delayed(pre=pre, ws=pre) == ALIAS
    # pre_out must not overlap the carried pre_in
    assert call_delayed(pre_in=pre, pre=pre) == ALIAS


def test_fused_specific():
    for k in ("y", "post_in", "comb_in", "xo", "pre_in", "li"):
        assert call_fused(**{k: None}) == NULL, k
    assert call_fused(post_in=0x80000000004) == ALIGN
    P = Ptrs()
    x = P()
    assert call_fused(x=x, xo=x) == ALIAS                      # not in place
    assert call_fused(x=x, xo=x + T * 4 * C * 2) != ALIAS      # adjacent is fine (then: no GPU)
    y = P()
    assert call_fused(y=y, li=y) == ALIAS
    g = P()
    assert call_fused(post_in=g, post=g) == ALIAS              # this seam's gates are new buffers
    assert call_fused(comb_in=g, comb=g + 32) == ALIAS
    assert call_fused(pre_in=g, pre=g) == ALIAS
    assert call_fused(T=0) == OK
    assert call_fused() == HIP


def test_entry_specific():
    assert call_entry(xo=None) == NULL
    assert call_entry(li=None, ws=None, T=0) == OK       # layer_input is optional
    P = Ptrs()
    h = P()
    assert call_entry(x=h, xo=h + 32) == ALIAS


def test_workspace_needs_by_form():
    # delayed, C = 5120, T > 4096: persistent form, partial sums go through the workspace
    assert call_delayed(T=6001, ws=None) == WS
    assert call_delayed(T=6001, ws_bytes=m.mhc_workspace_bytes(6001, 4, C) - 16) == WS
    assert call_delayed(T=6001, ws_bytes=m.mhc_workspace_bytes(6001, 4, C)) == HIP
    # delayed at 4096 tokens: split form (2 splits per tile), partials in the workspace
    assert call_delayed(T=4096, ws=None) == WS
    assert call_delayed(T=4096, ws_bytes=m.mhc_workspace_bytes(4096, 4, C)) == HIP
    # own pre-mix: split up to 128 tiles (T = 2048), then one workgroup per
    # 16-token tile (nothing to combine); beyond 4096 tokens with C = 5120 the
    # persistent gates-only form (workspace)
    assert call_pre(T=2048, ws=None) == WS
    assert call_pre(T=2049, ws=None) == HIP
    assert call_pre(T=4096, ws=None) == HIP
    assert call_pre(T=4097, ws=None) == WS
    assert call_pre(T=4097, ws_bytes=m.mhc_workspace_bytes(4097, 4, C)) == HIP
    assert call_pre(T=6001, C=4096, ws=None) == WS             # persistent gates-only form at C = 4096 too
    assert call_pre(T=6001, C=6144, ws=None) == HIP            # no persistent form: one workgroup per tile


class FarPtrs(Ptrs):
    """Fake device addresses 16 GiB apart: no two buffers of any token count here overlap."""
    def __call__(self, size=0):
        p = self.next
        self.next += 1 << 34
        return p


@pytest.mark.parametrize("Cx", [256, 5120, 7168])
def test_workspace_covers_every_plan(Cx):
    """mhc_workspace_bytes(T) is enough for every pre-stage entry point at every
    token count up to T, whichever kernel form the call plans (split with its
    partials, own-pre-mix records, persistent exchange): with exactly that many
    bytes each call passes validation and reaches the runtime."""
    lib = m.lib()
    Ts = [1, 15, 16, 17, 32, 33, 64, 255, 256, 257, 1024, 1025, 2048, 2049, 2100, 3072, 3073,
          4096, 4097, 6001, 16384]
    for T_ in Ts:
        P = FarPtrs()
        x, h, pin, y, po, cb = P(), P(), P(), P(), P(), P()
        w = m._Weights(P(), P(), P())
        nw, pre, post, comb, li, xo, ws = P(), P(), P(), P(), P(), P(), P()
        wb = m.mhc_workspace_bytes(T_, 4, Cx)
        assert wb == 0 or wb >= m.mhc_workspace_bytes(max(T_ - 1, 1), 4, Cx)   # grows with T
        args = (Cx, w, nw, 1e-6, 20)
        assert lib.mhc_pre(x, T_, 4, *args, pre, post, comb, li, ws, wb, None) == HIP, ("pre", T_)
        assert lib.mhc_pre_delayed(x, pin, T_, 4, *args, pre, post, comb, li, ws, wb, None) == HIP, ("delayed", T_)
        assert lib.mhc_post_pre_delayed(y, x, po, cb, pin, T_, 4, *args, xo, pre, post, comb, li, ws, wb,
                                        None) == HIP, ("fused", T_)
        assert lib.mhc_broadcast_entry(h, T_, 4, *args, xo, pre, post, comb, li, ws, wb, None) == HIP, ("entry", T_)


def test_valid_call_reaches_the_runtime():
    assert call_delayed() == HIP
    assert call_pre() == HIP


def _post(y, x, post, comb, T_, n, C_, out):
    return m.lib().mhc_post(y, x, post, comb, T_, n, C_, out, None)


def test_post_validation():
    P = Ptrs()
    y, x, po, cb, out = P(), P(), P(), P(), P()
    assert _post(y, x, po, cb, T, 3, C, out) == UNSUP
    assert _post(y, x, po, cb, T, 4, 1000, out) == UNSUP
    assert _post(y, x, po, cb, -2, 4, C, out) == SHAPE
    assert _post(None, x, po, cb, T, 4, C, out) == NULL
    assert _post(y, x, po, cb, T, 4, C, None) == NULL
    assert _post(y + 2, x, po, cb, T, 4, C, out) == ALIGN
    assert _post(y, x, po, cb, T, 4, C, x + 1024) == ALIAS        # partial overlap with x
    assert _post(y, x, po, cb, T, 4, C, y) == ALIAS               # over the sublayer output
    assert _post(y, x, po, cb, T, 4, C, po) == ALIAS
    assert _post(y, x, po, cb, 0, 4, C, x) == OK                  # exact in place, T = 0: no-op
    assert _post(y, x, po, cb, T, 4, C, x) == HIP                 # exact in place is legal
    assert _post(y, x, po, cb, T, 4, C, out) == HIP


def test_pack_validation():
    L = m.lib()
    P = Ptrs()
    assert L.mhc_pack_fn(None, 4 * C, P(), None) == NULL
    assert L.mhc_pack_fn(P(), 100, P(), None) == SHAPE
    assert L.mhc_pack_fn(P(), 0, P(), None) == SHAPE
    assert L.mhc_pack_fn(P() + 4, 4 * C, P(), None) == ALIGN
    f = P()
    assert L.mhc_pack_fn(f, 4 * C, f + 4096, None) == ALIAS
    assert L.mhc_pack_fn(P(), 4 * C, P(), None) == HIP


def _collapse(x, p, T_, n, C_, nw, eps, out):
    return m.lib().mhc_collapse(x, p, T_, n, C_, nw, eps, out, None)


def test_collapse_validation():
    P = Ptrs()
    x, p, nw, out = P(), P(), P(), P()
    assert _collapse(x, p, T, 3, C, nw, 1e-6, out) == UNSUP
    assert _collapse(x, p, T, 4, 1000, nw, 1e-6, out) == UNSUP
    assert _collapse(x, p, -1, 4, C, nw, 1e-6, out) == SHAPE
    assert _collapse(x, p, T, 4, C, nw, -1.0, out) == SHAPE           # eps matters with a norm
    assert _collapse(x, p, T, 4, C, None, -1.0, out) == HIP           # ... and is unused without
    assert _collapse(None, p, T, 4, C, nw, 1e-6, out) == NULL
    assert _collapse(x, None, T, 4, C, nw, 1e-6, out) == NULL
    assert _collapse(x, p, T, 4, C, nw, 1e-6, None) == NULL
    assert _collapse(x, p + 4, T, 4, C, nw, 1e-6, out) == ALIGN
    assert _collapse(x, p, T, 4, C, nw, 1e-6, x + 64) == ALIAS
    assert _collapse(x, p, T, 4, C, nw, 1e-6, p) == ALIAS
    assert _collapse(x, p, 0, 4, C, nw, 1e-6, out) == OK
    assert _collapse(x, p, T, 4, C, nw, 1e-6, out) == HIP


def test_wait_timeout_hook_validation():
    """The test hook for bounded waits takes 0 (normal bound) to 2^20 sleeps."""
    L = m.lib()
    assert L.mhc_debug_force_wait_timeouts(-1) == SHAPE
    assert L.mhc_debug_force_wait_timeouts((1 << 20) + 1) == SHAPE
    assert L.mhc_debug_force_wait_timeouts(1 << 20) == OK
    assert L.mhc_debug_force_wait_timeouts(0) == OK


def test_iteration_cap_matches_header():
    src = open(HEADER).read()
    mt = re.search(r"#define\s+MHC_MAX_SINKHORN_ITERS\s+(\d+)", src)
    assert mt and int(mt.group(1)) == m.MAX_SINKHORN_ITERS == 1024
    mt = re.search(r"#define\s+MHC_MAX_TOKENS\s+\(1 << (\d+)\)", src)
    assert mt and (1 << int(mt.group(1))) == m.MAX_TOKENS


def test_workspace_offsets_match_header():
    src = open(HEADER).read()
    vals = {}
    for name in ("MHC_WS_FLAG_BYTES", "MHC_WS_WAIT_ERROR_PERSIST", "MHC_WS_WAIT_ERROR_SPLIT"):
        mt = re.search(r"#define\s+%s\s+(.+)" % name, src)
        assert mt, name
        vals[name] = eval(mt.group(1).split("/*")[0], {})
    assert vals["MHC_WS_FLAG_BYTES"] == m.WS_FLAG_BYTES
    assert vals["MHC_WS_WAIT_ERROR_PERSIST"] == m.WS_WAIT_ERROR_PERSIST
    assert vals["MHC_WS_WAIT_ERROR_SPLIT"] == m.WS_WAIT_ERROR_SPLIT
    assert max(m.WS_WAIT_ERROR_PERSIST, m.WS_WAIT_ERROR_SPLIT) + 4 <= m.WS_FLAG_BYTES
    # every plan's workspace holds the whole flag region
    assert m.mhc_workspace_bytes(8) >= m.WS_FLAG_BYTES


def call_noalloc(**kw):
    a = _pre_args(**kw)
    P = Ptrs()
    P.next = 0x80000000000
    for k in ("y", "post_in", "comb_in", "xo"):
        a.setdefault(k, kw.get(k, P()))
    return m.lib().mhc_post_pre_delayed_noalloc(a["y"], a["x"], a["post_in"], a["comb_in"], a["pre_in"], a["T"],
                                                a["n"], a["C"], a["w"], a["nw"], a["eps"], a["iters"], a["xo"],
                                                a["pre"], a["post"], a["comb"], a["li"], None)


def test_noalloc_validation():
    """The no-allocation seam rejects what mhc_post_pre_delayed rejects, before it looks up its
    buffer (no GPU here: a call that passes every check then fails in the runtime)."""
    assert call_noalloc(n=3) == UNSUP
    assert call_noalloc(C=5000) == UNSUP
    assert call_noalloc(T=-1) == SHAPE
    assert call_noalloc(T=(1 << 22) + 1) == SHAPE
    assert call_noalloc(iters=0) == SHAPE
    assert call_noalloc(iters=1025) == SHAPE
    assert call_noalloc(eps=float("nan")) == SHAPE
    for k in ("y", "x", "post_in", "comb_in", "xo", "pre_in", "pre", "post", "comb", "li"):
        assert call_noalloc(**{k: None}) == NULL, k
    assert call_noalloc(post_in=0x80000000004) == ALIGN
    P = Ptrs()
    x = P()
    assert call_noalloc(x=x, xo=x) == ALIAS
    g = P()
    assert call_noalloc(pre_in=g, pre=g) == ALIAS
    assert call_noalloc(T=0) == OK
    assert call_noalloc() == HIP


def test_noalloc_scratch_covers_every_plan():
    """The library's own buffer holds the workspace of every shape the seam accepts."""
    hdr = open(os.path.join(ROOT, "include", "mhc.h")).read()
    mm = re.search(r"#define MHC_NOALLOC_SCRATCH_BYTES \((\d+)u << (\d+)\)", hdr)
    assert mm and int(mm.group(1)) << int(mm.group(2)) == m.NOALLOC_SCRATCH_BYTES
    for c in range(256, 16384 + 1, 256):
        for t in (1, 16, 33, 512, 2048, 3072, 3073, 4096, 4097, 1 << 22):
            assert m.mhc_workspace_bytes(t, 4, c) <= m.NOALLOC_SCRATCH_BYTES, (t, c)
