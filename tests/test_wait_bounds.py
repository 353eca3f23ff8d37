"""Bounded waits, forced from the host.

Calls that split a tile's projection over workgroups make some of them wait
for others (the own pre-mix collapse workgroups, the persistent kernels'
exchange).  The test hook makes every such wait unsatisfiable with a budget
of a few sleeps, so each wait runs out: the kernels must still end, report the
run-out in the documented workspace word, and, once the hook is off and the
workspace zero-filled again, give the same bits as before.  A form without
waits (the split delayed pre, whose last arriving workgroup finishes the tile)
is unaffected by the hook.
"""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
from gpu_util import dev_bf16, dev_f32, say, torch_mod

pytestmark = pytest.mark.gpu

C = mi.HIDDEN


def weights(d):
    return M.make_weights(dev_f32(d["fn"]), dev_f32(d["bias"]), dev_f32(d["alpha"]))


def words(ws):
    w = ws[:M.WS_FLAG_BYTES].view(torch_mod().int32)
    return int(w[M.WS_WAIT_ERROR_PERSIST // 4]), int(w[M.WS_WAIT_ERROR_SPLIT // 4])


def make_call(kind, T):
    torch = torch_mod()
    if kind == "entry":
        d = mi.entry_inputs(T, seed=4000 + T)
        h, w, nw = dev_bf16(d["h"]), weights(d), dev_bf16(d["norm_weight"])
        return lambda ws: M.mhc_broadcast_entry(h, w, nw, d["eps"], d["iters"], ws=ws)
    d = mi.pre_inputs(T, seed=4100 + T, delayed=True, norm=True)
    x, pin, nw, w = dev_bf16(d["x"]), dev_f32(d["pre_in"]), dev_bf16(d["norm_weight"]), weights(d)
    if kind == "own":
        return lambda ws: M.mhc_pre(x, w, nw, d["eps"], d["iters"], ws=ws)
    if kind == "delayed":
        return lambda ws: M.mhc_pre_delayed(x, pin, w, nw, d["eps"], d["iters"], ws=ws)
    p = mi.post_inputs(T, seed=4200 + T)
    y = dev_bf16(p["y"])
    post = dev_f32(2.0 / (1.0 + np.exp(-p["post_logit"])))
    e = np.exp(p["comb_logit"].astype(np.float64))
    comb = dev_f32(e / e.sum(axis=2, keepdims=True))
    return lambda ws: M.mhc_post_pre_delayed(y, x, post, comb, pin, w, nw, d["eps"], d["iters"], ws=ws)


def bits(outs):
    torch = torch_mod()
    return [None if o is None else (o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32)).clone()
            for o in outs]


# (form, T, word expected set: "persist" / "split" / None for a form without waits)
CASES = [("own", 8, "split"), ("entry", 16, "split"), ("own", 300, "split"),
         ("delayed", 4100, "persist"), ("fused", 3100, "persist"), ("own", 4100, "persist"),
         ("delayed", 7, None), ("fused", 5, None)]


@pytest.mark.parametrize("kind,T,word", CASES)
def test_forced_wait_run_out(kind, T, word):
    torch = torch_mod()
    call = make_call(kind, T)
    ws = torch.zeros(M.mhc_workspace_bytes(T), dtype=torch.uint8, device="cuda")
    say("wait bounds %s T=%d: reference" % (kind, T))
    ref = bits(call(ws))
    torch.cuda.synchronize()
    assert words(ws) == (0, 0)
    say("wait bounds %s T=%d: forced run-out" % (kind, T))
    M.mhc_debug_force_wait_timeouts(4)
    try:
        out = call(ws)
        torch.cuda.synchronize()
    finally:
        M.mhc_debug_force_wait_timeouts(0)
    wp, wsp = words(ws)
    if word == "persist":
        assert wp != 0 and wsp == 0, (wp, wsp)
    elif word == "split":
        assert wsp != 0 and wp == 0, (wp, wsp)
    else:
        assert (wp, wsp) == (0, 0)
        for a, b in zip(bits(out), ref):
            assert b is None or torch.equal(a, b)
    say("wait bounds %s T=%d: recovered" % (kind, T))
    ws.zero_()
    for _ in range(2):
        again = bits(call(ws))
        torch.cuda.synchronize()
        for a, b in zip(again, ref):
            assert b is None or torch.equal(a, b)
        assert int(ws[:M.WS_FLAG_BYTES].view(torch.int32).abs().sum()) == 0
