"""The Python binding on the GPU: every argument is checked before its pointer
reaches the library (which sees raw addresses only), and the default workspaces
survive graph capture.

Bad arguments -- strided or expanded views, wrong shapes, wrong element types,
out tensors of the wrong shape -- must raise before anything is enqueued: the
outputs passed in stay untouched.  The default workspace of a stream is
allocated once at the size that serves every token count, so a graph captured
with it at T = 1 still replays correctly after a call at T = 16384 on the same
stream (a grown-and-replaced workspace would leave the graph pointing at freed
memory)."""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
from gpu_util import dev_bf16, dev_f32, host_bits, host_f32, say, torch_mod

pytestmark = pytest.mark.gpu

C = mi.HIDDEN


def test_bad_arguments_raise_before_launch():
    torch = torch_mod()
    T = 8
    d = mi.pre_inputs(T, seed=5, delayed=True, norm=True)
    x, pin, nw = dev_bf16(d["x"]), dev_f32(d["pre_in"]), dev_bf16(d["norm_weight"])
    w = M.make_weights(dev_f32(d["fn"]), dev_f32(d["bias"]), dev_f32(d["alpha"]))
    outs = M._pre_outputs(T, C, x.device)
    for o in outs:
        o.view(torch.int32 if o.dtype == torch.float32 else torch.int16).fill_(0x7FC1)
    snap = [o.clone() for o in outs]
    h = x[:, 0, :]                                   # a strided view of one stream
    bad = [
        ("expanded residual", lambda: M.mhc_pre(h.unsqueeze(1).expand(T, 4, C), w, out=outs)),
        ("strided residual", lambda: M.mhc_pre_delayed(x[::2], pin[::2], w, out=outs)),
        ("float64 pre_in", lambda: M.mhc_pre_delayed(x, pin.double(), w, out=outs)),
        ("short pre_in", lambda: M.mhc_pre_delayed(x, pin[:4], w, out=outs)),
        ("transposed pre_in", lambda: M.mhc_pre_delayed(x, pin.t().contiguous().t(), w, out=outs)),
        ("float32 residual", lambda: M.mhc_pre(x.float(), w, out=outs)),
        ("norm weight too short", lambda: M.mhc_pre(x, w, nw[:100], out=outs)),
        ("float32 norm weight", lambda: M.mhc_pre(x, w, nw.float(), out=outs)),
        ("wrong out shape", lambda: M.mhc_pre(x, w, out=(outs[0][:4],) + tuple(outs[1:]))),
        ("out layer_input float32", lambda: M.mhc_pre(x, w, out=tuple(outs[:3]) + (outs[3].float(),))),
        ("iters above the cap", lambda: M.mhc_pre(x, w, iters=1025, out=outs)),
        ("negative eps", lambda: M.mhc_pre(x, w, eps=-1.0, out=outs)),
        ("weights for another K", lambda: M.mhc_broadcast_entry(h.contiguous(), w)),
        ("short y", lambda: M.mhc_post(x[:4, 0, :].contiguous(), x, pin, torch.zeros((T, 4, 4), device="cuda"))),
        ("comb float64", lambda: M.mhc_post(x[:, 0, :].contiguous(), x, pin,
                                            torch.zeros((T, 4, 4), device="cuda", dtype=torch.float64))),
        ("fused x_out wrong shape", lambda: M.mhc_post_pre_delayed(
            x[:, 0, :].contiguous(), x, pin, torch.zeros((T, 4, 4), device="cuda"), pin, w,
            out=(torch.empty((T, 4, C - 256), dtype=torch.bfloat16, device="cuda"),) + tuple(outs))),
        ("collapse p short", lambda: M.mhc_collapse(x, pin[:3])),
        ("workspace float32", lambda: M.mhc_pre(x, w, out=outs, ws=torch.zeros(1 << 20, device="cuda"))),
        ("workspace 2-D", lambda: M.mhc_pre(x, w, out=outs,
                                            ws=torch.zeros((2, 1 << 20), dtype=torch.uint8, device="cuda"))),
    ]
    for what, fn in bad:
        with pytest.raises((ValueError, TypeError)):
            fn()
        say("  refused: %s" % what)
    torch.cuda.synchronize()
    for o, s in zip(outs, snap):
        assert torch.equal(o.view(torch.int8), s.view(torch.int8))


def test_default_workspace_survives_capture_then_larger_call():
    """Capture a decode call (T = 1) with the default workspace, then call the
    same stream's default workspace at T = 16384, then replay: the replay must
    still give the eager bits, and the workspace object never changed."""
    torch = torch_mod()
    s = torch.cuda.Stream()
    d1 = mi.pre_inputs(1, seed=11, delayed=True, norm=True)
    x1, pin1, nw = dev_bf16(d1["x"]), dev_f32(d1["pre_in"]), dev_bf16(d1["norm_weight"])
    w = M.make_weights(dev_f32(d1["fn"]), dev_f32(d1["bias"]), dev_f32(d1["alpha"]))
    big = mi.pre_inputs(16384, seed=12, delayed=True, norm=True)
    xb, pinb = dev_bf16(big["x"]), dev_f32(big["pre_in"])
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        out = M._pre_outputs(1, C, x1.device)
        M.mhc_pre_delayed(x1, pin1, w, nw, out=out)            # creates the stream's default workspace
        ws0 = M.workspace(x1.device, 1, C, stream=s)
    s.synchronize()
    ref = [o.clone() for o in out]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            M.mhc_pre_delayed(x1, pin1, w, nw, out=out)
        for o in out:
            o.zero_()
        res_big = M.mhc_pre_delayed(xb, pinb, w, nw)           # same stream, many tokens
        ws1 = M.workspace(x1.device, 16384, C, stream=s)
    s.synchronize()
    assert ws1.data_ptr() == ws0.data_ptr()
    assert ws0.numel() >= M.mhc_workspace_bytes(M.MAX_TOKENS, 4, C)
    for _ in range(3):
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(out, ref):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o, r.view(torch.int16)
                               if r.dtype == torch.bfloat16 else r)
    assert host_f32(res_big[0]).shape == (16384, 4)
    M.check_workspace(ws0)
    del g


def test_default_workspaces_are_per_stream():
    torch = torch_mod()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        a = M.workspace(torch.device("cuda"), 8, C)
    with torch.cuda.stream(s2):
        b = M.workspace(torch.device("cuda"), 8, C)
    assert a.data_ptr() != b.data_ptr()
