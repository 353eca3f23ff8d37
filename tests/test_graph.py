"""Structure of the C-ABI calls on the GPU: HIP-graph capture and replay, and the
extent of every write.

Every pre-stage form (split with its partial sums, own-pre-mix records, the
persistent exchange, the gates-only pass followed by the collapse), the post
stage, the fused seam, the entry seam and the standalone collapse are captured
once in a HIP graph and replayed (1000 times at T <= 512, 100 above), with eager work and a
synchronisation between replays: every replay must give the eager call's bits
(the workspace's counters and records reset themselves inside each call), and
the workspace words that calls read before writing must be back at zero.  The
outputs are views into larger buffers whose guard bands hold a poison pattern:
nothing may be written outside [T, ...].  The captured graphs also give each
call's launch count: kernel nodes only, no memset or copy.
"""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
from gpu_util import dev_bf16, dev_f32, say, torch_mod

pytestmark = pytest.mark.gpu

C = mi.HIDDEN
PAD = 64                      # guard elements on each side (keeps 16-byte alignment)
POISON16 = 0x7FC1             # a bf16 NaN pattern the library never writes
POISON32 = 0x7FC00001         # a float32 NaN pattern the library never writes
COUNTER_BYTES = 192 * 1024    # workspace words read before written (counters, records)


def guarded(shape, kind):
    """(buffer, view): the view has `shape` and sits between two poisoned guard bands."""
    torch = torch_mod()
    n = int(np.prod(shape))
    if kind == "bf16":
        buf = torch.empty(n + 2 * PAD, dtype=torch.int16, device="cuda").fill_(POISON16)
        view = buf[PAD:PAD + n].view(torch.bfloat16).view(*shape)
    else:
        buf = torch.empty(n + 2 * PAD, dtype=torch.int32, device="cuda").fill_(POISON32)
        view = buf[PAD:PAD + n].view(torch.float32).view(*shape)
    return buf, view


def check_guards(bufs, what):
    for buf in bufs:
        poison = POISON16 if buf.dtype == torch_mod().int16 else POISON32
        head = buf[:PAD].cpu().numpy()
        tail = buf[-PAD:].cpu().numpy()
        assert np.all(head == poison) and np.all(tail == poison), what


def weights(d):
    return M.make_weights(dev_f32(d["fn"]), dev_f32(d["bias"]), dev_f32(d["alpha"]))


def gates_of(p):
    """Device post [T,4] in (0, 2) and a row-normalised positive comb [T,4,4] from the logits."""
    post = 2.0 / (1.0 + np.exp(-p["post_logit"].astype(np.float64)))
    e = np.exp(p["comb_logit"].astype(np.float64))
    return dev_f32(post), dev_f32(e / e.sum(axis=2, keepdims=True))


def case(kind, T):
    """Inputs, guarded outputs and a zero-argument call for one entry point."""
    if kind == "entry":
        d = mi.entry_inputs(T, seed=3000 + T)
        h = dev_bf16(d["h"])
        w, nw = weights(d), dev_bf16(d["norm_weight"])
        specs = [((T, 4, C), "bf16"), ((T, 4), "f32"), ((T, 4), "f32"), ((T, 4, 4), "f32"), ((T, C), "bf16")]
        gs = [guarded(s, k) for s, k in specs]
        outs = tuple(v for _, v in gs)
        ws = M.workspace(h.device, T, C)

        def call():
            M.mhc_broadcast_entry(h, w, nw, d["eps"], d["iters"], out=outs, ws=ws)
        return call, gs, outs, ws
    if kind == "post":
        p = mi.post_inputs(T, seed=3100 + T)
        y, x = dev_bf16(p["y"]), dev_bf16(p["x"])
        post, comb = gates_of(p)
        gs = [guarded((T, 4, C), "bf16")]
        outs = (gs[0][1],)

        def call():
            M.mhc_post(y, x, post, comb, out=outs[0])
        return call, gs, outs, None
    if kind == "collapse":
        d = mi.pre_inputs(T, seed=3200 + T, delayed=True, norm=True)
        x, pin, nw = dev_bf16(d["x"]), dev_f32(d["pre_in"]), dev_bf16(d["norm_weight"])
        gs = [guarded((T, C), "bf16")]
        outs = (gs[0][1],)

        def call():
            M.mhc_collapse(x, pin, nw, 1e-6, out=outs[0])
        return call, gs, outs, None
    d = mi.pre_inputs(T, seed=3300 + T, delayed=True, norm=True)
    x, pin, nw = dev_bf16(d["x"]), dev_f32(d["pre_in"]), dev_bf16(d["norm_weight"])
    w = weights(d)
    ws = M.workspace(x.device, T, C)
    specs = [((T, 4), "f32"), ((T, 4), "f32"), ((T, 4, 4), "f32"), ((T, C), "bf16")]
    if kind == "fused":
        specs = [((T, 4, C), "bf16")] + specs
    gs = [guarded(s, k) for s, k in specs]
    outs = tuple(v for _, v in gs)
    if kind == "own":
        def call():
            M.mhc_pre(x, w, nw, d["eps"], d["iters"], out=outs, ws=ws)
    elif kind == "delayed":
        def call():
            M.mhc_pre_delayed(x, pin, w, nw, d["eps"], d["iters"], out=outs, ws=ws)
    else:
        p = mi.post_inputs(T, seed=3400 + T)
        y = dev_bf16(p["y"])
        post, comb = gates_of(p)

        def call():
            M.mhc_post_pre_delayed(y, x, post, comb, pin, w, nw, d["eps"], d["iters"], out=outs, ws=ws)
    return call, gs, outs, ws


@pytest.mark.parametrize("kind,T", [
    ("delayed", 7), ("delayed", 128), ("delayed", 4100),        # split (32 / 16 splits), persistent
    ("own", 8), ("own", 2049), ("own", 4100),                   # records, one workgroup per tile, gates-only + collapse
    ("fused", 5), ("fused", 300), ("fused", 3100),              # split fused mode, persistent fused
    ("entry", 16), ("entry", 2100),                             # records, one workgroup per tile
    ("post", 64), ("collapse", 300)])
def test_graph_replay_and_guard_bands(kind, T):
    torch = torch_mod()
    call, gs, outs, ws = case(kind, T)
    say("graph %s T=%d" % (kind, T))
    call()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    check_guards([b for b, _ in gs], "%s T=%d eager" % (kind, T))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    reps = 1000 if T <= 512 else 100
    for r in range(reps):
        for b, _ in gs:                       # eager work between replays: re-poison everything
            b.fill_(POISON16 if b.dtype == torch.int16 else POISON32)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(o.view(torch.int16) if o.dtype == torch.bfloat16 else o.view(torch.int32),
                               e.view(torch.int16) if e.dtype == torch.bfloat16 else e.view(torch.int32)), \
                (kind, T, r)
        check_guards([b for b, _ in gs], "%s T=%d replay %d" % (kind, T, r))
    if ws is not None:
        assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0, (kind, T)
    del g


def _graph_node_types(graph):
    """Types of the nodes of a captured HIP graph (hipGraphNodeType: 0 kernel, 1 memcpy,
    2 memset, ...), read with the runtime's own graph queries."""
    import ctypes
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipGraphGetNodes.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]
    hip.hipGraphNodeGetType.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int)]
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(ctypes.c_void_p(graph), None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * max(1, n.value))()
    assert hip.hipGraphGetNodes(ctypes.c_void_p(graph), nodes, ctypes.byref(n)) == 0
    types = []
    for i in range(n.value):
        t = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(t)) == 0
        types.append(t.value)
    return types


@pytest.mark.parametrize("kind,T,launches", [
    ("delayed", 7, 1), ("delayed", 128, 1), ("delayed", 4100, 1),
    ("own", 8, 1), ("own", 2049, 1), ("own", 4100, 2),
    ("fused", 5, 1), ("fused", 300, 1), ("fused", 3100, 1),
    ("entry", 16, 1), ("entry", 2100, 1), ("post", 64, 1), ("collapse", 300, 1)])
def test_launches_per_call(kind, T, launches):
    """What a call enqueues, read from its captured graph: kernel launches only (no
    memset or copy node), one per call (a seam is one launch with the fused entry
    point) except the own pre-mix past the one-sweep threshold (gates, then the
    collapse with them)."""
    torch = torch_mod()
    call, gs, outs, ws = case(kind, T)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph(keep_graph=True)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    types = _graph_node_types(g.raw_cuda_graph())
    say("launches %s T=%d: node types %s" % (kind, T, types))
    assert types == [0] * launches, types
