"""mhc_post_pre_delayed_noalloc on the GPU: the seam with the library's own
per-GPU buffer gives the same bits as mhc_post_pre_delayed with a workspace.

Two calls in a row on one stream, the second with fewer tokens (the buffer
keeps the first call's contents: what the second call reads first must have
been left or made zero), over the plans the seam has: the persistent fused
kernel (C = 5120, 7168), the split kernel's fused mode (few tokens) and the
post kernel followed by the delayed split kernel (C = 6144, T > 3072).  Then a
graph captured with the no-allocation call replays to the eager bits."""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
from gpu_util import say, torch_mod

pytestmark = pytest.mark.gpu


def _inputs(T, C, seed):
    torch = torch_mod()
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    dev = torch.device("cuda")
    y = torch.randn((T, C), generator=g, device=dev).to(torch.bfloat16)
    x = torch.randn((T, 4, C), generator=g, device=dev).to(torch.bfloat16)
    post_in = 2.0 * torch.sigmoid(torch.randn((T, 4), generator=g, device=dev))
    comb_in = torch.rand((T, 4, 4), generator=g, device=dev)
    comb_in = comb_in / comb_in.sum(dim=-1, keepdim=True)
    pre_in = torch.rand((T, 4), generator=g, device=dev)
    return y, x, post_in, comb_in, pre_in


def _weights(C, seed):
    torch = torch_mod()
    fn, bias, alpha = mi.seam_weights(seed, 4 * C)
    w = M.make_weights(torch.from_numpy(fn).cuda(), torch.from_numpy(bias).cuda(),
                       torch.from_numpy(alpha).cuda())
    rng = np.random.default_rng(seed + 1)
    nw = torch.from_numpy(mi.f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(C).astype(np.float32))
                          .view(np.int16)).view(torch.bfloat16).cuda()
    return w, nw


def _same(a, b):
    torch = torch_mod()
    for u, v in zip(a, b):
        if u.dtype == torch.bfloat16:
            u, v = u.view(torch.int16), v.view(torch.int16)
        if not torch.equal(u, v):
            return False
    return True


@pytest.mark.parametrize("C,T1,T2", [(5120, 16384, 1000), (7168, 4100, 7), (5120, 4100, 3073),
                                     (4096, 8192, 64), (6144, 3500, 33), (5120, 64, 1)])
def test_noalloc_matches_workspace_form(C, T1, T2):
    torch = torch_mod()
    w, nw = _weights(C, seed=C + T1)
    for i, T in enumerate((T1, T2)):
        say("noalloc C=%d T=%d (call %d)" % (C, T, i + 1))
        y, x, post_in, comb_in, pre_in = _inputs(T, C, seed=7 * T + i)
        ref = M.mhc_post_pre_delayed(y, x, post_in, comb_in, pre_in, w, nw, 1e-6, 20)
        got = M.mhc_post_pre_delayed_noalloc(y, x, post_in, comb_in, pre_in, w, nw, 1e-6, 20)
        torch.cuda.synchronize()
        assert _same(got, ref), (C, T)


def test_noalloc_graph_replays():
    """Captured at T = 1 and T = 5000 (persistent form); replays between eager calls of the
    same entry point at other sizes give the eager bits each time."""
    torch = torch_mod()
    C = 5120
    w, nw = _weights(C, seed=5)
    s = torch.cuda.Stream()
    cases = []
    for T in (1, 5000):
        say("noalloc graph T=%d" % T)
        args = _inputs(T, C, seed=T)
        torch.cuda.synchronize()   # the inputs were drawn on the default stream; the calls run on s
        with torch.cuda.stream(s):
            out = [torch.empty_like(args[1])] + list(M._pre_outputs(T, C, args[1].device))
            M.mhc_post_pre_delayed_noalloc(*args, w, nw, 1e-6, 20, out=out)
        s.synchronize()
        ref = [o.clone() for o in out]
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                M.mhc_post_pre_delayed_noalloc(*args, w, nw, 1e-6, 20, out=out)
        s.synchronize()
        cases.append((g, out, ref, args))   # the graph reads these inputs: keep them alive
    other = _inputs(300, C, seed=3)
    for rep in range(3):
        for g, out, ref, _ in cases:
            for o in out:
                o.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert _same(out, ref), rep
            M.mhc_post_pre_delayed_noalloc(*other, w, nw, 1e-6, 20)   # eager work between replays
            torch.cuda.synchronize()
    del cases
