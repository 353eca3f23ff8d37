"""Run-to-run determinism of the persistent kernels at the benchmark's size.

The one-sweep kernels exchange partial sums between workgroups through device
memory with counters and bounded waits; every member sums the records in the
same order, so a call's outputs do not depend on which workgroup arrives
first.  Sixteen back-to-back calls of each form at T = 16384, C = 5120 (the
fused seam, the delayed pre and the own-pre-mix form, with the folded norm)
must all give the first call's bits, with the workspace counters back at zero
and no wait run out.  A race in the exchange, or a hazard that shows only under
load, would make some call differ.
"""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
from gpu_util import say, torch_mod

pytestmark = pytest.mark.gpu

T, C, CALLS = 16384, 5120, 16


def _inputs(seed):
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
    fn, bias, alpha = mi.seam_weights(seed, 4 * C)
    w = M.make_weights(torch.from_numpy(fn).cuda(), torch.from_numpy(bias).cuda(), torch.from_numpy(alpha).cuda())
    rng = np.random.default_rng(seed + 1)
    nw = torch.from_numpy(mi.f32_to_bf16_bits(1.0 + 0.1 * rng.standard_normal(C).astype(np.float32))
                          .view(np.int16)).cuda().view(torch.bfloat16)
    return y, x, post_in, comb_in, pre_in, w, nw


def _same(a, b):
    torch = torch_mod()
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("form", ["fused", "delayed", "own"])
def test_persistent_forms_repeat_bit_for_bit(form):
    torch = torch_mod()
    y, x, post_in, comb_in, pre_in, w, nw = _inputs(97)
    ws = torch.zeros(M.mhc_workspace_bytes(T, C=C), dtype=torch.uint8, device="cuda")

    def call():
        if form == "fused":
            return M.mhc_post_pre_delayed(y, x, post_in, comb_in, pre_in, w, nw, 1e-6, 20, ws=ws)
        if form == "delayed":
            return M.mhc_pre_delayed(x, pre_in, w, nw, 1e-6, 20, ws=ws)
        return M.mhc_pre(x, w, nw, 1e-6, 20, ws=ws)

    say("determinism %s T=%d: first call" % (form, T))
    ref = [o.clone() for o in call() if o is not None]
    torch.cuda.synchronize()
    for i in range(1, CALLS):
        out = [o for o in call() if o is not None]
        for a, b in zip(out, ref):
            assert _same(a, b), "call %d differs from the first" % i
    torch.cuda.synchronize()
    say("determinism %s T=%d: %d calls identical" % (form, T, CALLS))
    M.check_workspace(ws, clear=False)
    assert int(ws[:M.WS_FLAG_BYTES].view(torch.int32).abs().sum()) == 0
