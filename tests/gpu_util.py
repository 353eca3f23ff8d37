"""Helpers shared by the GPU tests: device transfer and the comparison bars.

Bars (the seam block's tolerances; the bf16 bound follows from one rounding to bf16
of a single-precision value that carries at most a few single-precision roundings
of the summed terms):
  * gates / comb: max relative error <= 1e-4 against the float64 oracle;
  * bf16 outputs: |gpu - v| <= ulp_bf16(v) + (8 * 2^-24 + d) * mag, where v is
    the oracle's exact value, mag the sum of |terms| that formed it, and d the
    relative error of any float gate that fed it (0 when the gate is an input);
  * the collapse without norm, given the same float pre-mix: bit-exact.
"""
import math
import sys

import numpy as np

import oracle

U32 = 2.0 ** -24
GATE_RTOL = 1e-4


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a ROCm GPU"
    return torch


def dev_bf16(bits: np.ndarray):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def dev_f32(a: np.ndarray):
    torch = torch_mod()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def host_bits(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f32(t) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    a = np.abs(np.asarray(v, dtype=np.float64))
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    u = np.exp2(e - 7)
    return np.where(a >= 2.0 ** -126, u, 2.0 ** -133)


def rel_err(g, o) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    return float(np.max(np.abs(g - o) / np.abs(o))) if o.size else 0.0


def check_gates(g_pre, g_post, g_comb, o_pre, o_post, o_comb, what=""):
    errs = dict(pre=rel_err(g_pre, o_pre), post=rel_err(g_post, o_post),
                comb=rel_err(np.asarray(g_comb).reshape(-1, 16), np.asarray(o_comb).reshape(-1, 16)))
    say("  gates max rel err %s: %s" % (what, {k: "%.2e" % v for k, v in errs.items()}))
    for k, v in errs.items():
        assert v <= GATE_RTOL, (what, k, v)
    return max(errs.values())


def check_bf16(g_bits, val, mag, d=0.0, what=""):
    g = oracle.bf16_to_f64(g_bits)
    val = np.asarray(val, dtype=np.float64)
    err = np.abs(g - val)
    bound = ulp_bf16(val) + (8 * U32 + d) * np.asarray(mag, dtype=np.float64)
    bad = err > bound
    n_bad = int(bad.sum())
    worst = float(np.max(err / bound)) if err.size else 0.0
    # share of outputs more than one bf16 ulp (of the exact value) away from it
    beyond = float(np.mean(err > ulp_bf16(val))) if err.size else 0.0
    say("  %s: %d values, worst err/bound %.3f, beyond 1 ulp %.2e, violations %d"
        % (what, err.size, worst, beyond, n_bad))
    if n_bad:
        idx = np.argwhere(bad)[:5]
        for i in idx:
            i = tuple(i)
            say("    at %s gpu %r exact %r bound %r" % (i, g[i], val[i], bound[i]))
    assert n_bad == 0, what


def rms_over_weight(li_bits, w_bits):
    li = oracle.bf16_to_f64(li_bits)
    w = oracle.bf16_to_f64(w_bits)
    return np.sqrt(np.square(li / w[None, :]).mean(1))
