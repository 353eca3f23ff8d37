"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Small sizes run the oracle on every token (several 16-token tiles and a ragged
tail); the full configuration sizes run the GPU on all tokens and the oracle on
sampled rows (tokens are independent).  Bars are in tests/gpu_util.py.
"""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
import oracle
from gpu_util import (check_bf16, check_gates, dev_bf16, dev_f32, host_bits, host_f32,
                      rel_err, rms_over_weight, say, torch_mod, ulp_bf16)

pytestmark = pytest.mark.gpu

C = mi.HIDDEN


def weights(d):
    return M.make_weights(dev_f32(d["fn"]), dev_f32(d["bias"]), dev_f32(d["alpha"]))


def run_delayed(d, rows=None):
    x = dev_bf16(d["x"])
    w = weights(d)
    nw = dev_bf16(d["norm_weight"]) if d["norm_weight"] is not None else None
    pre_out, post, comb, li = M.mhc_pre_delayed(x, dev_f32(d["pre_in"]), w, nw, d["eps"], d["iters"])
    torch_mod().cuda.synchronize()
    r = slice(None) if rows is None else rows
    return (host_f32(pre_out)[r], host_f32(post)[r], host_f32(comb)[r], host_bits(li)[r])


def oracle_delayed(d, rows=None):
    r = slice(None) if rows is None else rows
    return oracle.mhc_pre_delayed(d["x"][r], d["pre_in"][r], d["fn"], d["bias"], d["alpha"], d["eps"],
                                  d["iters"], norm_weight=d["norm_weight"])


# ----------------------------------------------------------------------------- packing

def test_pack_fn_split_and_layout():
    """Packed weight = nearest-even bf16 hi plus bf16 of the remainder, in the
    documented MFMA operand order."""
    torch = torch_mod()
    rng = np.random.default_rng(21)
    K = 4 * 256
    fn = (rng.standard_normal((K, 24)) * 0.02).astype(np.float32)
    packed = M.mhc_pack_fn(dev_f32(fn))
    torch.cuda.synchronize()
    pk = packed.cpu().numpy().view(np.uint16).reshape(K // 32, 3, 64, 8)
    # decode: lane L of tile q holds column 16q + (L & 15), rows 32 kb + 8 (L >> 4) + e
    cols = np.zeros((K, 48), dtype=np.uint16)
    for q in range(3):
        for L in range(64):
            for e in range(8):
                cols[np.arange(K // 32) * 32 + 8 * (L >> 4) + e, 16 * q + (L & 15)] = pk[:, q, L, e]
    hi = oracle.bf16_to_f64(cols[:, :24])
    lo = oracle.bf16_to_f64(cols[:, 24:])
    f = fn.astype(np.float64)
    assert np.array_equal(cols[:, :24], oracle.bf16_rne(f))
    assert np.array_equal(cols[:, 24:], oracle.bf16_rne(f - hi))
    assert np.all(np.abs(f - hi - lo) <= 2.0 ** -16 * np.abs(f))


# ----------------------------------------------------------------------------- pre, delayed, entry

@pytest.mark.parametrize("T", [1, 2, 7, 8, 17, 128, 1000, 2048, 2049, 4097])
def test_pre_no_norm(T):
    """Configuration 0 (T = 8, no norm) and neighbours: own pre-mix.  Up to 2048
    tokens the projection is split and one workgroup per token collapses once
    its tile's pre-mix is published; then each tile's workgroup collapses its
    tokens; from 4097 the persistent kernel's gates-only form runs, then the
    collapse kernel with those gates."""
    d = mi.pre_inputs(T, seed=100 + T)
    x = dev_bf16(d["x"])
    pre, post, comb, li = M.mhc_pre(x, weights(d), None, d["eps"], d["iters"])
    o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"])
    say("mhc_pre T=%d no norm" % T)
    ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"])
    check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="layer_input")


def test_config0_at_its_seed():
    """Configuration 0 exactly as stated: mhc_pre without norm, T = 8, seed 0."""
    d = mi.pre_inputs(8, seed=0)
    pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), None, d["eps"], d["iters"])
    o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"])
    say("config 0 (T=8, seed 0)")
    ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "cfg0")
    check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="cfg0 layer_input")


def _zero_rows(T):
    return sorted({0, min(17, T - 1), T // 2, T - 1})


@pytest.mark.parametrize("form,T", [("delayed", 40), ("delayed", 4100), ("own", 40), ("own", 4100),
                                    ("entry", 40), ("fused", 40), ("fused", 3100)])
def test_all_zero_rows(form, T):
    """Tokens whose whole residual row is zero: the row's RMS is eps alone
    (r = 1/sqrt(eps)), the logits are the bias, the collapse is zero and the folded
    norm gives zero (0 * 1/sqrt(eps) * w).  Mixed with ordinary rows in one call,
    on the split and the persistent forms."""
    torch = torch_mod()
    z = _zero_rows(T)
    say("zero rows %s T=%d rows %s" % (form, T, z))
    if form == "entry":
        d = mi.entry_inputs(T, seed=1900 + T)
        d["h"][z] = 0
        x_out, pre, post, comb, li = M.mhc_broadcast_entry(dev_bf16(d["h"]), weights(d), dev_bf16(d["norm_weight"]),
                                                          d["eps"], d["iters"])
        o = oracle.mhc_broadcast_entry(d["h"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                                       norm_weight=d["norm_weight"])
        assert np.array_equal(host_bits(x_out), o["x_out"])
        ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "entry")
        check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="entry layer_input")
        assert np.all(host_bits(li)[z] & 0x7FFF == 0)
        return
    d = mi.pre_inputs(T, seed=1950 + T, delayed=True, norm=True)
    d["x"][z] = 0
    if form == "own":
        pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"],
                                        d["iters"])
        o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                           norm_weight=d["norm_weight"])
        ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "own")
        li = host_bits(li)
        check_bf16(li, o["li_val"], o["li_mag"], d=2 * ge, what="own layer_input")
    elif form == "delayed":
        pre_out, post, comb, li = run_delayed(d)
        o = oracle_delayed(d)
        check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "delayed")
        check_bf16(li, o["li_val"], o["li_mag"], what="delayed layer_input")
    else:
        p, post_k, comb_k = post_gates(T, seed=1960 + T)
        y = p["y"].copy()
        y[z] = 0
        got = run_fused(d, y, post_k, comb_k)
        check_fused(got, d, y, post_k, comb_k, what="fused zero rows")
        assert np.all(got[0][z] & 0x7FFF == 0)
        li = got[4]
    assert np.all(li[z] & 0x7FFF == 0)


@pytest.mark.parametrize("form,T", [("delayed", 128), ("delayed", 4100), ("fused", 128), ("fused", 3100),
                                    ("own", 4100)])
@pytest.mark.parametrize("iters", [1, 7, 33, 1024])
def test_sinkhorn_iteration_counts(form, T, iters):
    """Iteration counts other than 20, up to the largest accepted (1024), on every
    kernel form (the persistent kernels spread the iterations over the steps of
    the next tile's sweep and finish any that are left when they write the gates)."""
    d = mi.pre_inputs(T, seed=2000 + T + iters, delayed=True, norm=True)
    d["iters"] = iters
    say("iters=%d %s T=%d" % (iters, form, T))
    if form == "delayed":
        pre_out, post, comb, li = run_delayed(d)
        o = oracle_delayed(d)
        check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "delayed iters=%d" % iters)
        check_bf16(li, o["li_val"], o["li_mag"], what="layer_input")
    elif form == "own":
        pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"], iters)
        o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], iters, norm_weight=d["norm_weight"])
        ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "own")
        check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="own layer_input")
    else:
        p, post_k, comb_k = post_gates(T, seed=2100 + T)
        check_fused(run_fused(d, p["y"], post_k, comb_k), d, p["y"], post_k, comb_k, what="fused iters=%d" % iters)


@pytest.mark.parametrize("form,T", [("delayed", 128), ("delayed", 4100), ("fused", 128), ("fused", 3100),
                                    ("own", 128), ("own", 4100), ("entry", 128)])
@pytest.mark.parametrize("eps", [0.0, 0.5])
def test_eps_values(form, T, eps):
    """eps enters both root mean squares (of the 4C row for the logits, of the
    collapsed row for the norm); at 0 and at a value comparable to the mean square
    (0.5, inputs ~N(0,1)) a misplaced eps would move the gates and layer_input far
    past the bar, on the split and the one-sweep forms alike."""
    d = mi.pre_inputs(T, seed=2300 + T, delayed=True, norm=True)
    d["eps"] = eps
    say("eps=%g %s T=%d" % (eps, form, T))
    if form == "delayed":
        pre_out, post, comb, li = run_delayed(d)
        o = oracle_delayed(d)
        check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "delayed eps=%g" % eps)
        check_bf16(li, o["li_val"], o["li_mag"], what="layer_input")
    elif form == "own":
        pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), eps, d["iters"])
        o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], eps, d["iters"], norm_weight=d["norm_weight"])
        ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "own")
        check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="own layer_input")
    elif form == "entry":
        e = mi.entry_inputs(T, seed=2400 + T)
        x_out, pre_e, post_e, comb_e, li_e = M.mhc_broadcast_entry(dev_bf16(e["h"]), weights(e),
                                                                  dev_bf16(e["norm_weight"]), eps, e["iters"])
        oe = oracle.mhc_broadcast_entry(e["h"], e["fn"], e["bias"], e["alpha"], eps, e["iters"],
                                        norm_weight=e["norm_weight"])
        assert np.array_equal(host_bits(x_out), oe["x_out"])
        ge = check_gates(host_f32(pre_e), host_f32(post_e), host_f32(comb_e), oe["pre"], oe["post"], oe["comb"],
                         "entry")
        check_bf16(host_bits(li_e), oe["li_val"], oe["li_mag"], d=2 * ge, what="entry layer_input")
    else:
        p, post_k, comb_k = post_gates(T, seed=2500 + T)
        check_fused(run_fused(d, p["y"], post_k, comb_k), d, p["y"], post_k, comb_k, what="fused eps=%g" % eps)


@pytest.mark.parametrize("form", ["delayed", "fused", "own"])
@pytest.mark.parametrize("T", [1, 2, 6, 7, 8, 64, 128, 256, 1024])
def test_token_list(form, T):
    """The token counts of the parity plan (the pages' test list 1/2/7/128/1024 and
    the decode sizes around it) on every pre form with the fused norm, every token
    against the oracle."""
    d = mi.pre_inputs(T, seed=2600 + T, delayed=True, norm=True)
    say("token list %s T=%d" % (form, T))
    if form == "delayed":
        pre_out, post, comb, li = run_delayed(d)
        o = oracle_delayed(d)
        check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "delayed T=%d" % T)
        check_bf16(li, o["li_val"], o["li_mag"], what="layer_input")
    elif form == "own":
        pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"], d["iters"])
        o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"], norm_weight=d["norm_weight"])
        ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "own")
        check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="own layer_input")
    else:
        p, post_k, comb_k = post_gates(T, seed=2700 + T)
        check_fused(run_fused(d, p["y"], post_k, comb_k), d, p["y"], post_k, comb_k, what="fused T=%d" % T)


@pytest.mark.parametrize("T", [1, 8, 33, 128, 4160])
def test_pre_with_norm(T):
    d = mi.pre_inputs(T, seed=200 + T, norm=True)
    pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"],
                                    d["iters"])
    o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                       norm_weight=d["norm_weight"])
    say("mhc_pre T=%d norm" % T)
    ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"])
    check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="layer_input")


def test_own_premix_repeat_and_workspace_reset():
    """The own-pre-mix forms' collapse workgroups wait on per-tile flags in the
    workspace: back-to-back mhc_pre and entry calls of different sizes on one
    workspace repeat bit for bit, and every flag, count and the wait-ran-out
    word are back at zero afterwards."""
    torch = torch_mod()
    ds = {T: mi.pre_inputs(T, seed=1600 + T, norm=True) for T in (1, 17, 300)}
    es = {T: mi.entry_inputs(T, seed=1700 + T) for T in (1, 17, 300)}

    def pre(T):
        d = ds[T]
        return [host_bits(t) if t.dtype == torch.bfloat16 else host_f32(t)
                for t in M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"], d["iters"])]

    def entry(T, li):
        d = es[T]
        out = M.mhc_broadcast_entry(dev_bf16(d["h"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"], d["iters"],
                                    layer_input=li)
        return [None if t is None else host_bits(t) if t.dtype == torch.bfloat16 else host_f32(t) for t in out]

    first = {T: (pre(T), entry(T, True), entry(T, False)) for T in (1, 17, 300)}
    for T in (17, 300, 1, 17):
        say("own pre-mix repeat T=%d" % T)
        again = (pre(T), entry(T, True), entry(T, False))
        for a, b in zip(first[T], again):
            for u, v in zip(a, b):
                assert (u is None and v is None) or np.array_equal(u, v)
    ws = M.workspace(torch.device("cuda"), 300, C)
    assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("T", [1, 2, 7, 16, 128, 1024])
def test_delayed_no_norm_bit_exact_collapse(T):
    """The pages' token list 1/2/7/128/1024: collapse with the carried pre-mix is bit-exact."""
    d = mi.pre_inputs(T, seed=300 + T, delayed=True)
    pre_out, post, comb, li = run_delayed(d)
    y32 = oracle.collapse32(d["x"], d["pre_in"])
    assert np.array_equal(li, mi.f32_to_bf16_bits(y32))
    o = oracle_delayed(d)
    say("mhc_pre_delayed T=%d no norm" % T)
    check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"])
    check_bf16(li, o["li_val"], o["li_mag"], what="layer_input")


@pytest.mark.parametrize("T", [1, 5, 128, 300])
def test_delayed_with_norm(T):
    """Configuration 1 (T = 128, fused RMSNorm) and ragged neighbours."""
    d = mi.pre_inputs(T, seed=400 + T, delayed=True, norm=True)
    pre_out, post, comb, li = run_delayed(d)
    o = oracle_delayed(d)
    say("mhc_pre_delayed T=%d norm" % T)
    check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"])
    check_bf16(li, o["li_val"], o["li_mag"], what="layer_input")


@pytest.mark.parametrize("T", [1, 8, 64, 256, 1024])
def test_unit_rms_of_fused_norm(T):
    """With weight 1 the folded norm has RMS sqrt(ms/(ms+eps)) ~ 1 per row; a
    half-wave sum of squares would show the page's sqrt(2) (token counts from
    the wavefront-bug PR, The bug)."""
    d = mi.pre_inputs(T, seed=500 + T, delayed=True, norm=True)
    d["norm_weight"] = np.full(C, 0x3F80, np.uint16)
    _, _, _, li = run_delayed(d)
    ratio = rms_over_weight(li, d["norm_weight"])
    say("unit RMS T=%d: min %.6f max %.6f" % (T, ratio.min(), ratio.max()))
    assert np.all(np.abs(ratio - 1.0) < 2.0 ** -8)


def test_delayed_with_own_pre_equals_pre():
    """Feeding mhc_pre's pre-mix back as pre_in reproduces mhc_pre: gates identical
    (delayed-pre PR, Purpose: only the collapse differs), layer_input bitwise without the
    norm and within one bf16 ulp with it (the two collapse forms add the row's sum of
    squares in different orders)."""
    torch = torch_mod()
    for T, norm in ((7, False), (130, True)):
        d = mi.pre_inputs(T, seed=600 + T, norm=norm)
        x = dev_bf16(d["x"])
        w = weights(d)
        nw = dev_bf16(d["norm_weight"]) if norm else None
        pre, post, comb, li = M.mhc_pre(x, w, nw, d["eps"], d["iters"])
        pre2, post2, comb2, li2 = M.mhc_pre_delayed(x, pre.clone(), w, nw, d["eps"], d["iters"])
        torch.cuda.synchronize()
        assert torch.equal(pre, pre2) and torch.equal(post, post2) and torch.equal(comb, comb2)
        if norm:
            va, vb = oracle.bf16_to_f64(host_bits(li)), oracle.bf16_to_f64(host_bits(li2))
            assert np.all(np.abs(va - vb) <= ulp_bf16(np.maximum(np.abs(va), np.abs(vb))))
        else:
            assert torch.equal(li.view(torch.int16), li2.view(torch.int16))


def test_collapse_order_golden_on_gpu():
    """The rounding-order case of tests/golden/collapse_order.txt, on the GPU."""
    T = 3
    xv = np.float32([1.0, 2.0 ** -8, 2.0 ** -24, 2.0 ** -24])
    x32 = np.broadcast_to(xv[None, :, None], (T, 4, C)).copy()
    d = mi.pre_inputs(T, seed=7, delayed=True)
    d["x"] = mi.f32_to_bf16_bits(x32)
    d["pre_in"] = np.ones((T, 4), np.float32)
    _, _, _, li = run_delayed(d)
    assert np.all(li == 0x3F80)


@pytest.mark.parametrize("T", [1, 16, 100, 2100])
def test_broadcast_entry(T):
    """Entry seam: split projection with per-token collapse workgroups (up to 128
    tiles), the tile's own workgroup collapsing past that (2100 tokens)."""
    torch = torch_mod()
    d = mi.entry_inputs(T, seed=900 + T)
    h = dev_bf16(d["h"])
    w = weights(d)
    x_out, pre, post, comb, li = M.mhc_broadcast_entry(h, w, dev_bf16(d["norm_weight"]), d["eps"],
                                                      d["iters"])
    o = oracle.mhc_broadcast_entry(d["h"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                                   norm_weight=d["norm_weight"])
    say("entry T=%d" % T)
    assert np.array_equal(host_bits(x_out), o["x_out"])
    ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"])
    check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="layer_input")
    # without layer_input: same gates, x_out still written
    x2, pre2, _, _, li2 = M.mhc_broadcast_entry(h, w, None, d["eps"], d["iters"], layer_input=False)
    torch.cuda.synchronize()
    assert li2 is None and torch.equal(pre, pre2)
    assert torch.equal(x2.view(torch.int16), x_out.view(torch.int16))


# ----------------------------------------------------------------------------- post

def post_gates(T, seed=3):
    p = mi.post_inputs(T, seed=seed)
    post = (2.0 / (1.0 + np.exp(-p["post_logit"].astype(np.float64)))).astype(np.float32)
    comb = np.stack([oracle.sinkhorn(np.exp(m.astype(np.float64)), 20) for m in p["comb_logit"]])
    return p, post, comb.astype(np.float32)


@pytest.mark.parametrize("Cx,T", [(1024, 37), (1280, 37), (256, 129), (768, 51)])
def test_post_hidden_sizes(Cx, T):
    """mhc_post on every token at hidden sizes where a wave's 64 threads always
    share one token (C / 8 a multiple of 64: 1024) and where waves straddle two
    tokens (1280, 256, 768), against the oracle's exact value and bit for bit
    against the single-precision post in the library's order."""
    torch = torch_mod()
    p = mi.post_inputs(T, seed=41 + Cx + T, C=Cx)
    post = (2.0 / (1.0 + np.exp(-p["post_logit"].astype(np.float64)))).astype(np.float32)
    comb = np.stack([oracle.sinkhorn(np.exp(m.astype(np.float64)), 20) for m in p["comb_logit"]]).astype(np.float32)
    out = host_bits(M.mhc_post(dev_bf16(p["y"]), dev_bf16(p["x"]), dev_f32(post), dev_f32(comb)))
    torch.cuda.synchronize()
    say("mhc_post C=%d T=%d" % (Cx, T))
    o = oracle.mhc_post(p["y"], p["x"], post, comb)
    check_bf16(out, o["out_val"], o["out_mag"], what="post C=%d" % Cx)
    assert np.array_equal(out, oracle.post32(p["y"], p["x"], post, comb))


@pytest.mark.parametrize("T", [1, 3, 64])
def test_post_small(T):
    torch = torch_mod()
    p, post, comb = post_gates(T, seed=30 + T)
    y, x = dev_bf16(p["y"]), dev_bf16(p["x"])
    out = M.mhc_post(y, x, dev_f32(post), dev_f32(comb))
    o = oracle.mhc_post(p["y"], p["x"], post, comb)
    say("mhc_post T=%d" % T)
    check_bf16(host_bits(out), o["out_val"], o["out_mag"], what="out")
    # exact in-place form gives the same bits
    M.mhc_post(y, x, dev_f32(post), dev_f32(comb), out=x)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(x), host_bits(out))


def test_post_bits_equal_single_precision_oracle():
    """mhc_post writes the single-precision post rounded once (the residual the next
    seam reads), bit for bit, and the hand-worked order case of
    tests/golden/post_order.txt."""
    T = 33
    p, post, comb = post_gates(T, seed=41)
    out = M.mhc_post(dev_bf16(p["y"]), dev_bf16(p["x"]), dev_f32(post), dev_f32(comb))
    assert np.array_equal(host_bits(out), oracle.post32(p["y"], p["x"], post, comb))
    # and, independently of any order, within the bf16 bar of the exact (double) post
    ex = oracle.mhc_post(p["y"], p["x"], post, comb)
    check_bf16(host_bits(out), ex["out_val"], ex["out_mag"], what="post vs exact")
    yb = np.full((1, C), 0x3F80, np.uint16)
    xb = np.full((1, 4, C), 0x3F80, np.uint16)
    pp = np.float32([[1.0 + 2.0 ** -8, 0, 0, 0]])
    cm = np.zeros((1, 4, 4), np.float32)
    cm[0, 0] = 2.0 ** -25
    out = M.mhc_post(dev_bf16(yb), dev_bf16(xb), dev_f32(pp), dev_f32(cm))
    assert np.all(host_bits(out)[0, 0] == 0x3F80)


def test_post_identity():
    torch = torch_mod()
    T = 5
    p, _, _ = post_gates(T)
    x = dev_bf16(p["x"])
    eye = np.tile(np.eye(4, dtype=np.float32), (T, 1, 1))
    out = M.mhc_post(dev_bf16(p["y"]), x, dev_f32(np.zeros((T, 4), np.float32)), dev_f32(eye))
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(out), p["x"])


# ----------------------------------------------------------------------------- full sizes, sampled

def _sample_rows(T, outliers, n=48, seed=0):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    rows |= set(outliers[:16].tolist()) | {0, T - 1}
    return np.array(sorted(rows))


def test_config2_prefill_delayed_norm_sampled():
    """T = 16384, fused norm, 1% outlier rows x100: GPU on all tokens (the
    benchmark's launch), oracle on sampled rows incl. outliers."""
    T = 16384
    d = mi.pre_inputs(T, seed=2, delayed=True, norm=True, outlier_frac=0.01)
    assert len(d["outliers"]) == 164
    rows = _sample_rows(T, d["outliers"])
    pre_out, post, comb, li = run_delayed(d, rows)
    o = oracle_delayed(d, rows)
    say("config 2 sampled rows: %d" % len(rows))
    check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "cfg2")
    check_bf16(li, o["li_val"], o["li_mag"], what="cfg2 layer_input")
    y32 = oracle.collapse32(d["x"][rows], d["pre_in"][rows])
    d2 = dict(d)
    d2["norm_weight"] = None
    _, _, _, li_nn = run_delayed(d2, rows)
    assert np.array_equal(li_nn, mi.f32_to_bf16_bits(y32))


def test_prefill_own_entry_collapse_sampled():
    """T = 16384, the launches the benchmark times for mhc_pre (the persistent
    gates-only pass, then the streaming collapse), the entry seam and the
    standalone collapse: GPU on all tokens, oracle on sampled rows incl. the 1%
    outlier rows."""
    torch = torch_mod()
    T = 16384
    d = mi.pre_inputs(T, seed=21, norm=True, outlier_frac=0.01)
    rows = _sample_rows(T, d["outliers"], seed=1)
    x = dev_bf16(d["x"])
    pre, post, comb, li = M.mhc_pre(x, weights(d), dev_bf16(d["norm_weight"]), d["eps"], d["iters"])
    torch.cuda.synchronize()
    o = oracle.mhc_pre(d["x"][rows], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                       norm_weight=d["norm_weight"])
    say("mhc_pre T=16384 sampled rows: %d" % len(rows))
    ge = check_gates(host_f32(pre)[rows], host_f32(post)[rows], host_f32(comb)[rows], o["pre"], o["post"],
                     o["comb"], "mhc_pre T=16384")
    check_bf16(host_bits(li)[rows], o["li_val"], o["li_mag"], d=2 * ge, what="mhc_pre T=16384 layer_input")
    # the standalone collapse at this size (streaming form), with the GPU's own pre-mix
    p = host_f32(pre)
    out = host_bits(M.mhc_collapse(x, dev_f32(p)))
    assert np.array_equal(out[rows], mi.f32_to_bf16_bits(oracle.collapse32(d["x"][rows], p[rows])))
    del x, pre, post, comb, li
    # the entry seam at this size
    e = mi.entry_inputs(T, seed=22)
    x_out, epre, epost, ecomb, eli = M.mhc_broadcast_entry(dev_bf16(e["h"]), weights(e), dev_bf16(e["norm_weight"]),
                                                           e["eps"], e["iters"])
    torch.cuda.synchronize()
    oe = oracle.mhc_broadcast_entry(e["h"][rows], e["fn"], e["bias"], e["alpha"], e["eps"], e["iters"],
                                    norm_weight=e["norm_weight"])
    say("entry T=16384 sampled rows: %d" % len(rows))
    assert np.array_equal(host_bits(x_out)[rows], oe["x_out"])
    ge = check_gates(host_f32(epre)[rows], host_f32(epost)[rows], host_f32(ecomb)[rows], oe["pre"], oe["post"],
                     oe["comb"], "entry T=16384")
    check_bf16(host_bits(eli)[rows], oe["li_val"], oe["li_mag"], d=2 * ge, what="entry T=16384 layer_input")


@pytest.mark.parametrize("T", [2113, 4096, 4097, 6001])
def test_delayed_many_tokens_every_token(T):
    """Many tokens, checked on every token: the split form with 2-4 splits per
    tile (2113, 4096 tokens) and the persistent delayed kernel from 4097 tokens
    (64-token tiles over groups of 16 workgroups; several tiles per group,
    ragged last tile, groups with unequal tile counts).  Without the norm the
    layer input is the exact-order collapse, bit for bit."""
    d = mi.pre_inputs(T, seed=40 + T, delayed=True, norm=True, outlier_frac=0.01)
    say("delayed many tokens T=%d" % T)
    pre_out, post, comb, li = run_delayed(d)
    o = oracle_delayed(d)
    check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "persist T=%d" % T)
    check_bf16(li, o["li_val"], o["li_mag"], what="persist T=%d layer_input" % T)
    d2 = dict(d)
    d2["norm_weight"] = None
    _, _, _, li_nn = run_delayed(d2)
    assert np.array_equal(li_nn, mi.f32_to_bf16_bits(oracle.collapse32(d["x"], d["pre_in"])))


def test_persistent_repeat_and_workspace_reset():
    """The persistent kernel's arrival counters are back at zero after every
    call: calls of different sizes on one workspace repeat bit for bit."""
    torch = torch_mod()
    ds = {T: mi.pre_inputs(T, seed=800 + T, delayed=True, norm=True) for T in (6001, 4160)}
    first = {T: run_delayed(ds[T]) for T in (6001, 4160)}
    for T in (4160, 6001, 4160):
        again = run_delayed(ds[T])
        for u, v in zip(first[T], again):
            assert np.array_equal(u, v)
    ws = M.workspace(torch.device("cuda"), 6001, C)
    assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


@pytest.mark.parametrize("T", [1, 7, 300, 6600])
def test_standalone_collapse(T):
    """mhc_collapse: without the norm bit-exact to the exact-order float collapse;
    with it within the bf16 bound of the oracle (6600 tokens: the streaming form,
    more bytes than the memory-side cache holds)."""
    rng = np.random.default_rng(60 + T)
    d = mi.pre_inputs(T, seed=60 + T, delayed=True, norm=True)
    p = rng.uniform(0, 1, (T, 4)).astype(np.float32)
    x = dev_bf16(d["x"])
    out = host_bits(M.mhc_collapse(x, dev_f32(p)))
    assert np.array_equal(out, mi.f32_to_bf16_bits(oracle.collapse32(d["x"], p)))
    outn = host_bits(M.mhc_collapse(x, dev_f32(p), dev_bf16(d["norm_weight"]), 1e-6))
    o = oracle.mhc_collapse(d["x"], p, d["norm_weight"], 1e-6)
    check_bf16(outn, o["li_val"], o["li_mag"], what="collapse T=%d" % T)


@pytest.mark.parametrize("T", [100, 4160, 6600])
def test_standalone_collapse_equals_delayed_layer_input(T):
    """Without the norm, mhc_collapse(x, p) is bit-identical to the layer_input of
    mhc_pre_delayed(x, pre_in = p), on both pre-kernel forms (split and persistent)."""
    d = mi.pre_inputs(T, seed=70 + T, delayed=True, norm=False)
    _, _, _, li = run_delayed(d)
    out = host_bits(M.mhc_collapse(dev_bf16(d["x"]), dev_f32(d["pre_in"])))
    assert np.array_equal(out, li)


def test_config3_post_sampled():
    T = 16384
    p, post, comb = post_gates(T, seed=3)
    out = M.mhc_post(dev_bf16(p["y"]), dev_bf16(p["x"]), dev_f32(post), dev_f32(comb))
    torch_mod().cuda.synchronize()
    rows = _sample_rows(T, np.zeros(0, np.int64), n=64, seed=3)
    ob = host_bits(out)[rows]
    o = oracle.mhc_post(p["y"][rows], p["x"][rows], post[rows], comb[rows])
    say("config 3 sampled rows: %d" % len(rows))
    check_bf16(ob, o["out_val"], o["out_mag"], what="cfg3 out")


# every counter of both kernel forms lies in the workspace's first 128 KiB
COUNTER_BYTES = 192 * 1024


def test_repeatable_and_workspace_reset():
    """Split-K runs leave the workspace counters at zero: back-to-back calls on
    one workspace, with different token counts, give identical bits."""
    torch = torch_mod()
    for T in (1, 64, 2113, 1):
        d = mi.pre_inputs(T, seed=700, delayed=True, norm=True)
        a = run_delayed(d)
        b = run_delayed(d)
        for u, v in zip(a, b):
            assert np.array_equal(u, v)
    ws = M.workspace(torch.device("cuda"), 1, C)
    assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


# ----------------------------------------------------------------------------- post -> delayed pre, fused

def fused_case(T, seed, norm=True, outlier_frac=0.0):
    """Seam k's post inputs (y, gates) and seam k+1's delayed pre inputs (x = the
    residual entering seam k, weights, pre_in = seam k's pre-mix)."""
    d = mi.pre_inputs(T, seed=seed, delayed=True, norm=norm, outlier_frac=outlier_frac)
    p, post, comb = post_gates(T, seed=seed + 1)
    return d, p["y"], post, comb


def run_fused(d, y, post, comb, rows=None):
    nw = dev_bf16(d["norm_weight"]) if d["norm_weight"] is not None else None
    xo, pre_out, po, co, li = M.mhc_post_pre_delayed(dev_bf16(y), dev_bf16(d["x"]), dev_f32(post), dev_f32(comb),
                                                     dev_f32(d["pre_in"]), weights(d), nw, d["eps"], d["iters"])
    torch_mod().cuda.synchronize()
    r = slice(None) if rows is None else rows
    return host_bits(xo)[r], host_f32(pre_out)[r], host_f32(po)[r], host_f32(co)[r], host_bits(li)[r]


def check_fused(got, d, y, post, comb, rows=None, what=""):
    r = slice(None) if rows is None else rows
    xo, pre_out, po, co, li = got
    o = oracle.mhc_post_pre_delayed(y[r], d["x"][r], post[r], comb[r], d["pre_in"][r], d["fn"], d["bias"],
                                    d["alpha"], d["eps"], d["iters"], norm_weight=d["norm_weight"])
    # the next residual: the single-precision post bit for bit, within the bar of the exact one
    assert np.array_equal(xo, o["x_out"]), what
    ex = oracle.mhc_post(y[r], d["x"][r], post[r], comb[r])
    check_bf16(xo, ex["out_val"], ex["out_mag"], what=what + " x_out")
    check_gates(pre_out, po, co, o["pre_out"], o["post"], o["comb"], what)
    if d["norm_weight"] is None:
        assert np.array_equal(li, mi.f32_to_bf16_bits(oracle.collapse32(o["x_out"], d["pre_in"][r]))), what
    check_bf16(li, o["li_val"], o["li_mag"], what=what + " layer_input")


@pytest.mark.parametrize("T,norm", [(1, True), (2, False), (7, True), (16, False), (128, True), (300, True),
                                    (1000, False)])
def test_post_pre_delayed(T, norm):
    """Post of seam k fused with the delayed pre of seam k+1: every token against the
    oracle's composition (single-precision post, then the delayed pre on its bits)."""
    d, y, post, comb = fused_case(T, 1100 + T, norm)
    say("mhc_post_pre_delayed T=%d norm=%s" % (T, norm))
    check_fused(run_fused(d, y, post, comb), d, y, post, comb, what="fused T=%d" % T)


@pytest.mark.parametrize("T", [5, 300, 1100, 4100])
def test_post_pre_delayed_equals_two_calls(T):
    """The fused form against mhc_post followed by mhc_pre_delayed: the residual bit
    for bit, layer_input without the norm bit for bit; the gates, and layer_input
    with the norm, to the bar (partial sums are added in another order)."""
    torch = torch_mod()
    for norm in (False, True):
        d, y, post, comb = fused_case(T, 1200 + T, norm)
        nw = dev_bf16(d["norm_weight"]) if norm else None
        a = run_fused(d, y, post, comb)
        xo = M.mhc_post(dev_bf16(y), dev_bf16(d["x"]), dev_f32(post), dev_f32(comb))
        pre_out, po, co, li = M.mhc_pre_delayed(xo, dev_f32(d["pre_in"]), weights(d), nw, d["eps"], d["iters"])
        torch.cuda.synchronize()
        say("fused vs two calls T=%d norm=%s" % (T, norm))
        assert np.array_equal(a[0], host_bits(xo))
        check_gates(a[1], a[2], a[3], host_f32(pre_out), host_f32(po), host_f32(co), "fused vs two calls")
        lb = host_bits(li)
        if norm:
            va, vb = oracle.bf16_to_f64(a[4]), oracle.bf16_to_f64(lb)
            assert np.all(np.abs(va - vb) <= ulp_bf16(np.maximum(np.abs(va), np.abs(vb))))
        else:
            assert np.array_equal(a[4], lb)


@pytest.mark.parametrize("T", [1281, 3072, 3073, 3999])
def test_fused_many_tokens_every_token(T):
    """Many tokens of the fused seam, every token against the oracle
    composition, with the norm and without it: the split kernel's fused mode
    (up to 3072 tokens) and the persistent fused kernel (the persistent delayed
    kernel with the post stage in front) from 3073."""
    for norm in (True, False):
        d, y, post, comb = fused_case(T, 1300 + T, norm, outlier_frac=0.01)
        say("fused many tokens T=%d norm=%s" % (T, norm))
        check_fused(run_fused(d, y, post, comb), d, y, post, comb, what="persist fused T=%d" % T)


def test_persistent_fused_repeat_and_workspace_reset():
    """Back-to-back fused calls of different sizes on one workspace repeat bit for
    bit, and the counters are back at zero."""
    torch = torch_mod()
    cs = {T: fused_case(T, 1400 + T, True) for T in (4096, 2048)}
    first = {T: run_fused(*cs[T]) for T in (4096, 2048)}
    for T in (2048, 4096, 2048):
        again = run_fused(*cs[T])
        for u, v in zip(first[T], again):
            assert np.array_equal(u, v)
    ws = M.workspace(torch.device("cuda"), 4096, C)
    assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


def test_fused_seam_prefill_sampled():
    """T = 16384, the prefill seam fused: post of seam k (configuration 3's shapes)
    into the delayed pre of seam k+1 with the norm and 1% outlier rows (configuration
    2's); GPU on all tokens in the benchmark's launch, oracle on sampled rows."""
    T = 16384
    d, y, post, comb = fused_case(T, 2, True, outlier_frac=0.01)
    rows = _sample_rows(T, d["outliers"])
    got = run_fused(d, y, post, comb, rows)
    say("fused prefill sampled rows: %d" % len(rows))
    check_fused(got, d, y, post, comb, rows=rows, what="fused T=16384")


def test_workspace_shared_by_split_and_persistent_forms():
    """One workspace serves both kernel forms: a split call (partial sums in the
    workspace) followed by persistent calls, and the reverse, stay correct, and
    every counter is back at zero after each call."""
    torch = torch_mod()
    ws = M.workspace(torch.device("cuda"), 4100, C)
    small = mi.pre_inputs(100, seed=1500, delayed=True, norm=True)   # split form, 4 splits per tile
    big = fused_case(4100, 1501, True)
    for rnd in range(2):
        say("shared workspace round %d: split T=100" % rnd)
        pre_out, post, comb, li = run_delayed(small)
        o = oracle_delayed(small)
        check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "split after persistent")
        assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0
        say("shared workspace round %d: persistent fused T=4100" % rnd)
        check_fused(run_fused(*big), *big, what="persistent fused after split")
        assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0
        run_delayed(small)
        say("shared workspace round %d: persistent delayed T=4100" % rnd)
        d = big[0]
        pre_out, post, comb, li = run_delayed(d)
        o = oracle_delayed(d)
        check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "persistent after split")
        assert int(ws[:COUNTER_BYTES].view(torch.int32).abs().sum()) == 0


# ----------------------------------------------------------------------------- configuration 4: seam chain

def _chain_weights(n_seams, C_):
    ws = []
    for k in range(n_seams):
        sw = mi.sweep_seam_weights(k, C=C_)
        ws.append(sw)
    return ws


# A free-running chain compounds each seam's rounding: gates within the 1e-4 bar
# feed the next post, the next seam's logits move by ~1e-4 of their size, and
# Sinkhorn's exponentials pass that on.  Measured over 80 seams at T = 1/7/64:
# gates drift up to 1e-1 relative, the final residual ~7e-3 (relative L2).
CHAIN_GATE_RTOL = 0.3
CHAIN_X_RTOL = 3e-2


@pytest.mark.parametrize("T", [1, 7, 64])
def test_config4_seam_chain(T):
    """Configuration 4: the model-entry seam, then 80 delayed seams (per-seam weights
    from seed 1000 + k, fused norm, the sublayer an identity stand-in: y = layer_input),
    each seam one mhc_post_pre_delayed call.  Every seam is checked to the tight bars
    on the oracle chain's own inputs (uploaded to the GPU); the GPU chain is also run
    free and held to drift bounds against the oracle chain."""
    torch = torch_mod()
    n_seams = 80
    e = mi.entry_inputs(T, seed=999)
    sws = _chain_weights(n_seams, C)
    gw = [M.make_weights(dev_f32(sw["fn"]), dev_f32(sw["bias"]), dev_f32(sw["alpha"])) for sw in sws]
    gnw = [dev_bf16(sw["norm_weight"]) for sw in sws]
    # free-running GPU chain
    we = M.make_weights(dev_f32(e["fn"]), dev_f32(e["bias"]), dev_f32(e["alpha"]))
    x, pre, post, comb, li = M.mhc_broadcast_entry(dev_bf16(e["h"]), we, dev_bf16(e["norm_weight"]), e["eps"],
                                                   e["iters"])
    g_gates = []
    for k in range(n_seams):
        x, pre, post, comb, li = M.mhc_post_pre_delayed(li, x, post, comb, pre, gw[k], gnw[k], 1e-6, 20)
        g_gates.append((host_f32(pre), host_f32(post), host_f32(comb)))
    x_final = M.mhc_post(li, x, post, comb)
    torch.cuda.synchronize()
    gx = host_bits(x_final)
    # oracle chain: every input is the oracle's own previous output; each seam is also
    # run on the GPU from the oracle's inputs and checked to the tight bars
    o = oracle.mhc_broadcast_entry(e["h"], e["fn"], e["bias"], e["alpha"], e["eps"], e["iters"],
                                   norm_weight=e["norm_weight"])
    ox, opre, opost, ocomb, oli = o["x_out"], o["pre"], o["post"], o["comb"], o["li"]
    worst = 0.0
    for k in range(n_seams):
        sw = sws[k]
        p32, c32, q32 = opost.astype(np.float32), ocomb.astype(np.float32), opre.astype(np.float32)
        f = oracle.mhc_post_pre_delayed(oli, ox, p32, c32, q32, sw["fn"], sw["bias"], sw["alpha"], 1e-6, 20,
                                        norm_weight=sw["norm_weight"])
        xs, ps, qs, cs, ls = M.mhc_post_pre_delayed(dev_bf16(oli), dev_bf16(ox), dev_f32(p32), dev_f32(c32),
                                                    dev_f32(q32), gw[k], gnw[k], 1e-6, 20)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(xs), f["x_out"]), k
        ge = check_gates(host_f32(ps), host_f32(qs), host_f32(cs), f["pre_out"], f["post"], f["comb"],
                         "seam %d" % k)
        check_bf16(host_bits(ls), f["li_val"], f["li_mag"], what="seam %d layer_input" % k)
        ox, opre, opost, ocomb, oli = f["x_out"], f["pre_out"], f["post"], f["comb"], f["li"]
        gp, gq, gc = g_gates[k]
        errs = (rel_err(gp, opre), rel_err(gq, opost), rel_err(gc.reshape(-1, 16), ocomb.reshape(-1, 16)))
        worst = max(worst, max(errs))
    oxf = oracle.bf16_to_f64(oracle.post32(oli, ox, opost.astype(np.float32), ocomb.astype(np.float32)))
    gxf = oracle.bf16_to_f64(gx)
    rel = np.linalg.norm(gxf - oxf) / np.linalg.norm(oxf)
    say("config 4 T=%d: free chain worst gate rel err over 80 seams %.2e, final residual rel L2 err %.2e"
        % (T, worst, rel))
    assert worst <= CHAIN_GATE_RTOL and rel <= CHAIN_X_RTOL


@pytest.mark.parametrize("T", [2048, 16384])
def test_config4_seam_chain_sampled(T):
    """Configuration 4 at the sizes the benchmark's chain reports beyond the decode
    sizes: T = 2048 (the split kernel's fused mode) and T = 16384 (the persistent
    fused kernel).  The GPU chain runs on all T tokens.  The oracle chain follows
    32 sampled token rows through the entry seam and all 80 seams (tokens are
    independent, so a row's chain does not depend on the others).  At every seam the
    GPU also runs one full-size launch on a copy of its own state in which the
    sampled rows are replaced by the oracle chain's values, and those rows are held
    to the tight per-seam bars against the oracle's next seam; the free-running GPU
    chain is held to the drift bounds of the small-T chain test."""
    torch = torch_mod()
    n_seams = 80
    rng = np.random.default_rng(T)
    rows = np.array(sorted({0, T - 1} | set(rng.choice(T, 30, replace=False).tolist())))
    idx = torch.from_numpy(rows).cuda()
    e = mi.entry_inputs(T, seed=999)
    sws = _chain_weights(n_seams, C)
    gw = [M.make_weights(dev_f32(sw["fn"]), dev_f32(sw["bias"]), dev_f32(sw["alpha"])) for sw in sws]
    gnw = [dev_bf16(sw["norm_weight"]) for sw in sws]
    we = M.make_weights(dev_f32(e["fn"]), dev_f32(e["bias"]), dev_f32(e["alpha"]))
    say("config 4 sampled T=%d: entry" % T)
    x, pre, post, comb, li = M.mhc_broadcast_entry(dev_bf16(e["h"]), we, dev_bf16(e["norm_weight"]), e["eps"],
                                                   e["iters"])
    o = oracle.mhc_broadcast_entry(e["h"][rows], e["fn"], e["bias"], e["alpha"], e["eps"], e["iters"],
                                   norm_weight=e["norm_weight"])
    assert np.array_equal(host_bits(x.index_select(0, idx)), o["x_out"])
    ox, opre, opost, ocomb, oli = o["x_out"], o["pre"], o["post"], o["comb"], o["li"]
    xs = torch.empty_like(x)
    worst = 0.0
    for k in range(n_seams):
        sw = sws[k]
        p32, c32, q32 = opost.astype(np.float32), ocomb.astype(np.float32), opre.astype(np.float32)
        f = oracle.mhc_post_pre_delayed(oli, ox, p32, c32, q32, sw["fn"], sw["bias"], sw["alpha"], 1e-6, 20,
                                        norm_weight=sw["norm_weight"])
        # one full-size launch with the oracle chain's rows scattered into the GPU state
        xc, lic = x.clone(), li.clone()
        prec, postc, combc = pre.clone(), post.clone(), comb.clone()
        xc.index_copy_(0, idx, dev_bf16(ox))
        lic.index_copy_(0, idx, dev_bf16(oli))
        prec.index_copy_(0, idx, dev_f32(q32))
        postc.index_copy_(0, idx, dev_f32(p32))
        combc.index_copy_(0, idx, dev_f32(c32))
        outs = M._pre_outputs(T, C, x.device)
        M.mhc_post_pre_delayed(lic, xc, postc, combc, prec, gw[k], gnw[k], 1e-6, 20, out=(xs,) + tuple(outs))
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(xs.index_select(0, idx)), f["x_out"]), k
        check_gates(host_f32(outs[0].index_select(0, idx)), host_f32(outs[1].index_select(0, idx)),
                    host_f32(outs[2].index_select(0, idx)), f["pre_out"], f["post"], f["comb"], "seam %d" % k)
        check_bf16(host_bits(outs[3].index_select(0, idx)), f["li_val"], f["li_mag"], what="seam %d layer_input" % k)
        del xc, lic, prec, postc, combc, outs
        # the free-running chain advances on its own outputs
        x, pre, post, comb, li = M.mhc_post_pre_delayed(li, x, post, comb, pre, gw[k], gnw[k], 1e-6, 20)
        ox, opre, opost, ocomb, oli = f["x_out"], f["pre_out"], f["post"], f["comb"], f["li"]
        errs = (rel_err(host_f32(pre.index_select(0, idx)), opre), rel_err(host_f32(post.index_select(0, idx)), opost),
                rel_err(host_f32(comb.index_select(0, idx)).reshape(-1, 16), ocomb.reshape(-1, 16)))
        worst = max(worst, max(errs))
    x_final = M.mhc_post(li, x, post, comb)
    torch.cuda.synchronize()
    gxf = oracle.bf16_to_f64(host_bits(x_final.index_select(0, idx)))
    oxf = oracle.bf16_to_f64(oracle.post32(oli, ox, opost.astype(np.float32), ocomb.astype(np.float32)))
    rel = np.linalg.norm(gxf - oxf) / np.linalg.norm(oxf)
    say("config 4 T=%d sampled: free chain worst gate rel err over 80 seams %.2e, final residual rel L2 err %.2e"
        % (T, worst, rel))
    assert worst <= CHAIN_GATE_RTOL and rel <= CHAIN_X_RTOL


# ----------------------------------------------------------------------------- other hidden sizes

@pytest.mark.parametrize("Cx,T", [(7168, 2100), (7168, 4100), (7168, 6001), (4096, 3100), (4096, 4100),
                                  (4096, 6001)])
def test_other_hidden_sizes_many_tokens(Cx, T):
    """Other hidden sizes with a persistent form (4096, 7168) at token counts past the
    decode sizes, every token: the fused seam (its x_out bit for bit equal to
    mhc_post's), the delayed pre and the own pre-mix form against the oracle.  At
    C = 7168 the fused and own forms are persistent from T = 2049, the delayed form
    from T = 4097 (at C = 4096: 3073 and 4097)."""
    torch = torch_mod()
    d = mi.pre_inputs(T, seed=2200 + Cx + T, C=Cx, delayed=True, norm=True, outlier_frac=0.01)
    say("hidden %d T=%d" % (Cx, T))
    p, post_k, comb_k = post_gates(T, seed=2300 + T)
    y = mi.post_inputs(T, seed=2301, C=Cx)["y"]
    got = run_fused(d, y, post_k, comb_k)
    check_fused(got, d, y, post_k, comb_k, what="fused C=%d T=%d" % (Cx, T))
    xo = M.mhc_post(dev_bf16(y), dev_bf16(d["x"]), dev_f32(post_k), dev_f32(comb_k))
    torch.cuda.synchronize()
    assert np.array_equal(got[0], host_bits(xo))
    del xo
    pre_out, post, comb, li = run_delayed(d)
    o = oracle_delayed(d)
    check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "delayed C=%d" % Cx)
    check_bf16(li, o["li_val"], o["li_mag"], what="delayed layer_input")
    pre, post, comb, li = M.mhc_pre(dev_bf16(d["x"]), weights(d), dev_bf16(d["norm_weight"]), d["eps"], d["iters"])
    o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"], norm_weight=d["norm_weight"])
    ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "own C=%d" % Cx)
    check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="own layer_input")


@pytest.mark.parametrize("Cx,T", [(256, 1), (256, 300), (1024, 37), (7168, 5), (7168, 300), (16384, 37)])
def test_other_hidden_sizes(Cx, T):
    """Hidden sizes other than 5120 (any multiple of 256 up to 16384; the split forms
    serve them at every T): own pre-mix, delayed with norm, the fused seam, the entry
    seam and the standalone collapse against the oracle."""
    torch = torch_mod()
    d = mi.pre_inputs(T, seed=1600 + Cx + T, C=Cx, delayed=True, norm=True)
    x, nw, pin = dev_bf16(d["x"]), dev_bf16(d["norm_weight"]), dev_f32(d["pre_in"])
    w = weights(d)
    say("hidden %d T=%d" % (Cx, T))
    pre, post, comb, li = M.mhc_pre(x, w, None, d["eps"], d["iters"])
    o = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"])
    ge = check_gates(host_f32(pre), host_f32(post), host_f32(comb), o["pre"], o["post"], o["comb"], "pre")
    check_bf16(host_bits(li), o["li_val"], o["li_mag"], d=2 * ge, what="pre layer_input")
    pre_out, post, comb, li = run_delayed(d)
    o = oracle_delayed(d)
    check_gates(pre_out, post, comb, o["pre_out"], o["post"], o["comb"], "delayed")
    check_bf16(li, o["li_val"], o["li_mag"], what="delayed layer_input")
    p, post_k, comb_k = post_gates(T, seed=1700 + T)
    y = mi.post_inputs(T, seed=1701, C=Cx)["y"]
    check_fused(run_fused(d, y, post_k, comb_k), d, y, post_k, comb_k, what="fused")
    e = mi.entry_inputs(T, seed=1800 + T, C=Cx)
    x_out, pre_e, post_e, comb_e, li_e = M.mhc_broadcast_entry(dev_bf16(e["h"]), weights(e), dev_bf16(e["norm_weight"]),
                                                              e["eps"], e["iters"])
    oe = oracle.mhc_broadcast_entry(e["h"], e["fn"], e["bias"], e["alpha"], e["eps"], e["iters"],
                                    norm_weight=e["norm_weight"])
    assert np.array_equal(host_bits(x_out), oe["x_out"])
    x2, pre2, _, _, li2 = M.mhc_broadcast_entry(dev_bf16(e["h"]), weights(e), dev_bf16(e["norm_weight"]), e["eps"],
                                                e["iters"], layer_input=False)
    torch.cuda.synchronize()
    assert li2 is None and np.array_equal(host_bits(x2), oe["x_out"]) and torch.equal(pre2, pre_e)
    ge = check_gates(host_f32(pre_e), host_f32(post_e), host_f32(comb_e), oe["pre"], oe["post"], oe["comb"], "entry")
    check_bf16(host_bits(li_e), oe["li_val"], oe["li_mag"], d=2 * ge, what="entry layer_input")
    out = host_bits(M.mhc_collapse(x, pin))
    torch.cuda.synchronize()
    assert np.array_equal(out, mi.f32_to_bf16_bits(oracle.collapse32(d["x"], d["pre_in"])))
