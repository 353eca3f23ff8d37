"""The largest token count the C ABI accepts (MHC_MAX_TOKENS = 2^22), at the
smallest hidden size (C = 256, so every buffer fits with room to spare): every
entry point runs on all 2^22 tokens in the launch it takes at that size (one
split per 16-token tile: more tiles than the split form's counters; the fused
seam as two launches), and the oracle checks sampled rows (the first and last
tiles, the middle, random rows).  Token offsets beyond 2^31 elements and grids of
millions of workgroups are what this exercises.  At C = 5120 the persistent
kernels run past the benchmark's 16384 tokens: T = 20001 is 313 tiles of 64 (the
last one 33 tokens), 20 tiles for some groups of 16 workgroups and 19 for others.

The residual and the sublayer output are drawn on the device with torch's
seeded generator (float32 N(0,1) rounded once to bf16, chunk by chunk): the host
generator would need 4.3e9 draws per tensor.  The weights come from the shared
input generator."""
import numpy as np
import pytest

import decode_mhc_pre_amd as M
import mhc_inputs as mi
import oracle
from gpu_util import check_bf16, check_gates, dev_bf16, dev_f32, host_bits, host_f32, say, torch_mod

pytestmark = pytest.mark.gpu

T = 1 << 22
CX = 256
CHUNK = 1 << 20


def device_normal_bf16(shape, seed):
    torch = torch_mod()
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    for a in range(0, shape[0], CHUNK):
        b = min(shape[0], a + CHUNK)
        out[a:b].copy_(torch.randn((b - a,) + tuple(shape[1:]), generator=g, device="cuda"))
    return out


def device_uniform(shape, seed):
    torch = torch_mod()
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    return torch.rand(shape, generator=g, device="cuda")


def sample_rows(seed, n=T):
    rng = np.random.default_rng(seed)
    fixed = [0, 1, 15, 16, 17, n // 2 - 1, n // 2, n - 33, n - 17, n - 16, n - 2, n - 1]
    return np.array(sorted(set(fixed) | set(int(v) for v in rng.choice(n, 48, replace=False))))


def rows_bits(t, rows):
    torch = torch_mod()
    idx = torch.from_numpy(rows).cuda()
    return host_bits(t.index_select(0, idx))


def rows_f32(t, rows):
    torch = torch_mod()
    idx = torch.from_numpy(rows).cuda()
    return host_f32(t.index_select(0, idx))


def weights_of(d):
    return M.make_weights(dev_f32(d["fn"]), dev_f32(d["bias"]), dev_f32(d["alpha"]))


@pytest.fixture(scope="module")
def residual():
    torch = torch_mod()
    say("max sizes: residual [%d, 4, %d] on the device" % (T, CX))
    x = device_normal_bf16((T, 4, CX), seed=90001)
    d = mi.pre_inputs(16, seed=90002, C=CX, delayed=True, norm=True)
    yield x, d
    del x
    torch.cuda.empty_cache()


def test_max_tokens_delayed_and_own(residual):
    torch = torch_mod()
    x, d = residual
    w, nw = weights_of(d), dev_bf16(d["norm_weight"])
    pin = device_uniform((T, 4), seed=90003)
    rows = sample_rows(1)
    xr, pr = rows_bits(x, rows), rows_f32(pin, rows)
    say("max sizes: mhc_pre_delayed T=%d" % T)
    pre_out, post, comb, li = M.mhc_pre_delayed(x, pin, w, nw, d["eps"], d["iters"])
    torch.cuda.synchronize()
    o = oracle.mhc_pre_delayed(xr, pr, d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                               norm_weight=d["norm_weight"])
    check_gates(rows_f32(pre_out, rows), rows_f32(post, rows), rows_f32(comb, rows), o["pre_out"], o["post"],
                o["comb"], "max delayed")
    check_bf16(rows_bits(li, rows), o["li_val"], o["li_mag"], what="max delayed layer_input")
    del pre_out, post, comb, li
    say("max sizes: mhc_pre T=%d" % T)
    pre, post, comb, li = M.mhc_pre(x, w, nw, d["eps"], d["iters"])
    torch.cuda.synchronize()
    o = oracle.mhc_pre(xr, d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"], norm_weight=d["norm_weight"])
    ge = check_gates(rows_f32(pre, rows), rows_f32(post, rows), rows_f32(comb, rows), o["pre"], o["post"],
                     o["comb"], "max own")
    check_bf16(rows_bits(li, rows), o["li_val"], o["li_mag"], d=2 * ge, what="max own layer_input")
    del pre, post, comb, li
    say("max sizes: mhc_collapse T=%d" % T)
    out = M.mhc_collapse(x, pin, nw, d["eps"])
    torch.cuda.synchronize()
    oc = oracle.mhc_collapse(xr, pr, norm_weight=d["norm_weight"], eps=d["eps"])
    check_bf16(rows_bits(out, rows), oc["li_val"], oc["li_mag"], what="max collapse")


def test_max_tokens_post_and_fused(residual):
    torch = torch_mod()
    x, d = residual
    w, nw = weights_of(d), dev_bf16(d["norm_weight"])
    y = device_normal_bf16((T, CX), seed=90004)
    pin = device_uniform((T, 4), seed=90005)
    post = 2.0 * device_uniform((T, 4), seed=90006)
    e = torch.exp(2.0 * device_uniform((T, 4, 4), seed=90007) - 1.0)
    comb = e / e.sum(dim=1, keepdim=True)            # column sums 1
    del e
    rows = sample_rows(2)
    xr, yr = rows_bits(x, rows), rows_bits(y, rows)
    pr, por, cr = rows_f32(pin, rows), rows_f32(post, rows), rows_f32(comb, rows)
    say("max sizes: mhc_post T=%d" % T)
    out = M.mhc_post(y, x, post, comb)
    torch.cuda.synchronize()
    op = oracle.mhc_post(yr, xr, por, cr)
    check_bf16(rows_bits(out, rows), op["out_val"], op["out_mag"], what="max post")
    del out
    torch.cuda.empty_cache()
    say("max sizes: mhc_post_pre_delayed T=%d" % T)
    xo, pre_out, po, co, li = M.mhc_post_pre_delayed(y, x, post, comb, pin, w, nw, d["eps"], d["iters"])
    torch.cuda.synchronize()
    of = oracle.mhc_post_pre_delayed(yr, xr, por, cr, pr, d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                                     norm_weight=d["norm_weight"])
    assert np.array_equal(rows_bits(xo, rows), of["x_out"])
    check_gates(rows_f32(pre_out, rows), rows_f32(po, rows), rows_f32(co, rows), of["pre_out"], of["post"],
                of["comb"], "max fused")
    check_bf16(rows_bits(li, rows), of["li_val"], of["li_mag"], what="max fused layer_input")


def test_max_tokens_entry():
    torch = torch_mod()
    h = device_normal_bf16((T, CX), seed=90008)
    e = mi.entry_inputs(16, seed=90009, C=CX)
    rows = sample_rows(3)
    hr = rows_bits(h, rows)
    say("max sizes: mhc_broadcast_entry T=%d" % T)
    x_out, pre, post, comb, li = M.mhc_broadcast_entry(h, weights_of(e), dev_bf16(e["norm_weight"]), e["eps"],
                                                      e["iters"])
    torch.cuda.synchronize()
    o = oracle.mhc_broadcast_entry(hr, e["fn"], e["bias"], e["alpha"], e["eps"], e["iters"],
                                   norm_weight=e["norm_weight"])
    assert np.array_equal(rows_bits(x_out, rows), o["x_out"])
    ge = check_gates(rows_f32(pre, rows), rows_f32(post, rows), rows_f32(comb, rows), o["pre"], o["post"],
                     o["comb"], "max entry")
    check_bf16(rows_bits(li, rows), o["li_val"], o["li_mag"], d=2 * ge, what="max entry layer_input")
    del x_out, h
    torch.cuda.empty_cache()


@pytest.mark.parametrize("form", ["delayed", "fused", "own"])
def test_persistent_beyond_benchmark_size(form):
    torch = torch_mod()
    n, C = 20001, mi.HIDDEN
    x = device_normal_bf16((n, 4, C), seed=91001)
    d = mi.pre_inputs(16, seed=91002, delayed=True, norm=True)
    w, nw = weights_of(d), dev_bf16(d["norm_weight"])
    pin = device_uniform((n, 4), seed=91003)
    rows = sample_rows(4, n)
    xr, pr = rows_bits(x, rows), rows_f32(pin, rows)
    say("persistent %s T=%d" % (form, n))
    if form == "delayed":
        pre_out, post, comb, li = M.mhc_pre_delayed(x, pin, w, nw, d["eps"], d["iters"])
        torch.cuda.synchronize()
        o = oracle.mhc_pre_delayed(xr, pr, d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                                   norm_weight=d["norm_weight"])
        check_gates(rows_f32(pre_out, rows), rows_f32(post, rows), rows_f32(comb, rows), o["pre_out"], o["post"],
                    o["comb"], form)
        check_bf16(rows_bits(li, rows), o["li_val"], o["li_mag"], what=form + " layer_input")
    elif form == "own":
        pre, post, comb, li = M.mhc_pre(x, w, nw, d["eps"], d["iters"])
        torch.cuda.synchronize()
        o = oracle.mhc_pre(xr, d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"], norm_weight=d["norm_weight"])
        ge = check_gates(rows_f32(pre, rows), rows_f32(post, rows), rows_f32(comb, rows), o["pre"], o["post"],
                         o["comb"], form)
        check_bf16(rows_bits(li, rows), o["li_val"], o["li_mag"], d=2 * ge, what=form + " layer_input")
    else:
        y = device_normal_bf16((n, C), seed=91004)
        post_in = 2.0 * device_uniform((n, 4), seed=91005)
        e = torch.exp(2.0 * device_uniform((n, 4, 4), seed=91006) - 1.0)
        comb_in = e / e.sum(dim=1, keepdim=True)
        xo, pre_out, po, co, li = M.mhc_post_pre_delayed(y, x, post_in, comb_in, pin, w, nw, d["eps"], d["iters"])
        torch.cuda.synchronize()
        of = oracle.mhc_post_pre_delayed(rows_bits(y, rows), xr, rows_f32(post_in, rows), rows_f32(comb_in, rows),
                                         pr, d["fn"], d["bias"], d["alpha"], d["eps"], d["iters"],
                                         norm_weight=d["norm_weight"])
        assert np.array_equal(rows_bits(xo, rows), of["x_out"])
        check_gates(rows_f32(pre_out, rows), rows_f32(po, rows), rows_f32(co, rows), of["pre_out"], of["post"],
                    of["comb"], form)
        check_bf16(rows_bits(li, rows), of["li_val"], of["li_mag"], what=form + " layer_input")
