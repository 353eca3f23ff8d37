"""Pins for the CPU oracle (no GPU).

Each test checks the oracle against something other than itself: closed forms,
invariants that the mathematics fixes, a library routine (numpy matmul) where
the step *is* that routine, a correctly rounded pure-Python brute force at
T = 1, and a high-precision reformulation of the Sinkhorn iteration.  Chosen so
that a plausible mistake (dropped term, wrong sign or index, transposed operand,
swapped row/column order, off-by-one iteration count) fails at least one.
"""
import math
import os

import numpy as np
import pytest

import mhc_inputs as mi
import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(vals):
    return mi.f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


# ----------------------------------------------------------------------------- bf16 rounding

def test_bf16_roundtrip_all_finite():
    b = np.arange(0x10000, dtype=np.uint16)
    v = oracle.bf16_to_f64(b)
    fin = np.isfinite(v)
    out = oracle.bf16_rne(v[fin])
    # -0.0 and +0.0 keep their sign; every finite bf16 maps to itself
    assert np.array_equal(out, b[fin])


def test_bf16_rne_matches_torch_from_float32():
    import torch
    rng = np.random.default_rng(5)
    a = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),     # subnormal range
        np.float32([3.3895314e38, 3.39e38, -3.4028235e38, 1e-45, 0.0, -0.0]),
    ])
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(a.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_ties_and_no_double_rounding():
    one = 1.0
    # exact tie between 1 and 1+2^-7 goes to the even neighbour (1.0)
    assert oracle.bf16_rne(np.array([one + 2.0**-8]))[0] == 0x3F80
    # tie between 1+2^-7 and 1+2^-6 goes to 1+2^-6 (even)
    assert oracle.bf16_rne(np.array([one + 2.0**-7 + 2.0**-8]))[0] == 0x3F82
    # just above the tie: must round up.  Via float32 this value would first
    # become the tie itself and then round to even (down) -- double rounding.
    assert oracle.bf16_rne(np.array([one + 2.0**-8 + 2.0**-40]))[0] == 0x3F81
    assert oracle.bf16_rne(np.array([-(one + 2.0**-8 + 2.0**-40)]))[0] == 0xBF81


# ----------------------------------------------------------------------------- logits

def test_logits_closed_form_rank1():
    """x = a everywhere, fn[k][j] = u_k v_j: s = K a^2, P_j = a v_j sum(u)."""
    T, C = 2, 256
    K = 4 * C
    a = 2.0
    x = np.full((T, 4, C), 0x4000, dtype=np.uint16)  # bf16 2.0
    k = np.arange(K)
    u = ((k % 7) - 3).astype(np.float64) / 8.0        # exact in fp32
    v = (np.arange(24) + 1).astype(np.float64) / 16.0
    fn = np.outer(u, v).astype(np.float32)
    assert np.array_equal(fn.astype(np.float64), np.outer(u, v))
    bias = (np.arange(24) * 0.25 - 3).astype(np.float32)
    alpha = np.float32([2.0, 3.0, 5.0])
    eps = 1e-6
    lg, r = oracle.logits(x.reshape(T, K), fn, bias, alpha, eps)
    r_exp = 1.0 / math.sqrt(a * a + eps)
    assert np.allclose(r, r_exp, rtol=1e-15, atol=0)
    P = a * v * u.sum()
    g = np.array([0] * 4 + [1] * 4 + [2] * 16)
    l_exp = alpha[g].astype(np.float64) * (r_exp * P) + bias.astype(np.float64)
    assert np.allclose(lg, l_exp[None, :], rtol=1e-13, atol=1e-13)


def test_projection_is_matmul():
    """With alpha = 1 and bias = 0, l / r is the plain product x @ fn (numpy)."""
    rng = np.random.default_rng(1)
    T, C = 5, 384
    x = _bits(rng.standard_normal((T, 4, C)))
    fn = (rng.standard_normal((4 * C, 24)) * 0.02).astype(np.float32)
    lg, r = oracle.logits(x.reshape(T, -1), fn, np.zeros(24, np.float32), np.ones(3, np.float32), 1e-6)
    xf = oracle.bf16_to_f64(x).reshape(T, -1)
    P = np.matmul(xf, fn.astype(np.float64))
    assert np.allclose(lg / r[:, None], P, rtol=1e-11, atol=1e-12)
    ms = np.square(xf).mean(axis=1)
    assert np.allclose(r, 1.0 / np.sqrt(ms + 1e-6), rtol=1e-13)


def test_logits_stream_permutation_and_scale():
    rng = np.random.default_rng(2)
    T, C = 3, 256
    x = _bits(rng.standard_normal((T, 4, C)))
    fn = (rng.standard_normal((4 * C, 24)) * 0.02).astype(np.float32)
    bias = (rng.standard_normal(24) * 0.1).astype(np.float32)
    alpha = np.float32([1.0, 0.5, 2.0])
    lg, _ = oracle.logits(x.reshape(T, -1), fn, bias, alpha, 1e-6)
    perm = [2, 0, 3, 1]
    xp = x[:, perm, :]
    fnp = fn.reshape(4, C, 24)[perm].reshape(4 * C, 24)
    lgp, _ = oracle.logits(xp.reshape(T, -1), fnp, bias, alpha, 1e-6)
    assert np.allclose(lg, lgp, rtol=1e-12, atol=1e-12)
    lgx, _ = oracle.logits(xp.reshape(T, -1), fn, bias, alpha, 1e-6)
    assert not np.allclose(lg, lgx, atol=1e-3)   # stream order matters to the projection
    # x -> 2x (exact in bf16): the logits move only through eps
    x2 = _bits(oracle.bf16_to_f64(x) * 2.0)
    lg2, _ = oracle.logits(x2.reshape(T, -1), fn, bias, alpha, 1e-6)
    ms = np.square(oracle.bf16_to_f64(x)).reshape(T, -1).mean(1)
    bound = np.abs(lg - bias) * (1e-6 / ms)[:, None] + 1e-12
    assert np.all(np.abs(lg2 - lg) <= bound)


def _brute_pre_T1(xf, fn, bias, alpha, eps, iters, p_in=None, w=None):
    """Pure Python, correctly rounded sums (math.fsum); one token."""
    K = len(xf)
    s = math.fsum(v * v for v in xf)
    r = 1.0 / math.sqrt(s / K + eps)
    P = [math.fsum(xf[k] * float(fn[k][j]) for k in range(K)) for j in range(24)]
    grp = lambda j: 0 if j < 4 else (1 if j < 8 else 2)
    l = [float(alpha[grp(j)]) * (r * P[j]) + float(bias[j]) for j in range(24)]
    pre = [1.0 / (1.0 + math.exp(-l[i])) for i in range(4)]
    post = [2.0 / (1.0 + math.exp(-l[4 + i])) for i in range(4)]
    M = [[math.exp(l[8 + 4 * i + j]) for j in range(4)] for i in range(4)]
    for _ in range(iters):
        for i in range(4):
            rs = math.fsum(M[i])
            M[i] = [m / rs for m in M[i]]
        for j in range(4):
            cs = math.fsum(M[i][j] for i in range(4))
            for i in range(4):
                M[i][j] /= cs
    C = K // 4
    p = pre if p_in is None else p_in
    y = [math.fsum(p[i] * xf[i * C + c] for i in range(4)) for c in range(C)]
    if w is not None:
        ry = 1.0 / math.sqrt(math.fsum(v * v for v in y) / C + eps)
        y = [(y[c] * ry) * w[c] for c in range(C)]
    return l, pre, post, M, y


def test_bruteforce_T1_full_size():
    """Whole pre op at T = 1, C = 5120 against a correctly rounded pure-Python evaluation."""
    d = mi.pre_inputs(1, seed=11, delayed=True, norm=True)
    xf = list(oracle.bf16_to_f64(d["x"]).reshape(-1))
    fn = d["fn"].astype(np.float64).tolist()
    w = list(oracle.bf16_to_f64(d["norm_weight"]))
    p_in = [float(v) for v in d["pre_in"][0]]
    l, pre, post, M, li = _brute_pre_T1(xf, fn, d["bias"], d["alpha"], 1e-6, 20, p_in=p_in, w=w)
    o = oracle.mhc_pre_delayed(d["x"], d["pre_in"], d["fn"], d["bias"], d["alpha"], 1e-6, 20,
                               norm_weight=d["norm_weight"])
    assert np.allclose(o["logits"][0], l, rtol=1e-11, atol=1e-12)
    assert np.allclose(o["pre_out"][0], pre, rtol=1e-12)
    assert np.allclose(o["post"][0], post, rtol=1e-12)
    assert np.allclose(o["comb"][0], np.array(M), rtol=1e-11)
    assert np.allclose(o["li_val"][0], li, rtol=1e-12, atol=1e-14)


# ----------------------------------------------------------------------------- gates / Sinkhorn

def test_gates_special_values_and_layout():
    """alpha = 0 makes l = bias: checks sigmoid, 2*sigmoid and the pre|post|comb layout."""
    T, C = 1, 256
    x = _bits(np.random.default_rng(3).standard_normal((T, 4, C)))
    bias = np.float32([0.0, math.log(3.0), -math.log(3.0), 1.0,
                       0.0, math.log(3.0), -2.0, 0.5] + [0.125 * q for q in range(16)])
    fn = np.ones((4 * C, 24), np.float32)
    lg, _ = oracle.logits(x.reshape(T, -1), fn, bias, np.zeros(3, np.float32), 1e-6)
    assert np.array_equal(lg[0], bias.astype(np.float64))
    pre, post, comb0 = oracle.gates(lg, 0)
    b = bias.astype(np.float64)
    assert pre[0, 0] == 0.5 and post[0, 0] == 1.0
    assert abs(pre[0, 1] - 0.75) < 1e-7 and abs(pre[0, 2] - 0.25) < 1e-7   # fp32 log(3)
    assert abs(post[0, 1] - 1.5) < 2e-7
    assert np.allclose(pre[0], 1 / (1 + np.exp(-b[:4])), rtol=1e-15)
    assert np.allclose(post[0], 2 / (1 + np.exp(-b[4:8])), rtol=1e-15)
    # zero iterations exposes the raw comb layout: comb[i][j] = exp(l[8 + 4i + j])
    assert np.allclose(comb0[0], np.exp(b[8:]).reshape(4, 4), rtol=1e-15)
    # post gates lie in (0, 2), pre in (0, 1)
    big = oracle.gates(np.float64([[30, -30, 0, 1, 30, -30, 0, 1] + [0] * 16]), 20)
    assert np.all(big[0] > 0) and np.all(big[0] < 1) and np.all(big[1] > 0) and np.all(big[1] < 2)


def test_sinkhorn_rank_one_is_uniform():
    u = np.array([1.0, 2.0, 0.5, 3.0])
    v = np.array([0.1, 4.0, 1.0, 2.0])
    S = oracle.sinkhorn(np.outer(u, v), 1)
    assert np.allclose(S, 0.25, rtol=1e-15, atol=1e-15)


def test_sinkhorn_column_sums_exact_rows_converge():
    rng = np.random.default_rng(4)
    M = np.exp(rng.standard_normal((4, 4)) * 2.0)
    prev = None
    for it in (1, 2, 5, 10, 20):
        S = oracle.sinkhorn(M, it)
        cs = S.sum(axis=0)
        assert np.all(np.abs(cs - 1.0) <= 4 * 2.0**-52), (it, cs)   # last step is the column step
        rerr = np.abs(S.sum(axis=1) - 1.0).max()
        if prev is not None:
            assert rerr <= prev * (1 + 1e-9)
        prev = rerr
    assert prev < 1e-6


def test_sinkhorn_row_first_order():
    """Row-first: a positive row scaling of the input changes nothing; a column
    scaling does, at a finite iteration count (a column-first variant would
    behave the other way round)."""
    rng = np.random.default_rng(6)
    M = np.exp(rng.standard_normal((4, 4)) * 3.0)
    d = np.array([0.5, 8.0, 3.0, 0.01])
    S = oracle.sinkhorn(M, 3)
    Sr = oracle.sinkhorn(d[:, None] * M, 3)
    Sc = oracle.sinkhorn(M * d[None, :], 3)
    assert np.allclose(S, Sr, rtol=1e-13, atol=1e-15)
    assert not np.allclose(S, Sc, rtol=1e-6)


def test_sinkhorn_permutation_equivariance():
    rng = np.random.default_rng(7)
    M = np.exp(rng.standard_normal((4, 4)))
    P = np.eye(4)[[1, 3, 0, 2]]
    Q = np.eye(4)[[2, 0, 3, 1]]
    S = oracle.sinkhorn(M, 20)
    S2 = oracle.sinkhorn(P @ M @ Q.T, 20)
    assert np.allclose(S2, P @ S @ Q.T, rtol=1e-12, atol=1e-15)


def _sinkhorn2x2_logodds(a11, a12, a21, a22, iters):
    """2x2 Sinkhorn through a different parametrisation, in 60-digit arithmetic.
    After a row step the matrix is [[a, 1-a], [b, 1-b]]; the cross ratio
    kappa = a(1-b)/((1-a)b) is invariant under diagonal scaling, so the state is
    the single number a.  A column step followed by a row step maps
    a -> (a/c1) / (a/c1 + (1-a)/c2) with c1 = a + b, c2 = 2 - a - b."""
    import mpmath as mp
    mp.mp.dps = 60
    a11, a12, a21, a22 = (mp.mpf(v) for v in (a11, a12, a21, a22))
    kappa = (a11 * a22) / (a12 * a21)
    a = a11 / (a11 + a12)                       # first row step

    def b_of(a):                                # second row from the invariant cross ratio
        # a(1-b)/((1-a) b) = kappa  ->  b = a / (a + kappa (1 - a))
        return a / (a + kappa * (1 - a))

    for it in range(iters):
        b = b_of(a)
        c1, c2 = a + b, 2 - a - b
        if it == iters - 1:                     # the last column step ends the iteration
            return [[a / c1, (1 - a) / c2], [b / c1, (1 - b) / c2]]
        a = (a / c1) / (a / c1 + (1 - a) / c2)
    raise AssertionError


def test_sinkhorn_iteration_count_via_kronecker():
    """Sinkhorn commutes with Kronecker products (row and column sums factor),
    so the 4x4 result on A (x) B is the product of two 2x2 results, each from
    the log-odds recurrence above.  The factors converge slowly, so 19, 20 and
    21 iterations differ far above rounding: this pins the count and order."""
    A = np.array([[2.0, 100.0], [1.0, 0.05]])
    B = np.array([[1.0, 30.0], [0.02, 1.0]])
    M = np.kron(A, B)
    SA = np.array(_sinkhorn2x2_logodds(*A.reshape(-1), 20), dtype=float)
    SB = np.array(_sinkhorn2x2_logodds(*B.reshape(-1), 20), dtype=float)
    exp = np.kron(SA, SB)
    got = oracle.sinkhorn(M, 20)
    assert np.allclose(got, exp, rtol=1e-11, atol=1e-14)
    for other in (19, 21):
        assert np.abs(oracle.sinkhorn(M, other) - exp).max() > 1e-6


# ----------------------------------------------------------------------------- collapse / norm

def test_collapse_one_hot_returns_stream():
    rng = np.random.default_rng(8)
    T, C = 4, 256
    x = _bits(rng.standard_normal((T, 4, C)))
    for i in range(4):
        p = np.zeros((T, 4), np.float32)
        p[:, i] = 1.0
        y32 = oracle.collapse32(x, p)
        assert np.array_equal(mi.f32_to_bf16_bits(y32), x[:, i, :])
        y64, _ = oracle.collapse64(x, p.astype(np.float64))
        assert np.array_equal(oracle.bf16_rne(y64), x[:, i, :])


def test_collapse_order_golden():
    with open(os.path.join(GOLDEN, "collapse_order.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    for ln in rows:
        xs, y_hex, li_hex = [s.strip() for s in ln.split("|")]
        xv = np.float32([float(s) for s in xs.split()])
        x = mi.f32_to_bf16_bits(xv).reshape(1, 4, 1).repeat(8, axis=2)
        assert np.array_equal(mi.bf16_bits_to_f32(x[0, :, 0]), xv)     # exact in bf16
        y32 = oracle.collapse32(x, np.ones((1, 4), np.float32))
        assert y32.view(np.uint32)[0, 0] == int(y_hex, 16)
        assert mi.f32_to_bf16_bits(y32)[0, 0] == int(li_hex, 16)
        assert oracle.bf16_rne(y32.astype(np.float64))[0, 0] == int(li_hex, 16)
        y64, _ = oracle.collapse64(x, np.ones((1, 4)))
        assert y64[0, 0] == 1.0 + 2.0**-8 + 2.0**-23


def test_collapse32_close_to_exact_and_broadcast():
    rng = np.random.default_rng(9)
    T, C = 6, 512
    x = _bits(rng.standard_normal((T, 4, C)))
    p = rng.uniform(0, 1, (T, 4)).astype(np.float32)
    y32 = oracle.collapse32(x, p).astype(np.float64)
    y64, mag = oracle.collapse64(x, p.astype(np.float64))
    assert np.all(np.abs(y32 - y64) <= 4 * 2.0**-24 * mag)
    h = x[:, 0, :]
    xb = np.repeat(h[:, None, :], 4, axis=1)
    yb, _ = oracle.collapse64(xb, p.astype(np.float64))
    assert np.allclose(yb, p.astype(np.float64).sum(1)[:, None] * oracle.bf16_to_f64(h), rtol=1e-15)


def test_norm_unit_rms_and_constant_row():
    rng = np.random.default_rng(10)
    T, C = 5, 1024
    y = rng.standard_normal((T, C)) * np.array([1.0, 100.0, 1e-3, 3.0, 0.5])[:, None]
    w1 = np.full(C, 0x3F80, np.uint16)     # weight 1.0
    out, ry = oracle.norm(y, w1, 1e-6)
    ms = np.square(y).mean(1)
    rms = np.sqrt(np.square(out).mean(1))
    assert np.allclose(rms, np.sqrt(ms / (ms + 1e-6)), rtol=1e-13)
    yc = np.full((1, C), 0.75)
    outc, _ = oracle.norm(yc, _bits(np.full(C, 1.5)), 1e-6)
    assert np.allclose(outc, 0.75 / math.sqrt(0.5625 + 1e-6) * 1.5, rtol=1e-15)


def rms_ratio(li_bits, w_bits):
    """RMS of layer_input / weight per row (the unit-RMS check used on the GPU)."""
    li = oracle.bf16_to_f64(li_bits)
    w = oracle.bf16_to_f64(w_bits)
    return np.sqrt(np.square(li / w[None, :]).mean(1))


def test_unit_rms_check_flags_half_sumsq():
    """Plant the half-sum-of-squares mistake in the oracle's norm (on the CPU):
    the unit-RMS check must see the sqrt(2) ratio the page reports."""
    with open(os.path.join(GOLDEN, "sqrt2_symptom.txt")) as f:
        kv = dict(ln.split(None, 1) for ln in f if ln.strip() and not ln.startswith("#"))
    counts = [int(v) for v in kv["token_counts"].split()]
    page_ratio = float(kv["measured_ratio"])
    w = np.full(512, 0x3F80, np.uint16)
    for T in counts[:3]:
        d = mi.pre_inputs(T, seed=T, C=128, delayed=True, norm=True)
        y, _ = oracle.collapse64(d["x"], d["pre_in"].astype(np.float64))
        good, ry = oracle.norm(y, np.full(128, 0x3F80, np.uint16), 1e-6)
        ok = rms_ratio(oracle.bf16_rne(good), np.full(128, 0x3F80, np.uint16))
        assert np.all(np.abs(ok - 1.0) < 2.0**-7)
        # the mistake: only half of the squares reach the sum
        ms_half = 0.5 * np.square(y).mean(1)
        bad = y / np.sqrt(ms_half + 1e-6)[:, None]
        r = rms_ratio(oracle.bf16_rne(bad), np.full(128, 0x3F80, np.uint16))
        assert np.all(np.abs(r - page_ratio) < 5e-3)
    assert abs(float(kv["sqrt2"]) - math.sqrt(2)) < 1e-6


# ----------------------------------------------------------------------------- post / entry / ops

def test_post_identity_zero_and_conservation():
    rng = np.random.default_rng(12)
    T, C = 3, 256
    y = _bits(rng.standard_normal((T, C)))
    x = _bits(rng.standard_normal((T, 4, C)))
    eye = np.tile(np.eye(4, dtype=np.float32), (T, 1, 1))
    o = oracle.mhc_post(y, x, np.zeros((T, 4), np.float32), eye)
    assert np.array_equal(o["out"], x)
    post = rng.uniform(0, 2, (T, 4)).astype(np.float32)
    o0 = oracle.mhc_post(y, x, post, np.zeros((T, 4, 4), np.float32))
    assert np.allclose(o0["out_val"], post[:, :, None] * oracle.bf16_to_f64(y)[:, None, :], rtol=1e-15)
    # column-stochastic comb conserves the stream sum: sum_i out_i = (sum post) y + sum_j x_j
    _, _, comb = oracle.gates(rng.standard_normal((T, 24)), 20)
    comb32 = comb.astype(np.float32)
    o2 = oracle.mhc_post(y, x, post, comb32)
    lhs = o2["out_val"].sum(1)
    colsum = comb32.astype(np.float64).sum(1)      # [T, 4] column sums of the fp32 comb
    rhs = post.astype(np.float64).sum(1)[:, None] * oracle.bf16_to_f64(y) + \
        np.einsum("tj,tjc->tc", colsum, oracle.bf16_to_f64(x))
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


def test_entry_equals_pre_on_broadcast():
    """Model-entry seam = pre op on the broadcast row when fn_e is the block sum
    of fn (the RMS over C of h equals the RMS over 4C of four copies)."""
    d = mi.entry_inputs(3, seed=13, C=256)
    rng = np.random.default_rng(14)
    # multiples of 2^-10 keep fn and its block sums exact in float32
    fn = (np.round(rng.standard_normal((4 * 256, 24)) * 20.0) / 1024.0).astype(np.float32)
    fn_e = fn.reshape(4, 256, 24).sum(0, dtype=np.float64).astype(np.float32)
    assert np.array_equal(fn_e.astype(np.float64), fn.astype(np.float64).reshape(4, 256, 24).sum(0))
    e = oracle.mhc_broadcast_entry(d["h"], fn_e, d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    xb = np.repeat(d["h"][:, None, :], 4, axis=1)
    p = oracle.mhc_pre(xb, fn, d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    assert np.array_equal(e["x_out"], xb)
    assert np.allclose(p["logits"], e["logits"], rtol=1e-12, atol=1e-12)
    assert np.allclose(p["comb"], e["comb"], rtol=1e-11, atol=1e-14)
    assert np.allclose(p["li_val"], e["li_val"], rtol=1e-11, atol=1e-14)


def test_delayed_gates_equal_non_delayed():
    """The carried pre-mix changes only the collapse (p1 Purpose): gates identical."""
    d = mi.pre_inputs(4, seed=15, C=256, delayed=True, norm=True)
    a = oracle.mhc_pre(d["x"], d["fn"], d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    b = oracle.mhc_pre_delayed(d["x"], d["pre_in"], d["fn"], d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    for k_a, k_b in (("pre", "pre_out"), ("post", "post"), ("comb", "comb"), ("logits", "logits")):
        assert np.array_equal(a[k_a], b[k_b])
    # feeding the seam's own pre-mix back in reproduces the non-delayed layer_input
    c = oracle.mhc_pre_delayed(d["x"], a["pre"].astype(np.float32), d["fn"], d["bias"], d["alpha"],
                               norm_weight=d["norm_weight"])
    assert np.allclose(c["li_val"], a["li_val"], rtol=1e-6, atol=1e-6)


def test_standalone_collapse_pins():
    """The standalone collapse (p1 Result) is steps 7-8 alone: one-hot weights give
    the stream back bit for bit; with w = 1 the folded norm has unit RMS; and it
    agrees with the delayed pre's layer_input for pre_in = p."""
    rng = np.random.default_rng(21)
    T, C = 5, 512
    x = _bits(rng.standard_normal((T, 4, C)))
    for i in range(4):
        p = np.zeros((T, 4), np.float32)
        p[:, i] = 1.0
        assert np.array_equal(oracle.mhc_collapse(x, p)["li"], x[:, i, :])
    p = rng.uniform(0, 1, (T, 4)).astype(np.float32)
    w1 = mi.f32_to_bf16_bits(np.ones(C, np.float32))
    r = oracle.mhc_collapse(x, p, norm_weight=w1, eps=0.0)
    rms = np.sqrt(np.mean(r["li_val"] ** 2, axis=1))
    assert np.all(np.abs(rms - 1.0) < 1e-12)
    fn = rng.standard_normal((4 * C, 24)) * 0.02
    d = oracle.mhc_pre_delayed(x, p, fn, np.zeros(24), np.ones(3), 1e-6, 20, norm_weight=w1)
    assert np.array_equal(oracle.mhc_collapse(x, p, norm_weight=w1)["li"], d["li"])


def test_post32_within_bar_identity_and_golden():
    """Single-precision post (the residual the next seam reads): the identity gates
    give x back; random gates stay within the bf16 bar of the exact value; the
    hand-worked order case of tests/golden/post_order.txt."""
    rng = np.random.default_rng(31)
    T, C = 6, 512
    y = _bits(rng.standard_normal((T, C)))
    x = _bits(rng.standard_normal((T, 4, C)))
    eye = np.tile(np.eye(4, dtype=np.float32), (T, 1, 1))
    assert np.array_equal(oracle.post32(y, x, np.zeros((T, 4), np.float32), eye), x)
    post = rng.uniform(0, 2, (T, 4)).astype(np.float32)
    _, _, comb = oracle.gates(rng.standard_normal((T, 24)), 20)
    comb32 = comb.astype(np.float32)
    o32 = oracle.post32(y, x, post, comb32)
    o = oracle.mhc_post(y, x, post, comb32)
    v = o["out_val"]
    a = np.abs(v)
    ulp = np.exp2(np.floor(np.log2(np.where(a > 0, a, 1.0))) - 7)
    err = np.abs(oracle.bf16_to_f64(o32) - v)
    assert np.all(err <= ulp + 6 * 2.0 ** -24 * o["out_mag"])
    # mostly the correctly rounded bits; the rest one bf16 step away
    assert np.mean(o32 == o["out"]) > 0.99
    with open(os.path.join(GOLDEN, "post_order.txt")) as f:
        rows = [ln for ln in f if ln.strip() and not ln.startswith("#")]
    for ln in rows:
        py, cr, xs, a_hex, b_hex, ex_hex = [s.strip() for s in ln.split("|")]
        pv, yv = [float(s) for s in py.split()]
        crow = np.float32([float(s) for s in cr.split()])
        xv = np.float32([float(s) for s in xs.split()])
        yb = mi.f32_to_bf16_bits(np.full((1, 8), yv, np.float32))
        xb = mi.f32_to_bf16_bits(np.broadcast_to(xv[None, :, None], (1, 4, 8)).copy())
        cm = np.zeros((1, 4, 4), np.float32)
        cm[0, 0] = crow
        pp = np.float32([[pv, 0, 0, 0]])
        assert mi.bf16_bits_to_f32(yb)[0, 0] == yv and np.array_equal(mi.bf16_bits_to_f32(xb)[0, :, 0], xv)
        out = oracle.post32(yb, xb, pp, cm)
        assert out[0, 0, 0] == int(b_hex, 16)
        ex = oracle.mhc_post(yb, xb, pp, cm)
        assert ex["out_val"][0, 0, 0] == 1.0 + 2.0 ** -8 + 2.0 ** -23
        assert ex["out"][0, 0, 0] == int(ex_hex, 16)
        assert np.float32(np.float32(pv) * np.float32(yv)).view(np.uint32) == int(a_hex, 16)


def test_post_pre_delayed_composition_pins():
    """Cross-seam composition (post of seam k into the delayed pre of seam k+1):
    with comb = I and post = 0 the residual passes through and everything equals
    mhc_pre_delayed on x; with comb = 0 and post = 1 every stream becomes y, and the
    gates equal the model-entry seam on y with the block-summed weight."""
    T, Cs = 5, 256
    d = mi.pre_inputs(T, seed=32, C=Cs, delayed=True, norm=True)
    rng = np.random.default_rng(33)
    y = _bits(rng.standard_normal((T, Cs)))
    eye = np.tile(np.eye(4, dtype=np.float32), (T, 1, 1))
    f = oracle.mhc_post_pre_delayed(y, d["x"], np.zeros((T, 4), np.float32), eye, d["pre_in"], d["fn"],
                                    d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    g = oracle.mhc_pre_delayed(d["x"], d["pre_in"], d["fn"], d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    assert np.array_equal(f["x_out"], d["x"])
    for k in ("pre_out", "post", "comb", "li"):
        assert np.array_equal(f[k], g[k])
    # multiples of 2^-10 keep fn and its block sums exact in float32
    fn = (np.round(rng.standard_normal((4 * Cs, 24)) * 20.0) / 1024.0).astype(np.float32)
    fn_e = fn.reshape(4, Cs, 24).sum(0, dtype=np.float64).astype(np.float32)
    f = oracle.mhc_post_pre_delayed(y, d["x"], np.ones((T, 4), np.float32), np.zeros((T, 4, 4), np.float32),
                                    d["pre_in"], fn, d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    assert np.array_equal(f["x_out"], np.repeat(y[:, None, :], 4, axis=1))
    e = oracle.mhc_broadcast_entry(y, fn_e, d["bias"], d["alpha"], norm_weight=d["norm_weight"])
    assert np.allclose(f["logits"], e["logits"], rtol=1e-12, atol=1e-12)
    assert np.allclose(f["pre_out"], e["pre"], rtol=1e-11, atol=1e-14)
    assert np.allclose(f["comb"], e["comb"], rtol=1e-11, atol=1e-14)
    # layer_input: the collapse of four copies of y with pre_in is (sum pre_in) * y
    s = d["pre_in"].astype(np.float64).sum(1)
    ybar = oracle.bf16_to_f64(y) * s[:, None]
    assert np.allclose(f["y"], ybar, rtol=1e-12, atol=1e-12)
