"""Pins of the CPU oracle against facts it does not compute itself.

Each test fixes the oracle to something independent of its own loops: values
worked by hand from the pages' update equations (tests/golden/), closed forms
(cumulative products and sums, geometric series, quadratic "attention" forms),
exact rational arithmetic on a different formula, special cases that reduce to
a textbook routine (a causal masked matmul), invariants, a second algorithm
(the chunked UT form of the delta rule, solved with numpy.linalg), and the
structural facts the pages assert (decay decomposability, segment
continuation).  Citations use the page titles:
  SunnyNet log  = "SunnyNet 工程化实录：一个 O(N) 架构如何长出自己的 C 推理运行时"
  vs llama.cpp  = "我拿同一份权重和 llama.cpp 正面比了一场：我手写的 C 内核，慢了 1.1–1.7 倍"
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel(x, y):
    """Normwise relative difference max|x-y| / max|y|."""
    x = np.asarray(x, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    d = np.max(np.abs(x - y)) if x.size else 0.0
    m = np.max(np.abs(y)) if y.size else 0.0
    return d / m if m > 0 else d


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# Hand-worked examples (tests/golden/*.json, each citing its equation)
# ----------------------------------------------------------------------------

def test_golden_fma_hand():
    d = _load("fma_hand.json")
    s, fin = oracle.scan_fma(np.array(d["a"]), np.array(d["b"]), np.array(d["s0"]))
    assert np.array_equal(s, np.array(d["s"]))
    assert np.array_equal(fin, np.array(d["s_final"]))


def test_golden_gated_hand():
    d = _load("gated_hand.json")
    s, fin = oracle.scan_gated(np.array(d["a"]), np.array(d["u"]), np.array(d["s0"]))
    assert np.array_equal(s, np.array(d["s"]))
    assert np.array_equal(fin, np.array(d["s_final"]))


@pytest.mark.parametrize("case", [0, 1])
def test_golden_diag_outer_hand(case):
    d = _load("diag_outer_hand.json")["cases"][case]
    g = np.log(np.array(d["alpha"]))
    ks = None if d["k_scale"] is None else np.array(d["k_scale"])
    s0 = None if d["s0"] is None else np.array(d["s0"])
    o, fin = oracle.scan_diag_outer(np.array(d["q"]), np.array(d["k"]), np.array(d["v"]), g,
                                    d["decay_mode"], ks, d["scale"], s0)
    assert rel(o, d["o"]) < 1e-15
    assert rel(fin, d["s_final"]) < 1e-15


@pytest.mark.parametrize("case", [0, 1])
@pytest.mark.parametrize("form", ["rank1", "explicit"])
def test_golden_delta_hand(case, form):
    d = _load("delta_hand.json")["cases"][case]
    fn = oracle.scan_delta if form == "rank1" else oracle.scan_delta_explicit
    s0 = None if d["s0"] is None else np.array(d["s0"])
    o, fin = fn(np.array(d["q"]), np.array(d["k"]), np.array(d["v"]), np.array(d["beta"]),
                d["scale"], s0)
    assert np.array_equal(o, np.array(d["o"]))
    assert np.array_equal(fin, np.array(d["s_final"]))


# ----------------------------------------------------------------------------
# Elementwise scans: closed forms [SunnyNet log §2.1; the pages' torch baseline
# is the cumsum closed form, §2.3]
# ----------------------------------------------------------------------------

def _rng(seed):
    return np.random.default_rng(seed)


def test_fma_cumprod_cumsum_closed_form():
    # s_t = P_t * (s0 + sum_{i<=t} b_i / P_i),  P_t = prod_{j<=t} a_j
    r = _rng(1)
    B, T, N = 3, 16, 5
    a = r.uniform(0.5, 1.0, (B, T, N))
    b = r.standard_normal((B, T, N))
    s0 = r.standard_normal((B, N))
    P = np.cumprod(a, axis=1)
    ref = P * (s0[:, None, :] + np.cumsum(b / P, axis=1))
    s, fin = oracle.scan_fma(a, b, s0)
    assert rel(s, ref) < 1e-12
    assert np.array_equal(fin, s[:, -1])


def test_fma_double_sum_exact_rational():
    # s_t = (prod_{j<=t} a_j) s0 + sum_{i<=t} (prod_{i<j<=t} a_j) b_i, in exact
    # rationals, with signed a (where the cumprod form would divide by ~0).
    r = _rng(2)
    B, T, N = 2, 9, 3
    a = r.integers(-6, 7, (B, T, N)) / 4.0
    b = r.integers(-8, 9, (B, T, N)) / 8.0
    s0 = r.integers(-4, 5, (B, N)) / 2.0
    s, fin = oracle.scan_fma(a, b, s0)
    for bi in range(B):
        for n in range(N):
            A = [Fraction(x) for x in a[bi, :, n]]
            Bv = [Fraction(x) for x in b[bi, :, n]]
            for t in range(T):
                val = Fraction(s0[bi, n])
                for j in range(t + 1):
                    val *= A[j]
                for i in range(t + 1):
                    term = Bv[i]
                    for j in range(i + 1, t + 1):
                        term *= A[j]
                    val += term
                # dyadic inputs with few bits: fp64 holds every partial result exactly
                assert s[bi, t, n] == float(val)
    assert np.array_equal(fin, s[:, -1])


def test_fma_special_cases():
    r = _rng(3)
    B, T, N = 2, 20, 4
    b = r.standard_normal((B, T, N))
    s0 = r.standard_normal((B, N))
    s, _ = oracle.scan_fma(np.ones((B, T, N)), b, s0)          # a = 1: running sum
    assert rel(s, s0[:, None, :] + np.cumsum(b, axis=1)) < 1e-14
    a = r.uniform(0.5, 1.0, (B, T, N))
    s, _ = oracle.scan_fma(a, np.zeros((B, T, N)), s0)         # b = 0: running product
    assert rel(s, s0[:, None, :] * np.cumprod(a, axis=1)) < 1e-14
    alpha, beta = 0.9, 0.3                                     # constants: geometric series
    s, _ = oracle.scan_fma(np.full((B, T, N), alpha), np.full((B, T, N), beta), s0)
    t = np.arange(1, T + 1)[None, :, None]
    ref = alpha ** t * s0[:, None, :] + beta * (1 - alpha ** t) / (1 - alpha)
    assert rel(s, ref) < 1e-13
    s, fin = oracle.scan_fma(np.ones((B, T, N)), b, None)      # NULL s0 means zeros
    assert rel(s, np.cumsum(b, axis=1)) < 1e-14


def test_gated_closed_forms():
    r = _rng(4)
    B, T, N = 2, 24, 3
    s0 = r.standard_normal((B, N))
    u = r.standard_normal((B, T, N))
    # a = 0 copies the input, a = 1 holds the state
    s, _ = oracle.scan_gated(np.zeros((B, T, N)), u, s0)
    assert np.array_equal(s, u)
    s, _ = oracle.scan_gated(np.ones((B, T, N)), u, s0)
    assert np.array_equal(s, np.broadcast_to(s0[:, None, :], (B, T, N)))
    # constant a = alpha, u = c: s_t = c + alpha^t (s0 - c)
    alpha, c = 0.75, 2.5
    s, _ = oracle.scan_gated(np.full((B, T, N), alpha), np.full((B, T, N), c), s0)
    t = np.arange(1, T + 1)[None, :, None]
    assert rel(s, c + alpha ** t * (s0[:, None, :] - c)) < 1e-13
    # fixed point: u = s0 = c everywhere stays c for any a in [0, 1]
    a = r.uniform(0.0, 1.0, (B, T, N))
    s, _ = oracle.scan_gated(a, np.full((B, T, N), 0.5), np.full((B, N), 0.5))
    assert np.all(np.abs(s - 0.5) <= 1e-15)


def test_gated_double_sum_exact_rational_and_convexity():
    # s_t = (prod_{j<=t} a_j) s0 + sum_{i<=t} (prod_{i<j<=t} a_j) (1 - a_i) u_i
    r = _rng(5)
    B, T, N = 2, 8, 2
    a = r.integers(0, 9, (B, T, N)) / 8.0
    u = r.integers(-8, 9, (B, T, N)) / 4.0
    s0 = r.integers(-4, 5, (B, N)) / 2.0
    s, _ = oracle.scan_gated(a, u, s0)
    for bi in range(B):
        for n in range(N):
            for t in range(T):
                val = Fraction(s0[bi, n])
                for j in range(t + 1):
                    val *= Fraction(a[bi, j, n])
                for i in range(t + 1):
                    term = (1 - Fraction(a[bi, i, n])) * Fraction(u[bi, i, n])
                    for j in range(i + 1, t + 1):
                        term *= Fraction(a[bi, j, n])
                    val += term
                assert s[bi, t, n] == float(val)
    # convex combination: the state stays inside [min, max] of s0 and the inputs so far
    a = r.uniform(0.0, 1.0, (3, 50, 4))
    u = r.standard_normal((3, 50, 4))
    s0 = r.standard_normal((3, 4))
    s, _ = oracle.scan_gated(a, u, s0)
    lo = np.minimum(s0[:, None, :], np.minimum.accumulate(u, axis=1))
    hi = np.maximum(s0[:, None, :], np.maximum.accumulate(u, axis=1))
    assert np.all(s >= lo - 1e-12) and np.all(s <= hi + 1e-12)


# ----------------------------------------------------------------------------
# Reverse (gradient) pass of the elementwise scans [SunnyNet log §8: the
# back-ends' reverse-scan entry].  The loss is L = sum_t <W_t, s_t> + <w_f, s_T>,
# so (W, w_f) are the incoming gradients (ds, ds_final).  Each pin derives the
# gradient without the backward recursion: every forward state is affine in
# any single input, so a unit difference of L is that input's exact partial
# derivative, and L is jointly linear in (b or u, s0).
# ----------------------------------------------------------------------------

def _states_exact(a, x, s0, gated):
    """All states of one channel in exact rationals, from the double-sum closed
    form (not the step-by-step recursion)."""
    T = len(a)
    out = []
    for t in range(T):
        val = s0
        for j in range(t + 1):
            val *= a[j]
        for i in range(t + 1):
            term = (1 - a[i]) * x[i] if gated else x[i]
            for j in range(i + 1, t + 1):
                term *= a[j]
            val += term
        out.append(val)
    return out


def _loss_exact(a, x, s0, W, wf, gated):
    st = _states_exact(a, x, s0, gated)
    return sum(w * v for w, v in zip(W, st)) + wf * st[-1]


@pytest.mark.parametrize("gated", [False, True])
def test_elem_backward_exact_unit_differences(gated):
    r = _rng(8 + gated)
    B, T, N = 2, 6, 2
    a = r.integers(-6, 7, (B, T, N)) / 4.0
    x = r.integers(-8, 9, (B, T, N)) / 8.0
    s0 = r.integers(-4, 5, (B, N)) / 2.0
    ds = r.integers(-4, 5, (B, T, N)) / 4.0
    dsf = r.integers(-4, 5, (B, N)) / 2.0
    fwd = oracle.scan_gated if gated else oracle.scan_fma
    s, _ = fwd(a, x, s0)
    if gated:
        da, dx, ds0 = oracle.scan_gated_backward(a, x, s, ds, s0, dsf)
    else:
        da, dx, ds0 = oracle.scan_fma_backward(a, s, ds, s0, dsf)
    for bi in range(B):
        for n in range(N):
            A = [Fraction(v) for v in a[bi, :, n]]
            X = [Fraction(v) for v in x[bi, :, n]]
            W = [Fraction(v) for v in ds[bi, :, n]]
            S0, WF = Fraction(s0[bi, n]), Fraction(dsf[bi, n])
            L0 = _loss_exact(A, X, S0, W, WF, gated)
            for t in range(T):
                Ap = list(A); Ap[t] += 1
                Xp = list(X); Xp[t] += 1
                assert da[bi, t, n] == pytest.approx(float(_loss_exact(Ap, X, S0, W, WF, gated) - L0),
                                                     rel=1e-14, abs=1e-14)
                assert dx[bi, t, n] == pytest.approx(float(_loss_exact(A, Xp, S0, W, WF, gated) - L0),
                                                     rel=1e-14, abs=1e-14)
            assert ds0[bi, n] == pytest.approx(float(_loss_exact(A, X, S0 + 1, W, WF, gated) - L0),
                                               rel=1e-14, abs=1e-14)


@pytest.mark.parametrize("gated", [False, True])
def test_elem_backward_central_differences(gated):
    # longer sequences in float64: L is affine in each single input, so the
    # central difference is exact up to the rounding of L itself
    r = _rng(10 + gated)
    B, T, N = 2, 64, 3
    a = r.uniform(0.5, 1.0, (B, T, N)) if gated else r.uniform(-1.1, 1.1, (B, T, N))
    x = r.standard_normal((B, T, N))
    s0 = r.standard_normal((B, N))
    ds = r.standard_normal((B, T, N))
    dsf = r.standard_normal((B, N))
    fwd = oracle.scan_gated if gated else oracle.scan_fma

    def loss(a_, x_, s0_):
        s_, fin_ = fwd(a_, x_, s0_)
        return np.sum(ds * s_, axis=(1, 2)) + np.sum(dsf * fin_, axis=1)   # one loss per batch row

    s, _ = fwd(a, x, s0)
    bwd = (lambda: oracle.scan_gated_backward(a, x, s, ds, s0, dsf)) if gated else \
          (lambda: oracle.scan_fma_backward(a, s, ds, s0, dsf))
    da, dx, ds0 = bwd()
    h = 0.25
    scale = np.max(np.abs(ds)) * T
    for t in (0, 1, T // 2, T - 2, T - 1):
        for n in range(N):
            e = np.zeros((B, T, N)); e[:, t, n] = h
            fd_a = (loss(a + e, x, s0) - loss(a - e, x, s0)) / (2 * h)
            fd_x = (loss(a, x + e, s0) - loss(a, x - e, s0)) / (2 * h)
            assert np.max(np.abs(fd_a - da[:, t, n])) < 1e-11 * scale
            assert np.max(np.abs(fd_x - dx[:, t, n])) < 1e-11 * scale
    for n in range(N):
        e = np.zeros((B, N)); e[:, n] = h
        fd = (loss(a, x, s0 + e) - loss(a, x, s0 - e)) / (2 * h)
        assert np.max(np.abs(fd - ds0[:, n])) < 1e-11 * scale


@pytest.mark.parametrize("gated", [False, True])
def test_elem_backward_linearity_identity(gated):
    # For fixed a the states are linear in (b or u, s0) jointly, so the loss
    # equals <dx, x> + <ds0, s0> exactly (Euler's identity for a linear map).
    r = _rng(12 + gated)
    B, T, N = 3, 200, 4
    a = r.uniform(0.5, 1.0, (B, T, N))
    x = r.standard_normal((B, T, N))
    s0 = r.standard_normal((B, N))
    ds = r.standard_normal((B, T, N))
    dsf = r.standard_normal((B, N))
    if gated:
        s, fin = oracle.scan_gated(a, x, s0)
        _, dx, ds0 = oracle.scan_gated_backward(a, x, s, ds, s0, dsf)
    else:
        s, fin = oracle.scan_fma(a, x, s0)
        _, dx, ds0 = oracle.scan_fma_backward(a, s, ds, s0, dsf)
    lhs = np.sum(ds * s, axis=(1, 2)) + np.sum(dsf * fin, axis=1)
    rhs = np.sum(dx * x, axis=(1, 2)) + np.sum(ds0 * s0, axis=1)
    assert np.max(np.abs(lhs - rhs)) < 1e-11 * np.max(np.abs(lhs))


def test_elem_backward_closed_forms():
    r = _rng(14)
    B, T, N = 2, 30, 3
    x = r.standard_normal((B, T, N))
    s0 = r.standard_normal((B, N))
    ds = r.standard_normal((B, T, N))
    dsf = r.standard_normal((B, N))
    # a = 1: the gradient of every state is the suffix sum of the incoming ones
    ones = np.ones((B, T, N))
    s, _ = oracle.scan_fma(ones, x, s0)
    _, db, ds0 = oracle.scan_fma_backward(ones, s, ds, s0, dsf)
    suffix = np.flip(np.cumsum(np.flip(ds, axis=1), axis=1), axis=1) + dsf[:, None, :]
    assert rel(db, suffix) < 1e-14
    assert rel(ds0, suffix[:, 0]) < 1e-14
    # a = 0: each state forgets the past, so only its own gradient reaches it
    zeros = np.zeros((B, T, N))
    s, _ = oracle.scan_fma(zeros, x, s0)
    da, db, ds0 = oracle.scan_fma_backward(zeros, s, ds, s0, dsf)
    own = ds.copy()
    own[:, -1] += dsf
    assert np.array_equal(db, own)
    assert np.array_equal(ds0, np.zeros((B, N)))
    # constant a = c with a single unit gradient at step k: gs_t = c^(k-t) for t <= k
    c, k = 0.8, 17
    ds1 = np.zeros((B, T, N)); ds1[:, k, :] = 1.0
    s, _ = oracle.scan_fma(np.full((B, T, N), c), x, s0)
    da, db, ds0 = oracle.scan_fma_backward(np.full((B, T, N), c), s, ds1, s0, None)
    t = np.arange(T)[None, :, None]
    ref = np.where(t <= k, c ** np.maximum(k - t, 0), 0.0) * np.ones((B, T, N))
    assert rel(db, ref) < 1e-14
    assert rel(ds0, np.full((B, N), c ** (k + 1))) < 1e-14
    # gated with a = 0: s_t = u_t, so du = ds (plus ds_final at the end) and da = ds (s_{t-1} - u_t)
    s, _ = oracle.scan_gated(zeros, x, s0)
    da, du, ds0 = oracle.scan_gated_backward(zeros, x, s, ds, s0, dsf)
    assert np.array_equal(du, own)
    prev = np.concatenate([s0[:, None, :], x[:, :-1]], axis=1)
    assert rel(da, own * (prev - x)) < 1e-15
    # gated with a = 1: the state never moves, so du = 0 and ds0 collects every gradient
    s, _ = oracle.scan_gated(ones, x, s0)
    da, du, ds0 = oracle.scan_gated_backward(ones, x, s, ds, s0, dsf)
    assert np.array_equal(du, np.zeros((B, T, N)))
    assert rel(ds0, ds.sum(axis=1) + dsf) < 1e-14


def test_elem_backward_float32_mode_and_nulls():
    r = _rng(15)
    a = r.uniform(0.5, 1.0, (2, 512, 8))
    x = r.standard_normal((2, 512, 8))
    ds = r.standard_normal((2, 512, 8))
    s, _ = oracle.scan_gated(a, x)
    g64 = oracle.scan_gated_backward(a, x, s, ds)
    g32 = oracle.scan_gated_backward(a, x, s, ds, dtype=np.float32)
    for u, v in zip(g32, g64):
        assert u.dtype == np.float32 and rel(u, v) < 5e-6
    # NULL s0 and ds_final mean zeros
    z = oracle.scan_gated_backward(a, x, s, ds, np.zeros((2, 8)), np.zeros((2, 8)))
    for u, v in zip(z, g64):
        assert np.array_equal(u, v)


# ----------------------------------------------------------------------------
# Decay-separable state scan [SunnyNet log §4.1, §4.3]
# ----------------------------------------------------------------------------

def _diag_inputs(r, B, T, H, Hg, K, V, mode, with_kscale, with_s0, gscale=0.3):
    q = r.standard_normal((B, T, Hg, K))
    k = r.standard_normal((B, T, Hg, K))
    v = r.standard_normal((B, T, H, V))
    gshape = (B, T, H) if mode == 0 else (B, T, H, K)
    g = -gscale * r.uniform(0.0, 1.0, gshape)
    ks = r.uniform(0.2, 2.0, (B, T, H)) if with_kscale else None
    s0 = r.standard_normal((B, H, K, V)) if with_s0 else None
    return q, k, v, g, ks, s0


def _diag_quadratic(q, k, v, g, mode, ks, scale, s0, H, ksk=None):
    """O(T^2) closed form: o_t = scale sum_{i<=t} sum_d q_td k_id kappa_i e^{G_td - G_id} v_i
    + scale sum_d q_td e^{G_td} S0_d,  S_T = e^{G_T} S0 + sum_i e^{G_T - G_i} kappa_i k_i v_i^T,
    with G_t = sum_{j<=t} g_j (kappa_i per key, kappa_id, when ksk is given)."""
    B, T, Hg, K = q.shape
    V = v.shape[-1]
    hpg = H // Hg
    o = np.zeros((B, T, H, V))
    fin = np.zeros((B, H, K, V))
    for b in range(B):
        for h in range(H):
            grp = h // hpg
            gg = g[b, :, h] if mode == 1 else np.repeat(g[b, :, h][:, None], K, axis=1)
            G = np.cumsum(gg, axis=0)                                   # [T, K]
            kap = ks[b, :, h] if ks is not None else np.ones(T)
            Q = q[b, :, grp]                                            # [T, K]
            Km = k[b, :, grp] * kap[:, None]
            if ksk is not None:
                Km = Km * ksk[b, :, h]                                  # per-key scale
            W = np.exp(G[:, None, :] - G[None, :, :])                   # [t, i, d]
            Pm = np.einsum("td,id,tid->ti", Q, Km, W)
            Pm = np.tril(Pm)
            o[b, :, h] = Pm @ v[b, :, h]
            S0 = s0[b, h] if s0 is not None else np.zeros((K, V))
            o[b, :, h] += (Q * np.exp(G)) @ S0
            o[b, :, h] *= scale
            fin[b, h] = np.exp(G[-1])[:, None] * S0 + (
                (Km * np.exp(G[-1][None, :] - G)).T @ v[b, :, h])
    return o, fin


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("with_s0", [False, True])
def test_diag_outer_quadratic_form(mode, with_s0):
    r = _rng(10 + mode + 2 * with_s0)
    B, T, H, Hg, K, V = 2, 23, 4, 2, 5, 7   # K != V and Hg < H: a wrong offset cannot hide
    q, k, v, g, ks, s0 = _diag_inputs(r, B, T, H, Hg, K, V, mode, True, with_s0)
    scale = 0.37
    o, fin = oracle.scan_diag_outer(q, k, v, g, mode, ks, scale, s0)
    ro, rf = _diag_quadratic(q, k, v, g, mode, ks, scale, s0, H)
    assert rel(o, ro) < 1e-12
    assert rel(fin, rf) < 1e-12


@pytest.mark.parametrize("with_s0", [False, True])
def test_diag_outer_per_key_scale_quadratic_form(with_s0):
    r = _rng(16 + with_s0)
    B, T, H, Hg, K, V = 2, 21, 4, 2, 6, 5
    q, k, v, g, _, s0 = _diag_inputs(r, B, T, H, Hg, K, V, 1, False, with_s0)
    ksk = r.uniform(-0.5, 1.5, (B, T, H, K))
    o, fin = oracle.scan_diag_outer(q, k, v, g, 1, None, 0.6, s0, k_scale_key=ksk)
    ro, rf = _diag_quadratic(q, k, v, g, 1, None, 0.6, s0, H, ksk=ksk)
    assert rel(o, ro) < 1e-12
    assert rel(fin, rf) < 1e-12


def test_diag_outer_per_key_scale_special_cases():
    r = _rng(18)
    B, T, H, Hg, K, V = 2, 30, 3, 3, 4, 6
    q, k, v, g, ks, s0 = _diag_inputs(r, B, T, H, Hg, K, V, 1, True, True)
    # a per-key scale equal on every key is the per-head scale, bit for bit
    o1, f1 = oracle.scan_diag_outer(q, k, v, g, 1, ks, 0.8, s0)
    o2, f2 = oracle.scan_diag_outer(q, k, v, g, 1, None, 0.8, s0,
                                    k_scale_key=np.repeat(ks[..., None], K, axis=-1))
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    # the associative memory with one key: S_t = p S_{t-1} + (1 - p) k v_t, the
    # gated elementwise scan with a = p and u = k v
    p = r.uniform(0.3, 0.99, (B, T, H, 1))
    k1 = r.uniform(-1.0, 1.0, (B, T, H, 1))
    q1 = r.standard_normal((B, T, H, 1))
    o, fin = oracle.scan_diag_outer(q1, k1, v, np.log(p), 1, None, 1.0, s0[:, :, :1],
                                    k_scale_key=1.0 - p)
    a = np.repeat(p, V, axis=-1).reshape(B, T, H * V)
    u = (k1 * v).reshape(B, T, H * V)
    s, sf = oracle.scan_gated(a, u, s0[:, :, 0, :].reshape(B, H * V))
    assert rel(fin[:, :, 0, :], sf.reshape(B, H, V)) < 1e-13
    assert rel(o, q1 * s.reshape(B, T, H, V)) < 1e-13
    # the memory is a convex combination: it stays within the range of S0 and of every k v^T
    K2 = 5
    p = r.uniform(0.0, 1.0, (B, T, H, K2))
    k2 = r.uniform(-1.0, 1.0, (B, T, H, K2))
    _, fin = oracle.scan_diag_outer(r.standard_normal((B, T, H, K2)), k2, v, np.log(p), 1, None, 1.0,
                                    np.zeros((B, H, K2, V)), k_scale_key=1.0 - p)
    bound = np.max(np.abs(k2)) * np.max(np.abs(v))
    assert np.all(np.abs(fin) <= bound * (1 + 1e-12))


def test_diag_outer_zero_decay_is_causal_linear_attention():
    # g = 0, kappa = 1: O = scale (tril(Q K^T) V + Q S0) per head (a masked matmul)
    r = _rng(20)
    B, T, H, Hg, K, V = 2, 17, 3, 3, 6, 4
    q, k, v, _, _, s0 = _diag_inputs(r, B, T, H, Hg, K, V, 1, False, True)
    g = np.zeros((B, T, H, K))
    o, fin = oracle.scan_diag_outer(q, k, v, g, 1, None, 0.5, s0)
    for b in range(B):
        for h in range(H):
            Q, Km, Vm = q[b, :, h], k[b, :, h], v[b, :, h]
            ref = 0.5 * (np.tril(Q @ Km.T) @ Vm + Q @ s0[b, h])
            assert rel(o[b, :, h], ref) < 1e-13
            assert rel(fin[b, h], s0[b, h] + Km.T @ Vm) < 1e-13


def test_diag_outer_k1_reduces_to_fma_scan():
    # K = V = 1: S_t = e^{g_t} S_{t-1} + kappa k v, o = scale S q, i.e. an FMA scan
    r = _rng(21)
    B, T, H = 2, 30, 3
    q, k, v, g, ks, s0 = _diag_inputs(r, B, T, H, H, 1, 1, 0, True, True)
    o, fin = oracle.scan_diag_outer(q, k, v, g, 0, ks, 1.0, s0)
    a = np.exp(g)                                           # [B,T,H]
    bb = ks * k[..., 0] * v[..., 0]
    s, sf = oracle.scan_fma(a, bb, s0[..., 0, 0])
    assert rel(o[..., 0], s * q[..., 0]) < 1e-14
    assert rel(fin[..., 0, 0], sf) < 1e-14


@pytest.mark.parametrize("mode", [0, 1])
def test_diag_outer_is_elementwise_decomposable(mode):
    # [SunnyNet log §4.3] asserts GLA decay is elementwise decomposable (and §4.1
    # says the same of Mamba-2).  Run the elementwise FMA scan on K*V channels with
    # a = exp(g_i) and b = (kappa k_i) v_j: its states equal S bit for bit.
    r = _rng(30 + mode)
    B, T, H, K, V = 2, 19, 2, 4, 3
    q, k, v, g, ks, s0 = _diag_inputs(r, B, T, H, H, K, V, mode, True, True)
    for t_end in (1, 7, T):
        _, fin = oracle.scan_diag_outer(q[:, :t_end], k[:, :t_end], v[:, :t_end],
                                        g[:, :t_end], mode, ks[:, :t_end], 1.0, s0)
        gi = g[:, :t_end] if mode == 1 else np.repeat(g[:, :t_end, :, None], K, axis=3)
        alpha = np.vectorize(math.exp)(gi)                   # libm exp, as the C oracle
        a = np.repeat(alpha[..., :, None], V, axis=4)        # [B,t,H,K,V]
        kk = ks[:, :t_end, :, None] * k[:, :t_end]           # [B,t,H,K]
        bb = kk[..., :, None] * v[:, :t_end, :, None, :]
        s, sf = oracle.scan_fma(a.reshape(B, t_end, -1), bb.reshape(B, t_end, -1),
                                s0.reshape(B, -1))
        assert np.array_equal(sf.reshape(B, H, K, V), fin)


def test_delta_rule_is_not_elementwise():
    # The converse [SunnyNet log §4.4]: the rank-1 term cannot be written as a
    # per-channel a*s + b, so the same mapping does not reproduce the delta rule.
    r = _rng(33)
    B, T, H, K, V = 1, 6, 1, 4, 3
    q = r.standard_normal((B, T, H, K))
    k = r.standard_normal((B, T, H, K))
    v = r.standard_normal((B, T, H, V))
    beta = np.full((B, T, H), 0.5)
    _, fin = oracle.scan_delta(q, k, v, beta)
    bb = (beta[..., None] * k)[..., :, None] * v[..., None, :]
    _, sf = oracle.scan_fma(np.ones((B, T, H * K * V)), bb.reshape(B, T, -1))
    assert rel(sf.reshape(B, H, K, V), fin) > 1e-3


# ----------------------------------------------------------------------------
# Delta rule [SunnyNet log §4.2; vs llama.cpp §3]
# ----------------------------------------------------------------------------

def _delta_inputs(r, B, T, H, K, V, with_s0=True, normalise=True):
    q = r.standard_normal((B, T, H, K))
    k = r.standard_normal((B, T, H, K))
    if normalise:
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = r.standard_normal((B, T, H, V))
    beta = r.uniform(0.0, 1.0, (B, T, H))
    s0 = r.standard_normal((B, H, K, V)) if with_s0 else None
    return q, k, v, beta, s0


@pytest.mark.parametrize("K,V", [(6, 10), (10, 6), (8, 8)])
def test_delta_rank1_matches_explicit(K, V):
    # The page requires the two forms to be built and checked separately, with
    # K != V so that a wrong-side product cannot pass silently.
    r = _rng(40 + K)
    q, k, v, beta, s0 = _delta_inputs(r, 2, 40, 3, K, V)
    o1, f1 = oracle.scan_delta(q, k, v, beta, 0.7, s0)
    o2, f2 = oracle.scan_delta_explicit(q, k, v, beta, 0.7, s0)
    assert rel(o1, o2) < 1e-12
    assert rel(f1, f2) < 1e-12


def test_delta_key_readback_invariant():
    # S_t^T k_t = (1 - beta ||k||^2) S_{t-1}^T k_t + beta ||k||^2 v_t, for any K, V;
    # a product taken on the wrong side of S breaks it.
    r = _rng(50)
    B, T, H, K, V = 1, 12, 2, 5, 9
    q, k, v, beta, s0 = _delta_inputs(r, B, T, H, K, V, normalise=False)
    prev = s0
    for t in range(T):
        _, cur = oracle.scan_delta(q[:, :t + 1], k[:, :t + 1], v[:, :t + 1], beta[:, :t + 1],
                                   1.0, s0)
        for h in range(H):
            kt, vt, bt = k[0, t, h], v[0, t, h], beta[0, t, h]
            nk = kt @ kt
            lhs = cur[0, h].T @ kt
            rhs = (1 - bt * nk) * (prev[0, h].T @ kt) + bt * nk * vt
            assert rel(lhs, rhs) < 1e-12
        prev = cur


def test_delta_beta_zero_and_one_hot_overwrite():
    r = _rng(51)
    B, T, H, K, V = 2, 9, 2, 4, 6
    q, k, v, _, s0 = _delta_inputs(r, B, T, H, K, V)
    o, fin = oracle.scan_delta(q, k, v, np.zeros((B, T, H)), 1.5, s0)
    assert np.array_equal(fin, s0)                     # beta = 0 leaves S unchanged
    assert rel(o, 1.5 * np.einsum("bhkv,bthk->bthv", s0, q)) < 1e-14
    # one-hot keys with beta = 1 overwrite row i_t of S with v_t
    idx = r.integers(0, K, (B, T, H))
    k1 = np.zeros((B, T, H, K))
    np.put_along_axis(k1, idx[..., None], 1.0, axis=-1)
    o, fin = oracle.scan_delta(q, k1, v, np.ones((B, T, H)), 1.0, s0)
    S = s0.copy()
    for t in range(T):
        for b in range(B):
            for h in range(H):
                S[b, h, idx[b, t, h]] = v[b, t, h]
        assert rel(o[:, t], np.einsum("bhkv,bhk->bhv", S, q[:, t])) < 1e-14
    # S + (v - S) equals v up to one rounding of the subtraction and the add
    assert rel(fin, S) < 1e-15


def test_delta_chunked_ut_form():
    # A second algorithm for the same map over one chunk (WY/UT form):
    #   A = strict_lower(diag(beta) K K^T),  Delta = (I + A)^{-1} diag(beta) (V - K S0),
    #   O = scale (Q S0 + tril(Q K^T) Delta),  S_L = S0 + K^T Delta.
    r = _rng(52)
    B, T, H, K, V = 1, 32, 2, 7, 5
    q, k, v, beta, s0 = _delta_inputs(r, B, T, H, K, V)
    o, fin = oracle.scan_delta(q, k, v, beta, 0.9, s0)
    for h in range(H):
        Q, Km, Vm, bt, S0 = q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], s0[0, h]
        A = np.tril(bt[:, None] * (Km @ Km.T), -1)
        Dl = np.linalg.solve(np.eye(T) + A, bt[:, None] * (Vm - Km @ S0))
        assert rel(o[0, :, h], 0.9 * (Q @ S0 + np.tril(Q @ Km.T) @ Dl)) < 1e-11
        assert rel(fin[0, h], S0 + Km.T @ Dl) < 1e-11


# ----------------------------------------------------------------------------
# Output epilogues: GLA's RMSNorm(o) * silu(g) [SunnyNet log §4.3] and
# Mamba-2's D x skip
# ----------------------------------------------------------------------------

def test_epilogue_norm_gate_hand_worked():
    # o = [3, 4]: mean square 12.5, so o / rms = [3, 4] / sqrt(12.5) = [0.6 sqrt2, 0.8 sqrt2];
    # weight [1, 2]; z = [0, ln 3]: silu(0) = 0, silu(ln 3) = (3/4) ln 3
    o = np.array([3.0, 4.0]).reshape(1, 1, 1, 2)
    z = np.array([0.0, math.log(3.0)]).reshape(1, 1, 1, 2)
    out = oracle.epilogue_norm_gate(o, z, np.array([1.0, 2.0]), eps=0.0)
    ref = np.array([0.0, 0.8 * math.sqrt(2.0) * 2.0 * 0.75 * math.log(3.0)])
    assert rel(out.reshape(2), ref) < 1e-15


def test_epilogue_norm_gate_invariants():
    r = _rng(90)
    B, T, H, V = 2, 7, 3, 16
    o = r.standard_normal((B, T, H, V)) * 5.0
    # z = 0 gates everything off
    assert np.array_equal(oracle.epilogue_norm_gate(o, np.zeros_like(o)), np.zeros_like(o))
    # constant gate c, unit weight: the mean square of a row is silu(c)^2 ms / (ms + eps)
    c, eps = 1.7, 1e-3
    out = oracle.epilogue_norm_gate(o, np.full_like(o, c), None, eps)
    ms = np.mean(o * o, axis=-1)
    sil = c / (1.0 + math.exp(-c))
    assert rel(np.mean(out * out, axis=-1), sil * sil * ms / (ms + eps)) < 1e-13
    # scale invariance: o and 10 o normalise to the same rows when eps = 0
    assert rel(oracle.epilogue_norm_gate(10 * o, o, None, 0.0), oracle.epilogue_norm_gate(o, o, None, 0.0)) < 1e-14
    # the weight multiplies each value column
    w = r.uniform(0.5, 2.0, V)
    assert rel(oracle.epilogue_norm_gate(o, o, w), oracle.epilogue_norm_gate(o, o) * w) < 1e-15


def test_epilogue_skip():
    r = _rng(91)
    B, T, H, V = 2, 5, 3, 4
    o = r.standard_normal((B, T, H, V))
    x = r.standard_normal((B, T, H, V))
    assert np.array_equal(oracle.epilogue_skip(o, np.zeros(H), x), o)
    assert np.array_equal(oracle.epilogue_skip(np.zeros_like(o), np.ones(H), x), x)
    dsk = np.array([0.5, -2.0, 3.0])
    assert rel(oracle.epilogue_skip(o, dsk, x)[:, :, 1], o[:, :, 1] - 2.0 * x[:, :, 1]) < 1e-15


# ----------------------------------------------------------------------------
# Delta rule with a per-key decay [SunnyNet log §5.1, RWKV-7's state update]
# ----------------------------------------------------------------------------

def _decay_inputs(r, B, T, H, K, V, with_s0=True, gmin=-0.6):
    q, k, v, beta, s0 = _delta_inputs(r, B, T, H, K, V, with_s0=with_s0)
    g = r.uniform(gmin, 0.0, (B, T, H, K))
    return q, k, v, g, beta, s0


@pytest.mark.parametrize("case", [0, 1])
@pytest.mark.parametrize("form", ["rank1", "explicit"])
def test_golden_delta_decay_hand(case, form):
    d = _load("delta_decay_hand.json")["cases"][case]
    fn = oracle.scan_delta_decay if form == "rank1" else oracle.scan_delta_decay_explicit
    s0 = None if d["s0"] is None else np.array(d["s0"])
    o, fin = fn(np.array(d["q"]), np.array(d["k"]), np.array(d["v"]), np.log(np.array(d["alpha"])),
                np.array(d["beta"]), d["scale"], s0)
    assert rel(o, d["o"]) < 1e-15
    assert rel(fin, d["s_final"]) < 1e-15


@pytest.mark.parametrize("K,V", [(6, 10), (10, 6), (8, 8)])
def test_delta_decay_rank1_matches_explicit(K, V):
    r = _rng(80 + K)
    q, k, v, g, beta, s0 = _decay_inputs(r, 2, 40, 3, K, V)
    g[0, 5] = 0.3            # a growing key now and then must not break the agreement
    o1, f1 = oracle.scan_delta_decay(q, k, v, g, beta, 0.7, s0)
    o2, f2 = oracle.scan_delta_decay_explicit(q, k, v, g, beta, 0.7, s0)
    assert rel(o1, o2) < 1e-12
    assert rel(f1, f2) < 1e-12


def test_delta_decay_without_decay_is_the_delta_rule():
    # w = 1 (g = 0) is DeltaNet's update, bit for bit
    r = _rng(81)
    q, k, v, g, beta, s0 = _decay_inputs(r, 2, 30, 2, 5, 7)
    z = np.zeros_like(g)
    o1, f1 = oracle.scan_delta_decay(q, k, v, z, beta, 0.8, s0)
    o2, f2 = oracle.scan_delta(q, k, v, beta, 0.8, s0)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)
    o1, f1 = oracle.scan_delta_decay_explicit(q, k, v, z, beta, 0.8, s0)
    o2, f2 = oracle.scan_delta_explicit(q, k, v, beta, 0.8, s0)
    assert np.array_equal(o1, o2) and np.array_equal(f1, f2)


def test_delta_decay_beta_zero_is_pure_decay():
    # beta = 0: S_t = diag(exp(G_t)) S0 with G_t the running sum of g
    r = _rng(82)
    B, T, H, K, V = 2, 25, 2, 4, 6
    q, k, v, g, _, s0 = _decay_inputs(r, B, T, H, K, V)
    o, fin = oracle.scan_delta_decay(q, k, v, g, np.zeros((B, T, H)), 1.3, s0)
    G = np.cumsum(g, axis=1)                                # [B,T,H,K]
    ref = 1.3 * np.einsum("bthk,bhkv,bthk->bthv", np.exp(G), s0, q)
    assert rel(o, ref) < 1e-13
    assert rel(fin, np.exp(G[:, -1])[..., None] * s0) < 1e-13


def test_delta_decay_k1_reduces_to_fma_scan():
    # K = 1: each state column is s_t = (w_t - beta_t k_t^2) s_{t-1} + beta_t k_t v_t[j]
    r = _rng(83)
    B, T, H, V = 2, 60, 3, 5
    q, k, v, g, beta, s0 = _decay_inputs(r, B, T, H, 1, V)
    k = r.uniform(-1.0, 1.0, (B, T, H, 1))
    o, fin = oracle.scan_delta_decay(q, k, v, g, beta, 1.0, s0)
    a = np.exp(g[..., 0]) - beta * k[..., 0] ** 2                      # [B,T,H]
    bb = (beta * k[..., 0])[..., None] * v                               # [B,T,H,V]
    # channels (h, j) of the FMA scan, in its [B,T,N] layout
    s, sf = oracle.scan_fma(np.repeat(a[..., None], V, axis=-1).reshape(B, T, H * V),
                            bb.reshape(B, T, H * V), s0[:, :, 0, :].reshape(B, H * V))
    assert rel(fin[:, :, 0, :], sf.reshape(B, H, V)) < 1e-13
    assert rel(o, q[..., 0:1] * s.reshape(B, T, H, V)) < 1e-13


def test_delta_decay_chunked_ut_form():
    # The chunked form the GPU kernels use, solved with numpy.linalg: with G the
    # within-chunk running sum of g (G_{-1} = 0) and, per key,
    #   a_t = exp(G_{t-1}) k_t,   b_t = exp(-G_t) k_t,   qt_t = exp(G_t) q_t,
    #   A = strict_lower(diag(beta) a b^T),  Delta = (I + A)^{-1} diag(beta) (V - a S0),
    #   O = scale (qt S0 + tril(qt b^T) Delta),
    #   S_L = diag(exp(G_L)) S0 + (exp(G_L - G_t) k_t)^T Delta.
    r = _rng(84)
    B, T, H, K, V = 1, 24, 2, 6, 5
    q, k, v, g, beta, s0 = _decay_inputs(r, B, T, H, K, V)
    o, fin = oracle.scan_delta_decay(q, k, v, g, beta, 0.9, s0)
    for h in range(H):
        Q, Km, Vm, bt, S0 = q[0, :, h], k[0, :, h], v[0, :, h], beta[0, :, h], s0[0, h]
        G = np.cumsum(g[0, :, h], axis=0)
        Gp = np.vstack([np.zeros((1, K)), G[:-1]])
        a, bk, qt = np.exp(Gp) * Km, np.exp(-G) * Km, np.exp(G) * Q
        A = np.tril(bt[:, None] * (a @ bk.T), -1)
        Dl = np.linalg.solve(np.eye(T) + A, bt[:, None] * (Vm - a @ S0))
        assert rel(o[0, :, h], 0.9 * (qt @ S0 + np.tril(qt @ bk.T) @ Dl)) < 1e-11
        khat = np.exp(G[-1][None, :] - G) * Km
        assert rel(fin[0, h], np.exp(G[-1])[:, None] * S0 + khat.T @ Dl) < 1e-11


# ----------------------------------------------------------------------------
# Segment continuation [SunnyNet log §4: two segments with the state carried
# across reproduce the full run exactly] and thread-count invariance
# ----------------------------------------------------------------------------

def _split_runs(run, T, splits):
    full = run(0, T, None)
    for t1 in splits:
        first = run(0, t1, None)
        second = run(t1, T, first[-1])
        yield full, first, second, t1


@pytest.mark.parametrize("dtype", [np.float64, np.float32])
def test_continuation_bit_exact(dtype):
    r = _rng(60)
    B, T, N = 2, 80, 6
    a = r.uniform(0.5, 1.0, (B, T, N)).astype(dtype)
    x = r.standard_normal((B, T, N)).astype(dtype)
    s0 = r.standard_normal((B, N)).astype(dtype)
    splits = (1, 37, T // 2, T - 1)
    for fn in (oracle.scan_fma, oracle.scan_gated):
        def run(lo, hi, init):
            return fn(a[:, lo:hi], x[:, lo:hi], s0 if init is None and lo == 0 else init,
                      dtype=dtype)
        for full, first, second, t1 in _split_runs(run, T, splits):
            assert np.array_equal(np.concatenate([first[0], second[0]], axis=1), full[0])
            assert np.array_equal(second[1], full[1])
    # matrix scans
    H, Hg, K, V = 2, 1, 5, 3
    q, k, v, g, ks, S0 = _diag_inputs(r, B, T, H, Hg, K, V, 1, True, True)
    q, k, v, g, ks, S0 = (z.astype(dtype) for z in (q, k, v, g, ks, S0))
    def run_d(lo, hi, init):
        return oracle.scan_diag_outer(q[:, lo:hi], k[:, lo:hi], v[:, lo:hi], g[:, lo:hi], 1,
                                      ks[:, lo:hi], 0.5, S0 if lo == 0 else init, dtype=dtype)
    for full, first, second, t1 in _split_runs(run_d, T, splits):
        assert np.array_equal(np.concatenate([first[0], second[0]], axis=1), full[0])
        assert np.array_equal(second[1], full[1])
    qd, kd, vd, bd, Sd = (z.astype(dtype) for z in _delta_inputs(r, B, T, H, K, V))
    def run_l(lo, hi, init):
        return oracle.scan_delta(qd[:, lo:hi], kd[:, lo:hi], vd[:, lo:hi], bd[:, lo:hi], 1.0,
                                 Sd if lo == 0 else init, dtype=dtype)
    for full, first, second, t1 in _split_runs(run_l, T, splits):
        assert np.array_equal(np.concatenate([first[0], second[0]], axis=1), full[0])
        assert np.array_equal(second[1], full[1])
    gd = r.uniform(-0.6, 0.0, (B, T, H, K)).astype(dtype)
    def run_w(lo, hi, init):
        return oracle.scan_delta_decay(qd[:, lo:hi], kd[:, lo:hi], vd[:, lo:hi], gd[:, lo:hi],
                                       bd[:, lo:hi], 1.0, Sd if lo == 0 else init, dtype=dtype)
    for full, first, second, t1 in _split_runs(run_w, T, splits):
        assert np.array_equal(np.concatenate([first[0], second[0]], axis=1), full[0])
        assert np.array_equal(second[1], full[1])


def test_thread_count_does_not_change_bits():
    r = _rng(70)
    a = r.uniform(0.5, 1.0, (3, 50, 700))
    x = r.standard_normal((3, 50, 700))
    s1 = oracle.scan_gated(a, x, nthreads=1)
    s4 = oracle.scan_gated(a, x, nthreads=4)
    assert np.array_equal(s1[0], s4[0]) and np.array_equal(s1[1], s4[1])
    q, k, v, beta, s0 = _delta_inputs(r, 2, 20, 3, 4, 6)
    d1 = oracle.scan_delta(q, k, v, beta, 1.0, s0, nthreads=1)
    d4 = oracle.scan_delta(q, k, v, beta, 1.0, s0, nthreads=4)
    assert np.array_equal(d1[0], d4[0]) and np.array_equal(d1[1], d4[1])


def test_float32_mode_tracks_float64():
    # The pages report fp32 scan accumulation error near 5e-7 relative
    # [SunnyNet log §9.3]; the single-precision mode must stay in that class.
    r = _rng(71)
    a = r.uniform(0.5, 1.0, (2, 2048, 16)).astype(np.float32)
    x = r.standard_normal((2, 2048, 16)).astype(np.float32)
    s64, _ = oracle.scan_gated(a, x)
    s32, _ = oracle.scan_gated(a, x, dtype=np.float32)
    assert rel(s32, s64) < 5e-6
