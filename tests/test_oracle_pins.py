"""Pins of the float64 oracle against facts the pages and the mathematics fix.

None of these re-run the oracle's own arithmetic to check itself: each compares
it with an independent route (an SVD closed form, a special case whose answer
is known, an invariant, or a constant printed on the pages), chosen so that a
wrong coefficient, sign, index, orientation or step order fails at least one.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest

from oracle import muon_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
PAGE = json.load(open(os.path.join(HERE, "golden", "page_constants.json")))


def svd_ns(G, steps=12, coeffs=(2.0, -1.5, 0.5), eps=1e-7):
    """NS via the SVD: U diag(p^steps(s / (||G||_F + eps))) V^T."""
    G = np.asarray(G, dtype=np.float64)
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    a, b, c = coeffs
    t = s / (math.sqrt(float(np.sum(G * G))) + eps)
    for _ in range(steps):
        t = a * t + b * t ** 3 + c * t ** 5
    return (U * t) @ Vt


def rel(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# --------------------------------------------------------------------------
# Page constants
# --------------------------------------------------------------------------

def test_defaults_match_page_table():
    cfg = O.OracleConfig()
    assert cfg.ns_steps == PAGE["ns"]["steps"]
    assert (cfg.ns_a, cfg.ns_b, cfg.ns_c) == (PAGE["ns"]["a"], PAGE["ns"]["b"], PAGE["ns"]["c"])
    assert cfg.ns_eps == PAGE["ns"]["norm_eps"]
    assert cfg.pp_iterations == PAGE["table"]["pp_iterations"]
    assert cfg.pp_beta == PAGE["table"]["pp_beta"]
    assert cfg.pp_eps == PAGE["aurora_signature"]["eps"]
    assert cfg.mu == PAGE["muon_update_signature"]["mu"]
    assert cfg.nesterov is PAGE["muon_update_signature"]["nesterov"]
    assert cfg.power_steps == PAGE["power_steps"]
    assert cfg.contra == PAGE["contra"]
    assert cfg.target_uw == PAGE["target_uw"]
    assert cfg.lr == PAGE["table"]["lr"]


# --------------------------------------------------------------------------
# Newton-Schulz
# --------------------------------------------------------------------------

def test_poly_fixed_point_and_flatness():
    a, b, c = PAGE["ns"]["a"], PAGE["ns"]["b"], PAGE["ns"]["c"]
    # a + b + c = 1: singular value 1 is a fixed point
    assert O.ns_poly(1.0) == pytest.approx(1.0, abs=1e-15)
    # p'(1) = a + 3b + 5c = 0: the fixed point is flat (quintic convergence)
    h = 1e-6
    d = (O.ns_poly(1 + h) - O.ns_poly(1 - h)) / (2 * h)
    assert abs(d) < 1e-9 and a + 3 * b + 5 * c == 0.0
    # p'(s) = 2 - 4.5 s^2 + 2.5 s^4 has its roots at s^2 in {0.8, 1}; max on [0,1] at sqrt(0.8)
    s = np.linspace(0, 1, 200001)
    pmax = O.ns_poly(s).max()
    assert pmax == pytest.approx(O.ns_poly(math.sqrt(0.8)), rel=1e-9)
    assert 1.0017 < pmax < 1.0018
    # p(0) = 0, odd polynomial
    assert O.ns_poly(0.0) == 0.0 and O.ns_poly(-0.3) == -O.ns_poly(0.3)


@pytest.mark.parametrize("shape", [(1, 1), (1, 7), (7, 1), (3, 5), (5, 3), (8, 8),
                                   (16, 40), (40, 16), (33, 9)])
def test_ns_equals_svd_closed_form(shape):
    rng = np.random.default_rng([11, *shape])
    G = rng.standard_normal(shape) * np.exp(rng.standard_normal((shape[0], 1)))
    got = O.newton_schulz(G)
    want = svd_ns(G)
    assert rel(got, want) < 1e-12


def test_ns_iteration_count_and_coefficients_matter():
    rng = np.random.default_rng(5)
    U = np.linalg.qr(rng.standard_normal((6, 6)))[0]
    V = np.linalg.qr(rng.standard_normal((10, 6)))[0]
    s = np.array([1.0, 0.9, 0.5, 0.3, 0.1, 3e-5])   # p'(0) = 2: s=3e-5 still grows at step 12
    G = (U * s) @ V.T
    base = O.newton_schulz(G)
    assert rel(base, svd_ns(G, steps=11)) > 1e-6
    assert rel(base, svd_ns(G, coeffs=(3.4445, -4.7750, 2.0315))) > 1e-2


def test_ns_close_to_exact_polar_when_well_conditioned():
    rng = np.random.default_rng(7)
    G = rng.standard_normal((20, 60))
    U, s, Vt = np.linalg.svd(G, full_matrices=False)
    assert s.min() / np.linalg.norm(G) > 1e-3       # inside the converged range
    assert rel(O.newton_schulz(G), U @ Vt) < 1e-5
    sv = np.linalg.svd(O.newton_schulz(G), compute_uv=False)
    assert sv.max() <= 1.00176 and sv.min() > 0.99


def test_ns_zero_matrix():
    Z = np.zeros((4, 9))
    assert not np.any(O.newton_schulz(Z))


def test_ns5_classic_closed_form():
    rng = np.random.default_rng(3)
    G = rng.standard_normal((12, 30))
    k = PAGE["ns5_classic"]
    want = svd_ns(G, steps=k["steps"], coeffs=(k["a"], k["b"], k["c"]))
    assert rel(O.ns5_classic(G), want) < 1e-12


# --------------------------------------------------------------------------
# Aurora
# --------------------------------------------------------------------------

def test_square_short_circuit():
    rng = np.random.default_rng(1)
    G = rng.standard_normal((9, 9)) * np.exp(rng.standard_normal((9, 1)))
    assert np.array_equal(O.aurora_orthogonalize(G), O.newton_schulz(G))
    assert rel(O.aurora_orthogonalize(G, pp_iterations=3, pp_beta=1.0), svd_ns(G)) < 1e-12


@pytest.mark.parametrize("shape", [(24, 8), (8, 24), (31, 5)])
def test_pp1_is_row_normalise_then_polar(shape):
    """pp_iterations = 1 is Muon-EQ: normalise each long-side row, then NS."""
    rng = np.random.default_rng([2, *shape])
    G = rng.standard_normal(shape) * np.exp(rng.standard_normal((shape[0], 1)))
    T = G if shape[0] > shape[1] else G.T
    Tn = T / np.linalg.norm(T, axis=1, keepdims=True)
    want = svd_ns(Tn)
    want = want if shape[0] > shape[1] else want.T
    assert rel(O.aurora_orthogonalize(G, pp_iterations=1), want) < 1e-11


@pytest.mark.parametrize("m", [2, 5, 17])
def test_column_vector_gets_uniform_entries(m):
    """An m x 1 matrix: D G = sign(g), whose polar is sign(g)/sqrt(m); rows are
    already uniform, so every later pass keeps D (closed form)."""
    rng = np.random.default_rng(m)
    g = rng.standard_normal((m, 1)) * np.exp(3 * rng.standard_normal((m, 1)))
    want = np.sign(g) / math.sqrt(m)
    # NS of a unit-norm vector: singular value 1/(1+1e-7) -> p^12 = 1 - O(1e-20)
    for pp in (1, 2, 3):
        got = O.aurora_orthogonalize(g, pp_iterations=pp)
        assert np.max(np.abs(got - want)) < 1e-12
        got_t = O.aurora_orthogonalize(g.T, pp_iterations=pp)
        assert np.max(np.abs(got_t - want.T)) < 1e-12


def test_transpose_equivariance():
    rng = np.random.default_rng(4)
    G = rng.standard_normal((10, 26)) * np.exp(rng.standard_normal((10, 1)))
    assert rel(O.aurora_orthogonalize(G.T), O.aurora_orthogonalize(G).T) < 1e-13


def test_long_side_scale_invariance():
    """D0 cancels any positive scaling of the long-side rows."""
    rng = np.random.default_rng(6)
    G = rng.standard_normal((30, 7))
    s = np.exp(rng.standard_normal((30, 1)))
    assert rel(O.aurora_orthogonalize(s * G), O.aurora_orthogonalize(G)) < 1e-12
    Gw = G.T            # wide: the long side is the columns
    assert rel(O.aurora_orthogonalize(Gw * s.T), O.aurora_orthogonalize(Gw)) < 1e-12
    # ...but not of the short side (so the orientation is pinned)
    t = np.exp(rng.standard_normal((1, 7)))
    assert rel(O.aurora_orthogonalize(G * t), O.aurora_orthogonalize(G)) > 1e-3


def test_beta_zero_reduces_to_pp1():
    rng = np.random.default_rng(8)
    G = rng.standard_normal((40, 12)) * np.exp(rng.standard_normal((40, 1)))
    a = O.aurora_orthogonalize(G, pp_iterations=2, pp_beta=0.0)
    b = O.aurora_orthogonalize(G, pp_iterations=1)
    assert rel(a, b) < 1e-13
    assert rel(O.aurora_orthogonalize(G, pp_iterations=2, pp_beta=0.5), b) > 1e-3


def _row_dev(U, shape):
    T = U if shape[0] > shape[1] else U.T
    m, n = T.shape
    return np.abs(np.linalg.norm(T, axis=1) / math.sqrt(n / m) - 1)


@pytest.mark.parametrize("shape", [(128, 512), (512, 128), (96, 384), (256, 1024)])
def test_row_norms_equilibrated(shape):
    """pp=2, beta=0.5 brings long-side row norms to within ~2 % of
    sqrt(min/max) (the page's claim; reading: typical deviation), and beats
    pp=1 on every seed."""
    for seed in range(3):
        rng = np.random.default_rng([9, seed, *shape])
        G = rng.standard_normal(shape)
        d2 = _row_dev(O.aurora_orthogonalize(G, 2, 0.5), shape)
        d1 = _row_dev(O.aurora_orthogonalize(G, 1, 0.5), shape)
        assert d2.mean() < 0.01 and d2.max() < 0.03
        assert d2.mean() < d1.mean()
        # converged polar of a full-rank tall T has sum_i ||U_i||^2 = n, i.e. mean row_sq = n/m
        T = O.aurora_orthogonalize(G, 2, 0.5)
        assert np.sum(T * T) == pytest.approx(min(shape), rel=1e-4)


def test_row_scaled_median_deviation_within_two_percent():
    shape = (256, 1024)
    devs = []
    for seed in range(1, 8):
        rng = np.random.default_rng([10, seed])
        G = rng.standard_normal(shape) * np.exp(rng.standard_normal((shape[0], 1)))
        devs.append(_row_dev(O.aurora_orthogonalize(G, 2, 0.5), shape).mean())
    assert np.median(devs) <= 0.02


# --------------------------------------------------------------------------
# Power iteration
# --------------------------------------------------------------------------

def test_power_rank_one_exact():
    rng = np.random.default_rng(12)
    u = rng.standard_normal(9); u /= np.linalg.norm(u)
    v = rng.standard_normal(5); v /= np.linalg.norm(v)
    assert abs(v.sum()) > 1e-3
    X = 3.7 * np.outer(u, v)
    assert O.power_sigma(X) == pytest.approx(3.7, rel=1e-13)


def test_power_bounds_and_monotone():
    rng = np.random.default_rng(13)
    X = rng.standard_normal((30, 20)) * np.exp(rng.standard_normal((30, 1)))
    smax = np.linalg.svd(X, compute_uv=False)[0]
    est = [O.power_sigma(X, k) for k in range(1, 40)]
    assert all(e <= smax * (1 + 1e-12) for e in est)
    assert all(est[i + 1] >= est[i] * (1 - 1e-12) for i in range(len(est) - 1))
    assert est[-1] == pytest.approx(smax, rel=1e-3)


def test_power_start_vector_is_ones():
    """With the top right singular vector equal to ones/sqrt(c) the first
    iterate is exact; with it orthogonal to ones the estimate is the second
    singular value (which pins the start vector)."""
    rng = np.random.default_rng(14)
    c = 4
    V = np.linalg.qr(np.column_stack([np.ones(c), rng.standard_normal((c, c - 1))]))[0]
    U = np.linalg.qr(rng.standard_normal((6, c)))[0]
    s = np.array([5.0, 2.0, 1.0, 0.5])
    X = (U * s) @ V.T
    assert O.power_sigma(X) == pytest.approx(5.0, rel=1e-12)
    X2 = (U * s) @ V[:, [1, 0, 2, 3]].T           # top vector now orthogonal to ones
    assert O.power_sigma(X2) < 2.0 + 1e-9


def test_power_restart_and_zero():
    X = np.array([[1.0, -1.0, 0.0], [2.0, 0.0, -2.0], [0.0, 3.0, -3.0]])   # rows sum to 0
    assert not np.any(X @ np.ones(3))
    smax = np.linalg.svd(X, compute_uv=False)[0]
    sig = O.power_sigma(X)
    assert 0.9 * smax < sig <= smax * (1 + 1e-12)
    assert O.power_sigma(np.zeros((3, 4))) == 0.0


# --------------------------------------------------------------------------
# muon_update
# --------------------------------------------------------------------------

def test_momentum_nesterov_closed_form():
    rng = np.random.default_rng(15)
    G = rng.standard_normal((5, 8)); M = rng.standard_normal((5, 8))
    cfg = O.OracleConfig(contra=0.0)
    Mn, V, _ = O.muon_update(G, M, None, cfg)
    assert np.allclose(Mn, 0.95 * M + 0.05 * G, rtol=0, atol=1e-15)
    # update direction comes from X = 0.0975 G + 0.9025 M
    X = 0.0975 * G + 0.9025 * M
    want = O.aurora_orthogonalize(X)
    assert rel(V, want) < 1e-12
    cfg2 = O.OracleConfig(contra=0.0, nesterov=False)
    _, V2, _ = O.muon_update(G, M, None, cfg2)
    assert rel(V2, O.aurora_orthogonalize(Mn)) < 1e-12


def test_contra_closed_form_square():
    """Square X with its top right singular vector = ones/sqrt(c): sigma_hat is
    exactly s1, NS is the SVD closed form, so V = (U - 0.2 X / s1) rescaled to
    ||U||_F. G is built so that the Nesterov update equals X for a given M."""
    rng = np.random.default_rng(16)
    c = 6
    V_ = np.linalg.qr(np.column_stack([np.ones(c), rng.standard_normal((c, c - 1))]))[0]
    U_ = np.linalg.qr(rng.standard_normal((c, c)))[0]
    s = np.array([4.0, 3.0, 2.0, 1.0, 0.7, 0.4])
    X = (U_ * s) @ V_.T
    M = rng.standard_normal((c, c))
    mu = 0.95
    G = (X - mu * mu * M) / (1 - mu * mu)            # X = (1-mu^2) G + mu^2 M
    cfg = O.OracleConfig(target_uw=0.0)
    _, V, _ = O.muon_update(G, M, None, cfg)
    Upol = svd_ns(X)
    raw = Upol - 0.2 * X / s[0]
    want = raw * (np.linalg.norm(Upol) / np.linalg.norm(raw))
    assert rel(V, want) < 1e-10
    # the wrong sign gives a clearly different answer
    raw_bad = Upol + 0.2 * X / s[0]
    assert rel(V, raw_bad * np.linalg.norm(Upol) / np.linalg.norm(raw_bad)) > 1e-2


@pytest.mark.parametrize("shape", [(24, 6), (6, 24), (10, 10)])
def test_frobenius_and_aspect(shape):
    rng = np.random.default_rng([17, *shape])
    G = rng.standard_normal(shape); M = rng.standard_normal(shape)
    cfg = O.OracleConfig(target_uw=0.0)
    Mn, V, _ = O.muon_update(G, M, None, cfg)
    X = G + 0.95 * (Mn - G)
    f = np.linalg.norm(O.aurora_orthogonalize(X))
    assert np.linalg.norm(V) == pytest.approx(f * math.sqrt(max(1.0, shape[0] / shape[1])), rel=1e-12)


def test_floor_forced_and_idle():
    rng = np.random.default_rng(18)
    shape = (16, 48)
    G = rng.standard_normal(shape); M = rng.standard_normal(shape)
    W_big = rng.standard_normal(shape)                      # ||V||/||W|| ~ 0.06 -> fires
    _, V, Wn = O.muon_update(G, M, W_big)
    assert np.linalg.norm(V) / np.linalg.norm(W_big) == pytest.approx(0.35, rel=1e-12)
    assert np.allclose(Wn, W_big - 0.0375 * V, rtol=0, atol=1e-15)
    W_small = 0.02 * rng.standard_normal(shape)             # ratio > 0.35 -> idle
    _, V2, Wn2 = O.muon_update(G, M, W_small)
    _, V3, _ = O.muon_update(G, M, None)
    assert np.array_equal(V2, V3)
    assert np.linalg.norm(V2) / np.linalg.norm(W_small) > 0.35
    assert np.linalg.norm(Wn2 - W_small) == pytest.approx(0.0375 * np.linalg.norm(V2), rel=1e-12)


def test_zero_inputs():
    Z = np.zeros((8, 20)); W = np.full((8, 20), 0.5)
    Mn, V, Wn = O.muon_update(Z, Z, W)
    assert not np.any(Mn) and not np.any(V) and np.array_equal(Wn, W)
    assert np.all(np.isfinite(V))


# --------------------------------------------------------------------------
# Classic five-step recipe (Track-1 page)
# --------------------------------------------------------------------------

def test_classic_config_matches_page():
    k, n = PAGE["classic_recipe"], PAGE["ns5_classic"]
    c = O.classic_config()
    assert (c.ns_steps, c.ns_a, c.ns_b, c.ns_c) == (n["steps"], n["a"], n["b"], n["c"])
    assert (c.lr, c.mu, c.nesterov) == (k["lr"], k["mu"], k["nesterov"])
    assert c.momentum == k["momentum_form"]
    # no Aurora preconditioner, no Contra term, no u/w-floor
    assert (c.pp_iterations, c.contra, c.target_uw) == (0, 0.0, 0.0)


def test_momentum_warmup_points_and_linearity():
    w = PAGE["classic_recipe"]["warmup"]

    def f(s):
        return O.momentum_warmup(s, w["mu_start"], w["mu_end"], w["steps"])

    assert f(0) == w["mu_start"] and f(-7) == w["mu_start"]
    assert f(w["steps"]) == w["mu_end"] and f(10 ** 7) == w["mu_end"]
    assert f(w["steps"] // 2) == pytest.approx(0.5 * (w["mu_start"] + w["mu_end"]), abs=1e-15)
    ys = np.array([f(s) for s in range(0, w["steps"] + 1)])
    assert np.all(np.diff(ys) > 0)                     # increasing over the warm-up
    assert np.max(np.abs(np.diff(ys, 2))) < 1e-15      # and linear
    assert O.momentum_warmup(3, 0.85, 0.95, 0) == 0.95


@pytest.mark.parametrize("shape", [(96, 40), (40, 96), (64, 64)])
def test_classic_update_closed_form(shape):
    """Classic step = SGD-momentum buffer and Nesterov blend -> NS5 (SVD closed
    form) -> sqrt(max(1, rows/cols)) -> W - lr V, with no further rescaling."""
    rng = np.random.default_rng(11)
    G, M, W = (rng.standard_normal(shape) for _ in range(3))
    cfg = dataclasses.replace(O.classic_config(), mu=O.momentum_warmup(123))
    M1, V, W1 = O.muon_update(G, M, W, cfg)
    buf = cfg.mu * M + G                       # heavy-ball buffer, no dampening
    X = G + cfg.mu * buf                       # Nesterov
    k = PAGE["ns5_classic"]
    want = svd_ns(X, steps=k["steps"], coeffs=(k["a"], k["b"], k["c"])) * math.sqrt(max(1.0, shape[0] / shape[1]))
    assert rel(M1, buf) < 1e-14
    assert rel(V, want) < 1e-10
    assert rel(W1, W - PAGE["classic_recipe"]["lr"] * want) < 1e-12


def _momentum_sums(Gs, mus, form):
    """Closed form of the momentum buffer after len(Gs) steps from zero, as an
    explicit weighted sum of the gradients (not the recursion): with
    P(j) = prod of mu_t for t > j, the SGD buffer is sum_j P(j) G_j and the
    moving average is sum_j (1 - mu_j) P(j) G_j."""
    k = len(Gs)
    tot = np.zeros_like(Gs[0])
    for j in range(k):
        P = float(np.prod(mus[j + 1:k]))
        w = P if form == "sgd" else (1.0 - mus[j]) * P
        tot = tot + w * Gs[j]
    return tot


def test_classic_sgd_momentum_over_warmup():
    """Five classic steps at the start of the momentum warm-up (mu from 0.85):
    the oracle's buffer equals the SGD-momentum closed form and not the
    moving-average one, and every step's update is NS5 of G_k + mu_k buf_k.
    Swapping the two momentum forms fails both checks."""
    shape = (48, 20)
    rng = np.random.default_rng(31)
    Gs = [rng.standard_normal(shape) * np.exp(rng.standard_normal((shape[0], 1))) for _ in range(5)]
    w = PAGE["classic_recipe"]["warmup"]
    k5 = PAGE["ns5_classic"]
    base = O.classic_config()
    M = np.zeros(shape)
    mus = []
    for step, G in enumerate(Gs):
        mu_k = O.momentum_warmup(step * 100, w["mu_start"], w["mu_end"], w["steps"])
        mus.append(mu_k)
        M, V, _ = O.muon_update(G, M, None, dataclasses.replace(base, mu=mu_k))
        sgd = _momentum_sums(Gs[:step + 1], mus, "sgd")
        ema = _momentum_sums(Gs[:step + 1], mus, "ema")
        assert rel(M, sgd) < 1e-13
        assert rel(M, ema) > 0.5                       # about 1 / (1 - mu) apart
        X = G + mu_k * sgd
        want = svd_ns(X, steps=k5["steps"], coeffs=(k5["a"], k5["b"], k5["c"])) * math.sqrt(shape[0] / shape[1])
        assert rel(V, want) < 1e-10
        if step >= 1:                                  # the two forms' directions part under the warm-up
            X_ema = (1 - mu_k) * G + mu_k * ema
            bad = svd_ns(X_ema, steps=k5["steps"], coeffs=(k5["a"], k5["b"], k5["c"])) * math.sqrt(shape[0] / shape[1])
            assert rel(V, bad) > 1e-3


def test_momentum_forms_agree_in_direction_at_constant_mu():
    """At constant mu and zero start the SGD buffer is the moving average
    divided by (1 - mu), so NS (which divides by the norm) gives the same
    update direction up to the 1e-7 norm guard."""
    shape = (30, 12)
    rng = np.random.default_rng(32)
    Ms, Me = np.zeros(shape), np.zeros(shape)
    for _ in range(3):
        G = rng.standard_normal(shape)
        Ms, Vs, _ = O.muon_update(G, Ms, None, dataclasses.replace(O.classic_config(), mu=0.9))
        Me, Ve, _ = O.muon_update(G, Me, None, dataclasses.replace(O.classic_config(), mu=0.9, momentum="ema"))
        assert rel(Ms * (1 - 0.9), Me) < 1e-13
        assert rel(Vs, Ve) < 1e-6


# --------------------------------------------------------------------------
# Aurora on a wide matrix's own rows (reading R7)
# --------------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(8, 24), (5, 31), (12, 40)])
def test_wide_rows_pp1_is_row_normalise_then_polar(shape):
    """pp = 1 on the wide matrix's own rows: normalise each row of G (no
    transpose), then the SVD closed form of NS."""
    rng = np.random.default_rng([33, *shape])
    G = rng.standard_normal(shape) * np.exp(rng.standard_normal((shape[0], 1)))
    Gn = G / np.linalg.norm(G, axis=1, keepdims=True)
    got = O.aurora_orthogonalize(G, pp_iterations=1, wide_rows=True)
    assert rel(got, svd_ns(Gn)) < 1e-11
    # and it is not the default column equilibration
    assert rel(got, O.aurora_orthogonalize(G, pp_iterations=1)) > 1e-3


def test_wide_rows_invariances():
    """Positive scaling of a wide G's rows cancels in D0 (but column scaling
    does not); tall and square inputs are unchanged by the option; the rows
    of the result are orthonormal for a well-conditioned input, so later
    passes stay at the first pass's D (the fixed point of target 1)."""
    rng = np.random.default_rng(34)
    G = rng.standard_normal((10, 36))
    s = np.exp(rng.standard_normal((10, 1)))
    t = np.exp(rng.standard_normal((1, 36)))
    for pp in (1, 2, 3):
        a = O.aurora_orthogonalize(G, pp, 0.5, wide_rows=True)
        assert rel(O.aurora_orthogonalize(s * G, pp, 0.5, wide_rows=True), a) < 1e-12
        assert rel(O.aurora_orthogonalize(G * t, pp, 0.5, wide_rows=True), a) > 1e-3
        assert np.max(np.abs(a @ a.T - np.eye(10))) < 1e-4
    assert rel(O.aurora_orthogonalize(G, 2, 0.5, wide_rows=True),
               O.aurora_orthogonalize(G, 1, 0.5, wide_rows=True)) < 1e-4
    T = G.T
    assert np.array_equal(O.aurora_orthogonalize(T, 2, 0.5, wide_rows=True), O.aurora_orthogonalize(T, 2, 0.5))
    S = rng.standard_normal((9, 9))
    assert np.array_equal(O.aurora_orthogonalize(S, 2, 0.5, wide_rows=True), O.newton_schulz(S))


def test_wide_rows_moves_d_when_rows_are_ill_conditioned():
    """Where NS has not converged (two nearly parallel rows, a singular value
    near 1e-4 of the largest), the leverage of those rows is below 1 and the
    second pass reweights them: pp = 2 then differs from pp = 1."""
    rng = np.random.default_rng(35)
    G = rng.standard_normal((6, 40))
    G[1] = G[0] + 1e-4 * rng.standard_normal(40)
    a1 = O.aurora_orthogonalize(G, 1, 0.5, wide_rows=True)
    a2 = O.aurora_orthogonalize(G, 2, 0.5, wide_rows=True)
    lev1 = np.sum(a1 * a1, axis=1)
    assert lev1[0] < 0.9 and lev1[1] < 0.9
    assert rel(a2, a1) > 1e-3
