"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a textbook
matrix or routine, a closed form, an invariant, brute force on tiny inputs,
or a number printed on the pages. Statistical tests redraw the QJL sketch for
every pair, because the estimator is unbiased over the sketch, not for one
fixed sketch.
"""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import scipy.stats
from scipy import integrate

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# --------------------------------------------------------------------------
# rotation
# --------------------------------------------------------------------------


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_hadamard_is_sylvester(d):
    """H equals scipy's Sylvester construction (natural order)."""
    np.testing.assert_array_equal(O.hadamard(d), scipy.linalg.hadamard(d))


def _fwht_textbook(v):
    """In-place iterative butterflies (the textbook fast transform), unnormalised."""
    v = np.array(v, dtype=np.float64)
    h = 1
    n = v.shape[-1]
    while h < n:
        for i in range(0, n, 2 * h):
            a = v[..., i:i + h].copy()
            b = v[..., i + h:i + 2 * h].copy()
            v[..., i:i + h] = a + b
            v[..., i + h:i + 2 * h] = a - b
        h *= 2
    return v


@pytest.mark.parametrize("d", [4, 64, 128])
def test_rotation_matches_fast_transform_and_is_orthogonal(d):
    rng = np.random.default_rng(d)
    s = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((50, d))
    y = O.rotate(x, s)
    np.testing.assert_allclose(y, _fwht_textbook(x * s) / math.sqrt(d), rtol=0, atol=1e-12)
    # explicit matrix from scipy
    R = scipy.linalg.hadamard(d) @ np.diag(s) / math.sqrt(d)
    np.testing.assert_allclose(y, x @ R.T, rtol=0, atol=1e-12)
    # norms preserved, inverse is the transpose
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    np.testing.assert_allclose(O.rotate_inverse(y, s), x, rtol=0, atol=1e-12)
    np.testing.assert_allclose(R.T @ R, np.eye(d), atol=1e-12)


def test_rotation_all_sign_vectors_d4():
    """d = 4: every one of the 16 sign vectors gives the explicit matrix."""
    H = np.array([[1, 1, 1, 1], [1, -1, 1, -1], [1, 1, -1, -1], [1, -1, -1, 1]], dtype=float)
    x = np.eye(4)
    for s in itertools.product([-1.0, 1.0], repeat=4):
        R = H @ np.diag(s) / 2.0
        np.testing.assert_allclose(O.rotate(x, np.array(s)), x @ R.T, atol=1e-15)


# --------------------------------------------------------------------------
# codebook
# --------------------------------------------------------------------------


def _quad_mass_moment(a, b, d):
    f = lambda x: O.sphere_coord_density(np.array([x]), d)[0]
    m0 = integrate.quad(f, a, b, epsabs=1e-15, epsrel=1e-13, limit=400)[0]
    m1 = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-15, epsrel=1e-13, limit=400)[0]
    return m0, m1


@pytest.mark.parametrize("d", [3, 4, 16, 128])
def test_density_is_the_sphere_marginal(d):
    """f_d integrates to 1 and matches the Beta law of X^2 (scipy.stats)."""
    f = lambda x: O.sphere_coord_density(np.array([x]), d)[0]
    assert abs(integrate.quad(f, -1, 1, limit=400)[0] - 1) < 1e-10
    for t in (0.05, 0.2, 0.5):
        p = integrate.quad(f, -t, t, limit=400)[0]
        assert abs(p - scipy.stats.beta(0.5, (d - 1) / 2).cdf(t * t)) < 1e-10
    # empirical: coordinates of normalised Gaussian vectors
    rng = np.random.default_rng(1)
    g = rng.standard_normal((200000, d))
    u = g[:, 0] / np.linalg.norm(g, axis=1)
    h, edges = np.histogram(u, bins=20, range=(-1, 1))
    expected = [integrate.quad(f, a, b)[0] * len(u) for a, b in zip(edges[:-1], edges[1:])]
    chi2 = np.sum((h - expected) ** 2 / np.maximum(expected, 1e-9))
    assert chi2 < 60


@pytest.mark.parametrize("d", [4, 5, 64, 128])
def test_codebook_one_bit_closed_form(d):
    """1 bit: c = +-E|X| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))."""
    c, t = O.make_codebook(d, 1, return_fp64=True)
    e = math.exp(scipy.special.gammaln(d / 2) - scipy.special.gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    np.testing.assert_allclose(c, [-e, e], rtol=1e-13)
    assert t[0] == 0.0


def test_codebook_one_bit_printed_values():
    for d, v in ((4, 4 / (3 * math.pi)), (64, 0.1001259), (128, 0.0706616)):
        c, _ = O.make_codebook(d, 1, return_fp64=True)
        assert abs(c[1] - v) < 5e-8


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_d3_uniform(bits):
    """d = 3: f_3 is uniform on [-1, 1]; the Lloyd-Max quantizer is uniform,
    c_k = -1 + (2k+1)/L, with MSE per coordinate 1/(3 L^2)."""
    L = 1 << bits
    c, t = O.make_codebook(3, bits, return_fp64=True)
    np.testing.assert_allclose(c, -1 + (2 * np.arange(L) + 1) / L, atol=1e-12)
    edges = np.concatenate(([-1.0], t, [1.0]))
    mse = sum(integrate.quad(lambda x: (x - c[j]) ** 2 * 0.5, edges[j], edges[j + 1])[0]
              for j in range(L))
    assert abs(mse - 1 / (3 * L * L)) < 1e-12


def test_codebook_d4_semicircle_brute_force():
    """d = 4: f_4 = (2/pi) sqrt(1 - x^2). A symmetric 2-bit quantizer has one
    free threshold tau; brute-force grid search over tau (with conditional-
    mean centroids, integrated numerically) must land on the oracle."""
    f = lambda x: 2 / math.pi * math.sqrt(max(0.0, 1 - x * x))

    def distortion(tau):
        tot = 0.0
        for a, b in ((0.0, tau), (tau, 1.0)):
            m0 = integrate.quad(f, a, b)[0]
            m1 = integrate.quad(lambda x: x * f(x), a, b)[0]
            c = m1 / m0
            tot += integrate.quad(lambda x: (x - c) ** 2 * f(x), a, b)[0]
        return 2 * tot

    taus = np.linspace(0.30, 0.60, 301)
    best = taus[np.argmin([distortion(x) for x in taus])]
    fine = np.linspace(best - 0.001, best + 0.001, 201)
    best = fine[np.argmin([distortion(x) for x in fine])]
    c, t = O.make_codebook(4, 2, return_fp64=True)
    assert abs(t[2] - best) < 2e-5
    np.testing.assert_allclose(c[2:], [0.21945, 0.67440], atol=5e-5)


@pytest.mark.parametrize("d,bits", [(4, 2), (64, 2), (64, 4), (128, 1), (128, 2), (128, 3), (128, 4)])
def test_codebook_fixed_point(d, bits):
    """Both Lloyd conditions hold at the returned point: thresholds are
    midpoints, and each centroid is its cell's conditional mean (checked by
    adaptive quadrature of the density, independent of the closed forms)."""
    c, t = O.make_codebook(d, bits, return_fp64=True)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    edges = np.concatenate(([-1.0], t, [1.0]))
    for j in range(len(c)):
        m0, m1 = _quad_mass_moment(edges[j], edges[j + 1], d)
        assert abs(m1 / m0 - c[j]) < 1e-12
    assert np.all(np.diff(c) > 0)
    np.testing.assert_array_equal(c, -c[::-1])


def _gaussian_lloyd_max(bits):
    """Lloyd-Max for N(0,1) (Max 1960), iterated with scipy.stats.norm."""
    L = 1 << bits
    c = scipy.stats.norm.ppf((np.arange(L) + 0.5) / L)
    for _ in range(20000):
        t = np.concatenate(([-np.inf], 0.5 * (c[:-1] + c[1:]), [np.inf]))
        m0 = scipy.stats.norm.cdf(t[1:]) - scipy.stats.norm.cdf(t[:-1])
        m1 = scipy.stats.norm.pdf(t[:-1]) - scipy.stats.norm.pdf(t[1:])
        c = m1 / m0
    return c


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_codebook_gaussian_limit(bits):
    """sqrt(d) c tends to the Gaussian Lloyd-Max levels as d grows; the gap
    shrinks like 1/d."""
    g = _gaussian_lloyd_max(bits)
    # textbook (Max 1960) positive levels, to 3-4 digits
    table = {1: [0.7979], 2: [0.4528, 1.510], 3: [0.2451, 0.7560, 1.344, 2.152],
             4: [0.1284, 0.3881, 0.6568, 0.9424, 1.256, 1.618, 2.069, 2.733]}
    np.testing.assert_allclose(g[len(g) // 2:], table[bits], atol=1.5e-3)
    gaps = []
    for d in (128, 512, 1024):
        c, _ = O.make_codebook(d, bits, return_fp64=True)
        gaps.append(np.max(np.abs(c * math.sqrt(d) - g)))
    # O(1/d): quadrupling d divides the gap by about four
    assert 0.2 < gaps[1] / gaps[0] < 0.3
    assert 0.4 < gaps[2] / gaps[1] < 0.6
    assert gaps[2] * 1024 < 50


def _analytic_total_mse(d, bits):
    c, t = O.make_codebook(d, bits, return_fp64=True)
    edges = np.concatenate(([-1.0], t, [1.0]))
    f = lambda x: O.sphere_coord_density(np.array([x]), d)[0]
    per = sum(integrate.quad(lambda x: (x - c[j]) ** 2 * f(x), edges[j], edges[j + 1],
                             epsabs=1e-15, limit=400)[0] for j in range(len(c)))
    return d * per


@pytest.mark.parametrize("d", [64, 128])
def test_distortion_within_stated_factor(d):
    """Total MSE per unit vector against 4^-bits, the information-theoretic
    distortion at `bits` per coordinate: the ratio stays within the 2.7x the
    pages quote (classmethod article, PolarQuant + QJL section)."""
    expected = {128: [0.3609, 0.1160, 0.03397, 0.009315]}
    for bits in (1, 2, 3, 4):
        mse = _analytic_total_mse(d, bits)
        assert mse / 4.0 ** (-bits) <= 2.7
        if d in expected:
            assert abs(mse - expected[d][bits - 1]) / expected[d][bits - 1] < 2e-3


@pytest.mark.parametrize("bits", [2, 3])
def test_empirical_distortion_matches_analytic(bits):
    """Encode 1e5 Gaussian rows (uniform directions) and compare the measured
    total MSE of the rotated unit vectors with the analytic value (3 sigma)."""
    d = 128
    rng = np.random.default_rng(7 + bits)
    s = rng.choice([-1.0, 1.0], size=d)
    c, t = O.make_codebook(d, bits)
    x = rng.standard_normal((100000, d))
    enc = O.encode(x, s, c, t)
    err = np.sum((enc["y"] - c.astype(np.float64)[enc["idx"]]) ** 2, axis=1)
    mse = _analytic_total_mse(d, bits)
    assert abs(err.mean() - mse) < 3 * err.std() / math.sqrt(len(err))


# --------------------------------------------------------------------------
# quantizer decisions
# --------------------------------------------------------------------------


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_threshold_compare_is_nearest_centroid(bits):
    """idx from threshold counts equals argmin |y - c_v|; exact ties go up."""
    d = 64
    c, t = O.make_codebook(d, bits)
    rng = np.random.default_rng(bits)
    t32 = t.astype(np.float32)
    y = np.concatenate([rng.standard_normal(20000).astype(np.float32) / np.float32(math.sqrt(d)),
                        t32,                                        # exact ties
                        np.nextafter(t32, np.float32(-np.inf)),     # one ulp below
                        np.nextafter(t32, np.float32(np.inf))])     # one ulp above
    idx = np.sum(y[:, None] >= t32[None, :], axis=1)
    # the decision is taken on the fp32 value; brute force in fp64 on that value
    dist = np.abs(y.astype(np.float64)[:, None] - c.astype(np.float64)[None, :])
    best = np.argmin(dist, axis=1)
    # away from the thresholds both agree
    near = np.min(np.abs(y.astype(np.float64)[:, None] - t.astype(np.float64)[None, :]), axis=1) < 1e-7
    np.testing.assert_array_equal(idx[~near], best[~near])
    # at and around a threshold: exact tie -> upper cell, one ulp off -> that side
    L = 1 << bits
    n = len(t32)
    np.testing.assert_array_equal(idx[20000:20000 + n], np.arange(1, L))
    np.testing.assert_array_equal(idx[20000 + n:20000 + 2 * n], np.arange(0, L - 1))
    np.testing.assert_array_equal(idx[20000 + 2 * n:], np.arange(1, L))


def test_d4_per_coordinate_choice_is_best_codeword():
    """d = 4: the per-coordinate quantizer picks the best of all L^4
    codewords (the distortion is separable)."""
    d, bits = 4, 2
    c, t = O.make_codebook(d, bits)
    L = 1 << bits
    words = np.array(list(itertools.product(range(L), repeat=d)))
    cw = c.astype(np.float64)[words]                                   # [L^4, 4]
    rng = np.random.default_rng(3)
    s = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((300, d))
    enc = O.encode(x, s, c, t)
    dist = np.sum((enc["y"][:, None, :] - cw[None]) ** 2, axis=2)
    best = words[np.argmin(dist, axis=1)]
    np.testing.assert_array_equal(enc["idx"], best)


def test_zero_vector_encodes_to_zero_norm():
    d = 64
    c, t = O.make_codebook(d, 2)
    s = np.ones(d)
    S = np.random.default_rng(0).standard_normal((d, d)).astype(np.float16)
    enc = O.encode(np.zeros((3, d)), s, c, t, S)
    assert np.all(enc["nhat"] == 0)
    q = np.random.default_rng(1).standard_normal((2, d))
    lg = O.key_logits(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], enc["ghat"])
    assert np.all(lg == 0)


@pytest.mark.parametrize("d,bits", [(16, 2), (64, 3), (128, 2)])
def test_requantize_key_with_the_encoders_indices_reproduces_encode(d, bits):
    """Given the indices encode() chose, requantize_key recomputes the key's
    residual, its norm, the projection and the sign bits exactly as encode()
    did (the second stage applied to the same first-stage codes)."""
    rng = np.random.default_rng(1000 + d + bits)
    c, t = O.make_codebook(d, bits)
    s = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    x = rng.standard_normal((40, d)) * np.exp(rng.standard_normal(d))
    enc = O.encode(x, s, c, t, S)
    rq = O.requantize_key(enc["y"], enc["idx"], c, S)
    for k in ("r", "gamma", "z"):
        np.testing.assert_array_equal(rq[k], enc[k])
    np.testing.assert_array_equal(rq["sigma"], enc["sigma"])
    np.testing.assert_array_equal(rq["ghat"].view(np.uint16), enc["ghat"].view(np.uint16))


def test_requantize_key_with_a_moved_index_is_the_explicit_residual_projection():
    """After one index is moved to a neighbouring cell (what the parity rule
    does when the GPU crossed a threshold the oracle did not), the residual is
    y - c[idx'] coordinate by coordinate, gamma its Euclidean norm and z_j the
    sum over k of S[j][k] r_k, written out here as plain Python loops with
    exactly rounded sums; sigma_j = [fp32(z_j) >= 0]."""
    d, bits = 16, 3
    rng = np.random.default_rng(77)
    c, t = O.make_codebook(d, bits)
    s = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    x = rng.standard_normal((6, d))
    enc = O.encode(x, s, c, t, S)
    idx = enc["idx"].copy()
    L = 1 << bits
    for row in range(idx.shape[0]):
        col = (3 * row + 1) % d
        idx[row, col] = idx[row, col] + 1 if idx[row, col] < L - 1 else idx[row, col] - 1
    rq = O.requantize_key(enc["y"], idx, c, S)
    c32 = [float(np.float32(v)) for v in c]
    for row in range(idx.shape[0]):
        y = [float(v) for v in enc["y"][row]]
        r = [y[k] - c32[int(idx[row, k])] for k in range(d)]
        gamma = math.sqrt(math.fsum(v * v for v in r))
        z = [math.fsum(float(S[j, k]) * r[k] for k in range(d)) for j in range(d)]
        np.testing.assert_allclose(rq["r"][row], r, rtol=0, atol=0)
        assert abs(rq["gamma"][row] - gamma) <= 1e-15 * max(gamma, 1.0)
        np.testing.assert_allclose(rq["z"][row], z, rtol=0, atol=1e-14)
        np.testing.assert_array_equal(rq["sigma"][row], [1 if np.float32(v) >= 0 else 0 for v in z])
        assert rq["ghat"][row] == np.float16(gamma)
        # the moved coordinate really changed the residual: the old one differs there
        col = (3 * row + 1) % d
        assert rq["r"][row, col] != enc["r"][row, col]


# --------------------------------------------------------------------------
# QJL estimator: unbiasedness, test power, variance, d = 4 brute force
# --------------------------------------------------------------------------


def _fresh_sketches(rng, n, d):
    return rng.standard_normal((n, d, d), dtype=np.float32).astype(np.float16)


def _pair_errors(d, bits, n_pairs, seed, with_qjl=True, batch=2000):
    """Estimation error est - <q, k> over correlated pairs k ~ N(0, I),
    q = k + N(0, I), with a fresh sketch and fresh signs per batch of pairs
    (the sketch is fresh for every pair)."""
    rng = np.random.default_rng(seed)
    c, t = O.make_codebook(d, bits)
    errs = []
    for b0 in range(0, n_pairs, batch):
        n = min(batch, n_pairs - b0)
        s = rng.choice([-1.0, 1.0], size=d)
        S = _fresh_sketches(rng, n, d)
        k = rng.standard_normal((n, d))
        q = k + rng.standard_normal((n, d))
        enc = O.encode(k, s, c, t, S)
        if with_qjl:
            est = O.pair_logits(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], enc["ghat"])
        else:
            est = O.pair_logits(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"],
                                np.zeros(n, dtype=np.float16))
        errs.append(est - np.sum(q * k, axis=1))
    return np.concatenate(errs)


@pytest.mark.slow
def test_qjl_unbiased_1e5_pairs():
    """Mean error within 3 standard errors over 1e5 pairs (d = 128, 2-bit
    Lloyd-Max + 1 QJL bit): the QJL term makes the estimate unbiased."""
    e = _pair_errors(128, 2, 100000, seed=11)
    z = e.mean() / (e.std() / math.sqrt(len(e)))
    assert abs(z) < 3, z


def test_qjl_negative_control():
    """Without the QJL term the same test has power: the MSE-optimal quantizer
    shrinks inner products (mean relative error about -D(w) = -0.116 at 2 bits)."""
    d = 128
    rng = np.random.default_rng(5)
    c, t = O.make_codebook(d, 2)
    s = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    k = rng.standard_normal((20000, d))
    q = k + rng.standard_normal((20000, d))
    enc = O.encode(k, s, c, t, S)
    lm_only = O.pair_logits(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"],
                            np.zeros(len(k), dtype=np.float16))
    e = lm_only - np.sum(q * k, axis=1)
    z = e.mean() / (e.std() / math.sqrt(len(e)))
    assert z < -20
    rel = np.mean(lm_only) / np.mean(np.sum(q * k, axis=1)) - 1
    assert abs(rel - (-0.116)) < 0.01


def test_qjl_variance_closed_form():
    """Over fresh sketches, Var of the QJL term equals
    [(pi/2) g^2 |q'|^2 - (g/gamma)^2 <q', r>^2] / d, g the stored gamma."""
    d = 64
    rng = np.random.default_rng(9)
    c, t = O.make_codebook(d, 2)
    s = rng.choice([-1.0, 1.0], size=d)
    k = rng.standard_normal((1, d))
    q = k + rng.standard_normal((1, d))
    n_draw = 20000
    S = _fresh_sketches(rng, n_draw, d)
    kk = np.repeat(k, n_draw, axis=0)
    qq = np.repeat(q, n_draw, axis=0)
    enc = O.encode(kk, s, c, t, S)
    full = O.pair_logits(qq, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], enc["ghat"])
    lm = O.pair_logits(qq, s, c, S, enc["idx"], enc["sigma"], enc["nhat"],
                       np.zeros(n_draw, dtype=np.float16))
    term = (full - lm) / enc["nhat"].astype(np.float64)
    qr = O.rotate(q, s)[0]
    r = enc["r"][0]
    gamma = enc["gamma"][0]
    g = float(enc["ghat"][0])
    var = ((math.pi / 2) * g * g * qr @ qr - (g / gamma) ** 2 * (qr @ r) ** 2) / d
    # sampling error of a variance estimate: sd ~ var * sqrt(2 / n) (Gaussian-ish)
    assert abs(term.var() - var) < 5 * var * math.sqrt(2.0 / n_draw) * 1.5
    # and the mean is (g / gamma) <q', r>
    assert abs(term.mean() - (g / gamma) * (qr @ r)) < 4 * math.sqrt(var / n_draw)


def test_d4_expectation_over_sketch_brute_force():
    """d = 4, every sign vector, inputs on a grid (including exact ties):
    E over S of the estimate equals n_hat (<q', c[idx]> + (g/gamma) <q', r>),
    by 2e5 Monte-Carlo sketches per case."""
    d = 4
    c, t = O.make_codebook(d, 2)
    rng = np.random.default_rng(21)
    grid = [np.array([1.0, 0.0, 0.0, 0.0]), np.array([1.0, 1.0, 0.0, 0.0]),
            np.array([0.5, -0.25, 1.0, 2.0]), np.array([1.0, 1.0, 1.0, 1.0])]
    q = np.array([0.3, -1.2, 0.7, 0.1])
    n_draw = 200000
    for s in itertools.product([-1.0, 1.0], repeat=4):
        s = np.array(s)
        for k in grid:
            S = _fresh_sketches(rng, n_draw, d)
            kk = np.repeat(k[None], n_draw, axis=0)
            qq = np.repeat(q[None], n_draw, axis=0)
            enc = O.encode(kk, s, c, t, S)
            est = O.pair_logits(qq, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], enc["ghat"])
            qr = O.rotate(q[None], s)[0]
            n = float(enc["nhat"][0])
            gamma = enc["gamma"][0]
            g = float(enc["ghat"][0])
            lm = qr @ c.astype(np.float64)[enc["idx"][0]]
            expect = n * (lm + (g / gamma if gamma > 0 else 0.0) * (qr @ enc["r"][0]))
            se = est.std() / math.sqrt(n_draw)
            assert abs(est.mean() - expect) < 4.5 * se + 1e-12, (s, k)


# --------------------------------------------------------------------------
# packing
# --------------------------------------------------------------------------


def _golden_lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def test_pack_matches_hand_derived_records():
    for row in _golden_lines("pack_d8.txt"):
        kind = row[0]
        kv = dict(x.split("=", 1) for x in row[1:])
        w = int(kv["lm_bits"])
        if kind == "key":
            idx = np.array([int(v) for v in kv["idx"].split(",")])[None]
            sig = np.array([int(v) for v in kv["sigma"].split(",")])[None]
            rec = O.pack_key_codes(idx, sig, w)[0]
            assert [int(b) for b in rec] == [int(v, 16) for v in kv["bytes"].split(",")]
            i2, s2 = O.unpack_key_codes(rec[None], 8, w)
            np.testing.assert_array_equal(i2, idx)
            np.testing.assert_array_equal(s2, sig)
        elif "pattern" in kv:
            n = int(kv["tokens"])
            idx = np.zeros((1, n, 8), dtype=np.int64)
            for tk in range(n):
                idx[0, tk, tk % 8] = 3
            words = O.pack_value_codes(idx, w)
            b0 = [int(v, 16) for v in kv["block0"].split(",")]
            b1 = [int(v, 16) for v in kv["block1"].split(",")]
            for p in range(w):
                assert list(words[0, 0, p]) == b0
                assert list(words[0, 1, p]) == b1
            np.testing.assert_array_equal(O.unpack_value_codes(words, n), idx)
        else:
            n = int(kv["tokens"])
            idx = np.array([[int(v) for v in tok.split(",")] for tok in kv["idx"].split(";")])
            words = O.pack_value_codes(idx[None], w)
            assert list(words[0, 0, 0]) == [int(v) for v in kv["words"].split(",")]
            np.testing.assert_array_equal(O.unpack_value_codes(words, n)[0], idx)


@pytest.mark.parametrize("w", [1, 2, 3, 4])
def test_pack_roundtrip(w):
    rng = np.random.default_rng(w)
    idx = rng.integers(0, 1 << w, size=(3, 77, 64))
    sig = rng.integers(0, 2, size=(3, 77, 64))
    rec = O.pack_key_codes(idx, sig, w)
    assert rec.shape == (3, 77, (w + 1) * 8)
    i2, s2 = O.unpack_key_codes(rec, 64, w)
    np.testing.assert_array_equal(i2, idx)
    np.testing.assert_array_equal(s2, sig)
    words = O.pack_value_codes(idx, w, cap=128)
    assert words.shape == (3, 4, w, 64)
    np.testing.assert_array_equal(O.unpack_value_codes(words, 77), idx)
    assert np.all(O.unpack_value_codes(words, 128)[:, 77:] == 0)


def test_page_cache_size_arithmetic():
    """The TinyLlama cache sizes the ainew page prints follow from its own
    formula; and at that shape our 3-bit key record (with its two fp16
    scalars) costs 28 bytes against 128 bytes of fp16."""
    for tok, bits, mb in [(int(a), int(b), float(c)) for a, b, c in _golden_lines("p5_cache_sizes.txt")]:
        elements = 22 * 32 * 64 * tok * 2
        assert round(elements * bits / (8 * 1024 * 1024), 2) == mb
    assert 3 * 64 // 8 + 4 == 28
    # 4-bit key (3 LM + 1 QJL) at d = 128 vs fp32 keys
    assert abs(128 * 4 / (4 * 128 // 8 + 4) - 7.53) < 0.01


# --------------------------------------------------------------------------
# logits and decode attention
# --------------------------------------------------------------------------


def _toy_codec(d, w, seed):
    rng = np.random.default_rng(seed)
    s = rng.choice([-1.0, 1.0], size=d)
    S = rng.standard_normal((d, d)).astype(np.float16)
    c, t = O.make_codebook(d, w)
    return rng, s, S, c, t


def test_key_logits_matrix_form_equals_explicit_matrices():
    """key_logits against explicit scipy matrices and against the pairwise form."""
    d, w = 64, 3
    rng, s, S, c, t = _toy_codec(d, w, 4)
    k = rng.standard_normal((40, d))
    q = rng.standard_normal((5, d))
    enc = O.encode(k, s, c, t, S)
    lg = O.key_logits(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], enc["ghat"])
    R = scipy.linalg.hadamard(d) @ np.diag(s) / math.sqrt(d)
    S64 = S.astype(np.float64)
    chat = c.astype(np.float64)[enc["idx"]]
    pm = 2.0 * enc["sigma"] - 1.0
    explicit = (enc["nhat"].astype(np.float64)[None, :] *
                ((R @ q.T).T @ chat.T + math.sqrt(math.pi / 2) / d *
                 enc["ghat"].astype(np.float64)[None, :] * ((S64 @ R @ q.T).T @ pm.T)))
    np.testing.assert_allclose(lg, explicit, rtol=1e-12, atol=1e-12)
    for i in range(5):
        pl = O.pair_logits(np.repeat(q[i:i + 1], 40, 0), s, c, S, enc["idx"], enc["sigma"],
                           enc["nhat"], enc["ghat"])
        np.testing.assert_allclose(pl, lg[i], rtol=1e-12, atol=1e-12)


def test_zero_residual_drops_qjl_term():
    """gamma = 0 makes the QJL term vanish whatever the sign bits."""
    d, w = 64, 2
    rng, s, S, c, t = _toy_codec(d, w, 6)
    idx = rng.integers(0, 4, size=(10, d))
    sig = rng.integers(0, 2, size=(10, d))
    nh = np.full(10, 2.0, dtype=np.float16)
    q = rng.standard_normal((3, d))
    a = O.key_logits(q, s, c, S, idx, sig, nh, np.zeros(10, dtype=np.float16))
    b = O.key_logits(q, s, c, S, idx, 1 - sig, nh, np.zeros(10, dtype=np.float16))
    np.testing.assert_array_equal(a, b)
    np.testing.assert_allclose(a, 2.0 * O.rotate(q, s) @ c.astype(np.float64)[idx].T, rtol=1e-13)


def test_key_logits_mse_is_the_first_term():
    """key_logits_mse against explicit matrices, and against key_logits with
    the residual norms set to zero (which drops the QJL term)."""
    d, w = 64, 3
    rng, s, S, c, t = _toy_codec(d, w, 9)
    k = rng.standard_normal((50, d))
    q = rng.standard_normal((6, d))
    enc = O.encode(k, s, c, t, S)
    got = O.key_logits_mse(q, s, c, enc["idx"], enc["nhat"])
    R = scipy.linalg.hadamard(d) @ np.diag(s) / math.sqrt(d)
    explicit = enc["nhat"].astype(np.float64)[None, :] * ((R @ q.T).T @ c.astype(np.float64)[enc["idx"]].T)
    np.testing.assert_allclose(got, explicit, rtol=1e-12, atol=1e-12)
    zero_g = O.key_logits(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], np.zeros(50, dtype=np.float16))
    np.testing.assert_allclose(got, zero_g, rtol=1e-12, atol=1e-12)


def _toy_cache(B, Hkv, T, d, kw, vw, seed):
    rng, s, S, c, t = _toy_codec(d, kw, seed)
    sv = rng.choice([-1.0, 1.0], size=d)
    cv, tv = O.make_codebook(d, vw)
    K = rng.standard_normal((B * Hkv, T, d))
    V = rng.standard_normal((B * Hkv, T, d))
    ek = O.encode(K, s, c, t, S)
    ev = O.encode(V, sv, cv, tv)
    return rng, (s, c, S), (sv, cv), ek, ev


def test_decode_attend_special_cases_and_textbook_softmax():
    B, Hkv, G, T, d = 2, 2, 3, 37, 64
    rng, (s, c, S), (sv, cv), ek, ev = _toy_cache(B, Hkv, T, d, 2, 4, 8)
    q = rng.standard_normal((B, Hkv * G, d))
    scale = 1 / math.sqrt(d)
    args = (s, c, S, ek["idx"], ek["sigma"], ek["nhat"], ek["ghat"], sv, cv, ev["idx"], ev["nhat"])
    # reconstructed values in the original domain with an explicit matrix
    Rv = scipy.linalg.hadamard(d) @ np.diag(sv) / math.sqrt(d)
    Vhat = ev["nhat"].astype(np.float64)[..., None] * (cv.astype(np.float64)[ev["idx"]] @ Rv)
    # N = 1: output is the single reconstructed value
    out1 = O.decode_attend(q, *args, ctx_lens=[1, 1], sm_scale=scale, group=G)
    for b in range(B):
        for h in range(Hkv * G):
            np.testing.assert_allclose(out1[b, h], Vhat[b * Hkv + h // G, 0], atol=1e-12)
    # ragged lengths, including an empty context: textbook softmax(scale * l) V
    lens = [T, 5]
    out = O.decode_attend(q, *args, ctx_lens=lens, sm_scale=scale, group=G)
    for b in range(B):
        for h in range(Hkv * G):
            sq = b * Hkv + h // G
            Tb = lens[b]
            lg = O.key_logits(q[b, h:h + 1], s, c, S, ek["idx"][sq, :Tb], ek["sigma"][sq, :Tb],
                              ek["nhat"][sq, :Tb], ek["ghat"][sq, :Tb])[0]
            a = scipy.special.softmax(scale * lg)
            np.testing.assert_allclose(out[b, h], a @ Vhat[sq, :Tb], rtol=1e-10, atol=1e-12)
    out0 = O.decode_attend(q, *args, ctx_lens=[0, 3], sm_scale=scale, group=G)
    assert np.all(out0[0] == 0)
    # equal logits (all keys identical) -> plain mean of the values
    ek2 = dict(ek)
    for key in ("idx", "sigma", "nhat", "ghat"):
        ek2[key] = np.repeat(ek[key][:, :1], T, axis=1)
    out_eq = O.decode_attend(q, s, c, S, ek2["idx"], ek2["sigma"], ek2["nhat"], ek2["ghat"],
                             sv, cv, ev["idx"], ev["nhat"], ctx_lens=[T, T], sm_scale=scale, group=G)
    for b in range(B):
        for h in range(Hkv * G):
            np.testing.assert_allclose(out_eq[b, h], Vhat[b * Hkv + h // G].mean(0), atol=1e-12)


def test_append_decode_attend_places_the_new_token():
    """Appending row T-1 of every sequence to a cache holding rows < T-1 and
    attending equals attending over the full encoding (slot, KV-head and
    batch placement); ctx_lens = 1 gives the new value itself, rebuilt with an
    explicit rotation matrix; a row with ctx_lens = 0 appends nothing."""
    B, Hkv, G, T, d, kw, vw = 2, 3, 2, 21, 64, 2, 3
    rng, s, S, c, t = _toy_codec(d, kw, 12)
    sv = rng.choice([-1.0, 1.0], size=d)
    cv, tv = O.make_codebook(d, vw)
    K = rng.standard_normal((B * Hkv, T, d))
    V = rng.standard_normal((B * Hkv, T, d))
    q = rng.standard_normal((B, Hkv * G, d))
    ek, ev = O.encode(K, s, c, t, S), O.encode(V, sv, cv, tv)
    scale = 1 / math.sqrt(d)
    full = O.decode_attend(q, s, c, S, ek["idx"], ek["sigma"], ek["nhat"], ek["ghat"], sv, cv, ev["idx"],
                           ev["nhat"], [T, T], scale, G)
    # the cache's slot T-1 holds another token's codes before the append
    stale = lambda a: np.concatenate([a[:, :T - 1], a[:, :1]], axis=1)
    args = (s, c, t, S, stale(ek["idx"]), stale(ek["sigma"]), stale(ek["nhat"]), stale(ek["ghat"]), sv, cv, tv,
            stale(ev["idx"]), stale(ev["nhat"]))
    k_new = K[:, T - 1].reshape(B, Hkv, d)
    v_new = V[:, T - 1].reshape(B, Hkv, d)
    out, cache, nk, nv = O.append_decode_attend(q, k_new, v_new, *args, ctx_lens=[T, T], sm_scale=scale, group=G)
    np.testing.assert_allclose(out, full, rtol=1e-12, atol=1e-14)
    np.testing.assert_array_equal(cache["kidx"], ek["idx"])
    np.testing.assert_array_equal(cache["vidx"], ev["idx"])
    np.testing.assert_array_equal(nk["sigma"].reshape(B * Hkv, d), ek["sigma"][:, T - 1])
    # an empty cache: the output is the new value, n R_v^T c_v[idx], from an explicit matrix
    out1, cache1, _, nv1 = O.append_decode_attend(q, k_new, v_new, *args, ctx_lens=[1, 0], sm_scale=scale, group=G)
    Rv = scipy.linalg.hadamard(d) @ np.diag(sv) / math.sqrt(d)
    for h in range(Hkv * G):
        vh = nv1["nhat"][0, h // G].astype(np.float64) * (cv.astype(np.float64)[nv1["idx"][0, h // G]] @ Rv)
        np.testing.assert_allclose(out1[0, h], vh, atol=1e-12)
    assert np.all(out1[1] == 0)
    np.testing.assert_array_equal(cache1["kidx"][Hkv:], args[4][Hkv:])     # row 1 untouched
    np.testing.assert_array_equal(cache1["vnhat"][Hkv:], args[12][Hkv:])


def test_prefill_attend_is_masked_softmax_attention():
    """Causal chunk attention against an explicit mask matrix and scipy's
    softmax over the full logit matrix, values rebuilt with an explicit
    rotation matrix; chunk position i equals decode_attend with
    pos0 + i + 1 tokens."""
    B, Hkv, G, T, d, C = 2, 2, 3, 40, 64, 6
    rng, (s, c, S), (sv, cv), ek, ev = _toy_cache(B, Hkv, T, d, 2, 3, 13)
    q = rng.standard_normal((B, C, Hkv * G, d))
    pos0 = [20, 34]
    scale = 0.37
    args = (s, c, S, ek["idx"], ek["sigma"], ek["nhat"], ek["ghat"], sv, cv, ev["idx"], ev["nhat"])
    out = O.prefill_attend(q, *args, pos0=pos0, sm_scale=scale, group=G)
    Rv = scipy.linalg.hadamard(d) @ np.diag(sv) / math.sqrt(d)
    Vhat = ev["nhat"].astype(np.float64)[..., None] * (cv.astype(np.float64)[ev["idx"]] @ Rv)
    for b in range(B):
        for h in range(Hkv * G):
            sq = b * Hkv + h // G
            lg = O.key_logits(q[b, :, h], s, c, S, ek["idx"][sq], ek["sigma"][sq], ek["nhat"][sq],
                              ek["ghat"][sq])                                  # [C, T]
            mask = np.arange(T)[None, :] <= (pos0[b] + np.arange(C))[:, None]
            a = scipy.special.softmax(np.where(mask, scale * lg, -np.inf), axis=1)
            np.testing.assert_allclose(out[b, :, h], a @ Vhat[sq], rtol=1e-10, atol=1e-12)
    for i in (0, C - 1):
        dec = O.decode_attend(q[:, i], *args, ctx_lens=[p + i + 1 for p in pos0], sm_scale=scale, group=G)
        np.testing.assert_allclose(out[:, i], dec, rtol=1e-13, atol=1e-15)


def test_mse_key_record_is_the_key_record_without_its_sign_plane():
    """MSE-only key records against the hand-derived key records (their first
    w planes) and a round trip."""
    n = 0
    for row in _golden_lines("pack_d8.txt"):
        kv = dict(x.split("=", 1) for x in row[1:])
        if row[0] != "key":
            continue
        w = int(kv["lm_bits"])
        idx = np.array([int(v) for v in kv["idx"].split(",")])[None]
        want = [int(v, 16) for v in kv["bytes"].split(",")][:w]          # d = 8: one byte per plane
        rec = O.pack_mse_key_codes(idx, w)[0]
        assert [int(b) for b in rec] == want
        np.testing.assert_array_equal(O.unpack_mse_key_codes(rec[None], 8, w), idx)
        n += 1
    assert n > 0
    rng = np.random.default_rng(5)
    for w in (1, 2, 3, 4):
        idx = rng.integers(0, 1 << w, size=(2, 33, 128))
        rec = O.pack_mse_key_codes(idx, w)
        assert rec.shape == (2, 33, w * 16)
        np.testing.assert_array_equal(O.unpack_mse_key_codes(rec, 128, w), idx)


def test_attention_over_mse_only_keys_is_the_zero_residual_case():
    """With sketch None (MSE-only keys) decode, prefill and append attention
    equal the full estimator's with every residual norm 0 (which drops the
    QJL term), and decode equals scipy's softmax over key_logits_mse."""
    B, Hkv, G, T, d = 2, 2, 3, 29, 64
    rng, (s, c, S), (sv, cv), ek, ev = _toy_cache(B, Hkv, T, d, 3, 2, 21)
    q = rng.standard_normal((B, Hkv * G, d))
    scale = 0.29
    zg = np.zeros_like(ek["ghat"])
    lens = [T, 11]
    mse = O.decode_attend(q, s, c, None, ek["idx"], None, ek["nhat"], None, sv, cv, ev["idx"], ev["nhat"],
                          lens, scale, G)
    full0 = O.decode_attend(q, s, c, S, ek["idx"], ek["sigma"], ek["nhat"], zg, sv, cv, ev["idx"], ev["nhat"],
                            lens, scale, G)
    np.testing.assert_allclose(mse, full0, rtol=1e-12, atol=1e-14)
    Rv = scipy.linalg.hadamard(d) @ np.diag(sv) / math.sqrt(d)
    Vhat = ev["nhat"].astype(np.float64)[..., None] * (cv.astype(np.float64)[ev["idx"]] @ Rv)
    for b in range(B):
        for h in range(Hkv * G):
            sq = b * Hkv + h // G
            lg = O.key_logits_mse(q[b, h:h + 1], s, c, ek["idx"][sq, :lens[b]], ek["nhat"][sq, :lens[b]])[0]
            a = scipy.special.softmax(scale * lg)
            np.testing.assert_allclose(mse[b, h], a @ Vhat[sq, :lens[b]], rtol=1e-10, atol=1e-12)
    C = 4
    qc = rng.standard_normal((B, C, Hkv * G, d))
    pm = O.prefill_attend(qc, s, c, None, ek["idx"], None, ek["nhat"], None, sv, cv, ev["idx"], ev["nhat"],
                          [3, 20], scale, G)
    pf = O.prefill_attend(qc, s, c, S, ek["idx"], ek["sigma"], ek["nhat"], zg, sv, cv, ev["idx"], ev["nhat"],
                          [3, 20], scale, G)
    np.testing.assert_allclose(pm, pf, rtol=1e-12, atol=1e-14)
    # append: the new token lands in slot T-1 and is attended like the rest
    t = O.make_codebook(d, 3)[1]
    tv = O.make_codebook(d, 2)[1]
    K = rng.standard_normal((B * Hkv, d))
    V = rng.standard_normal((B * Hkv, d))
    out, cache, nk, _ = O.append_decode_attend(q, K.reshape(B, Hkv, d), V.reshape(B, Hkv, d), s, c, t, None,
                                               ek["idx"], None, ek["nhat"], None, sv, cv, tv, ev["idx"],
                                               ev["nhat"], [T, T], scale, G)
    assert cache["ksigma"] is None and cache["kghat"] is None and "sigma" not in nk
    e_new = O.encode(K, s, c, t)
    np.testing.assert_array_equal(cache["kidx"][:, T - 1], e_new["idx"])
    ref = O.decode_attend(q, s, c, None, cache["kidx"], None, cache["knhat"], None, sv, cv, cache["vidx"],
                          cache["vnhat"], [T, T], scale, G)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-15)


def test_rate_plan_mixes_neighbouring_widths_evenly():
    """The plan's average is the nearest achievable to the target, its widths
    are the two integers around the Lloyd-Max average, and every prefix of
    layers holds the proportional count of wide layers up to one (checked
    directly, for many rates and depths); 3.5-bit keys over an even depth
    alternate 2 and 3 Lloyd-Max bits."""
    for n in (1, 2, 3, 7, 22, 32, 80):
        for bits in (1.0, 1.5, 2.0, 2.25, 2.5, 3.0, 3.3, 3.5, 3.75, 4.0):
            for is_key in (False, True):
                avg = bits - (1 if is_key else 0)
                if avg < 1 or avg > 4:
                    continue
                plan = O.rate_plan(bits, n, is_key)
                lo = math.floor(avg)
                assert set(plan) <= {lo, lo + 1}
                n_hi = sum(w - lo for w in plan)
                # nearest achievable average
                assert all(abs(n_hi / n - (avg - lo)) <= abs(k / n - (avg - lo)) + 1e-12 for k in range(n + 1))
                for m in range(n + 1):
                    assert abs(sum(w - lo for w in plan[:m]) - m * n_hi / n) < 1.0
    assert O.rate_plan(3.5, 22, True) == [2, 3] * 11
    assert O.rate_plan(2.5, 4, False) == [2, 3, 2, 3]
    with pytest.raises(ValueError):
        O.rate_plan(5.5, 4, True)


def test_e4m3_format_against_torch_and_brute_force():
    """The e4m3fn decode table from its bit fields against torch's
    float8_e4m3fn (all 256 codes, NaN at 0x7f and 0xff); encoding against
    brute-force nearest-value search with ties to an even mantissa (every
    midpoint between neighbouring values, random values across the range)
    and against torch's cast, saturation at +-448, the scale applied to the
    float32 quotient."""
    import torch
    codes = np.arange(256)
    v = O.e4m3_value(codes)
    t = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    assert np.array_equal(np.isnan(v), np.isnan(t)) and np.all(np.isnan(v) == np.isin(codes, [0x7F, 0xFF]))
    np.testing.assert_array_equal(v[~np.isnan(v)], t[~np.isnan(t)])
    finite = [(v[c], c) for c in range(256) if not np.isnan(v[c])]
    pos = sorted({val for val, _ in finite if val >= 0})
    mids = [(a + b) / 2 for a, b in zip(pos[:-1], pos[1:])]
    rng = np.random.default_rng(3)
    xs = np.array(mids + [-m for m in mids] + list(rng.standard_normal(3000) * 30) + [0.0, -0.0, 1e-9, -1e-9],
                  dtype=np.float32)
    got = O.e4m3_encode(xs)
    for x, c in zip(xs.astype(np.float64), got):
        # nearest value (a zero keeps the input's sign); among equal distances the even mantissa
        cands = [(val, cc) for val, cc in finite if val != 0 or np.signbit(val) == np.signbit(x)]
        dist = min(abs(val - x) for val, _ in cands)
        ties = [cc for val, cc in cands if abs(val - x) == dist]
        expect = min(ties, key=lambda cc: (cc & 1, cc))
        assert int(c) == int(expect), (x, c, expect)
    tc = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(got, tc)
    np.testing.assert_array_equal(O.e4m3_encode(np.array([500.0, -1e30, 448.0], dtype=np.float32)), [0x7E, 0xFE, 0x7E])
    assert O.e4m3_encode(np.array([np.nan], dtype=np.float32))[0] == 0xFF
    # x / scale taken in float32
    x = np.array([1.3, -7.7, 200.0], dtype=np.float32)
    np.testing.assert_array_equal(O.e4m3_encode(x, 0.6), O.e4m3_encode(x / np.float32(0.6)))


def test_decode_attend_k8_is_softmax_attention_over_decoded_keys():
    """fp8-key attention against scipy's softmax over logits from the explicit
    decoded key matrix; one token gives the value itself."""
    B, Hkv, G, T, d = 2, 2, 3, 33, 64
    rng = np.random.default_rng(21)
    sv = rng.choice([-1.0, 1.0], size=d)
    cv, tv = O.make_codebook(d, 4)
    V = rng.standard_normal((B * Hkv, T, d))
    ev = O.encode(V, sv, cv, tv)
    K = rng.standard_normal((B * Hkv, T, d)) * 5
    kc = O.e4m3_encode(K.astype(np.float32), 0.5)
    q = rng.standard_normal((B, Hkv * G, d))
    out = O.decode_attend_k8(q, kc, 0.5, sv, cv, ev["idx"], ev["nhat"], [T, 9], 0.3, G)
    Rv = scipy.linalg.hadamard(d) @ np.diag(sv) / math.sqrt(d)
    Vhat = ev["nhat"].astype(np.float64)[..., None] * (cv.astype(np.float64)[ev["idx"]] @ Rv)
    Kd = O.e4m3_value(kc) * 0.5
    for b, Tb in enumerate([T, 9]):
        for h in range(Hkv * G):
            sq = b * Hkv + h // G
            a = scipy.special.softmax(0.3 * (Kd[sq, :Tb] @ q[b, h]))
            np.testing.assert_allclose(out[b, h], a @ Vhat[sq, :Tb], rtol=1e-10, atol=1e-12)
    out1 = O.decode_attend_k8(q, kc, 0.5, sv, cv, ev["idx"], ev["nhat"], [1, 1], 0.3, G)
    for b in range(B):
        for h in range(Hkv * G):
            np.testing.assert_allclose(out1[b, h], Vhat[b * Hkv + h // G, 0], atol=1e-12)


# ---------------------------------------------------------------- search


def _brute_top_k(row, k):
    """Plain Python ranking: score descending, column ascending on ties."""
    order = sorted(range(len(row)), key=lambda i: (-float(row[i]), i))[:k]
    return [float(row[i]) for i in order], order


@pytest.mark.parametrize("k", [1, 3, 7, 16])
def test_top_k_matches_brute_force_with_ties(k):
    rng = np.random.default_rng(11)
    s = rng.integers(-3, 4, size=(6, 16)).astype(np.float32)      # many ties
    s[0, :] = 0.0
    s[1, ::2] = -0.0                                               # -0.0 ties with +0.0
    s[2, :] = np.float32(np.inf)
    s[2, 5] = np.float32(-np.inf)
    vals, idx = O.top_k(s, k)
    for r in range(s.shape[0]):
        bv, bi = _brute_top_k(s[r], k)
        assert list(idx[r]) == bi
        assert list(vals[r]) == bv


def test_search_is_explicit_scores_ranked():
    """search() on a small coded database: the explicit-matrix estimator
    (R, S, centroids as matrices) ranked by brute force."""
    d, w = 64, 3
    rng, s, S, c, t = _toy_codec(d, w, 21)
    db = rng.standard_normal((300, d))
    q = rng.standard_normal((4, d))
    enc = O.encode(db, s, c, t, S)
    vals, idx = O.search(q, s, c, S, enc["idx"], enc["sigma"], enc["nhat"], enc["ghat"], 10)
    R = scipy.linalg.hadamard(d) @ np.diag(s) / math.sqrt(d)
    chat = c.astype(np.float64)[enc["idx"]]
    pm = 2.0 * enc["sigma"] - 1.0
    est = (enc["nhat"].astype(np.float64)[None, :] *
           ((R @ q.T).T @ chat.T + math.sqrt(math.pi / 2) / d *
            enc["ghat"].astype(np.float64)[None, :] * ((S.astype(np.float64) @ R @ q.T).T @ pm.T)))
    for r in range(4):
        bv, bi = _brute_top_k(est[r], 10)
        assert list(idx[r]) == bi
        np.testing.assert_allclose(vals[r], bv, rtol=1e-12)
    # the estimator ranks the exact inner products well: the true best match
    # of each query is among the estimated top 10
    exact = q @ db.T
    for r in range(4):
        assert int(np.argmax(exact[r])) in set(idx[r].tolist())
