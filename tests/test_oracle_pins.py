"""Pins of the CPU oracle against what the pages and mathematics fix (no GPU).

Each test ties one oracle function to something other than itself: a closed form, a
textbook table, numerical quadrature by SciPy, an invariant, brute force at tiny d, or a
Monte-Carlo expectation.  A dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one of them (see the notes on each test).
"""
import itertools
import math
import os

import numpy as np
import pytest
from scipy import integrate, special, stats

import oracle
from workloads import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------- helpers

def _load_max_table():
    table = {}
    with open(os.path.join(GOLDEN, "lloyd_max_gaussian_max1960.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            table[(int(parts[0]), parts[1])] = parts[2:]
    return table


def _tol(printed: str) -> float:
    decimals = len(printed.split(".")[1]) if "." in printed else 0
    return 0.5 * 10.0 ** (-decimals) + 1e-4


def _sphere_marginal_pdf(d):
    """Density of one coordinate of a uniform point on the unit sphere in R^d."""
    logc = special.gammaln(d / 2.0) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2.0)
    return lambda t: math.exp(logc + 0.5 * (d - 3) * math.log1p(-t * t)) if abs(t) < 1 else 0.0


def _sphere_expectations(d, bits_mse):
    """kappa = d E[u Q(u)] and D = d E[(u - Q(u))^2] for u a sphere coordinate (quadrature)."""
    c, t = oracle.codebook(bits_mse, d)
    f = _sphere_marginal_pdf(d)
    edges = [-1.0] + list(t) + [1.0]
    kappa = 0.0
    dist = 0.0
    for i, ci in enumerate(c):
        a, b = edges[i], edges[i + 1]
        kappa += ci * integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-13, epsrel=1e-12)[0]
        dist += integrate.quad(lambda x: (x - ci) ** 2 * f(x), a, b, epsabs=1e-13,
                               epsrel=1e-12)[0]
    return d * kappa, d * dist


# ----------------------------------------------------------------------- codebook pins

def test_one_bit_codebook_closed_form():
    # 1-bit Lloyd-Max for N(0, 1): centroids +-E|X| = +-sqrt(2/pi), threshold 0.
    c, t = oracle.lloyd_max_gaussian(1)
    assert np.allclose(c, [-math.sqrt(2 / math.pi), math.sqrt(2 / math.pi)], atol=1e-14, rtol=0)
    assert t.tolist() == [0.0]
    # Scaled to N(0, 1/d): +-sqrt(2/pi) * sigma.
    d = 128
    cs, ts = oracle.codebook(1, d)
    assert np.allclose(cs, np.array([-1, 1]) * math.sqrt(2 / math.pi) / math.sqrt(d), rtol=1e-14)
    # Distortion of the 1-bit quantizer: 1 - 2/pi.
    assert abs(oracle.gaussian_distortion(c, t) - (1 - 2 / math.pi)) < 1e-14


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_matches_textbook_table(bits):
    table = _load_max_table()
    L = 1 << bits
    c, t = oracle.lloyd_max_gaussian(bits)
    pos_c = c[L // 2:]
    for got, printed in zip(pos_c, table[(L, "y")]):
        assert abs(got - float(printed)) <= _tol(printed), (bits, got, printed)
    if (L, "x") in table:
        pos_t = t[L // 2 - 1:]
        for got, printed in zip(pos_t, table[(L, "x")]):
            assert abs(got - float(printed)) <= _tol(printed), (bits, got, printed)
    printed_d = table[(L, "D")][0]
    assert abs(oracle.gaussian_distortion(c, t) - float(printed_d)) <= _tol(printed_d)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_lloyd_max_fixed_point_by_quadrature(bits):
    # Optimality conditions checked with SciPy's own Gaussian pdf and adaptive quadrature:
    # every centroid is the conditional mean of its cell, every threshold the midpoint.
    c, t = oracle.lloyd_max_gaussian(bits)
    assert np.allclose(t, 0.5 * (c[:-1] + c[1:]), atol=1e-15, rtol=0)
    edges = [-np.inf] + list(t) + [np.inf]
    for i in range(len(c)):
        a, b = edges[i], edges[i + 1]
        p = stats.norm.cdf(b) - stats.norm.cdf(a) if a < 0 else stats.norm.sf(a) - stats.norm.sf(b)
        m = integrate.quad(lambda x: x * stats.norm.pdf(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(m / p - c[i]) < 1e-10, (bits, i, m / p, c[i])
    # distortion by quadrature against the oracle's closed-form moments
    dq = sum(integrate.quad(lambda x: (x - c[i]) ** 2 * stats.norm.pdf(x), edges[i], edges[i + 1],
                            epsabs=1e-14, epsrel=1e-13)[0] for i in range(len(c)))
    assert abs(dq - oracle.gaussian_distortion(c, t)) < 1e-11


def test_codebook_is_odd_symmetric_with_zero_middle_threshold():
    for bits in (1, 2, 3, 4, 5):
        c, t = oracle.lloyd_max_gaussian(bits)
        assert np.array_equal(c, -c[::-1])
        assert t[len(t) // 2] == 0.0
        assert np.all(np.diff(c) > 0) and np.all(np.diff(t) > 0)


# ----------------------------------------------------------------------- rotation pins

def test_rotation_preserves_norms_and_is_orthogonal():
    # [news]: the rotation must not spoil the geometry (distances, inner products).
    for d in (128, 1536):
        Pi = gen.haar_orthogonal(d, cfg=900)
        P64 = Pi.astype(np.float64)
        assert np.abs(P64.T @ P64 - np.eye(d)).max() <= 1e-6
        x = gen.unit_sphere(64, d, cfg=900, role=gen.ROLE_DATA) * 3.0
        nu, xn, u = oracle.normalize_rotate(x, Pi)
        assert np.allclose(nu, 3.0, rtol=1e-6)
        assert np.abs(np.linalg.norm(u, axis=1) - 1.0).max() <= 1e-6


def test_rotation_orientation_with_explicit_permutation():
    # u = Pi x / nu, not Pi^T x: with a permutation matrix Pi[t, sigma(t)] = 1 the rotated
    # coordinate t must be x[sigma(t)] / nu (a transposed Pi would give x[sigma^-1(t)]).
    d = 8
    sigma = np.array([3, 0, 6, 1, 7, 2, 5, 4])
    Pi = np.zeros((d, d), dtype=np.float32)
    Pi[np.arange(d), sigma] = 1.0
    x = np.arange(1, d + 1, dtype=np.float32)[None, :]
    nu, xn, u = oracle.normalize_rotate(x, Pi)
    assert nu[0] == pytest.approx(math.sqrt(sum(i * i for i in range(1, d + 1))))
    assert np.allclose(u[0], x[0, sigma] / nu[0], rtol=1e-15)
    # 2-D rotation by +30 degrees maps e_1 to (cos, sin)
    th = math.pi / 6
    R = np.array([[math.cos(th), -math.sin(th)], [math.sin(th), math.cos(th)]])
    _, _, u2 = oracle.normalize_rotate(np.array([[2.0, 0.0]]), R)
    assert np.allclose(u2[0], [math.cos(th), math.sin(th)], atol=1e-15)


def test_zero_vector_gets_zero_norm_and_zero_rotation():
    nu, xn, u = oracle.normalize_rotate(np.zeros((2, 4)), np.eye(4))
    assert nu.tolist() == [0.0, 0.0] and not xn.any() and not u.any()


# ----------------------------------------------------------------------- bucketize pins

@pytest.mark.parametrize("d", [2, 3, 4])
@pytest.mark.parametrize("bits", [1, 2, 3])
def test_bucketize_equals_bruteforce_nearest_product_codebook(d, bits):
    # Brute force: the nearest point of the whole product codebook (L^d candidates) must be
    # the per-coordinate threshold decision.  Ties cannot occur for random u.
    c, t = oracle.codebook(bits, d)
    g = np.random.default_rng(1000 * d + bits)
    u = g.standard_normal((40, d)) / math.sqrt(d)
    idx = oracle.bucketize(u, t)
    cands = np.array(list(itertools.product(range(len(c)), repeat=d)))
    pts = c[cands]                                             # [L^d][d]
    for row in range(u.shape[0]):
        dist = np.sum((pts - u[row]) ** 2, axis=1)
        best = cands[np.argmin(dist)]
        assert np.array_equal(best, idx[row])


def test_bucketize_threshold_tie_goes_away_from_zero():
    # Ties keep the quantizer odd: on a positive threshold the upper cell, on a negative one
    # the lower cell (both farther from zero); exactly 0 (either zero) to the positive side.
    c, t = oracle.codebook(3, 128)
    L = len(c)
    on = oracle.bucketize(t[None, :].repeat(1, 0), t)[0]
    for i, tau in enumerate(t):
        expect = i + 1 if tau >= 0 else i
        assert on[i] == expect, (i, tau, on[i])
    below = oracle.bucketize(np.nextafter(t, -np.inf)[None, :], t)[0]
    above = oracle.bucketize(np.nextafter(t, np.inf)[None, :], t)[0]
    assert below.tolist() == list(range(0, L - 1))
    assert above.tolist() == list(range(1, L))
    assert oracle.bucketize(np.array([-0.0]), np.array([0.0]))[0] == 1
    assert oracle.bucketize(np.array([0.0]), np.array([0.0]))[0] == 1


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_bucketize_is_odd_symmetric_including_ties(bits):
    # Q(-u) = -Q(u) for u != 0: index(-u) = L - 1 - index(u), also on every threshold.
    c, t = oracle.codebook(bits, 64)
    g = np.random.default_rng(77 + bits)
    u = np.concatenate([g.standard_normal(500) / 8.0, t[t != 0], -t[t != 0]])
    i_pos = oracle.bucketize(u, t)
    i_neg = oracle.bucketize(-u, t)
    assert np.array_equal(i_neg, len(c) - 1 - i_pos)


def test_bucketize_float32_decision_matches_float64_away_from_thresholds():
    c, t = oracle.codebook(3, 128)
    u = np.random.default_rng(5).standard_normal((2000, 128)) / math.sqrt(128)
    i32 = oracle.bucketize(u, t, decide_dtype=np.float32)
    i64 = oracle.bucketize(u, t)
    near = np.min(np.abs(u[..., None] - t), axis=-1) <= 1e-7
    assert np.array_equal(i32[~near], i64[~near])


# -------------------------------------------------------------------- residual / gamma

def test_gamma_closed_form_one_bit():
    # b = 2: chat_t = sign(u_t) c0/sqrt(d), c0 = sqrt(2/pi), so
    # gamma^2 = |u - chat|^2 = 1 - 2 c0/sqrt(d) sum|u_t| + c0^2   (rotation keeps norms).
    d = 128
    Pi = gen.haar_orthogonal(d, cfg=901)
    S = gen.gaussian_matrix(d, d, cfg=901)
    c, t = oracle.codebook(1, d)
    x = gen.unit_sphere(200, d, cfg=901, role=gen.ROLE_DATA) * 5.0
    res = oracle.quantize(x, Pi, S, c, t)
    c0 = math.sqrt(2 / math.pi)
    expect = 1 - 2 * c0 / math.sqrt(d) * np.abs(res["u"]).sum(axis=1) + c0 * c0
    assert np.allclose(res["gamma"] ** 2, expect, atol=2e-6, rtol=0)


@pytest.mark.parametrize("b,expect", [(2, 0.36089), (3, 0.11601), (4, 0.03398)])
def test_mean_gamma_squared_is_sphere_distortion(b, expect):
    # E[gamma^2] = d E[(u_1 - Q(u_1))^2] with u_1 a sphere coordinate (quadrature, and the
    # value recomputed here); the sample mean over 4000 vectors must lie within 5 SE.
    d = 128
    kappa, dist = _sphere_expectations(d, b - 1)
    assert abs(dist - expect) < 2e-5
    Pi = gen.haar_orthogonal(d, cfg=902)
    S = gen.gaussian_matrix(d, d, cfg=902)
    c, t = oracle.codebook(b - 1, d)
    x = gen.unit_sphere(4000, d, cfg=902, role=gen.ROLE_DATA)
    g2 = oracle.quantize(x, Pi, S, c, t)["gamma"] ** 2
    se = g2.std(ddof=1) / math.sqrt(len(g2))
    assert abs(g2.mean() - dist) < 5 * se


# ---------------------------------------------------------------------------- QJL pins

def test_qjl_signs_special_case_identity_matrices():
    # With Pi = S = I the sign bits are those of x/nu - chat, coordinate by coordinate.
    d = 64
    c, t = oracle.codebook(2, d)
    x = gen.unit_sphere(50, d, cfg=903, role=gen.ROLE_DATA) * 2.0
    eye = np.eye(d, dtype=np.float32)
    res = oracle.quantize(x, eye, eye, c, t)
    xn = x.astype(np.float64) / np.linalg.norm(x.astype(np.float64), axis=1, keepdims=True)
    chat = c[oracle.bucketize(xn, t)]
    assert np.array_equal(res["z"], (xn - chat >= 0).astype(np.int64))
    assert np.allclose(res["gamma"], np.linalg.norm(xn - chat, axis=1), rtol=1e-15)


def test_qjl_uses_S_rows_not_columns():
    # A non-symmetric S with one nonzero entry per row: y_i = S[i, j(i)] r_j(i).
    d = 4
    S = np.zeros((d, d))
    S[0, 2], S[1, 0], S[2, 3], S[3, 1] = 2.0, -1.0, 1.0, -3.0
    r = np.array([[0.5, -0.25, 0.125, -2.0]])
    y, z = oracle.qjl_signs(S, r)
    assert np.allclose(y[0], [0.25, -0.5, -2.0, 0.75])
    assert z[0].tolist() == [1, 0, 0, 1]
    _, z0 = oracle.qjl_signs(np.eye(1), np.array([[-0.0]]))
    assert z0[0, 0] == 1                                     # sign(0) counts as +1


# ----------------------------------------------------------------------- estimator pins

def _setup(d=64, b=3, n=300, nq=5, cfg=904, rep=0, scale=1.0):
    Pi = gen.haar_orthogonal(d, cfg=cfg, rep=rep)
    S = gen.gaussian_matrix(d, d, cfg=cfg, rep=rep)
    c, t = oracle.codebook(b - 1, d)
    x = gen.unit_sphere(n, d, cfg=cfg, role=gen.ROLE_DATA) * scale
    q = gen.unit_sphere(nq, d, cfg=cfg, role=gen.ROLE_QUERY) * 1.7
    return Pi, S, c, t, x, q


@pytest.mark.parametrize("mode", ["prod", "mse"])
def test_estimator_equals_inner_product_with_dequantized_vector(mode):
    # <q, x~> computed from the reconstruction must equal the direct estimate.
    Pi, S, c, t, x, q = _setup(scale=3.0)
    r = oracle.quantize(x, Pi, S, c, t)
    est = oracle.estimate_ip(q, Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c, mode)
    xt = oracle.dequantize(Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c, mode)
    ref = q.astype(np.float64) @ xt.T
    assert np.allclose(est, ref, rtol=1e-12, atol=1e-12)


def test_prod_estimator_is_unbiased_over_S_for_fixed_rotation():
    # E_S[estimate] = <q, x> exactly for any rotation; the variance over S is
    # (pi/2) nu^2 gamma^2 / m (|q|^2 - (2/pi) <q, r/gamma>^2).  A wrong QJL scale, sign,
    # residual or transposed S shifts the mean or the variance.
    d, b, N = 32, 3, 6000
    Pi = gen.haar_orthogonal(d, cfg=905)
    c, t = oracle.codebook(b - 1, d)
    x = gen.unit_sphere(1, d, cfg=905, role=gen.ROLE_DATA) * 2.5
    q0 = gen.unit_sphere(1, d, cfg=905, role=gen.ROLE_QUERY)
    # query with cosine 0.6 to x
    xh = x[0] / np.linalg.norm(x[0])
    perp = q0[0] - (q0[0] @ xh) * xh
    perp /= np.linalg.norm(perp)
    q = (0.6 * xh + 0.8 * perp)[None, :] * 1.3
    truth = float(q[0].astype(np.float64) @ x[0].astype(np.float64))
    ests = np.empty(N)
    for s in range(N):
        S = gen.gaussian_matrix(d, d, cfg=905, rep=s)
        r = oracle.quantize(x, Pi, S, c, t)
        ests[s] = oracle.estimate_ip(q, Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c)[0, 0]
    se = ests.std(ddof=1) / math.sqrt(N)
    assert abs(ests.mean() - truth) < 4 * se, (ests.mean(), truth, se)
    # predicted variance (nu, gamma, r do not depend on S)
    r0 = oracle.quantize(x, Pi, gen.gaussian_matrix(d, d, cfg=905), c, t)
    nu, gamma = r0["nu"][0], r0["gamma"][0]
    _, xn, _ = oracle.normalize_rotate(x, Pi)
    resid, _ = oracle.residual(xn, Pi, c[r0["idx"]])
    rho = resid[0] / gamma
    q64 = q[0].astype(np.float64)
    var = (math.pi / 2) * nu ** 2 * gamma ** 2 / d * (q64 @ q64 - (2 / math.pi) * (q64 @ rho) ** 2)
    assert abs(ests.var(ddof=1) / var - 1.0) < 0.08


@pytest.mark.parametrize("d,b", [(2, 2), (16, 2), (16, 3)])
def test_mse_only_estimator_is_biased_by_kappa(d, b):
    # Averaged over Haar rotations, E[nu <Pi q, chat>] = kappa <q, x> with
    # kappa = d E[u_1 Q(u_1)] (sphere quadrature); d = 2, 1 bit: kappa = 4 / pi^(3/2).
    # [review, experiments] / [news, bias paragraph]: the MSE quantizer is biased.
    kappa, _ = _sphere_expectations(d, b - 1)
    if d == 2 and b == 2:
        assert abs(kappa - 4 / math.pi ** 1.5) < 1e-10
    N = 6000
    c, t = oracle.codebook(b - 1, d)
    x = gen.unit_sphere(1, d, cfg=906, role=gen.ROLE_DATA) * 1.5
    q = gen.unit_sphere(1, d, cfg=906, role=gen.ROLE_QUERY)
    q = q + 0.8 * x / 1.5
    truth = float(q[0].astype(np.float64) @ x[0].astype(np.float64))
    S = gen.gaussian_matrix(d, d, cfg=906)
    mse = np.empty(N)
    prod = np.empty(N)
    for s in range(N):
        Pi = gen.haar_orthogonal(d, cfg=906, rep=s)
        S = gen.gaussian_matrix(d, d, cfg=906, rep=s)
        r = oracle.quantize(x, Pi, S, c, t)
        args = (q, Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c)
        mse[s] = oracle.estimate_ip(*args, mode="mse")[0, 0]
        prod[s] = oracle.estimate_ip(*args, mode="prod")[0, 0]
    se_m = mse.std(ddof=1) / math.sqrt(N)
    se_p = prod.std(ddof=1) / math.sqrt(N)
    assert abs(mse.mean() - kappa * truth) < 4 * se_m, (mse.mean(), kappa * truth, se_m)
    assert abs(mse.mean() - truth) > 4 * se_m                 # biased
    assert abs(prod.mean() - truth) < 4 * se_p                # unbiased


def test_estimator_scales_with_key_norm_and_handles_zero_keys():
    Pi, S, c, t, x, q = _setup(n=20)
    x2 = x.copy()
    x2[3] = 0.0
    r1 = oracle.quantize(x2, Pi, S, c, t)
    r5 = oracle.quantize(x2 * 5.0, Pi, S, c, t)
    e1 = oracle.estimate_ip(q, Pi, S, r1["idx"], r1["z"], r1["nu"], r1["gamma"], c)
    e5 = oracle.estimate_ip(q, Pi, S, r5["idx"], r5["z"], r5["nu"], r5["gamma"], c)
    assert np.array_equal(r1["idx"], r5["idx"]) and np.array_equal(r1["z"], r5["z"])
    assert np.allclose(e5, 5.0 * e1, rtol=1e-6)
    assert np.all(e1[:, 3] == 0.0)
    assert np.all(oracle.dequantize(Pi, S, r1["idx"], r1["z"], r1["nu"], r1["gamma"], c)[3] == 0)


# -------------------------------------------------------------------------- layout pins

def test_pack_layout_hand_built():
    d, b = 64, 4
    idx = np.zeros((1, d), dtype=np.int64)
    z = np.zeros((1, d), dtype=np.int64)
    idx[0, 37] = 5                   # bits 0 and 2 of coordinate 37: group 1, bit 5
    idx[0, 0] = 2                    # bit 1 of coordinate 0: group 0, bit 0
    z[0, 31] = 1                     # sign of coordinate 31: group 0, bit 31
    z[0, 63] = 1
    codes = oracle.pack_codes(idx, z, b)
    assert codes.shape == (1, 2, 4) and codes.dtype == np.uint32
    assert codes[0, 0].tolist() == [0, 1, 0, 1 << 31]
    assert codes[0, 1].tolist() == [1 << 5, 0, 1 << 5, 1 << 31]
    i2, z2 = oracle.unpack_codes(codes, b)
    assert np.array_equal(i2, idx) and np.array_equal(z2, z)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_pack_roundtrip_random(b):
    g = np.random.default_rng(b)
    idx = g.integers(0, 1 << (b - 1), size=(17, 128))
    z = g.integers(0, 2, size=(17, 128))
    i2, z2 = oracle.unpack_codes(oracle.pack_codes(idx, z, b), b)
    assert np.array_equal(i2, idx) and np.array_equal(z2, z)


# ----------------------------------------------------------------------------- top-k pin

def test_topk_matches_python_sort_with_index_tiebreak():
    g = np.random.default_rng(7)
    s = np.round(g.standard_normal((6, 300)), 1)           # many exact ties
    ids, vals = oracle.topk(s, 10, index_offset=1000)
    for a in range(6):
        ref = sorted(range(300), key=lambda j: (-s[a, j], j))[:10]
        assert ids[a].tolist() == [j + 1000 for j in ref]
        assert vals[a].tolist() == [s[a, j] for j in ref]


# ------------------------------------------------------- value quantizer and attention pins

@pytest.mark.parametrize("b,expect", [(2, 0.36089), (3, 0.11601), (4, 0.03398)])
def test_mse_value_reconstruction_error_is_sphere_distortion(b, expect):
    # |x - v~|^2 for unit x equals |u - chat|^2 (the rotation keeps norms), whose mean is
    # the sphere distortion of the (b-1)-bit Lloyd-Max quantizer (same quadrature values as
    # the gamma pin); a transposed Pi in dequantize_mse or a wrong centroid index fails it.
    d = 128
    Pi = gen.haar_orthogonal(d, cfg=905)
    c, t = oracle.codebook(b - 1, d)
    x = gen.unit_sphere(4000, d, cfg=905, role=gen.ROLE_DATA).astype(np.float64)
    r = oracle.quantize_mse(x * 2.5, Pi, c, t)
    assert np.allclose(r["nu"], 2.5, rtol=1e-6)
    v = oracle.dequantize_mse(Pi, r["idx"], r["nu"], c) / 2.5
    e2 = np.sum((x - v) ** 2, axis=1)
    se = e2.std(ddof=1) / math.sqrt(len(e2))
    assert abs(e2.mean() - expect) < 5 * se + 2e-5


def test_mse_value_index_matches_prod_encoder_index():
    # the MSE stage of the inner-product encoder is the same bucketization
    Pi, S, c, t, x, _ = _setup(d=64, b=4, n=200, cfg=906, scale=0.7)
    assert np.array_equal(oracle.quantize_mse(x, Pi, c, t)["idx"], oracle.quantize(x, Pi, S, c, t)["idx"])


def test_index_planes_hand_built_and_roundtrip():
    idx = np.zeros((1, 64), dtype=np.int64)
    idx[0, 37] = 5                   # bits 0 and 2 of coordinate 37: word 1, bit 5
    idx[0, 0] = 2                    # bit 1 of coordinate 0: word 0, bit 0
    idx[0, 63] = 7
    codes = oracle.pack_index_planes(idx, 3)
    assert codes.shape == (1, 2, 3) and codes.dtype == np.uint32
    assert codes[0, 0].tolist() == [0, 1, 0]
    assert codes[0, 1].tolist() == [(1 << 5) | (1 << 31), 1 << 31, (1 << 5) | (1 << 31)]
    g = np.random.default_rng(11)
    r = g.integers(0, 8, size=(9, 128))
    assert np.array_equal(oracle.unpack_index_planes(oracle.pack_index_planes(r, 3), 3), r)


def test_attention_constant_logits_give_the_mean_value():
    g = np.random.default_rng(12)
    vals = g.standard_normal((2, 37, 16))
    logits = np.full((2, 3, 37), 4.25)
    out = oracle.attention_decode(logits, vals, scale=0.3)
    for h in range(3):
        assert np.allclose(out[:, h], vals.mean(axis=1), rtol=1e-13, atol=1e-13)


def test_attention_single_key_and_dominant_key():
    g = np.random.default_rng(13)
    vals = g.standard_normal((1, 1, 8))
    assert np.allclose(oracle.attention_decode(g.standard_normal((1, 2, 1)), vals, 1.0)[0],
                       vals[0, 0], rtol=0, atol=0)
    vals = g.standard_normal((1, 50, 8))
    logits = g.standard_normal((1, 1, 50))
    logits[0, 0, 17] = 5.0
    out = oracle.attention_decode(logits, vals, scale=200.0)   # exp(-200 * gap) vanishes
    assert np.allclose(out[0, 0], vals[0, 17], rtol=0, atol=1e-12)


def test_attention_brute_force_tiny_and_shift_invariance():
    # pure-Python softmax sums on a tiny case; adding a constant per head changes nothing
    g = np.random.default_rng(14)
    vals = g.standard_normal((2, 5, 3))
    logits = g.standard_normal((2, 2, 5)) * 3.0
    scale = 0.7
    out = oracle.attention_decode(logits, vals, scale)
    for gi in range(2):
        for h in range(2):
            w = [math.exp(scale * float(logits[gi, h, t])) for t in range(5)]
            tot = sum(w)
            for c in range(3):
                ref = sum(w[t] * float(vals[gi, t, c]) for t in range(5)) / tot
                assert abs(out[gi, h, c] - ref) < 1e-12
    shifted = logits + np.array([[[100.0], [-40.0]], [[3.0], [0.5]]])
    assert np.allclose(oracle.attention_decode(shifted, vals, scale), out, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ variants: sphere codebook

@pytest.mark.parametrize("bits", [1, 2, 3])
def test_sphere_codebook_is_uniform_grid_at_d3(bits):
    # In R^3 a coordinate of a uniform unit vector is uniform on [-1, 1] (Archimedes), and the
    # Lloyd-Max quantizer of a uniform law is the uniform grid of cell midpoints.
    L = 1 << bits
    c, t = oracle.codebook_sphere(bits, 3)
    np.testing.assert_allclose(c, [-1 + (2 * i + 1) / L for i in range(L)], atol=1e-9)
    np.testing.assert_allclose(t, [-1 + 2 * (i + 1) / L for i in range(L - 1)], atol=1e-9)


@pytest.mark.parametrize("d,bits", [(4, 2), (16, 3), (128, 3), (64, 2)])
def test_sphere_codebook_is_a_fixed_point_by_quadrature(d, bits):
    # both Lloyd-Max conditions, with the cell means by numerical integration of the sphere
    # marginal density (independent of the incomplete-beta and closed-form moments)
    c, t = oracle.codebook_sphere(bits, d)
    np.testing.assert_allclose(t, 0.5 * (c[:-1] + c[1:]), rtol=0, atol=1e-15)
    f = _sphere_marginal_pdf(d)
    edges = [-1.0] + list(t) + [1.0]
    for i in range(len(c)):
        mass = integrate.quad(f, edges[i], edges[i + 1], epsabs=1e-14, epsrel=1e-13)[0]
        mom = integrate.quad(lambda x: x * f(x), edges[i], edges[i + 1], epsabs=1e-14,
                             epsrel=1e-13)[0]
        assert abs(mom / mass - c[i]) < 1e-9, (i, mom / mass, c[i])


@pytest.mark.parametrize("d", [3, 7, 64, 1000])
def test_sphere_cell_functions_against_quadrature(d):
    f = _sphere_marginal_pdf(d)
    assert abs(oracle.sphere_cell_prob(-1.0, 1.0, d) - 1.0) < 1e-14
    for a, b in [(-0.3, 0.1), (0.05, 0.2), (-1.0, -0.01), (0.5, 1.0)]:
        p = integrate.quad(f, a, b, epsabs=1e-14, epsrel=1e-13)[0]
        m = integrate.quad(lambda x: x * f(x), a, b, epsabs=1e-14, epsrel=1e-13)[0]
        assert abs(oracle.sphere_cell_prob(a, b, d) - p) < 1e-11
        assert abs(oracle.sphere_cell_moment(a, b, d) - m) < 1e-11


@pytest.mark.parametrize("bits", [1, 2, 3])
def test_sphere_codebook_tends_to_scaled_gaussian(bits):
    # the sphere marginal tends to N(0, 1/d); the gap in sigma units shrinks like 1/d
    gaps = []
    for d in (256, 4096):
        cs, _ = oracle.codebook_sphere(bits, d)
        cg, _ = oracle.codebook(bits, d)
        gaps.append(np.max(np.abs(cs - cg)) * math.sqrt(d))
    assert gaps[1] < 3.0 / 4096
    assert 15.0 < gaps[0] / gaps[1] < 17.0


@pytest.mark.parametrize("d", [2, 3, 5, 64, 1536])
def test_sphere_one_bit_centroid_is_mean_absolute_coordinate(d):
    # with two cells split at 0 the centroid is E[u | u > 0] = E|w_1|
    # = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)), which the orthogonal QJL scale also uses
    ew = math.exp(math.lgamma(d / 2) - math.lgamma((d + 1) / 2)) / math.sqrt(math.pi)
    c, t = oracle.codebook_sphere(1, d)
    assert t[0] == 0.0
    assert abs(c[1] - ew) < 1e-12 and c[0] == -c[1]


@pytest.mark.parametrize("d,bits", [(3, 2), (8, 2), (32, 3)])
def test_sphere_codebook_has_lower_distortion_on_the_sphere(d, bits):
    # optimal for the exact law, so its mean squared error on sphere coordinates is below the
    # Gaussian-approximation codebook's (Monte Carlo with one shared sample)
    u = gen.unit_sphere(20000, d, cfg=931, role=gen.ROLE_DATA).astype(np.float64).ravel()

    def mse(c, t):
        return float(np.mean((u - c[np.searchsorted(t, u, side="right")]) ** 2))
    cs, ts = oracle.codebook_sphere(bits, d)
    cg, tg = oracle.codebook(bits, d)
    assert mse(cs, ts) < mse(cg, tg)


# ------------------------------------------------------------------ variants: orthogonal QJL

@pytest.mark.parametrize("d,expect", [(2, 2.0 / math.pi), (3, 0.5), (4, 4.0 / (3.0 * math.pi))])
def test_orthogonal_qjl_scale_closed_forms(d, expect):
    # E|w_1| for a uniform unit vector: 2/pi on the circle, 1/2 in R^3 (uniform coordinate),
    # 4/(3 pi) in R^4; alpha = 1 / (m E|w_1|)
    assert abs(oracle.qjl_alpha_orthogonal(5, d) - 1.0 / (5 * expect)) < 1e-14
    f = _sphere_marginal_pdf(d) if d > 2 else None
    if f is not None:
        ew = 2 * integrate.quad(lambda x: x * f(x), 0, 1, epsabs=1e-14)[0]
        assert abs(ew - expect) < 1e-10


def test_orthogonal_qjl_estimator_is_unbiased_over_S():
    # every row of a Haar orthogonal S is a uniform unit vector, so with alpha = 1/(m E|w_1|)
    # the estimate is unbiased over S; the Gaussian scale on these unit rows would be off by
    # a factor of about sqrt(d), a transposed S or a wrong sign shifts the mean too
    d, b, N = 32, 3, 4000
    Pi = gen.haar_orthogonal(d, cfg=907)
    c, t = oracle.codebook_sphere(b - 1, d)
    x = gen.unit_sphere(1, d, cfg=907, role=gen.ROLE_DATA) * 1.7
    q0 = gen.unit_sphere(1, d, cfg=907, role=gen.ROLE_QUERY)
    xh = x[0] / np.linalg.norm(x[0])
    perp = q0[0] - (q0[0] @ xh) * xh
    perp /= np.linalg.norm(perp)
    q = (0.5 * xh + math.sqrt(0.75) * perp)[None, :] * 0.9
    truth = float(q[0].astype(np.float64) @ x[0].astype(np.float64))
    alpha = oracle.qjl_alpha_orthogonal(d, d)
    ests = np.empty(N)
    for s in range(N):
        S = gen.haar_orthogonal(d, cfg=907, rep=s + 1, role=gen.ROLE_S)
        r = oracle.quantize(x, Pi, S, c, t)
        ests[s] = oracle.estimate_ip(q, Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c,
                                     alpha=alpha)[0, 0]
    se = ests.std(ddof=1) / math.sqrt(N)
    assert abs(ests.mean() - truth) < 4 * se, (ests.mean(), truth, se)
    # variance below the Gaussian S's (predicted in closed form, as in the Gaussian test):
    # orthonormal rows do not repeat directions, so the signs carry more of <q, r>
    nu, gamma = r["nu"][0], r["gamma"][0]
    _, xn, _ = oracle.normalize_rotate(x, Pi)
    resid, _ = oracle.residual(xn, Pi, c[r["idx"]])
    q64 = q[0].astype(np.float64)
    rho = resid[0] / gamma
    var_gauss = (math.pi / 2) * nu ** 2 * gamma ** 2 / d * (q64 @ q64 - (2 / math.pi) * (q64 @ rho) ** 2)
    assert ests.var(ddof=1) < 0.8 * var_gauss, (ests.var(ddof=1), var_gauss)
    # the same S used through dequantize gives the same numbers
    r = oracle.quantize(x, Pi, S, c, t)
    xh_ = oracle.dequantize(Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c, alpha=alpha)
    assert abs(float(q[0].astype(np.float64) @ xh_[0]) - ests[-1]) < 1e-9


# -------------------------------------------------------- fractional rates: channel groups

def _split_groups(d_a, b_a, d_b, b_b, cfg, rep=0):
    gs = []
    for k, (off, w, b) in enumerate(((0, d_a, b_a), (d_a, d_b, b_b))):
        if w == 0:
            continue
        c, t = oracle.codebook(b - 1, w)
        gs.append({"off": off, "width": w, "b": b, "Pi": gen.haar_orthogonal(w, cfg + k, rep),
                   "S": gen.gaussian_matrix(w, w, cfg + k, rep), "centroids": c, "thresholds": t})
    return gs


def test_split_with_one_group_is_the_plain_quantizer():
    d, b = 32, 3
    x = gen.unit_sphere(50, d, cfg=940, role=gen.ROLE_DATA) * 2.0
    q = gen.unit_sphere(4, d, cfg=940, role=gen.ROLE_QUERY)
    g = _split_groups(d, b, 0, 2, 940)
    r = oracle.quantize_split(x, g)[0]
    r0 = oracle.quantize(x, g[0]["Pi"], g[0]["S"], g[0]["centroids"], g[0]["thresholds"])
    assert np.array_equal(r["idx"], r0["idx"]) and np.array_equal(r["z"], r0["z"])
    e = oracle.estimate_ip_split(q, g, [r])
    e0 = oracle.estimate_ip(q, g[0]["Pi"], g[0]["S"], r0["idx"], r0["z"], r0["nu"], r0["gamma"],
                            g[0]["centroids"])
    assert np.array_equal(e, e0)


@pytest.mark.parametrize("mode", ["prod", "mse"])
def test_split_estimate_is_inner_product_with_concatenated_reconstruction(mode):
    # each group reconstructs its own channels; the split estimate is <q, [xhat_A; xhat_B]>
    x = gen.unit_sphere(40, 24, cfg=941, role=gen.ROLE_DATA) * 1.5
    q = gen.unit_sphere(3, 24, cfg=941, role=gen.ROLE_QUERY)
    g = _split_groups(16, 4, 8, 2, 941)
    codes = oracle.quantize_split(x, g)
    xhat = np.concatenate([oracle.dequantize(gg["Pi"], gg["S"], c["idx"], c["z"], c["nu"], c["gamma"],
                                             gg["centroids"], mode) for gg, c in zip(g, codes)], axis=1)
    est = oracle.estimate_ip_split(q, g, codes, mode)
    np.testing.assert_allclose(est, q.astype(np.float64) @ xhat.T, rtol=0, atol=1e-12)
    # the groups see only their own channels: changing group B's channels leaves group A's codes
    x2 = x.copy()
    x2[:, 16:] *= -3.0
    c2 = oracle.quantize_split(x2, g)
    assert np.array_equal(c2[0]["idx"], codes[0]["idx"]) and np.array_equal(c2[0]["z"], codes[0]["z"])


def test_split_estimate_is_unbiased_over_both_instances():
    # 2.5 bits per channel on 16 channels: 8 at b = 3, 8 at b = 2
    d, N = 16, 3000
    x = gen.unit_sphere(1, d, cfg=942, role=gen.ROLE_DATA) * 2.0
    q = gen.unit_sphere(1, d, cfg=942, role=gen.ROLE_QUERY) * 1.2
    truth = float(q[0].astype(np.float64) @ x[0].astype(np.float64))
    ests = np.empty(N)
    for s in range(N):
        g = _split_groups(8, 3, 8, 2, 942, rep=s)
        ests[s] = oracle.estimate_ip_split(q, g, oracle.quantize_split(x, g))[0, 0]
    se = ests.std(ddof=1) / math.sqrt(N)
    assert abs(ests.mean() - truth) < 4 * se, (ests.mean(), truth, se)


def test_split_mse_distortion_is_the_sum_of_the_groups():
    # MSE-only reconstruction over Haar rotations: E|x - xhat|^2 = sum_g nu_g^2 D(d_g, b_g - 1),
    # D from the sphere law by quadrature; groups at different norms and bit widths, so a group
    # run at the other's codebook or bit width moves the mean by many SE
    d_a, d_b, N = 8, 8, 3000
    xa = gen.unit_sphere(1, d_a, cfg=943, role=gen.ROLE_DATA) * 3.0
    xb = gen.unit_sphere(1, d_b, cfg=944, role=gen.ROLE_DATA) * 1.0
    x = np.concatenate([xa, xb], axis=1)
    errs = np.empty(N)
    for s in range(N):
        g = _split_groups(d_a, 4, d_b, 2, 943, rep=s)
        codes = oracle.quantize_split(x, g)
        xhat = np.concatenate([oracle.dequantize(gg["Pi"], gg["S"], c["idx"], c["z"], c["nu"], c["gamma"],
                                                 gg["centroids"], "mse") for gg, c in zip(g, codes)], axis=1)
        errs[s] = float(np.sum((x[0].astype(np.float64) - xhat[0]) ** 2))
    expect = 9.0 * _sphere_expectations(d_a, 3)[1] + 1.0 * _sphere_expectations(d_b, 1)[1]
    se = errs.std(ddof=1) / math.sqrt(N)
    assert abs(errs.mean() - expect) < 4 * se, (errs.mean(), expect, se)
