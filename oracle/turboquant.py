"""Plain, slow, float64 CPU oracle of the TurboQuant quantize / inner-product path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares no code,
table or constant with the HIP library (``kv_cache_embedding_amd``) and imports nothing
from it; the two meet only in the seeded input arrays of ``workloads``.

Sources (web pages; cited by short name and the passage on the page):
  [review]    TurboQuant paper review, quant_prune_distill channel (tgviewer.app, post 674)
  [news]      "Google ускоряет LLM в 8 раз" (comuna.ru, post 6696)
  [explainer] "TurboQuant: Redefining AI efficiency with extreme compression"
              (RecSysChannel, tgstat.ru, post 256)
  [tldr]      TurboQuant two-step TLDR, seeallochnaya channel (postsniper.ru, post 3476)

The pages give the method in prose only.  Readings taken where they are silent:
  * the codebook is Lloyd-Max for N(0, 1/d) (coordinates of a rotated unit vector are
    "almost normal"), with L = 2**(b-1) levels for a total budget of b bits;
  * a coordinate lying exactly on a threshold goes to the cell farther from zero, and a
    coordinate equal to 0 to the positive side: the quantizer of the symmetric law stays odd,
    Q(-u) = -Q(u), at ties too;
  * the QJL matrix S is Gaussian N(0, 1) with m = d rows, separate from the rotation;
  * the QJL scale is sqrt(pi/2)/m times the residual norm gamma (the value that makes the
    estimate exactly unbiased: E|<s, r/|r|>| sign terms average sqrt(2/pi)|r|);
  * sign(0) is +1 (z = [y >= 0]);
  * vectors are normalised and their norm nu is stored next to gamma (no other constant);
  * integer decisions (bucket index, sign bit) are taken in float64 on the float64 values
    (the pages fix no precision; a decision within rounding of a threshold is what the
    parity tests excuse);
  * variants ([review, QJL paragraph]: an orthogonal QJL matrix; the exact sphere law of a
    rotated coordinate): codebook_sphere is Lloyd-Max on that law, and an orthogonal S
    takes the scale 1/(m E|w_1|);
  * decode attention: values are quantized by the MSE stage alone (index and nu, no QJL
    bit: they are reconstructed, not inner-producted) and the softmax is over the raw
    estimated logits times a caller-given scale;
  * fractional rates ([review, experiments paragraph] and [news, results paragraph]: 2.5 and
    3.5 bits per channel, mechanism not given): two channel groups, each its own TurboQuant
    instance (rotation, QJL matrix, nu, gamma) at its own b, the estimate being the sum of
    the groups' estimates; half the channels at b + 1 and half at b give b + 1/2.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "gauss_cell_prob", "gauss_cell_mean", "lloyd_max_gaussian", "gaussian_distortion",
    "codebook", "normalize_rotate", "bucketize", "residual", "qjl_signs", "quantize",
    "pack_codes", "unpack_codes", "estimate_ip", "dequantize", "topk", "qjl_alpha",
    "quantize_mse", "pack_index_planes", "unpack_index_planes", "dequantize_mse",
    "attention_decode", "sphere_cell_prob", "sphere_cell_moment", "codebook_sphere",
    "qjl_alpha_orthogonal", "quantize_split", "estimate_ip_split",
]

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


# ------------------------------------------------------------------------ codebook
# [review, MSE paragraph]: after the random rotation an optimal scalar grid is fitted with
# the Max-Lloyd algorithm for the target bit width.  [tldr, step 1]: the grid is a 1-D
# k-means solved in advance for the known bell-shaped coordinate law, denser in the centre.
# [explainer, step 1]: the optimal thresholds are computed once, ahead of time.

def _phi(t: float) -> float:
    if math.isinf(t):
        return 0.0
    return _INV_SQRT_2PI * math.exp(-0.5 * t * t)


def gauss_cell_prob(a: float, b: float) -> float:
    """P(a < X < b) for X ~ N(0, 1), written to keep tail cells accurate."""
    if a >= 0.0:
        return 0.5 * (math.erfc(a / _SQRT2) - math.erfc(b / _SQRT2))
    if b <= 0.0:
        return 0.5 * (math.erfc(-b / _SQRT2) - math.erfc(-a / _SQRT2))
    return 0.5 * (math.erf(b / _SQRT2) - math.erf(a / _SQRT2))


def gauss_cell_mean(a: float, b: float) -> float:
    """E[X | a < X < b] for X ~ N(0, 1): (phi(a) - phi(b)) / P(a < X < b)."""
    return (_phi(a) - _phi(b)) / gauss_cell_prob(a, b)


def lloyd_max_gaussian(bits: int, tol: float = 1e-14, max_iter: int = 200000):
    """Lloyd-Max quantizer for N(0, 1) with 2**bits levels.

    Alternates the two optimality conditions until the centroids move by less than
    ``tol``: every threshold is the midpoint of its two neighbouring centroids, and every
    centroid is the mean of the density over its cell.  Starts from a symmetric grid, and
    symmetrises the result exactly, so the middle threshold is exactly 0.0.

    Returns (centroids[L] ascending, thresholds[L-1] ascending), in units of sigma = 1.
    """
    L = 1 << bits
    c = [(-(L - 1) + 2.0 * i) / L * 2.0 for i in range(L)]
    for _ in range(max_iter):
        t = [0.5 * (c[i] + c[i + 1]) for i in range(L - 1)]
        edges = [-math.inf] + t + [math.inf]
        new_c = [gauss_cell_mean(edges[i], edges[i + 1]) for i in range(L)]
        delta = max(abs(new_c[i] - c[i]) for i in range(L))
        c = new_c
        if delta < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max did not converge")
    c = np.array(c, dtype=np.float64)
    c = 0.5 * (c - c[::-1])                     # exact odd symmetry
    t = 0.5 * (c[:-1] + c[1:])
    return c, t


def gaussian_distortion(centroids: np.ndarray, thresholds: np.ndarray) -> float:
    """E[(X - Q(X))^2] for X ~ N(0, 1) under the given quantizer (sigma = 1 units)."""
    edges = [-math.inf] + list(thresholds) + [math.inf]
    total = 0.0
    for i, c in enumerate(centroids):
        a, b = edges[i], edges[i + 1]
        p = gauss_cell_prob(a, b)
        m1 = _phi(a) - _phi(b)                  # integral of x phi(x) over the cell
        # integral of x^2 phi(x) = P + a phi(a) - b phi(b)   (with x phi(x) -> 0 at +-inf)
        ea = 0.0 if math.isinf(a) else a * _phi(a)
        eb = 0.0 if math.isinf(b) else b * _phi(b)
        m2 = p + ea - eb
        total += m2 - 2.0 * c * m1 + c * c * p
    return total


def sphere_cell_prob(a: float, b: float, d: int) -> float:
    """P(a < u < b) for u one coordinate of a uniform point of the unit sphere in R^d.

    u^2 ~ Beta(1/2, (d-1)/2), so P(|u| < t) is the regularized incomplete beta function
    I_{t^2}(1/2, (d-1)/2) (taken from SciPy as a library primitive)."""
    from scipy.special import betainc

    def cdf(t):
        if t <= -1.0:
            return 0.0
        if t >= 1.0:
            return 1.0
        half = 0.5 * float(betainc(0.5, 0.5 * (d - 1), t * t))
        return 0.5 + half if t >= 0.0 else 0.5 - half
    return cdf(b) - cdf(a)


def sphere_cell_moment(a: float, b: float, d: int) -> float:
    """Integral of u f(u) over (a, b), f the sphere marginal density
    f(u) = Gamma(d/2) / (sqrt(pi) Gamma((d-1)/2)) (1 - u^2)^((d-3)/2): the antiderivative of
    u (1 - u^2)^((d-3)/2) is -(1 - u^2)^((d-1)/2) / (d - 1)."""
    logc = math.lgamma(0.5 * d) - math.lgamma(0.5 * (d - 1)) - 0.5 * math.log(math.pi)

    def g(t):
        t = min(max(t, -1.0), 1.0)
        return 0.0 if abs(t) >= 1.0 else math.exp(0.5 * (d - 1) * math.log1p(-t * t))
    return math.exp(logc) * (g(a) - g(b)) / (d - 1)


def codebook_sphere(bits_mse: int, d: int, tol: float | None = None, max_iter: int = 200000):
    """Lloyd-Max quantizer with 2**bits_mse levels for the exact law of a rotated coordinate
    of a unit vector in R^d (the sphere marginal, which the Gaussian N(0, 1/d) approximates):
    the same two optimality conditions as lloyd_max_gaussian, iterated from the scaled
    Gaussian grid (from the uniform grid when that one reaches past 0.9), then symmetrised
    exactly.  Stops once no centroid moves by more than ``tol`` (default 1e-14 / sqrt(d), the
    noise floor of the incomplete-beta masses).  Returns (centroids, thresholds) in the units
    of u."""
    if tol is None:
        tol = 1e-14 / math.sqrt(d)
    g, _ = lloyd_max_gaussian(bits_mse)
    L = 1 << bits_mse
    if g[-1] / math.sqrt(d) < 0.9:
        c = list(g / math.sqrt(d))                        # near the Gaussian limit
    else:
        c = [-1.0 + (2 * i + 1) / L for i in range(L)]    # broad law (small d): uniform start
    for _ in range(max_iter):
        t = [0.5 * (c[i] + c[i + 1]) for i in range(L - 1)]
        edges = [-1.0] + t + [1.0]
        new_c = [sphere_cell_moment(edges[i], edges[i + 1], d) / sphere_cell_prob(edges[i], edges[i + 1], d)
                 for i in range(L)]
        delta = max(abs(new_c[i] - c[i]) for i in range(L))
        c = new_c
        if delta < tol:
            break
    else:
        raise RuntimeError("Lloyd-Max (sphere) did not converge")
    c = np.array(c, dtype=np.float64)
    c = 0.5 * (c - c[::-1])
    return c, 0.5 * (c[:-1] + c[1:])


def codebook(bits_mse: int, d: int):
    """Centroids and thresholds for a rotated coordinate of a unit vector in R^d.

    [explainer, per-component reduction]: a coordinate of a random point of the unit
    sphere is almost normal with variance 1/d, so the sigma = 1 grid is scaled by 1/sqrt(d).
    """
    c, t = lloyd_max_gaussian(bits_mse)
    s = 1.0 / math.sqrt(d)
    return c * s, t * s


# ------------------------------------------------------------------------ quantizer

def normalize_rotate(x: np.ndarray, Pi: np.ndarray):
    """nu = |x|, x_n = x / nu and u = Pi x_n, row by row (float64).

    [explainer, caveats]: the vectors must be normalised and multiplied by a random
    matrix.  [review, MSE paragraph]: the matrix is random orthogonal (not Hadamard).
    A zero vector gets nu = 0 and x_n = u = 0.
    """
    x = np.asarray(x, dtype=np.float64)
    Pi = np.asarray(Pi, dtype=np.float64)
    nu = np.sqrt(np.sum(x * x, axis=1))
    safe = np.where(nu > 0.0, nu, 1.0)
    xn = np.where((nu > 0.0)[:, None], x / safe[:, None], 0.0)
    u = xn @ Pi.T
    return nu, xn, u


def bucketize(u: np.ndarray, thresholds: np.ndarray, decide_dtype=np.float64) -> np.ndarray:
    """Lloyd-Max cell index of every coordinate: the number of thresholds below u_t.

    [tldr, step 1] / [explainer, step 1]: each coordinate is rounded on its own against the
    precomputed grid.  The grid of the symmetric law is odd-symmetric, and ties keep the
    quantizer odd: a value equal to a threshold goes to the cell farther from zero (for
    u >= 0 the thresholds with u >= tau count, for u < 0 those with u > tau), so u = 0
    goes to the positive side.  The comparison is made in ``decide_dtype`` (float64 by
    default).
    """
    uu = np.asarray(u).astype(decide_dtype)
    tt = np.asarray(thresholds).astype(decide_dtype)
    at_or_above = np.zeros(uu.shape, dtype=np.int64)       # #{tau : tau <= u}
    strictly_above = np.zeros(uu.shape, dtype=np.int64)    # #{tau : tau < u}
    for tau in tt.ravel():
        at_or_above += uu >= tau
        strictly_above += uu > tau
    return np.where(uu >= 0, at_or_above, strictly_above)


def residual(xn: np.ndarray, Pi: np.ndarray, chat: np.ndarray):
    """r = x_n - Pi^T chat (original space) and gamma = |r|.

    [tldr, step 2]: the residual is the difference between the original vector and its
    compressed version.
    """
    Pi = np.asarray(Pi, dtype=np.float64)
    r = xn - chat @ Pi
    return r, np.sqrt(np.sum(r * r, axis=1))


def qjl_signs(S: np.ndarray, r: np.ndarray, decide_dtype=np.float64):
    """y = S r and z_i = [y_i >= 0] (1 bit per projected dimension).

    [tldr, step 2]: the residual is multiplied by another random matrix and only the sign
    of each result is kept.  [review, inner-product paragraph]: this is the 1-bit QJL stage.
    """
    S = np.asarray(S, dtype=np.float64)
    y = r @ S.T
    z = (y.astype(decide_dtype) >= 0).astype(np.int64)
    return y, z


def quantize(x, Pi, S, centroids, thresholds):
    """TurboQuant-prod encoding of each row of x: (b-1)-bit MSE code + 1-bit QJL of the residual.

    [review, inner-product paragraph]: quantize with the MSE-optimal quantizer at one bit
    less, then the 1-bit residual with QJL.  Returns a dict with idx [n][d], z [n][m],
    nu [n], gamma [n] and, for diagnostics, u, y.
    """
    nu, xn, u = normalize_rotate(x, Pi)
    idx = bucketize(u, thresholds)
    chat = np.asarray(centroids, dtype=np.float64)[idx]
    r, gamma = residual(xn, Pi, chat)
    y, z = qjl_signs(S, r)
    return {"idx": idx, "z": z, "nu": nu, "gamma": gamma, "u": u, "y": y}


# ------------------------------------------------------------------- canonical layout
# The pages fix no bit layout.  Layout used by this project: per vector, for each group w
# of 32 consecutive coordinates, b consecutive little-endian uint32 words; word p < b-1
# holds bit p of idx, word b-1 holds the QJL signs z; coordinate 32w + j is bit j.

def pack_codes(idx: np.ndarray, z: np.ndarray, b: int) -> np.ndarray:
    """Pack idx [n][d] (values < 2**(b-1)) and z [n][d] into uint32 codes [n][d/32][b]."""
    idx = np.asarray(idx, dtype=np.int64)
    z = np.asarray(z, dtype=np.int64)
    n, d = idx.shape
    assert d % 32 == 0 and z.shape == (n, d)
    planes = [(idx >> p) & 1 for p in range(b - 1)] + [z & 1]
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    out = np.empty((n, d // 32, b), dtype=np.uint32)
    for p, bits in enumerate(planes):
        grouped = bits.reshape(n, d // 32, 32).astype(np.uint64)
        out[:, :, p] = np.sum(grouped * weights, axis=-1).astype(np.uint32)
    return out


def unpack_codes(codes: np.ndarray, b: int):
    """Inverse of pack_codes: uint32 [n][d/32][b] -> (idx [n][d], z [n][d])."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, groups, bb = codes.shape
    assert bb == b
    shifts = np.arange(32, dtype=np.uint32)
    bits = (codes[:, :, :, None] >> shifts) & 1          # [n][groups][b][32]
    bits = bits.transpose(0, 2, 1, 3).reshape(n, b, groups * 32).astype(np.int64)
    idx = np.zeros((n, groups * 32), dtype=np.int64)
    for p in range(b - 1):
        idx |= bits[:, p] << p
    return idx, bits[:, b - 1]


# ------------------------------------------------------------------------ estimator

def qjl_alpha(m: int) -> float:
    """Scale of the QJL term: sqrt(pi/2) / m.

    For s ~ N(0, I) and a unit vector rho, E[sign<s, rho> <s, q>] = sqrt(2/pi) <q, rho>, so
    summing m rows and multiplying by gamma sqrt(pi/2)/m gives <q, r> in expectation.
    """
    return math.sqrt(math.pi / 2.0) / m


def qjl_alpha_orthogonal(m: int, d: int) -> float:
    """Scale of the QJL term for a matrix with m orthonormal rows: 1 / (m E|w_1|), w_1 one
    coordinate of a uniform unit vector in R^d, E|w_1| = Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2)).

    For a unit row s uniform on the sphere, E[sign<s, rho> <s, q>] = E|w_1| <q, rho>, so m
    rows times gamma / (m E|w_1|) give <q, r> in expectation."""
    ew = math.exp(math.lgamma(0.5 * d) - math.lgamma(0.5 * (d + 1))) / math.sqrt(math.pi)
    return 1.0 / (m * ew)


def estimate_ip(q, Pi, S, idx, z, nu, gamma, centroids, mode: str = "prod",
                alpha: float | None = None) -> np.ndarray:
    """Estimated inner products <q_a, x_k> for every query row a and key row k -> [nq][n].

    [review, problem statement]: one vector of the pair (the key) is quantized, the other
    (the query) is kept exact, and the inner-product estimate must be unbiased.
    prod: nu * (<Pi q, chat> + sqrt(pi/2)/m * gamma * <S q, 2z - 1>)   (MSE + QJL)
    mse : nu * <Pi q, chat>   (the MSE part alone; biased, [news, bias paragraph])
    """
    q = np.asarray(q, dtype=np.float64)
    Pi = np.asarray(Pi, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    nu = np.asarray(nu, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    chat = np.asarray(centroids, dtype=np.float64)[np.asarray(idx)]
    qh = q @ Pi.T
    mse = qh @ chat.T
    if mode == "mse":
        return mse * nu[None, :]
    if mode != "prod":
        raise ValueError(mode)
    sh = q @ S.T
    sgn = 2.0 * np.asarray(z, dtype=np.float64) - 1.0
    qjl = sh @ sgn.T
    a = qjl_alpha(S.shape[0]) if alpha is None else alpha
    return nu[None, :] * (mse + a * gamma[None, :] * qjl)


def dequantize(Pi, S, idx, z, nu, gamma, centroids, mode: str = "prod",
               alpha: float | None = None) -> np.ndarray:
    """Reconstruction x~ [n][d].

    [review, QJL paragraph]: dequantization is the inverse rotation and a renormalisation.
    prod: x~ = nu (Pi^T chat + sqrt(pi/2)/m * gamma * S^T (2z - 1));  mse: x~ = nu Pi^T chat.
    """
    Pi = np.asarray(Pi, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    nu = np.asarray(nu, dtype=np.float64)
    gamma = np.asarray(gamma, dtype=np.float64)
    chat = np.asarray(centroids, dtype=np.float64)[np.asarray(idx)]
    xt = chat @ Pi
    if mode == "prod":
        sgn = 2.0 * np.asarray(z, dtype=np.float64) - 1.0
        a = qjl_alpha(S.shape[0]) if alpha is None else alpha
        xt = xt + a * gamma[:, None] * (sgn @ S)
    elif mode != "mse":
        raise ValueError(mode)
    return nu[:, None] * xt


def topk(scores: np.ndarray, k: int, index_offset: int = 0):
    """The k largest scores of each row; equal scores are ordered by smaller index.

    [news, vector-search paragraph]: search is a flat scan of estimated inner products.
    Returns (indices [nq][k] int64, values [nq][k] float64).
    """
    scores = np.asarray(scores, dtype=np.float64)
    nq, n = scores.shape
    k = min(k, n)
    ids = np.empty((nq, k), dtype=np.int64)
    vals = np.empty((nq, k), dtype=np.float64)
    cols = np.arange(n)
    for a in range(nq):
        order = np.lexsort((cols, -scores[a]))[:k]
        ids[a] = order + index_offset
        vals[a] = scores[a, order]
    return ids, vals


# ------------------------------------------------------------- decode attention (values)
# [review, problem statement]: the MSE-optimal quantizer rotates the vector with a random
# orthogonal matrix and applies Lloyd-Max at the target bit width.  Values of a KV cache
# are reconstructed (not inner-producted), so they take this quantizer alone: the MSE stage
# of the same encoder, its (b-1)-bit index and the norm nu, without the QJL bit.

def quantize_mse(x, Pi, centroids, thresholds):
    """TurboQuant-mse encoding of each row of x: idx [n][d] (Lloyd-Max cell of u = Pi x/nu)
    and nu [n].  The centroids are not used by the encoding; they are taken for symmetry
    with quantize()."""
    del centroids
    nu, _, u = normalize_rotate(x, Pi)
    return {"idx": bucketize(u, thresholds), "nu": nu, "u": u}


def pack_index_planes(idx: np.ndarray, bits: int) -> np.ndarray:
    """Pack idx [n][d] (values < 2**bits) into uint32 [n][d/32][bits]: plane p holds bit p
    of every coordinate's index, coordinate t in word t // 32, bit t % 32."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    assert d % 32 == 0
    weights = (np.uint64(1) << np.arange(32, dtype=np.uint64))
    out = np.empty((n, d // 32, bits), dtype=np.uint32)
    for p in range(bits):
        grouped = ((idx >> p) & 1).reshape(n, d // 32, 32).astype(np.uint64)
        out[:, :, p] = np.sum(grouped * weights, axis=-1).astype(np.uint32)
    return out


def unpack_index_planes(codes: np.ndarray, bits: int) -> np.ndarray:
    """Inverse of pack_index_planes: uint32 [n][d/32][bits] -> idx [n][d]."""
    codes = np.asarray(codes, dtype=np.uint32)
    n, groups, bb = codes.shape
    assert bb == bits
    shifts = np.arange(32, dtype=np.uint32)
    bitsarr = ((codes[:, :, :, None] >> shifts) & 1).transpose(0, 2, 1, 3).reshape(n, bits, groups * 32)
    idx = np.zeros((n, groups * 32), dtype=np.int64)
    for p in range(bits):
        idx |= bitsarr[:, p].astype(np.int64) << p
    return idx


def dequantize_mse(Pi, idx, nu, centroids) -> np.ndarray:
    """Value reconstruction v~ = nu Pi^T chat [n][d] ([review, QJL paragraph]: inverse
    rotation and renormalisation)."""
    Pi = np.asarray(Pi, dtype=np.float64)
    chat = np.asarray(centroids, dtype=np.float64)[np.asarray(idx)]
    return np.asarray(nu, dtype=np.float64)[:, None] * (chat @ Pi)


def attention_decode(logits: np.ndarray, values: np.ndarray, scale: float) -> np.ndarray:
    """One decode step of attention per group: for every query head h of group g,
        o[g][h] = sum_t softmax_t(scale * logits[g][h][t]) * values[g][t].
    logits [groups][G][T] (the estimated <q, k>), values [groups][T][d] (reconstructed
    values) -> o [groups][G][d].  The softmax is taken as exp(w - max w) / sum, which is the
    same function for finite w."""
    logits = np.asarray(logits, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    groups, G, T = logits.shape
    out = np.empty((groups, G, values.shape[2]), dtype=np.float64)
    for g in range(groups):
        w = scale * logits[g]
        w = w - np.max(w, axis=1, keepdims=True)
        p = np.exp(w)
        p /= np.sum(p, axis=1, keepdims=True)
        out[g] = p @ values[g]
    return out


# ---------------------------------------------------------------- fractional rates
# [review, experiments paragraph], [news, results paragraph]: KV caches at 2.5 and 3.5 bits per
# channel.  Reading: the channels form groups, given as (first channel, width) pairs that
# tile [0, d); each group is a separate TurboQuant instance with its own rotation, QJL
# matrix, codebook and bit budget, and the inner product is the sum over groups.  Each
# group's estimate is unbiased, so the sum is.

def quantize_split(x, groups):
    """Encode the channel groups of x [n][d] separately.

    groups: list of dicts with keys off, width, Pi, S, centroids, thresholds (the group's
    instance).  Returns the list of quantize() results, one per group."""
    x = np.asarray(x)
    return [quantize(x[:, g["off"]:g["off"] + g["width"]], g["Pi"], g["S"], g["centroids"],
                     g["thresholds"]) for g in groups]


def estimate_ip_split(q, groups, codes, mode: str = "prod") -> np.ndarray:
    """Sum over channel groups of estimate_ip on the query's matching channels -> [nq][n].

    codes: per group a dict with idx, z, nu, gamma (as quantize_split returns); each group
    may carry its own QJL scale under the key alpha (None or absent: Gaussian S)."""
    q = np.asarray(q, dtype=np.float64)
    total = None
    for g, c in zip(groups, codes):
        est = estimate_ip(q[:, g["off"]:g["off"] + g["width"]], g["Pi"], g["S"], c["idx"], c["z"],
                          c["nu"], c["gamma"], g["centroids"], mode, alpha=g.get("alpha"))
        total = est if total is None else total + est
    return total
