"""The error bound of the d = 128 scorer's integer query digits (CPU).

The scorer evaluates the estimate nu (<Pi q, chat> + alpha gamma <S q, 2z - 1>) through the
Walsh form of the odd-symmetric codebook: chat_t = sum_w e_w (2 B_w,t - 1) over the index
bit planes B_w (b = 4 adds the plane b0 ^ b1 ^ b2), so
    <Pi q, chat> = 2 sum_w e_w sum_t (Pi q)_t B_w,t - (sum_w e_w) sum_t (Pi q)_t,
    <S q, 2z - 1> = 2 sum_t (S q)_t z_t - sum_t (S q)_t.
It rounds each value e_w (Pi q)_t and (S q)_t to an integer digit at the scale
DIGIT_RANGE / max|row|, the odd coordinates stored halved against key bytes of 0/2, sums the
digits selected by the key bits exactly and subtracts float constants formed from the
unrounded values.  This file emulates those steps in float64 and checks that the bound the
GPU parity tests use (tq_testutil.logit_bound) holds, that it is reached up to a small factor
by a query whose roundings all go the same way, and that without rounding the emulation is
the oracle's estimate.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import tq_testutil as U

D = 128


def planes(idx: np.ndarray, b: int) -> list:
    """The scorer's key planes for (b-1)-bit indices: b0, b1, [b2, b0^b1^b2]."""
    bits = [(idx >> p) & 1 for p in range(b - 1)]
    if b == 4:
        bits = bits + [bits[0] ^ bits[1] ^ bits[2]]
    return bits


def emulate(pq, sq, idx, z, e, rounding=True):
    """Per-key estimate / nu with the digit arithmetic: (<Pi q, chat>, <S q, 2z - 1>)."""
    b = {1: 2, 2: 3, 4: 4}[len(e)]       # Walsh words -> total bits
    odd = (np.arange(D) % 2) == 1

    def digits(v, mx):
        scale = U.DIGIT_RANGE / mx if mx > 0 else 1.0
        if not rounding:
            return v * scale, scale
        dv = np.where(odd, 2.0 * np.rint(0.5 * scale * v), np.rint(scale * v))
        return dv, scale

    emax = max(abs(x) for x in e)
    pl = planes(idx, b)
    mx = emax * np.max(np.abs(pq))
    ai = np.zeros(idx.shape[0])
    for w, ew in enumerate(e):
        dv, sa = digits(ew * pq, mx)
        ai += pl[w].astype(np.float64) @ dv
    mse = ai * 2.0 / sa - sum(e) * pq.sum()
    dz, sb = digits(sq, np.max(np.abs(sq)))
    qjl = (z.astype(np.float64) @ dz) * 2.0 / sb - sq.sum()
    return mse, qjl


def _case(b, seed):
    rng = np.random.default_rng(seed)
    c, t = oracle.codebook(b - 1, D)
    n = 400
    idx = rng.integers(0, 2 ** (b - 1), size=(n, D))
    z = rng.integers(0, 2, size=(n, D))
    pq = rng.standard_normal(D) * rng.uniform(0.1, 3.0)
    sq = rng.standard_normal(D) * rng.uniform(0.1, 3.0)
    return c, idx, z, pq, sq


@pytest.mark.parametrize("b", [2, 3, 4])
def test_unrounded_emulation_is_the_estimate(b):
    c, idx, z, pq, sq = _case(b, 100 + b)
    e = U.walsh_coefficients(c)
    assert len(e) == {2: 1, 3: 2, 4: 4}[b]
    mse, qjl = emulate(pq, sq, idx, z, e, rounding=False)
    np.testing.assert_allclose(mse, c[idx] @ pq, rtol=0, atol=1e-12 * np.abs(pq).sum())
    np.testing.assert_allclose(qjl, (2.0 * z - 1.0) @ sq, rtol=0, atol=1e-12 * np.abs(sq).sum())


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("seed", range(5))
def test_digit_rounding_within_bound(b, seed):
    c, idx, z, pq, sq = _case(b, 1000 * b + seed)
    e = U.walsh_coefficients(c)
    mse, qjl = emulate(pq, sq, idx, z, e)
    b_mse, b_qjl = U.digit_error_terms(e, 1.0, np.max(np.abs(pq)), np.max(np.abs(sq)), D)
    assert np.all(np.abs(mse - c[idx] @ pq) <= b_mse)
    assert np.all(np.abs(qjl - (2.0 * z - 1.0) @ sq) <= b_qjl)


def _aligned_values():
    """Scaled values just below k + 1/2 (even coordinates) or 2 k + 1 (odd ones, stored halved),
    so that every digit errs by almost its maximum in the same direction; coordinate 0 is the
    row maximum (an exact digit)."""
    k = np.arange(D) % 50 + 10
    v = np.where(np.arange(D) % 2 == 1, 2.0 * k + 0.999, k + 0.4999)
    v[0] = U.DIGIT_RANGE
    return v


@pytest.mark.parametrize("b", [2, 3, 4])
def test_qjl_bound_is_reached_by_aligned_rounding(b):
    c, _, _, pq, _ = _case(b, 7)
    e = U.walsh_coefficients(c)
    sq = _aligned_values() / U.DIGIT_RANGE           # row max 1, digits = the values above
    idx = np.zeros((1, D), dtype=np.int64)
    z = np.ones((1, D), dtype=np.int64)               # every sign bit selects its digit
    _, qjl = emulate(pq, sq, idx, z, e)
    _, b_qjl = U.digit_error_terms(e, 1.0, np.max(np.abs(pq)), np.max(np.abs(sq)), D)
    err = abs(qjl[0] - (2.0 * z[0] - 1.0) @ sq)
    assert 0.99 * b_qjl <= err <= b_qjl, (err, b_qjl)


def test_mse_bound_is_reached_by_aligned_rounding():
    # one Walsh word (b = 2): e_0 (Pi q)_t at the row scale are the aligned values when
    # (Pi q)_t = v_t / (DIGIT_RANGE e_0); index 1 (the positive level) sets every plane bit
    c, _, _, _, sq = _case(2, 7)
    e = U.walsh_coefficients(c)
    pq = _aligned_values() / (U.DIGIT_RANGE * e[0])
    idx = np.ones((1, D), dtype=np.int64)
    z = np.zeros((1, D), dtype=np.int64)
    mse, _ = emulate(pq, sq, idx, z, e)
    b_mse, _ = U.digit_error_terms(e, 1.0, np.max(np.abs(pq)), np.max(np.abs(sq)), D)
    err = abs(mse[0] - c[idx[0]] @ pq)
    assert 0.99 * b_mse <= err <= b_mse, (err, b_mse)
