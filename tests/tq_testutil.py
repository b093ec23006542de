"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Acceptance rules (the pages fix no tolerances; these follow the stated targets):
  * index codes: bit-exact, except a coordinate whose oracle value u lies within 1e-5 of a
    threshold that separates the two indices (excused);
  * sign bits: compared with the oracle's QJL re-run on the GPU's indices (so one excused
    index flip does not cascade), bit-exact except |y_i| <= 1e-5 |S_i| gamma (excused);
  * excused rate <= 1e-4, unexcused = 0;
  * nu within 1e-5 relative, gamma within 1e-5 absolute (gamma is a norm of a unit-vector
    residual);
  * logits with the oracle fed the GPU's codes: |l_gpu - l_oracle| <= 1e-3 |q| nu.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen

EXCUSE_U = 1e-5
EXCUSE_Y = 1e-5
MAX_EXCUSED_RATE = 1e-4
LOGIT_TOL = 1e-3

DEV = torch.device("cuda:0")


@dataclasses.dataclass
class Setup:
    d: int
    b: int
    Pi: np.ndarray
    S: np.ndarray
    c_or: np.ndarray
    t_or: np.ndarray
    params: torch.Tensor
    alpha: float | None = None     # QJL scale for the oracle (None: Gaussian S)


def make_setup(d: int, b: int, cfg: int, rep: int = 0, sphere: bool = False,
               orthogonal_s: bool = False) -> Setup:
    """Parameters of one configuration.  sphere: Lloyd-Max on the exact sphere law instead of
    N(0, 1/d); orthogonal_s: a Haar orthogonal QJL matrix instead of Gaussian entries."""
    Pi = gen.haar_orthogonal(d, cfg, rep)
    if orthogonal_s:
        S = gen.haar_orthogonal(d, cfg, rep, role=gen.ROLE_S)
    else:
        S = gen.gaussian_matrix(d, d, cfg, rep)
    build = tq.tq_codebook_build_sphere if sphere else tq.tq_codebook_build
    c, t = build(b - 1, d)
    params = torch.empty(tq.tq_params_bytes(d, b), dtype=torch.uint8, device=DEV)
    prepare = tq.tq_prepare_orthogonal_qjl if orthogonal_s else tq.tq_prepare
    prepare(d, b, Pi, S, c, t, params)
    c_or, t_or = (oracle.codebook_sphere if sphere else oracle.codebook)(b - 1, d)
    alpha = oracle.qjl_alpha_orthogonal(d, d) if orthogonal_s else None
    return Setup(d, b, Pi, S, c_or, t_or, params, alpha)


def to_device(x: np.ndarray, bf16: bool) -> torch.Tensor:
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV)


def host64(x: np.ndarray, bf16: bool) -> np.ndarray:
    """The exact input values as the oracle sees them (float64)."""
    return (gen.bf16_bits_to_f32(x) if bf16 else np.asarray(x, np.float32)).astype(np.float64)


def gpu_quantize(st: Setup, xd: torch.Tensor):
    n = xd.shape[0]
    codes = torch.full((n * (st.d // 32) * st.b,), -1, dtype=torch.int32, device=DEV)
    nu = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    gamma = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_quantize(st.params, st.d, st.b, xd, codes, nu, gamma)
    torch.cuda.synchronize()
    return codes, nu, gamma


def codes_np(codes: torch.Tensor, n: int, d: int, b: int) -> np.ndarray:
    return codes.cpu().numpy().view(np.uint32).reshape(n, d // 32, b)


def compare_codes(st: Setup, x64: np.ndarray, codes: np.ndarray, nu: np.ndarray,
                  gamma: np.ndarray) -> dict:
    """Compare GPU codes with the oracle on the same inputs; returns a report dict."""
    d, b = st.d, st.b
    idx_g, z_g = oracle.unpack_codes(codes, b)
    nu_o, xn, u = oracle.normalize_rotate(x64, st.Pi)
    idx_o = oracle.bucketize(u, st.t_or)
    mism = idx_g != idx_o
    unexcused_idx = 0
    excused_idx = 0
    if mism.any():
        rows, cols = np.nonzero(mism)
        lo = np.minimum(idx_g[rows, cols], idx_o[rows, cols])
        hi = np.maximum(idx_g[rows, cols], idx_o[rows, cols])
        for k in range(rows.size):
            taus = st.t_or[lo[k]:hi[k]]
            dist = np.min(np.abs(u[rows[k], cols[k]] - taus)) if taus.size else np.inf
            if dist <= EXCUSE_U:
                excused_idx += 1
            else:
                unexcused_idx += 1
    # QJL stage re-run on the GPU's indices
    chat = st.c_or[idx_g]
    r, gam = oracle.residual(xn, st.Pi, chat)
    y, z_o = oracle.qjl_signs(st.S, r)
    srow = np.linalg.norm(st.S.astype(np.float64), axis=1)
    zm = z_g != z_o
    tol_y = EXCUSE_Y * srow[None, :] * gam[:, None]
    excused_z = int(np.sum(zm & (np.abs(y) <= tol_y)))
    unexcused_z = int(np.sum(zm & (np.abs(y) > tol_y)))
    nu_err = float(np.max(np.abs(nu - nu_o) / np.maximum(nu_o, 1e-30))) if nu.size else 0.0
    gamma_err = float(np.max(np.abs(gamma - gam))) if gamma.size else 0.0
    total = idx_g.size
    return {
        "n": x64.shape[0], "unexcused_idx": unexcused_idx, "excused_idx": excused_idx,
        "unexcused_z": unexcused_z, "excused_z": excused_z,
        "excused_rate": (excused_idx + excused_z) / max(2 * total, 1),
        "nu_rel_err": nu_err, "gamma_abs_err": gamma_err, "idx": idx_g, "z": z_g,
    }


def assert_codes_ok(rep: dict):
    assert rep["unexcused_idx"] == 0, rep["unexcused_idx"]
    assert rep["unexcused_z"] == 0, rep["unexcused_z"]
    assert rep["excused_rate"] <= MAX_EXCUSED_RATE, rep["excused_rate"]
    assert rep["nu_rel_err"] <= 1e-5, rep["nu_rel_err"]
    assert rep["gamma_abs_err"] <= 1e-5, rep["gamma_abs_err"]


def logit_errors(st: Setup, q64: np.ndarray, idx, z, nu, gamma, logits: np.ndarray,
                 mode: str = "prod") -> float:
    """max |l_gpu - l_oracle| / (|q| nu) over all (query, key), oracle fed the GPU's codes.

    q64 [groups][G][d], idx/z [groups*T][d], nu/gamma [groups*T], logits [groups][G][T].
    """
    groups, G, _ = q64.shape
    T = logits.shape[2]
    worst = 0.0
    for g in range(groups):
        sl = slice(g * T, (g + 1) * T)
        ref = oracle.estimate_ip(q64[g], st.Pi, st.S, idx[sl], z[sl], nu[sl], gamma[sl], st.c_or,
                                 mode, alpha=st.alpha)
        scale = np.linalg.norm(q64[g], axis=1)[:, None] * np.maximum(nu[sl][None, :], 1e-30)
        err = np.abs(logits[g].astype(np.float64) - ref) / scale
        worst = max(worst, float(np.max(err)))
    return worst


def gpu_score(st: Setup, qd: torch.Tensor, codes, nu, gamma, groups: int, G: int, T: int,
              mode: int) -> np.ndarray:
    logits = torch.full((groups * G * T,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(tq.tq_score_ws_bytes(st.d, st.b, groups, G, T), 256), dtype=torch.uint8,
                     device=DEV)
    tq.tq_score_ip(st.params, st.d, st.b, qd, codes, nu, gamma, groups, G, T, mode, logits, ws)
    torch.cuda.synchronize()
    return logits.cpu().numpy().reshape(groups, G, T)


def describe(rep: dict) -> str:
    return (f"n={rep['n']} idx unexcused={rep['unexcused_idx']} excused={rep['excused_idx']} "
            f"z unexcused={rep['unexcused_z']} excused={rep['excused_z']} "
            f"rate={rep['excused_rate']:.2e} nu_err={rep['nu_rel_err']:.1e} "
            f"gamma_err={rep['gamma_abs_err']:.1e}")


def gpu_topk(st: Setup, qd: torch.Tensor, codes, nu, gamma, n: int, k: int, mode: int):
    nq = qd.shape[0]
    idx = torch.full((nq * k,), -7, dtype=torch.int32, device=DEV)
    score = torch.full((nq * k,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_topk_ws_bytes(st.d, st.b, nq, n, k), dtype=torch.uint8, device=DEV)
    tq.tq_topk(st.params, st.d, st.b, qd, codes, nu, gamma, n, k, mode, idx, score, ws)
    torch.cuda.synchronize()
    return idx.cpu().numpy().reshape(nq, k), score.cpu().numpy().reshape(nq, k)


def check_topk(idx_g: np.ndarray, score_g: np.ndarray, ref: np.ndarray, scale: np.ndarray):
    """Compare GPU top-k with the oracle's scores of every key (oracle fed the GPU codes).

    ref [nq][n] float64 oracle scores; scale [nq][n] = |q| nu for the score tolerance.
    Rules: every returned score within LOGIT_TOL * scale of the oracle's score of that key;
    scores non-increasing; the returned set equals the oracle's top-k except swaps between
    keys whose oracle scores differ by at most 4x the largest score error seen for that
    query (near ties).  Returns (max relative score error, number of queries with swaps).
    """
    nq, k = idx_g.shape
    worst = 0.0
    swapped = 0
    for a in range(nq):
        ids = idx_g[a]
        assert np.all((ids >= 0) & (ids < ref.shape[1])), ids
        assert len(set(ids.tolist())) == k
        err = np.abs(score_g[a].astype(np.float64) - ref[a, ids])
        rel = err / np.maximum(scale[a, ids], 1e-30)
        worst = max(worst, float(rel.max()))
        assert np.all(np.diff(score_g[a]) <= 0), score_g[a]
        o_ids, o_vals = oracle.topk(ref[a:a + 1], k)
        o_set, g_set = set(o_ids[0].tolist()), set(ids.tolist())
        if o_set != g_set:
            swapped += 1
            tol = 4.0 * float(err.max()) + 1e-12
            kth = o_vals[0, -1]
            for j in g_set - o_set:
                assert ref[a, j] >= kth - tol, (a, j, ref[a, j], kth, tol)
            g_min = min(ref[a, j] for j in g_set)
            for j in o_set - g_set:
                assert ref[a, j] <= g_min + tol, (a, j, ref[a, j], g_min, tol)
    return worst, swapped
