"""Shared helpers of the GPU parity tests: run the HIP path, run the oracle, compare.

Acceptance rules (the pages fix no tolerances; these follow the stated targets):
  * index codes: bit-exact, except a coordinate whose oracle value u lies within 1e-5 of a
    threshold that separates the two indices (excused);
  * sign bits: compared with the oracle's QJL re-run on the GPU's indices (so one excused
    index flip does not cascade), bit-exact except |y_i| <= 1e-5 |S_i| gamma (excused);
  * excused rate <= 1e-4, unexcused = 0;
  * nu within 1e-5 relative, gamma within 1e-5 absolute (gamma is a norm of a unit-vector
    residual);
  * logits with the oracle fed the GPU's codes, per (query, key), within the bound of the scoring
    path's own arithmetic (logit_bound): the d = 128 scorer rounds each query value to an integer
    digit of at most DIGIT_RANGE in magnitude (everything after that is exact integer work and
    float32 epilogue arithmetic), the general path sums in float32;
  * rotated coordinates (where the encoder reports them): max |u_gpu - u_oracle| <= 1e-5
    (u is a unit vector, so this is relative to |x|).
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import itertools
import math
import os

import numpy as np
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen

EXCUSE_U = 1e-5
EXCUSE_Y = 1e-5
MAX_EXCUSED_RATE = 1e-4
# d = 128 scorer: query values of a row become integers round(DIGIT_RANGE v / max |v|) (the
# value 128 hi + lo in two int8 digits); the general path: float32 sums over 2d terms
DIGIT_RANGE = 16000.0
FP32_LOGIT_TOL = 1e-5
ROTATION_TOL = 1e-5
# top-k scores are float32 estimates (the fused fp16 scan only picks candidates): float32
# rounding over a 2d-term sum, far inside the logit tolerance
TOPK_SCORE_TOL = 1e-5


def worker_count() -> int:
    """Host threads for the oracle side of the full-size checks (at most 16)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:   # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def parallel_map(fn, items, label: str | None = None, every: int = 16):
    """fn over items on host threads, BLAS limited to one thread each; results in order.
    NumPy releases the GIL in its array loops and BLAS calls, so chunks of an oracle check
    run side by side.  With a label, a progress line is printed every `every` items."""
    import threading

    from threadpoolctl import threadpool_limits
    items = list(items)
    lock = threading.Lock()
    done = [0]

    def run(item):
        out = fn(item)
        if label:
            with lock:
                done[0] += 1
                if done[0] % every == 0 or done[0] == len(items):
                    print(f"  [{label}] {done[0]}/{len(items)}", flush=True)
        return out

    with threadpool_limits(limits=1), concurrent.futures.ThreadPoolExecutor(worker_count()) as ex:
        return list(ex.map(run, items))


def merge_reports(reps: list) -> dict:
    """Totals and worst cases of several compare_codes reports (their idx / z dropped)."""
    out = {"n": 0, "unexcused_idx": 0, "excused_idx": 0, "unexcused_z": 0, "excused_z": 0,
           "nu_rel_err": 0.0, "gamma_abs_err": 0.0, "u_abs_err": None, "coords": 0}
    for r in reps:
        for k in ("n", "unexcused_idx", "excused_idx", "unexcused_z", "excused_z", "coords"):
            out[k] += r[k]
        out["nu_rel_err"] = max(out["nu_rel_err"], r["nu_rel_err"])
        out["gamma_abs_err"] = max(out["gamma_abs_err"], r["gamma_abs_err"])
        if r.get("u_abs_err") is not None:
            out["u_abs_err"] = max(out["u_abs_err"] or 0.0, r["u_abs_err"])
    out["excused_rate"] = (out["excused_idx"] + out["excused_z"]) / max(2 * out["coords"], 1)
    return out

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
                  gamma: np.ndarray, u_gpu: np.ndarray | None = None, keep: bool = True) -> dict:
    """Compare GPU codes with the oracle on the same inputs; returns a report dict.
    u_gpu: the rotated coordinates the encoder reported (checked against the oracle's u);
    keep: also return the unpacked GPU idx and z."""
    d, b = st.d, st.b
    idx_g, z_g = oracle.unpack_codes(codes, b)
    nu_o, xn, u = oracle.normalize_rotate(x64, st.Pi)
    u_err = None
    if u_gpu is not None:
        u_err = float(np.max(np.abs(np.asarray(u_gpu, np.float64) - u))) if u.size else 0.0
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
    rep = {
        "n": x64.shape[0], "unexcused_idx": unexcused_idx, "excused_idx": excused_idx,
        "unexcused_z": unexcused_z, "excused_z": excused_z, "coords": total,
        "excused_rate": (excused_idx + excused_z) / max(2 * total, 1),
        "nu_rel_err": nu_err, "gamma_abs_err": gamma_err, "u_abs_err": u_err,
    }
    if keep:
        rep["idx"], rep["z"] = idx_g, z_g
    return rep


def assert_codes_ok(rep: dict):
    assert rep["unexcused_idx"] == 0, rep["unexcused_idx"]
    assert rep["unexcused_z"] == 0, rep["unexcused_z"]
    assert rep["excused_rate"] <= MAX_EXCUSED_RATE, rep["excused_rate"]
    assert rep["nu_rel_err"] <= 1e-5, rep["nu_rel_err"]
    assert rep["gamma_abs_err"] <= 1e-5, rep["gamma_abs_err"]
    if rep.get("u_abs_err") is not None:
        assert rep["u_abs_err"] <= ROTATION_TOL, rep["u_abs_err"]


def walsh_coefficients(c) -> list:
    """Odd-subset Walsh coefficients of an odd-symmetric codebook c[2^m]:
    c[idx] = sum_P e_P prod_{p in P} (2 bit_p(idx) - 1) over the odd subsets P of the m index bits."""
    c = np.asarray(c, dtype=np.float64)
    m = len(c).bit_length() - 1
    idx = np.arange(len(c))
    sig = [2 * ((idx >> p) & 1) - 1 for p in range(m)]
    out = []
    for r in range(1, m + 1, 2):
        for P in itertools.combinations(range(m), r):
            out.append(float(np.mean(c * np.prod([sig[p] for p in P], axis=0))))
    return out


def digit_path(d: int, G: int) -> bool:
    """Whether tq_score_ip runs the d = 128 integer-digit scorer for this shape."""
    return d == 128 and G % 4 == 0


def logit_bound(st: Setup, qg: np.ndarray, nu: np.ndarray, gamma: np.ndarray, mode: str = "prod",
                digits: bool | None = None) -> np.ndarray:
    """Largest |l_gpu - l_exact| [G][T] that the scoring path's arithmetic allows, given the codes.

    Digit scorer: the MSE rows hold e_w (Pi q)_t and the QJL rows (S q)_t as integers rounded from
    DIGIT_RANGE v / max|v| (max over the row); a digit errs by at most 1/2, and the odd coordinates
    (half of them), stored halved against key bytes of 0/2, by 1.  The masked sums over key bits
    are exact and the row constants are float32 sums of the unrounded values, so per word the
    rounding adds at most 96 digits, scaled by 2 (the Walsh form 2 sum - const):
      |dl| <= nu (2 * 96 ne e_max max|Pi q| + gamma 2 * 96 alpha max|S q|) / DIGIT_RANGE  (d = 128)
    plus float32 rounding of the query prep and the epilogue (1e-5 |q| nu covers it).
    General path: float32 sums only, FP32_LOGIT_TOL |q| nu.
    """
    G, d = qg.shape
    if digits is None:
        digits = digit_path(d, G)
    qn = np.linalg.norm(qg, axis=1)[:, None]
    nu = nu[None, :]
    if not digits:
        return FP32_LOGIT_TOL * qn * nu
    pq = np.max(np.abs(qg @ st.Pi.astype(np.float64).T), axis=1)[:, None]
    sq = np.max(np.abs(qg @ st.S.astype(np.float64).T), axis=1)[:, None]
    alpha = st.alpha if st.alpha is not None else oracle.qjl_alpha(st.S.shape[0])
    b_mse, b_qjl = digit_error_terms(walsh_coefficients(st.c_or), alpha, pq, sq, d)
    bound = nu * b_mse
    if mode == "prod":
        bound = bound + nu * gamma[None, :] * b_qjl
    return bound + FP32_LOGIT_TOL * qn * nu


def digit_error_terms(e, alpha, pq_max, sq_max, d: int = 128):
    """The digit rounding's share of the logit error bound (see logit_bound): the MSE term and
    the QJL term per unit gamma, both per unit nu, for rows with max |Pi q| = pq_max and
    max |S q| = sq_max.  Per word, d/2 coordinates err by at most 1/2 digit and d/2 (the
    halved odd ones) by 1 digit: 3 d / 4 digits."""
    per_word = 0.75 * d
    b_mse = 2.0 * per_word * len(e) * max(abs(v) for v in e) * pq_max / DIGIT_RANGE
    b_qjl = 2.0 * per_word * alpha * sq_max / DIGIT_RANGE
    return b_mse, b_qjl


def logit_errors(st: Setup, q64: np.ndarray, idx, z, nu, gamma, logits: np.ndarray,
                 mode: str = "prod", digits: bool | None = None) -> float:
    """Asserts |l_gpu - l_oracle| <= logit_bound for every (query, key), the oracle fed the GPU's
    codes; returns max |l_gpu - l_oracle| / (|q| nu) for the record.

    q64 [groups][G][d], idx/z [groups*T][d], nu/gamma [groups*T], logits [groups][G][T].
    """
    groups, G, _ = q64.shape
    T = logits.shape[2]
    worst = 0.0
    for g in range(groups):
        sl = slice(g * T, (g + 1) * T)
        ref = oracle.estimate_ip(q64[g], st.Pi, st.S, idx[sl], z[sl], nu[sl], gamma[sl], st.c_or,
                                 mode, alpha=st.alpha)
        dl = np.abs(logits[g].astype(np.float64) - ref)
        bound = logit_bound(st, q64[g], nu[sl], gamma[sl], mode, digits)
        bad = np.argwhere(~(dl <= bound))
        assert bad.size == 0, (g, bad[:4].tolist(), dl[tuple(bad[0])], bound[tuple(bad[0])])
        scale = np.linalg.norm(q64[g], axis=1)[:, None] * np.maximum(nu[sl][None, :], 1e-30)
        worst = max(worst, float(np.max(dl / scale)))
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
    u = rep.get("u_abs_err")
    return (f"n={rep['n']} idx unexcused={rep['unexcused_idx']} excused={rep['excused_idx']} "
            f"z unexcused={rep['unexcused_z']} excused={rep['excused_z']} "
            f"rate={rep['excused_rate']:.2e} nu_err={rep['nu_rel_err']:.1e} "
            f"gamma_err={rep['gamma_abs_err']:.1e}" + ("" if u is None else f" u_err={u:.1e}"))


def gpu_quantize_rotation(st: Setup, xd: torch.Tensor):
    """tq_quantize_with_rotation: codes, nu, gamma and the encoder's u [n][d] (on the GPU)."""
    n = xd.shape[0]
    codes = torch.full((n * (st.d // 32) * st.b,), -1, dtype=torch.int32, device=DEV)
    nu = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    gamma = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    u = torch.full((n * st.d,), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_quantize_with_rotation(st.params, st.d, st.b, xd, codes, nu, gamma, u)
    torch.cuda.synchronize()
    return codes, nu, gamma, u.view(n, st.d)


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
    Rules: every returned score within TOPK_SCORE_TOL * scale of the oracle's score of that
    key (float32 estimates); scores non-increasing; the returned set equals the oracle's top-k
    except swaps between keys whose oracle scores differ by at most 4x the largest score error
    seen for that query, i.e. by float32 rounding.  Returns (max relative score error, number
    of queries with swaps).
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
        assert rel.max() <= TOPK_SCORE_TOL, (a, float(rel.max()))
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
