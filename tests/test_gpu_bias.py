"""Bias of the MSE-only and MSE+QJL logits over 100 random (Pi, S) pairs.

Workload: 16 sequences x 8 KV heads x 8192 tokens, d = 128, bf16 keys with outlier
channels, 32 query heads per sequence, b = 2 and 3 ([review, experiments] and [news, bias
paragraph]: the MSE-optimal quantizer gives biased inner products; the 1-bit QJL residual
removes the bias).  For each seed s the slope beta_s = sum_p e_p l_s(p) / sum_p e_p^2 over
all (query head, key) pairs p, with e_p the exact <q, k>.  For a Haar rotation the rotated
key is uniform on the sphere whatever the key, so E[beta] = kappa = d E[u Q(u)] for the
MSE-only estimate (sphere quadrature below) and exactly 1 for MSE+QJL.

The QJL variants are compared on the same keys and rotations: a Gaussian S (sqrt(pi/2)/m
scale) and a Haar orthogonal S (1/(m E|w_1|) scale, [review, QJL paragraph]).  Both must be
unbiased; the mean squared logit error sum_p (l_s(p) - e_p)^2 / sum_p e_p^2 over the seeds
measures their variance.
"""
import math

import numpy as np
import pytest
import torch
from scipy import integrate, special

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu

SEEDS = 100


def _kappa(d, bits_mse):
    c, t = oracle.codebook(bits_mse, d)
    logc = special.gammaln(d / 2.0) - 0.5 * math.log(math.pi) - special.gammaln((d - 1) / 2.0)
    f = lambda x: math.exp(logc + 0.5 * (d - 3) * math.log1p(-x * x))
    edges = [-1.0] + list(t) + [1.0]
    return d * sum(ci * integrate.quad(lambda x: x * f(x), edges[i], edges[i + 1], epsabs=1e-14)[0]
                   for i, ci in enumerate(c))


@pytest.mark.timeout(900)
def test_bias_over_100_seeds():
    w = gen.DECODE_BATCH16
    d, T, G = w.d, w.T, w.G
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    keys = np.concatenate([gen.kv_keys_chunk(w.cfg, s, h, T, d, chans[h])
                           for s in range(w.n_seq) for h in range(w.n_kv)])
    q = gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d).reshape(-1, d)
    xd = U.to_device(keys, True)
    qd = U.to_device(q, True)
    # exact logits e_p (float32 on the GPU from the exact bf16 values)
    kf = xd.float().view(w.groups, T, d)
    qf = qd.float().view(w.groups, G, d)
    exact = torch.bmm(qf, kf.transpose(1, 2).contiguous())
    ee = float((exact.double() ** 2).sum())
    n = w.n_keys
    lines = []
    for b in w.bits:
        kappa = _kappa(d, b - 1)
        slopes = {tq.TQ_EST_MSE: [], tq.TQ_EST_PROD: [], "orth": []}
        err2 = {tq.TQ_EST_PROD: [], "orth": []}
        codes = torch.empty(n * (d // 32) * b, dtype=torch.int32, device=U.DEV)
        nu = torch.empty(n, device=U.DEV)
        gamma = torch.empty(n, device=U.DEV)
        logits = torch.empty(w.groups * G * T, device=U.DEV)
        ws = torch.empty(tq.tq_score_ws_bytes(d, b, w.groups, G, T), dtype=torch.uint8, device=U.DEV)
        c, t = tq.tq_codebook_build(b - 1, d)
        params = torch.empty(tq.tq_params_bytes(d, b), dtype=torch.uint8, device=U.DEV)
        for rep in range(SEEDS):
            Pi = gen.haar_orthogonal(d, w.cfg, rep)
            for kind in ("gauss", "orth"):
                if kind == "gauss":
                    tq.tq_prepare(d, b, Pi, gen.gaussian_matrix(d, d, w.cfg, rep), c, t, params)
                else:
                    tq.tq_prepare_orthogonal_qjl(d, b, Pi, gen.haar_orthogonal(d, w.cfg, rep, role=gen.ROLE_S),
                                                 c, t, params)
                tq.tq_quantize(params, d, b, xd, codes, nu, gamma)
                for mode in ((tq.TQ_EST_MSE, tq.TQ_EST_PROD) if kind == "gauss" else (tq.TQ_EST_PROD,)):
                    tq.tq_score_ip(params, d, b, qd, codes, nu, gamma, w.groups, G, T, mode, logits, ws)
                    lv = logits.view(w.groups, G, T).double()
                    key = "orth" if kind == "orth" else mode
                    slopes[key].append(float((exact.double() * lv).sum()) / ee)
                    if mode == tq.TQ_EST_PROD:
                        err2[key].append(float(((lv - exact.double()) ** 2).sum()) / ee)
        for mode, name in ((tq.TQ_EST_MSE, "MSE-only"), (tq.TQ_EST_PROD, "MSE+QJL"), ("orth", "MSE+QJL orthogonal S")):
            s = np.array(slopes[mode])
            mean, se = s.mean(), s.std(ddof=1) / math.sqrt(len(s))
            expect = kappa if mode == tq.TQ_EST_MSE else 1.0
            lines.append(f"b={b} {name:8s}: slope {mean:.5f} +- {se:.5f} (SE, {SEEDS} seeds); expected {expect:.5f}")
            print(lines[-1], flush=True)
            assert abs(mean - expect) <= 4 * se + 1e-4, (b, name, mean, se, expect)
        ms = np.array(slopes[tq.TQ_EST_MSE])
        assert 1.0 - ms.mean() > 20 * ms.std(ddof=1) / math.sqrt(SEEDS)   # clearly biased
        eg, eo = np.array(err2[tq.TQ_EST_PROD]), np.array(err2["orth"])
        lines.append(f"b={b} relative mean squared logit error: Gaussian S {eg.mean():.5f} +- "
                     f"{eg.std(ddof=1) / math.sqrt(SEEDS):.5f}, orthogonal S {eo.mean():.5f} +- "
                     f"{eo.std(ddof=1) / math.sqrt(SEEDS):.5f} (ratio {eo.mean() / eg.mean():.3f})")
        print(lines[-1], flush=True)
        assert eo.mean() < eg.mean()
