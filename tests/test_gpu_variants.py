"""GPU parity of the method variants against the oracle run with the same variant: the
Lloyd-Max codebook of the exact sphere law (tq_codebook_build_sphere) and an orthogonal QJL
matrix (tq_prepare_orthogonal_qjl), through every call that reads them: both encoders, both
scoring kernels, dequantize, the fused top-k scan and the large-k path."""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu

# (sphere codebook, orthogonal S)
VARIANTS = [(True, False), (False, True), (True, True)]


def _name(sphere, orth):
    return "+".join(n for n, on in (("sphere", sphere), ("orth", orth)) if on)


@pytest.mark.parametrize("sphere,orth", VARIANTS)
@pytest.mark.parametrize("d,b,G,bf16", [(128, 4, 4, False), (128, 2, 8, True), (128, 3, 3, False),
                                        (256, 3, 5, False), (1536, 4, 2, True)])
def test_quantize_and_score_variants(d, b, G, bf16, sphere, orth):
    # d = 128 with G % 4 == 0 takes the fused encoder and the d = 128 scoring kernel; G = 3
    # and d != 128 the general scoring kernel; d != 128 the tiled encoder
    cfg = 50 + b
    st = U.make_setup(d, b, cfg=cfg, sphere=sphere, orthogonal_s=orth)
    n = 1500 + 13
    x = gen.unit_sphere(n, d, cfg=cfg, role=gen.ROLE_DATA) * np.float32(2.0)
    if bf16:
        x = gen.f32_to_bf16_bits(x)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, bf16))
    rep = U.compare_codes(st, U.host64(x, bf16), U.codes_np(codes, n, d, b), nu.cpu().numpy(),
                          gamma.cpu().numpy())
    print(f"[variant {_name(sphere, orth)} d={d} b={b}] {U.describe(rep)}", flush=True)
    U.assert_codes_ok(rep)
    q = gen.unit_sphere(G, d, cfg=cfg, role=gen.ROLE_QUERY) * np.float32(1.5)
    q64 = q.astype(np.float64).reshape(1, G, d)
    for mode, name in ((tq.TQ_EST_PROD, "prod"), (tq.TQ_EST_MSE, "mse")):
        lg = U.gpu_score(st, U.to_device(q, False), codes, nu, gamma, 1, G, n, mode)
        err = U.logit_errors(st, q64, rep["idx"], rep["z"], nu.cpu().numpy(), gamma.cpu().numpy(),
                             lg, name)
        print(f"  score {name}: max |dl|/(|q|nu) = {err:.2e}", flush=True)


@pytest.mark.parametrize("sphere,orth", VARIANTS)
def test_dequantize_variants(sphere, orth):
    d, b, n = 128, 3, 400
    st = U.make_setup(d, b, cfg=57, sphere=sphere, orthogonal_s=orth)
    x = gen.unit_sphere(n, d, cfg=57, role=gen.ROLE_DATA) * np.float32(3.0)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, d, b), b)
    for mode, name in ((tq.TQ_EST_PROD, "prod"), (tq.TQ_EST_MSE, "mse")):
        xhat = torch.full((n * d,), float("nan"), dtype=torch.float32, device=U.DEV)
        tq.tq_dequantize(st.params, d, b, codes, nu, gamma, mode, xhat)
        torch.cuda.synchronize()
        ref = oracle.dequantize(st.Pi, st.S, idx, z, nu.cpu().numpy(), gamma.cpu().numpy(), st.c_or,
                                name, alpha=st.alpha)
        err = np.max(np.abs(xhat.cpu().numpy().reshape(n, d) - ref)) / 3.0
        assert err <= 1e-5, (name, err)


@pytest.mark.parametrize("d,b,n,nq,k", [(128, 4, 6000, 40, 10), (128, 2, 3001, 9, 32),
                                        (256, 3, 4000, 5, 100)])
def test_topk_variants(d, b, n, nq, k):
    # k <= 32: the fused MFMA scan (its key operand carries sqrt(d) alpha gamma, alpha from
    # the parameter header); k = 100: the scoring + radix-select path
    st = U.make_setup(d, b, cfg=58, sphere=True, orthogonal_s=True)
    x = gen.unit_sphere(n, d, cfg=58, role=gen.ROLE_DATA)
    q = gen.unit_sphere(nq, d, cfg=58, role=gen.ROLE_QUERY)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, d, b), b)
    q64 = q.astype(np.float64)
    nu_h, ga_h = nu.cpu().numpy(), gamma.cpu().numpy()
    for mode, name in ((tq.TQ_EST_PROD, "prod"), (tq.TQ_EST_MSE, "mse")):
        idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, mode)
        ref = oracle.estimate_ip(q64, st.Pi, st.S, idx, z, nu_h, ga_h, st.c_or, name, alpha=st.alpha)
        scale = np.linalg.norm(q64, axis=1)[:, None] * np.maximum(nu_h[None, :], 1e-30)
        worst, swapped = U.check_topk(idx_g, sc_g, ref, scale)
        print(f"[topk variant d={d} b={b} k={k} {name}] max err {worst:.2e} swaps {swapped}", flush=True)
        assert worst <= U.TOPK_SCORE_TOL


def test_orthogonal_and_gaussian_scales_differ():
    # the same codes scored under the two preparations differ exactly in the QJL term's
    # scale: (l_orth - l_mse) / (l_gauss - l_mse) = alpha_orth / alpha_gauss for every key
    d, b, n, G = 128, 4, 700, 4
    Pi = gen.haar_orthogonal(d, 59)
    S = gen.haar_orthogonal(d, 59, role=gen.ROLE_S)
    c, t = tq.tq_codebook_build(b - 1, d)
    pg = torch.empty(tq.tq_params_bytes(d, b), dtype=torch.uint8, device=U.DEV)
    po = torch.empty_like(pg)
    tq.tq_prepare(d, b, Pi, S, c, t, pg)
    tq.tq_prepare_orthogonal_qjl(d, b, Pi, S, c, t, po)
    c_or, t_or = oracle.codebook(b - 1, d)
    stg = U.Setup(d, b, Pi, S, c_or, t_or, pg, None)
    sto = U.Setup(d, b, Pi, S, c_or, t_or, po, oracle.qjl_alpha_orthogonal(d, d))
    x = gen.unit_sphere(n, d, cfg=59, role=gen.ROLE_DATA)
    codes, nu, gamma = U.gpu_quantize(stg, U.to_device(x, False))
    codes_o, _, _ = U.gpu_quantize(sto, U.to_device(x, False))
    assert torch.equal(codes, codes_o)            # the encoder does not read alpha
    q = gen.unit_sphere(G, d, cfg=59, role=gen.ROLE_QUERY)
    qd = U.to_device(q, False)
    lg = U.gpu_score(stg, qd, codes, nu, gamma, 1, G, n, tq.TQ_EST_PROD).astype(np.float64)
    lo = U.gpu_score(sto, qd, codes, nu, gamma, 1, G, n, tq.TQ_EST_PROD).astype(np.float64)
    lm = U.gpu_score(stg, qd, codes, nu, gamma, 1, G, n, tq.TQ_EST_MSE).astype(np.float64)
    ratio = oracle.qjl_alpha_orthogonal(d, d) / oracle.qjl_alpha(d)
    qjl_g, qjl_o = lg - lm, lo - lm
    big = np.abs(qjl_g) > 0.25 * np.max(np.abs(qjl_g))
    assert np.max(np.abs(qjl_o[big] / qjl_g[big] - ratio)) < 1e-2 * ratio
