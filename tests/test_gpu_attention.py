"""GPU decode attention over a TurboQuant KV cache vs the oracle.

Values: tq_quantize_mse against oracle.quantize_mse (index decisions within the 1e-5 band
of a threshold excused, as for the keys).  Attention: tq_attention against
oracle.attention_decode fed the GPU's own key and value codes (end to end, logit tolerance
propagated through the softmax), and against the oracle fed the GPU's own logits (the value
aggregation alone, float32 accumulation bound).
"""
import math

import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu
DEV = U.DEV


def _mse_quantize(st, xd, n):
    codes = torch.full((n * (st.d // 32) * (st.b - 1),), -1, dtype=torch.int32, device=DEV)
    nu = torch.full((n,), float("nan"), dtype=torch.float32, device=DEV)
    tq.tq_quantize_mse(st.params, st.d, st.b, xd, codes, nu)
    torch.cuda.synchronize()
    return codes, nu


def _idx_report(st, x64, idx_g):
    _, _, u = oracle.normalize_rotate(x64, st.Pi)
    idx_o = oracle.bucketize(u, st.t_or)
    rows, cols = np.nonzero(idx_g != idx_o)
    unexcused = 0
    for r, c in zip(rows, cols):
        lo, hi = sorted((idx_g[r, c], idx_o[r, c]))
        taus = st.t_or[lo:hi]
        if not taus.size or np.min(np.abs(u[r, c] - taus)) > U.EXCUSE_U:
            unexcused += 1
    return unexcused, rows.size


@pytest.mark.parametrize("d,b,bf16", [(128, 4, True), (128, 2, False), (192, 3, True), (1536, 4, False)])
def test_quantize_mse_parity(d, b, bf16):
    n = 1500 + 17
    st = U.make_setup(d, b, cfg=40)
    x = gen.unit_sphere(n, d, cfg=40, role=gen.ROLE_DATA) * 3.0
    if bf16:
        x = gen.f32_to_bf16_bits(x)
    codes, nu = _mse_quantize(st, U.to_device(x, bf16), n)
    idx_g = oracle.unpack_index_planes(codes.cpu().numpy().view(np.uint32).reshape(n, d // 32, b - 1), b - 1)
    x64 = U.host64(x, bf16)
    unexcused, mism = _idx_report(st, x64, idx_g)
    print(f"[mse d={d} b={b}] index mismatches {mism}, unexcused {unexcused}", flush=True)
    assert unexcused == 0 and mism <= 1e-4 * idx_g.size
    nu_o = np.linalg.norm(x64, axis=1)
    assert np.max(np.abs(nu.cpu().numpy() - nu_o) / nu_o) < 1e-6
    # the same GEMM and bucketization as tq_quantize (fused at d = 128, tiled otherwise):
    # identical index planes
    if True:
        ck, _, _ = U.gpu_quantize(st, U.to_device(x, bf16))
        idx_k, _ = oracle.unpack_codes(U.codes_np(ck, n, d, b), b)
        assert np.array_equal(idx_k, idx_g)


def _kv_case(d, b_k, b_v, groups, G, T, cfg, q_bf16=True, zero_values=(), variant=""):
    # variant "sphere": exact sphere-law codebooks for keys and values; "orth": orthogonal
    # QJL matrix for the keys
    stk = U.make_setup(d, b_k, cfg=cfg, sphere="sphere" in variant, orthogonal_s="orth" in variant)
    stv = U.make_setup(d, b_v, cfg=cfg + 1, sphere="sphere" in variant)
    chans = gen.outlier_channels(cfg, groups, d)
    keys = np.concatenate([gen.kv_keys_chunk(cfg, 0, h, T, d, chans[h]) for h in range(groups)])
    vals = np.concatenate([gen.kv_keys_chunk(cfg, 1, h, T, d, chans[h], scale=1.0) for h in range(groups)])
    for t in zero_values:
        vals[t] = 0
    q = gen.kv_queries(cfg, 1, groups * G, d)[0]
    if not q_bf16:
        q = gen.bf16_bits_to_f32(q)
    ck, nk, gk = U.gpu_quantize(stk, U.to_device(keys, True))
    cv, nv = _mse_quantize(stv, U.to_device(vals, True), groups * T)
    return stk, stv, q, ck, nk, gk, cv, nv


def _gpu_attention(stk, stv, d, q, q_bf16, ck, nk, gk, cv, nv, groups, G, T, scale, mode):
    out = torch.full((groups * G * d,), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_attention_ws_bytes(d, stk.b, groups, G, T), dtype=torch.uint8, device=DEV)
    tq.tq_attention(stk.params, stv.params, d, stk.b, stv.b, U.to_device(q, q_bf16), ck, nk, gk, cv, nv,
                    groups, G, T, scale, mode, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(groups, G, d)


def _oracle_parts(stk, stv, d, q, q_bf16, ck, nk, gk, cv, nv, groups, G, T, mode):
    n = groups * T
    idx_k, z_k = oracle.unpack_codes(U.codes_np(ck, n, d, stk.b), stk.b)
    nuk, gak = nk.cpu().numpy().astype(np.float64), gk.cpu().numpy().astype(np.float64)
    q64 = U.host64(q, q_bf16).reshape(groups, G, d)
    name = "prod" if mode == tq.TQ_EST_PROD else "mse"
    logits = np.stack([oracle.estimate_ip(q64[g], stk.Pi, stk.S, idx_k[g * T:(g + 1) * T],
                                          z_k[g * T:(g + 1) * T], nuk[g * T:(g + 1) * T],
                                          gak[g * T:(g + 1) * T], stk.c_or, name, alpha=stk.alpha)
                       for g in range(groups)])
    idx_v = oracle.unpack_index_planes(cv.cpu().numpy().view(np.uint32).reshape(n, d // 32, stv.b - 1),
                                       stv.b - 1)
    vhat = oracle.dequantize_mse(stv.Pi, idx_v, nv.cpu().numpy(), stv.c_or).reshape(groups, T, d)
    return logits, vhat, q64


@pytest.mark.parametrize("d,b_k,b_v,G,T,q_bf16,mode,variant", [
    (128, 4, 4, 4, 1000, True, tq.TQ_EST_PROD, ""),
    (128, 3, 3, 4, 257, False, tq.TQ_EST_MSE, ""),
    (128, 4, 2, 5, 600, True, tq.TQ_EST_PROD, ""),
    (64, 3, 4, 3, 300, True, tq.TQ_EST_PROD, ""),
    (256, 2, 3, 4, 513, False, tq.TQ_EST_PROD, ""),
    (128, 4, 3, 4, 700, True, tq.TQ_EST_PROD, "sphere+orth"),
    (128, 2, 3, 8, 777, False, tq.TQ_EST_PROD, ""),
    (128, 3, 2, 12, 1333, True, tq.TQ_EST_PROD, ""),
    (128, 4, 4, 4, 256, False, tq.TQ_EST_MSE, ""),
    (128, 2, 4, 4, 65, True, tq.TQ_EST_PROD, ""),
    (192, 3, 4, 2, 333, True, tq.TQ_EST_PROD, "sphere+orth"),
    (1024, 3, 3, 4, 300, False, tq.TQ_EST_PROD, ""),     # the largest d of the four-wave combine
    (1536, 4, 3, 4, 300, False, tq.TQ_EST_PROD, "")])    # d > 1024: the 1024-thread combine
def test_attention_parity(d, b_k, b_v, G, T, q_bf16, mode, variant):
    groups = 3
    scale = 1.0 / math.sqrt(d)
    stk, stv, q, ck, nk, gk, cv, nv = _kv_case(d, b_k, b_v, groups, G, T, cfg=41, q_bf16=q_bf16,
                                               zero_values=(5, T + 7), variant=variant)
    out = _gpu_attention(stk, stv, d, q, q_bf16, ck, nk, gk, cv, nv, groups, G, T, scale, mode)
    assert np.all(np.isfinite(out))
    logits, vhat, q64 = _oracle_parts(stk, stv, d, q, q_bf16, ck, nk, gk, cv, nv, groups, G, T, mode)
    ref = oracle.attention_decode(logits, vhat, scale)
    vmax = float(np.max(nv.cpu().numpy()))
    lg = U.gpu_score(stk, U.to_device(q, q_bf16), ck, nk, gk, groups, G, T, mode)
    # the GPU logits stay within the scoring path's own error bound of the oracle's ...
    dl = np.abs(lg.astype(np.float64) - logits)
    nk_h, gk_h = nk.cpu().numpy(), gk.cpu().numpy()
    for g in range(groups):
        sl = slice(g * T, (g + 1) * T)
        assert np.all(dl[g] <= U.logit_bound(stk, q64[g], nk_h[sl], gk_h[sl],
                                             "prod" if mode == tq.TQ_EST_PROD else "mse"))
    # ... and a logit error delta moves each softmax weight by at most a factor
    # exp(2 scale delta); outputs are convex sums of values of norm <= max nu_v
    tol = (math.exp(2 * scale * float(dl.max())) - 1.0) * vmax + 2e-5 * vmax
    err = float(np.max(np.abs(out - ref)))
    # the aggregation alone: the oracle fed the GPU's own logits
    ref_own = oracle.attention_decode(lg.astype(np.float64), vhat, scale)
    err_own = float(np.max(np.abs(out - ref_own)))
    print(f"[attention d={d} bk={b_k} bv={b_v} G={G} T={T} mode={mode}] err {err / vmax:.2e} "
          f"(bound {tol / vmax:.2e}), own-logit err {err_own / vmax:.2e}", flush=True)
    assert err <= tol
    assert err_own <= 2e-5 * vmax


def test_attention_single_key_returns_that_value():
    d, groups, G, T = 128, 2, 4, 1
    stk, stv, q, ck, nk, gk, cv, nv = _kv_case(d, 4, 4, groups, G, T, cfg=42)
    out = _gpu_attention(stk, stv, d, q, True, ck, nk, gk, cv, nv, groups, G, T, 0.1, tq.TQ_EST_PROD)
    _, vhat, _ = _oracle_parts(stk, stv, d, q, True, ck, nk, gk, cv, nv, groups, G, T, tq.TQ_EST_PROD)
    for g in range(groups):
        for h in range(G):
            assert np.max(np.abs(out[g, h] - vhat[g, 0])) <= 1e-5 * np.max(np.abs(vhat[g, 0]))


def test_attention_long_sequence_many_blocks():
    # 40000 keys per group: 157 key blocks merged per head
    d, groups, G, T = 128, 2, 4, 40000
    scale = 1.0 / math.sqrt(d)
    stk, stv, q, ck, nk, gk, cv, nv = _kv_case(d, 3, 4, groups, G, T, cfg=43)
    out = _gpu_attention(stk, stv, d, q, True, ck, nk, gk, cv, nv, groups, G, T, scale, tq.TQ_EST_PROD)
    lg = U.gpu_score(stk, U.to_device(q, True), ck, nk, gk, groups, G, T, tq.TQ_EST_PROD)
    _, vhat, _ = _oracle_parts(stk, stv, d, q, True, ck, nk, gk, cv, nv, groups, G, T, tq.TQ_EST_PROD)
    ref = oracle.attention_decode(lg.astype(np.float64), vhat, scale)
    vmax = float(np.max(nv.cpu().numpy()))
    err = float(np.max(np.abs(out - ref)))
    print(f"[attention long T={T}] own-logit err {err / vmax:.2e}", flush=True)
    assert err <= 2e-5 * vmax


@pytest.mark.parametrize("d,bf16", [(128, True), (192, False)])
def test_append_matches_oracle_and_bulk_encoding(d, bf16):
    # a cache filled token by token through tq_append holds, in every written slot, the
    # oracle's encoding of that token (keys: oracle.quantize, values: oracle.quantize_mse,
    # under the excuse rule of the bulk parity tests) and the bulk encoders' bytes; slots not
    # yet written keep their contents
    groups, T, b = 3, 40, 4
    st = U.make_setup(d, b, cfg=44)
    x = gen.unit_sphere(groups * T, d, cfg=44, role=gen.ROLE_DATA) * 2.0
    if bf16:
        x = gen.f32_to_bf16_bits(x)
    xd = U.to_device(x, bf16).reshape(groups, T, d)
    bulk_c, bulk_n, bulk_g = U.gpu_quantize(st, U.to_device(x, bf16))
    bulk_vc, bulk_vn = _mse_quantize(st, U.to_device(x, bf16), groups * T)
    W = d // 32
    ck = torch.full((groups * T * W * b,), -1, dtype=torch.int32, device=DEV)
    nk = torch.full((groups * T,), -1.0, dtype=torch.float32, device=DEV)
    gk = torch.full((groups * T,), -1.0, dtype=torch.float32, device=DEV)
    cv = torch.full((groups * T * W * (b - 1),), -1, dtype=torch.int32, device=DEV)
    nv = torch.full((groups * T,), -1.0, dtype=torch.float32, device=DEV)
    ws = torch.empty(tq.tq_append_ws_bytes(d, b, groups), dtype=torch.uint8, device=DEV)
    filled = [t for t in range(T) if t != 17]      # slot 17 stays empty
    for t in filled:
        tok = xd[:, t, :].contiguous()
        tq.tq_append(st.params, d, b, tq.TQ_EST_PROD, tok, T, t, ck, nk, gk, ws)
        tq.tq_append(st.params, d, b, tq.TQ_EST_MSE, tok, T, t, cv, nv, None, ws)
    torch.cuda.synchronize()
    rows = np.array([g * T + t for g in range(groups) for t in filled])
    empty = np.array([g * T + 17 for g in range(groups)])
    ckn = ck.cpu().numpy().reshape(groups * T, W * b)
    cvn = cv.cpu().numpy().reshape(groups * T, W * (b - 1))
    assert np.array_equal(ckn[rows], bulk_c.cpu().numpy().reshape(groups * T, W * b)[rows])
    assert np.array_equal(cvn[rows], bulk_vc.cpu().numpy().reshape(groups * T, W * (b - 1))[rows])
    for got, ref in ((nk, bulk_n), (gk, bulk_g), (nv, bulk_vn)):
        assert np.array_equal(got.cpu().numpy()[rows], ref.cpu().numpy()[rows])
        assert np.all(got.cpu().numpy()[empty] == -1.0)
    assert np.all(ckn[empty] == -1) and np.all(cvn[empty] == -1)
    # against the oracle, slot by slot: token t of group g sits at row g * T + t
    x64 = U.host64(x, bf16)[rows]
    rep = U.compare_codes(st, x64, ckn[rows].view(np.uint32).reshape(rows.size, W, b),
                          nk.cpu().numpy()[rows], gk.cpu().numpy()[rows])
    print(f"[append d={d}] keys vs oracle: {U.describe(rep)}", flush=True)
    U.assert_codes_ok(rep)
    idx_v = oracle.unpack_index_planes(cvn[rows].view(np.uint32).reshape(rows.size, W, b - 1), b - 1)
    unexcused, mism = _idx_report(st, x64, idx_v)
    print(f"[append d={d}] values vs oracle: index mismatches {mism}, unexcused {unexcused}", flush=True)
    assert unexcused == 0 and mism <= 1e-4 * idx_v.size
    nu_o = np.linalg.norm(x64, axis=1)
    assert np.max(np.abs(nv.cpu().numpy()[rows] - nu_o) / nu_o) <= 1e-5
