"""GPU parity: HIP path vs the CPU oracle on identical seeded inputs (MI355X only)."""
import math

import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def _report(tag, rep):
    print(f"[{tag}] {U.describe(rep)}", flush=True)


# ------------------------------------------------------------------------- quantize

@pytest.mark.parametrize("n", [4096, 4096 - 37, 1, 33])
def test_quantize_toy_f32(n):
    # Toy workload: unit vectors in R^128 (float32), b = 4.
    st = U.make_setup(128, 4, cfg=0)
    x = gen.unit_sphere(n, 128, cfg=0, role=gen.ROLE_DATA)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    rep = U.compare_codes(st, U.host64(x, False), U.codes_np(codes, n, 128, 4),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report(f"toy n={n}", rep)
    U.assert_codes_ok(rep)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_quantize_kv_bf16_outliers(b):
    # KV keys: N(0,1) bf16 with 4 outlier channels per head (x20); 3 heads x 1000 tokens.
    st = U.make_setup(128, b, cfg=1)
    chans = gen.outlier_channels(1, 3, 128)
    keys = np.concatenate([gen.kv_keys_chunk(1, 0, h, 1000, 128, chans[h]) for h in range(3)])
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(keys, True))
    rep = U.compare_codes(st, U.host64(keys, True), U.codes_np(codes, keys.shape[0], 128, b),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report(f"kv b={b}", rep)
    U.assert_codes_ok(rep)


@pytest.mark.parametrize("b", [2, 3, 4])
def test_quantize_f32_nonunit(b):
    st = U.make_setup(128, b, cfg=5)
    x = gen.unit_sphere(2000, 128, cfg=5, role=gen.ROLE_DATA) * np.float32(7.5)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    rep = U.compare_codes(st, U.host64(x, False), U.codes_np(codes, 2000, 128, b),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report(f"f32 nonunit b={b}", rep)
    U.assert_codes_ok(rep)


@pytest.mark.parametrize("d", [128, 192])     # the fused encoder and the tiled one
def test_quantize_zero_vectors_and_empty(d):
    st = U.make_setup(d, 4, cfg=6)
    x = gen.unit_sphere(40, d, cfg=6, role=gen.ROLE_DATA)
    x[[0, 7, 39]] = 0.0
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    rep = U.compare_codes(st, U.host64(x, False), U.codes_np(codes, 40, d, 4),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    U.assert_codes_ok(rep)
    assert nu.cpu().numpy()[[0, 7, 39]].tolist() == [0.0, 0.0, 0.0]
    # zero vector: all indices L/2 (u = 0 sits on the middle threshold, upper cell)
    assert np.all(rep["idx"][[0, 7, 39]] == 4)
    # n = 0: no-op
    e = torch.empty((0, d), dtype=torch.float32, device=U.DEV)
    z = torch.empty(0, dtype=torch.int32, device=U.DEV)
    f = torch.empty(0, dtype=torch.float32, device=U.DEV)
    tq.tq_quantize(st.params, d, 4, e, z, f, f)


@pytest.mark.parametrize("d", [128, 192])
def test_quantize_nonfinite_inputs_do_not_fault(d):
    # a vector with a NaN or an infinite coordinate gets unspecified codes; every other vector
    # of the launch is encoded as usual
    st = U.make_setup(d, 3, cfg=7)
    x = gen.unit_sphere(300, d, cfg=7, role=gen.ROLE_DATA)
    x[3, 5] = np.nan
    x[9, 0] = np.inf
    x[290, d - 1] = -np.inf
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    good = np.array([i not in (3, 9, 290) for i in range(300)])
    rep = U.compare_codes(st, U.host64(x[good], False),
                          U.codes_np(codes, 300, d, 3)[good], nu.cpu().numpy()[good],
                          gamma.cpu().numpy()[good])
    U.assert_codes_ok(rep)


# --------------------------------------------------------------------------- scoring

def _kv_case(b, cfg, groups, T, G=4):
    st = U.make_setup(128, b, cfg=cfg)
    chans = gen.outlier_channels(cfg, groups, 128)
    keys = np.concatenate([gen.kv_keys_chunk(cfg, 0, h, T, 128, chans[h]) for h in range(groups)])
    q = gen.kv_queries(cfg, 1, groups * G, 128)[0]
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(keys, True))
    cn = U.codes_np(codes, groups * T, 128, b)
    idx, z = oracle.unpack_codes(cn, b)
    q64 = U.host64(q, True).reshape(groups, G, 128)
    return st, keys, q, codes, nu, gamma, idx, z, q64


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("mode", [tq.TQ_EST_PROD, tq.TQ_EST_MSE])
def test_score_kv_parity(b, mode):
    groups, T = 3, 1000
    st, keys, q, codes, nu, gamma, idx, z, q64 = _kv_case(b, 11, groups, T)
    lg = U.gpu_score(st, U.to_device(q, True), codes, nu, gamma, groups, 4, T, mode)
    err = U.logit_errors(st, q64, idx, z, nu.cpu().numpy(), gamma.cpu().numpy(), lg,
                         "prod" if mode == tq.TQ_EST_PROD else "mse")
    print(f"[score b={b} mode={mode}] max |dl|/(|q|nu) = {err:.2e}", flush=True)


@pytest.mark.parametrize("T", [1, 15, 17, 257])
def test_score_ragged_lengths(T):
    groups = 2
    st, keys, q, codes, nu, gamma, idx, z, q64 = _kv_case(4, 12, groups, T)
    lg = U.gpu_score(st, U.to_device(q, True), codes, nu, gamma, groups, 4, T, tq.TQ_EST_PROD)
    err = U.logit_errors(st, q64, idx, z, nu.cpu().numpy(), gamma.cpu().numpy(), lg)


def test_score_wide_group_f32_queries():
    # Toy workload: 64 unit queries against 4096 unit keys in one group (G = 64), float32.
    st = U.make_setup(128, 4, cfg=0)
    x = gen.unit_sphere(4096, 128, cfg=0, role=gen.ROLE_DATA)
    q = gen.unit_sphere(64, 128, cfg=0, role=gen.ROLE_QUERY)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx, z = oracle.unpack_codes(U.codes_np(codes, 4096, 128, 4), 4)
    lg = U.gpu_score(st, U.to_device(q, False), codes, nu, gamma, 1, 64, 4096, tq.TQ_EST_PROD)
    err = U.logit_errors(st, q.astype(np.float64)[None], idx, z, nu.cpu().numpy(),
                         gamma.cpu().numpy(), lg)
    print(f"[score toy G=64] max err {err:.2e}", flush=True)


@pytest.mark.parametrize("d,b,G,T,bf16", [
    (64, 4, 4, 300, True), (192, 3, 3, 257, False), (256, 2, 5, 1000, True),
    (128, 4, 3, 513, True), (128, 3, 1, 77, False), (1024, 4, 2, 260, False)])
@pytest.mark.parametrize("mode", [tq.TQ_EST_PROD, tq.TQ_EST_MSE])
def test_score_general_shapes(d, b, G, T, bf16, mode):
    # shapes outside the tuned kernel (d != 128, or G not a multiple of 4): the general path
    groups = 3
    st = U.make_setup(d, b, cfg=14)
    chans = gen.outlier_channels(14, groups, d)
    keys = np.concatenate([gen.kv_keys_chunk(14, 0, h, T, d, chans[h]) for h in range(groups)])
    q = gen.kv_queries(14, 1, groups * G, d)[0]
    if not bf16:
        q = gen.bf16_bits_to_f32(q)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(keys, True))
    idx, z = oracle.unpack_codes(U.codes_np(codes, groups * T, d, b), b)
    lg = U.gpu_score(st, U.to_device(q, bf16), codes, nu, gamma, groups, G, T, mode)
    q64 = U.host64(q, bf16).reshape(groups, G, d)
    err = U.logit_errors(st, q64, idx, z, nu.cpu().numpy(), gamma.cpu().numpy(), lg,
                         "prod" if mode == tq.TQ_EST_PROD else "mse")
    print(f"[score general d={d} b={b} G={G} T={T} mode={mode}] max err {err:.2e}", flush=True)
    assert np.all(np.isfinite(lg))


def test_score_zero_keys_give_zero_logits():
    st = U.make_setup(128, 3, cfg=13)
    x = gen.unit_sphere(64, 128, cfg=13, role=gen.ROLE_DATA)
    x[[2, 50]] = 0.0
    q = gen.unit_sphere(4, 128, cfg=13, role=gen.ROLE_QUERY)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    lg = U.gpu_score(st, U.to_device(q, False), codes, nu, gamma, 1, 4, 64, tq.TQ_EST_PROD)
    assert np.all(lg[0][:, [2, 50]] == 0.0)


# ------------------------------------------------------------------------ dequantize

@pytest.mark.parametrize("b", [2, 4])
@pytest.mark.parametrize("mode", [tq.TQ_EST_PROD, tq.TQ_EST_MSE])
def test_dequantize_parity(b, mode):
    st = U.make_setup(128, b, cfg=14)
    x = gen.unit_sphere(300, 128, cfg=14, role=gen.ROLE_DATA) * np.float32(3.0)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    xhat = torch.full((300 * 128,), float("nan"), dtype=torch.float32, device=U.DEV)
    tq.tq_dequantize(st.params, 128, b, codes, nu, gamma, mode, xhat)
    torch.cuda.synchronize()
    idx, z = oracle.unpack_codes(U.codes_np(codes, 300, 128, b), b)
    ref = oracle.dequantize(st.Pi, st.S, idx, z, nu.cpu().numpy(), gamma.cpu().numpy(), st.c_or,
                            "prod" if mode == tq.TQ_EST_PROD else "mse")
    err = np.max(np.abs(xhat.cpu().numpy().reshape(300, 128) - ref)) / 3.0
    assert err <= 1e-5, err


# ------------------------------------------------------- tiled encoder (d != 128)

@pytest.mark.parametrize("b,n", [(2, 3000), (4, 16384 + 300)])
def test_quantize_d1536_lowrank_f32(b, n):
    # embedding-search law (low rank + noise, unit norm, fp32), d = 1536; one chunk of the
    # tiled encoder with a ragged last row block
    st = U.make_setup(1536, b, cfg=3)
    x = gen.lowrank_vectors(n, 1536, 64, 3.0, cfg=3)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    rep = U.compare_codes(st, U.host64(x, False), U.codes_np(codes, n, 1536, b),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report(f"d1536 b={b} n={n}", rep)
    U.assert_codes_ok(rep)


def test_quantize_d1536_three_chunks_sampled():
    # 32768-vector chunks: the split rows of chunk 2 reuse chunk 0's buffers while chunk 1 is
    # encoded; rows on both sides of each chunk boundary and the ragged end are checked
    n = 2 * 32768 + 300
    st = U.make_setup(1536, 4, cfg=3)
    x = gen.lowrank_vectors(n, 1536, 64, 3.0, cfg=3)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    rows = np.r_[0:256, 32768 - 256:32768 + 256, 65536 - 256:n]
    rep = U.compare_codes(st, U.host64(x[rows], False), U.codes_np(codes, n, 1536, 4)[rows],
                          nu.cpu().numpy()[rows], gamma.cpu().numpy()[rows])
    _report(f"d1536 b=4 n={n} sampled", rep)
    U.assert_codes_ok(rep)


@pytest.mark.parametrize("bf16", [False, True])
def test_quantize_d256_four_chunks(bf16):
    # four chunks of the tiled encoder, the last one ragged, every row checked
    n = 3 * 32768 + 123
    st = U.make_setup(256, 4, cfg=5)
    x = gen.lowrank_vectors(n, 256, 32, 3.0, cfg=5)
    if bf16:
        x = gen.f32_to_bf16_bits(x)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, bf16))
    rep = U.compare_codes(st, U.host64(x, bf16), U.codes_np(codes, n, 256, 4),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report(f"d256 b=4 n={n} {'bf16' if bf16 else 'f32'}", rep)
    U.assert_codes_ok(rep)


@pytest.mark.parametrize("d,b,bf16", [(64, 4, False), (64, 2, True), (192, 3, False), (192, 4, True)])
def test_quantize_d64_multiples(d, b, bf16):
    # dimensions that are multiples of 64 but not of 128 (two and six K stages of the tiled
    # encoder, one column tile mostly padding); ragged row count
    n = 2000 + 37
    st = U.make_setup(d, b, cfg=6)
    x = gen.unit_sphere(n, d, 6, 0)
    if bf16:
        x = gen.f32_to_bf16_bits(x)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, bf16))
    rep = U.compare_codes(st, U.host64(x, bf16), U.codes_np(codes, n, d, b),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report(f"d{d} b={b} {'bf16' if bf16 else 'f32'}", rep)
    U.assert_codes_ok(rep)


def test_quantize_d256_bf16_and_zero_vectors():
    st = U.make_setup(256, 3, cfg=8)
    chans = gen.outlier_channels(8, 1, 256)
    keys = gen.kv_keys_chunk(8, 0, 0, 1000, 256, chans[0])
    keys[[0, 999]] = 0
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(keys, True))
    rep = U.compare_codes(st, U.host64(keys, True), U.codes_np(codes, 1000, 256, 3),
                          nu.cpu().numpy(), gamma.cpu().numpy())
    _report("d256 bf16 b=3", rep)
    U.assert_codes_ok(rep)
    assert nu.cpu().numpy()[[0, 999]].tolist() == [0.0, 0.0]


@pytest.mark.parametrize("d,b,G", [(128, 3, 4), (128, 4, 8), (64, 3, 3), (128, 2, 5)])
def test_score_prepared_matches_score_ip(d, b, G):
    # the query operands prepared once serve two key caches of different lengths; each scan
    # gives exactly tq_score_ip's logits (same kernels, same operands)
    groups = 5
    st = U.make_setup(d, b, cfg=81)
    q = U.to_device(gen.f32_to_bf16_bits(gen.unit_sphere(groups * G, d, cfg=81, role=gen.ROLE_QUERY) * 2.0),
                    True)
    ws = torch.empty(max(tq.tq_score_ws_bytes(d, b, groups, G, 1), 256), dtype=torch.uint8, device=U.DEV)
    tq.tq_score_prepare(st.params, d, b, q, groups, G, ws)
    for i, T in enumerate((3000, 517)):
        x = gen.f32_to_bf16_bits(gen.unit_sphere(groups * T, d, cfg=82 + i, role=gen.ROLE_DATA) * 3.0)
        codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, True))
        ref = U.gpu_score(st, q, codes, nu, gamma, groups, G, T, tq.TQ_EST_PROD)
        for mode in (tq.TQ_EST_PROD, tq.TQ_EST_MSE):
            if mode == tq.TQ_EST_MSE:
                ref = U.gpu_score(st, q, codes, nu, gamma, groups, G, T, mode)
            out = torch.full((groups * G * T,), float("nan"), dtype=torch.float32, device=U.DEV)
            tq.tq_score_ip_prepared(st.params, d, b, codes, nu, gamma, groups, G, T, mode, out, ws)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy().reshape(groups, G, T), ref), (T, mode)
