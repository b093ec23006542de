"""GPU top-k search vs the oracle's scores of every key (oracle fed the GPU's codes)."""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def _oracle_scores(st, q64, idx, z, nu, gamma, mode="prod"):
    ref = oracle.estimate_ip(q64, st.Pi, st.S, idx, z, nu, gamma, st.c_or, mode, alpha=st.alpha)
    scale = np.linalg.norm(q64, axis=1)[:, None] * np.maximum(nu[None, :], 1e-30)
    return ref, scale


@pytest.mark.parametrize("n,nq,k", [(4096, 64, 10), (5000, 130, 7), (2049, 3, 1), (3000, 17, 32), (3000, 40, 26), (3000, 40, 27), (3000, 40, 11),
                                    (9000, 300, 10)])
def test_topk_d128_gpu_codes(n, nq, k):
    # toy workload shape (unit vectors, b = 4) plus ragged tiles, query tiles and k values
    st = U.make_setup(128, 4, cfg=0)
    x = gen.unit_sphere(n, 128, cfg=0, role=gen.ROLE_DATA)
    q = gen.unit_sphere(nq, 128, cfg=0, role=gen.ROLE_QUERY)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, tq.TQ_EST_PROD)
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, 128, 4), 4)
    ref, scale = _oracle_scores(st, q.astype(np.float64), idx, z, nu.cpu().numpy(), gamma.cpu().numpy())
    worst, swapped = U.check_topk(idx_g, sc_g, ref, scale)
    print(f"[topk d=128 n={n} nq={nq} k={k}] max score err {worst:.2e}, near-tie swaps {swapped}", flush=True)
    assert worst <= U.TOPK_SCORE_TOL


def test_topk_mse_mode_and_long_key_ranges():
    # 200000 keys with one query tile: each workgroup scans several 256-key blocks, so the
    # running lists and thresholds carry across blocks before the cross-range merge
    st = U.make_setup(128, 2, cfg=31)
    n, nq, k = 200000, 9, 10
    x = gen.unit_sphere(n, 128, cfg=31, role=gen.ROLE_DATA)
    q = gen.unit_sphere(nq, 128, cfg=31, role=gen.ROLE_QUERY)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, 128, 2), 2)
    for mode, name in ((tq.TQ_EST_PROD, "prod"), (tq.TQ_EST_MSE, "mse")):
        idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, mode)
        ref, scale = _oracle_scores(st, q.astype(np.float64), idx, z, nu.cpu().numpy(),
                                    gamma.cpu().numpy(), name)
        worst, swapped = U.check_topk(idx_g, sc_g, ref, scale)
        print(f"[topk chunks mode={name}] max err {worst:.2e} swaps {swapped}", flush=True)
        assert worst <= U.TOPK_SCORE_TOL


def test_topk_b3_bf16_queries_and_zero_query():
    # KV-key law (bf16, outlier channels), b = 3, bf16 queries; query 5 is all zero, so every
    # score is 0 and the result is the k smallest indices
    st = U.make_setup(128, 3, cfg=32)
    chans = gen.outlier_channels(32, 1, 128)
    keys = gen.kv_keys_chunk(32, 0, 0, 6000, 128, chans[0])
    q = gen.kv_queries(32, 1, 12, 128)[0]
    q[5] = 0
    n, nq, k = keys.shape[0], q.shape[0], 10
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(keys, True))
    idx_g, sc_g = U.gpu_topk(st, U.to_device(q, True), codes, nu, gamma, n, k, tq.TQ_EST_PROD)
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, 128, 3), 3)
    q64 = U.host64(q, True)
    ref, scale = _oracle_scores(st, q64, idx, z, nu.cpu().numpy(), gamma.cpu().numpy())
    keep = [a for a in range(nq) if a != 5]
    worst, swapped = U.check_topk(idx_g[keep], sc_g[keep], ref[keep], scale[keep])
    print(f"[topk b=3 bf16] max err {worst:.2e} swaps {swapped}", flush=True)
    assert worst <= U.TOPK_SCORE_TOL
    assert idx_g[5].tolist() == list(range(k)) and np.all(sc_g[5] == 0.0)


@pytest.mark.parametrize("b", [2, 4])
def test_topk_d1536_oracle_codes(b):
    # embedding-search shape (d = 1536, low-rank + noise, unit norm) on codes packed by the
    # oracle: top-k alone, independent of the encoder
    d, n, nq, k = 1536, 3000, 20, 10
    st = U.make_setup(d, b, cfg=3)
    x = gen.lowrank_vectors(n, d, 64, 3.0, cfg=3)
    q = gen.lowrank_queries(nq, d, 64, 3.0, cfg=3)
    r = oracle.quantize(x.astype(np.float64), st.Pi, st.S, st.c_or, st.t_or)
    cn = oracle.pack_codes(r["idx"], r["z"], b)
    codes = torch.from_numpy(cn.view(np.int32).reshape(-1).copy()).to(U.DEV)
    nu = torch.from_numpy(r["nu"].astype(np.float32)).to(U.DEV)
    gamma = torch.from_numpy(r["gamma"].astype(np.float32)).to(U.DEV)
    idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, tq.TQ_EST_PROD)
    ref, scale = _oracle_scores(st, q.astype(np.float64), r["idx"], r["z"], nu.cpu().numpy().astype(np.float64),
                                gamma.cpu().numpy().astype(np.float64))
    worst, swapped = U.check_topk(idx_g, sc_g, ref, scale)
    print(f"[topk d=1536 b={b}] max err {worst:.2e} swaps {swapped}", flush=True)
    assert worst <= U.TOPK_SCORE_TOL


def test_topk_rejects_k_beyond_1024():
    st = U.make_setup(128, 4, cfg=0)
    x = gen.unit_sphere(2000, 128, cfg=0, role=gen.ROLE_DATA)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    with pytest.raises(tq.TQError) as e:
        U.gpu_topk(st, U.to_device(x[:2], False), codes, nu, gamma, 2000, 1025, tq.TQ_EST_PROD)
    assert e.value.status == tq.TQ_EINVAL


@pytest.mark.parametrize("d,n,nq,k,mode", [(128, 5000, 40, 33, tq.TQ_EST_PROD),
                                           (128, 3000, 7, 1024, tq.TQ_EST_MSE),
                                           (192, 2000, 5, 100, tq.TQ_EST_PROD)])
def test_topk_large_k(d, n, nq, k, mode):
    # k beyond the fused scan's lists: scores of every key, then a radix select per query;
    # query 0 is all zero, so its k results are the k smallest indices with score 0
    st = U.make_setup(d, 4, cfg=33)
    x = gen.unit_sphere(n, d, cfg=33, role=gen.ROLE_DATA)
    q = gen.unit_sphere(nq, d, cfg=33, role=gen.ROLE_QUERY)
    q[0] = 0.0
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, mode)
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, d, 4), 4)
    name = "prod" if mode == tq.TQ_EST_PROD else "mse"
    ref, scale = _oracle_scores(st, q.astype(np.float64), idx, z, nu.cpu().numpy(), gamma.cpu().numpy(),
                                name)
    assert idx_g[0].tolist() == list(range(k)) and np.all(sc_g[0] == 0.0)
    worst, swapped = U.check_topk(idx_g[1:], sc_g[1:], ref[1:], scale[1:])
    print(f"[topk large k d={d} n={n} nq={nq} k={k} {name}] max err {worst:.2e} swaps {swapped}",
          flush=True)
    assert worst <= U.TOPK_SCORE_TOL


def test_topk_large_k_two_query_batches():
    # 600000 keys: 256 MiB of scores hold 111 queries, so 150 queries run as two batches
    st = U.make_setup(128, 3, cfg=34)
    n, nq, k = 600000, 150, 50
    x = gen.unit_sphere(n, 128, cfg=34, role=gen.ROLE_DATA)
    q = gen.unit_sphere(nq, 128, cfg=34, role=gen.ROLE_QUERY)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, tq.TQ_EST_PROD)
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, 128, 3), 3)
    ref, scale = _oracle_scores(st, q.astype(np.float64), idx, z, nu.cpu().numpy(), gamma.cpu().numpy())
    worst, swapped = U.check_topk(idx_g, sc_g, ref, scale)
    print(f"[topk large k two batches] max err {worst:.2e} swaps {swapped}", flush=True)
    assert worst <= U.TOPK_SCORE_TOL


@pytest.mark.parametrize("b", [2, 4])
def test_topk_d1536_gpu_codes(b):
    # end to end at d = 1536: tiled encoder, then search
    d, n, nq, k = 1536, 5000, 40, 10
    st = U.make_setup(d, b, cfg=3)
    x = gen.lowrank_vectors(n, d, 64, 3.0, cfg=3)
    q = gen.lowrank_queries(nq, d, 64, 3.0, cfg=3)
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(x, False))
    idx_g, sc_g = U.gpu_topk(st, U.to_device(q, False), codes, nu, gamma, n, k, tq.TQ_EST_PROD)
    idx, z = oracle.unpack_codes(U.codes_np(codes, n, d, b), b)
    ref, scale = _oracle_scores(st, q.astype(np.float64), idx, z, nu.cpu().numpy().astype(np.float64),
                                gamma.cpu().numpy().astype(np.float64))
    worst, swapped = U.check_topk(idx_g, sc_g, ref, scale)
    print(f"[topk d=1536 gpu codes b={b}] max err {worst:.2e} swaps {swapped}", flush=True)
    assert worst <= U.TOPK_SCORE_TOL
