"""Embedding search at full size: 10^6 unit vectors in R^1536 (low rank + noise, fp32),
b = 2 and 4, 1000 queries, top-10, in the launch configuration the benchmark uses.

Parity, per bit width:
  * every code, nu and gamma of the 10^6 vectors against the oracle, and every rotated
    coordinate (tq_quantize_with_rotation must encode exactly as tq_quantize);
  * the top-10 of queries 0..99 against the oracle's scores of all 10^6 keys (oracle fed
    the GPU's codes).
recall@10 against exact brute force on the unquantized vectors is reported for all 1000
queries (parity unpinned: the pages print no value).  The oracle side runs on host threads,
one 16384-vector block per task.
"""
import time

import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu

W = gen.EMBED_SEARCH
NCHK = 100          # queries whose top-10 is checked against the oracle
_RECALL = {}


def _exact_top10(xd, qd, k):
    """Exact top-k by float32 inner product on the GPU (reference for recall only)."""
    best_s = torch.full((qd.shape[0], k), -float("inf"), device=U.DEV)
    best_i = torch.zeros((qd.shape[0], k), dtype=torch.int64, device=U.DEV)
    for c0 in range(0, xd.shape[0], 65536):
        s = qd @ xd[c0:c0 + 65536].T
        cs, ci = torch.topk(s, k, dim=1)
        alls = torch.cat([best_s, cs], 1)
        alli = torch.cat([best_i, ci + c0], 1)
        o = torch.topk(alls, k, dim=1)
        best_s, best_i = o.values, torch.gather(alli, 1, o.indices)
    return best_i.cpu().numpy()


@pytest.fixture(scope="module")
def search_data():
    d, n, nq, k = W.d, W.n, W.nq, W.k
    rank, snr = W.lowrank
    t0 = time.time()
    basis = gen.lowrank_basis(d, rank, W.cfg)
    nblk = (n + gen.LOWRANK_BLOCK - 1) // gen.LOWRANK_BLOCK
    blocks = U.parallel_map(lambda blk: gen.lowrank_block(blk, d, rank, snr, W.cfg, 0, basis, n_total=n),
                            range(nblk))
    x = np.concatenate(blocks)
    del blocks
    q = gen.lowrank_queries(nq, d, rank, snr, cfg=W.cfg)
    print(f"  generated {n} x {d} in {time.time() - t0:.0f} s", flush=True)
    xd = U.to_device(x, False)
    qd = U.to_device(q, False)
    exact = _exact_top10(xd, qd, k)
    yield x, q, xd, qd, exact
    del xd, qd
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("b", W.bits)
def test_embedding_search_full(search_data, b):
    x, q, xd, qd, exact = search_data
    d, n, nq, k = W.d, W.n, W.nq, W.k
    st = U.make_setup(d, b, cfg=W.cfg)
    codes, nu, gamma = U.gpu_quantize(st, xd)
    c2, nu2, ga2, u = U.gpu_quantize_rotation(st, xd)
    assert torch.equal(codes, c2) and torch.equal(nu, nu2) and torch.equal(gamma, ga2), \
        "tq_quantize_with_rotation must encode exactly as tq_quantize"
    del c2, nu2, ga2
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    idx_g = torch.empty(nq * k, dtype=torch.int32, device=U.DEV)
    sc_g = torch.empty(nq * k, dtype=torch.float32, device=U.DEV)
    ws = torch.empty(tq.tq_topk_ws_bytes(d, b, nq, n, k), dtype=torch.uint8, device=U.DEV)
    e0.record()
    tq.tq_topk(st.params, d, b, qd, codes, nu, gamma, n, k, tq.TQ_EST_PROD, idx_g, sc_g, ws)
    e1.record()
    torch.cuda.synchronize()
    print(f"  [b={b}] tq_topk {e0.elapsed_time(e1):.1f} ms", flush=True)
    idx_g = idx_g.cpu().numpy().reshape(nq, k)
    sc_g = sc_g.cpu().numpy().reshape(nq, k)
    cn = codes.cpu().numpy().view(np.uint32).reshape(n, d // 32, b)
    nu_h, ga_h = nu.cpu().numpy(), gamma.cpu().numpy()
    u_h = u.cpu().numpy()
    del u, codes, nu, gamma, ws
    torch.cuda.empty_cache()

    # every code and rotated coordinate, one seeded block per task
    B = gen.LOWRANK_BLOCK

    def one_block(blk):
        sl = slice(blk * B, min(n, (blk + 1) * B))
        return U.compare_codes(st, x[sl].astype(np.float64), cn[sl], nu_h[sl], ga_h[sl], u_gpu=u_h[sl],
                               keep=False)

    reps = U.parallel_map(one_block, range((n + B - 1) // B), label=f"b={b} oracle code blocks")
    tot = U.merge_reports(reps)
    print(f"  [b={b}] all codes: {U.describe(tot)}", flush=True)
    U.assert_codes_ok(tot)
    del u_h

    # top-10 of queries 0..NCHK-1 against the oracle's scores of every key
    q64 = q[:NCHK].astype(np.float64)

    def one_scores(c0):
        sl = slice(c0, min(n, c0 + 8192))
        ic, zc = oracle.unpack_codes(cn[sl], b)
        return oracle.estimate_ip(q64, st.Pi, st.S, ic, zc, nu_h[sl], ga_h[sl], st.c_or)

    ref = np.concatenate(U.parallel_map(one_scores, range(0, n, 8192), label=f"b={b} oracle scores",
                                        every=32), axis=1)
    scale = np.linalg.norm(q64, axis=1)[:, None] * nu_h[None, :]
    worst, swapped = U.check_topk(idx_g[:NCHK], sc_g[:NCHK], ref, scale)
    print(f"  [b={b}] top-10 of queries 0..{NCHK - 1}: max score err {worst:.2e} of |q| nu, "
          f"queries with near-tie swaps {swapped}", flush=True)
    assert worst <= U.TOPK_SCORE_TOL
    _RECALL[b] = float(np.mean([len(set(idx_g[a]) & set(exact[a])) / k for a in range(nq)]))
    print(f"  [b={b}] recall@10 over {nq} queries = {_RECALL[b]:.4f}", flush=True)
    if len(_RECALL) == len(W.bits):
        assert _RECALL[4] > _RECALL[2]
