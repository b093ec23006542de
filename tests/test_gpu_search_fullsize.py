"""Embedding search at full size: 10^6 unit vectors in R^1536 (low rank + noise, fp32),
b = 2 and 4, 1000 queries, top-10.

Parity: codes of a deterministic sample of 4000 vectors (plus the last 100) against the
oracle; the top-10 of queries 0..19 against the oracle's scores of all 10^6 keys (oracle fed
the GPU's codes).  recall@10 against exact brute force on the unquantized vectors is
reported for all 1000 queries (parity unpinned: the pages print no value).
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


@pytest.mark.timeout(1200)
def test_embedding_search_full():
    d, n, nq, k = W.d, W.n, W.nq, W.k
    rank, snr = W.lowrank
    t0 = time.time()
    x = gen.lowrank_vectors(n, d, rank, snr, cfg=W.cfg)
    q = gen.lowrank_queries(nq, d, rank, snr, cfg=W.cfg)
    print(f"  generated {n} x {d} in {time.time() - t0:.0f} s", flush=True)
    xd = U.to_device(x, False)
    qd = U.to_device(q, False)
    exact = _exact_top10(xd, qd, k)
    sample = np.concatenate([np.arange(0, n, n // 4000), np.arange(n - 100, n)])
    recall = {}
    for b in W.bits:
        st = U.make_setup(d, b, cfg=W.cfg)
        codes, nu, gamma = U.gpu_quantize(st, xd)
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
        # codes of the sample
        rep = U.compare_codes(st, x[sample].astype(np.float64), cn[sample], nu_h[sample], ga_h[sample])
        print(f"  [b={b}] sample codes: {U.describe(rep)}", flush=True)
        U.assert_codes_ok(rep)
        # top-10 of queries 0..19 against the oracle's scores of every key
        nchk = 20
        q64 = q[:nchk].astype(np.float64)
        ref = np.empty((nchk, n))
        for c0 in range(0, n, 8192):
            ic, zc = oracle.unpack_codes(cn[c0:c0 + 8192], b)
            ref[:, c0:c0 + 8192] = oracle.estimate_ip(q64, st.Pi, st.S, ic, zc, nu_h[c0:c0 + 8192],
                                                      ga_h[c0:c0 + 8192], st.c_or)
            if c0 % (8192 * 32) == 0:
                print(f"    oracle scores {c0}/{n}", flush=True)
        scale = np.linalg.norm(q64, axis=1)[:, None] * nu_h[None, :]
        worst, swapped = U.check_topk(idx_g[:nchk], sc_g[:nchk], ref, scale)
        print(f"  [b={b}] top-10 parity: max score err {worst:.2e}, near-tie swaps {swapped}", flush=True)
        assert worst <= U.LOGIT_TOL
        recall[b] = float(np.mean([len(set(idx_g[a]) & set(exact[a])) / k for a in range(nq)]))
        print(f"  [b={b}] recall@10 over {nq} queries = {recall[b]:.4f}", flush=True)
    assert recall[4] > recall[2]
