"""Parity at the full workload sizes, in the launch configuration the benchmark uses.

decode_layer   (8 KV heads x 32768 tokens, b=4)
decode_batch16 (16 seq x 8 heads x 8192 tokens, b=2 and b=3)
long_context   (16 seq x 8 heads x 131072 tokens, b=3)

Each case quantizes the whole cache with tq_quantize (the benchmark's call) and scores
every query head.  Every code, nu and gamma of the whole cache is checked against the
oracle, and every rotated coordinate u = Pi x / nu: tq_quantize_with_rotation runs on the
same input and must return the same codes, nu and gamma bit for bit.  Logits: every group
of decode_layer and decode_batch16, sequences 0 and 15 of long_context (the oracle's cost).
The oracle side runs on host threads, one KV group per task.
"""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def _load_cache(w, channels):
    """Whole key cache on the GPU, filled chunk by chunk from the seeded generator."""
    x = torch.empty((w.n_keys, w.d), dtype=torch.bfloat16, device=U.DEV)

    def fill(gi):
        s, h = divmod(gi, w.n_kv)
        return gi, gen.kv_keys_chunk(w.cfg, s, h, w.T, w.d, channels[h])

    for gi, chunk in U.parallel_map(fill, range(w.groups)):
        x[gi * w.T:(gi + 1) * w.T] = U.to_device(chunk, True)
    print(f"  [{w.name}] generated {w.groups} groups of {w.T} keys", flush=True)
    return x


def _run(w, b, logit_groups):
    d, T, G = w.d, w.T, w.G
    st = U.make_setup(d, b, cfg=w.cfg)
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    x = _load_cache(w, chans)
    codes, nu, gamma = U.gpu_quantize(st, x)
    c2, nu2, ga2, u = U.gpu_quantize_rotation(st, x)
    assert torch.equal(codes, c2) and torch.equal(nu, nu2) and torch.equal(gamma, ga2), \
        "tq_quantize_with_rotation must encode exactly as tq_quantize"
    del c2, nu2, ga2, x
    q = gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d).reshape(-1, d)
    lg = U.gpu_score(st, U.to_device(q, True), codes, nu, gamma, w.groups, G, T, tq.TQ_EST_PROD)
    cn = codes.cpu().numpy().view(np.uint32).reshape(w.groups, T, d // 32, b)
    nu_h = nu.cpu().numpy().reshape(w.groups, T)
    ga_h = gamma.cpu().numpy().reshape(w.groups, T)
    u_h = u.cpu().numpy().reshape(w.groups, T, d)
    del u, codes, nu, gamma
    torch.cuda.empty_cache()
    q64 = U.host64(q, True).reshape(w.groups, G, d)
    with_logits = set(logit_groups)

    def one(gi):
        s, h = divmod(gi, w.n_kv)
        keys = gen.kv_keys_chunk(w.cfg, s, h, T, d, chans[h])
        rep = U.compare_codes(st, U.host64(keys, True), cn[gi], nu_h[gi], ga_h[gi], u_gpu=u_h[gi],
                              keep=gi in with_logits)
        err = None
        if gi in with_logits:
            err = U.logit_errors(st, q64[gi:gi + 1], rep.pop("idx"), rep.pop("z"), nu_h[gi], ga_h[gi],
                                 lg[gi:gi + 1])
        return rep, err

    results = U.parallel_map(one, range(w.groups), label=f"{w.name} b={b} oracle groups")
    tot = U.merge_reports([r for r, _ in results])
    worst = max(e for _, e in results if e is not None)
    print(f"[{w.name} b={b}] all {w.groups} groups: {U.describe(tot)}; logits of "
          f"{len(with_logits)} groups: max err {worst:.2e} of |q| nu", flush=True)
    U.assert_codes_ok(tot)


@pytest.mark.timeout(300)
def test_decode_layer_full():
    w = gen.DECODE_LAYER
    _run(w, 4, range(w.groups))


@pytest.mark.timeout(300)
@pytest.mark.parametrize("b", [2, 3])
def test_decode_batch16_full(b):
    w = gen.DECODE_BATCH16
    _run(w, b, range(w.groups))


@pytest.mark.timeout(600)
def test_long_context_full():
    w = gen.LONG_CONTEXT
    last = (w.n_seq - 1) * w.n_kv
    _run(w, 3, list(range(w.n_kv)) + list(range(last, last + w.n_kv)))
