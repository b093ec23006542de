"""Parity at the full workload sizes, in the launch configuration the benchmark uses.

decode_layer   (8 KV heads x 32768 tokens, b=4): every code and every logit is checked.
decode_batch16 (16 seq x 8 heads x 8192 tokens, b=2 and b=3): every code; logits of a
               deterministic sample of 16 of the 128 groups.
long_context   (16 seq x 8 heads x 131072 tokens, b=3): the whole cache is quantized and
               scored on the GPU; codes and logits of sequences 0 and 15 are checked.
"""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def _load_cache(w, channels, seqs=None):
    """Whole key cache on the GPU, filled chunk by chunk from the seeded generator."""
    n = w.n_keys
    x = torch.empty((n, w.d), dtype=torch.bfloat16, device=U.DEV)
    for s in range(w.n_seq):
        for h in range(w.n_kv):
            gi = s * w.n_kv + h
            chunk = gen.kv_keys_chunk(w.cfg, s, h, w.T, w.d, channels[h])
            x[gi * w.T:(gi + 1) * w.T] = U.to_device(chunk, True)
        if s % 4 == 3:
            print(f"  [{w.name}] generated {s + 1}/{w.n_seq} sequences", flush=True)
    return x


def _run(w, b, check_groups):
    d, T, G = w.d, w.T, w.G
    st = U.make_setup(d, b, cfg=w.cfg)
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    x = _load_cache(w, chans)
    codes, nu, gamma = U.gpu_quantize(st, x)
    del x
    q = gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d).reshape(-1, d)
    lg = U.gpu_score(st, U.to_device(q, True), codes, nu, gamma, w.groups, G, T, tq.TQ_EST_PROD)
    cn = codes.view(w.groups, T * (d // 32) * b)
    nu_h = nu.view(w.groups, T)
    ga_h = gamma.view(w.groups, T)
    q64 = U.host64(q, True).reshape(w.groups, G, d)
    worst = 0.0
    excused = 0
    total = 0
    for gi in check_groups:
        s, h = divmod(gi, w.n_kv)
        keys = gen.kv_keys_chunk(w.cfg, s, h, T, d, chans[h])
        c_np = cn[gi].cpu().numpy().view(np.uint32).reshape(T, d // 32, b)
        rep = U.compare_codes(st, U.host64(keys, True), c_np, nu_h[gi].cpu().numpy(),
                              ga_h[gi].cpu().numpy())
        U.assert_codes_ok(rep)
        excused += rep["excused_idx"] + rep["excused_z"]
        total += 2 * T * d
        err = U.logit_errors(st, q64[gi:gi + 1], rep["idx"], rep["z"], nu_h[gi].cpu().numpy(),
                             ga_h[gi].cpu().numpy(), lg[gi:gi + 1])
        worst = max(worst, err)
    print(f"[{w.name} b={b}] groups checked {len(check_groups)}; excused {excused}/{total} "
          f"= {excused / total:.2e}; max logit err {worst:.2e} of |q| nu", flush=True)
    assert excused / total <= U.MAX_EXCUSED_RATE
    assert worst <= U.LOGIT_TOL


def test_decode_layer_full():
    w = gen.DECODE_LAYER
    _run(w, 4, list(range(w.groups)))


@pytest.mark.parametrize("b", [2, 3])
def test_decode_batch16_full(b):
    w = gen.DECODE_BATCH16
    _run(w, b, [i * 8 + (i % 8) for i in range(16)])


@pytest.mark.timeout(600)
def test_long_context_full():
    w = gen.LONG_CONTEXT
    last = (w.n_seq - 1) * w.n_kv
    _run(w, 3, list(range(w.n_kv)) + list(range(last, last + w.n_kv)))
