"""The quantize + score step captured in a HIP graph replays to the eager result, replay
after replay, with eager work and synchronisation in between (the benchmark replays it)."""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager():
    d, b, groups, G, T = 128, 4, 4, 4, 700
    st = U.make_setup(d, b, cfg=21)
    chans = gen.outlier_channels(21, groups, d)
    keys = np.concatenate([gen.kv_keys_chunk(21, 0, h, T, d, chans[h]) for h in range(groups)])
    q = U.to_device(gen.kv_queries(21, 1, groups * G, d)[0], True)
    x = U.to_device(keys, True)
    n = groups * T
    codes = torch.zeros(n * (d // 32) * b, dtype=torch.int32, device=U.DEV)
    nu = torch.zeros(n, dtype=torch.float32, device=U.DEV)
    gamma = torch.zeros(n, dtype=torch.float32, device=U.DEV)
    logits = torch.zeros(groups * G * T, dtype=torch.float32, device=U.DEV)
    ws = torch.empty(tq.tq_score_ws_bytes(d, b, groups, G, T), dtype=torch.uint8, device=U.DEV)

    def step():
        tq.tq_quantize(st.params, d, b, x, codes, nu, gamma)
        tq.tq_score_ip(st.params, d, b, q, codes, nu, gamma, groups, G, T, tq.TQ_EST_PROD, logits, ws)

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (codes, nu, gamma, logits)]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(4):
        for t in (codes, nu, gamma, logits):
            t.zero_()
        ws.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip((codes, nu, gamma, logits), ref):
            assert torch.equal(a, r), f"replay {rep} differs from eager"


def _replays_match(step, outs, ws_list, reps=4):
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(reps):
        for t in outs:
            t.zero_()
        for w in ws_list:
            w.fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, r in zip(outs, ref):
            assert torch.equal(a, r), f"replay {rep} differs from eager"


def test_graph_replay_fractional_rate_and_attention():
    # the split calls of a fractional-rate cache (fused split encoder for keys and values,
    # general scoring with accumulate, per-group value stages of attention) in one graph
    d, d0, groups, G, T = 128, 64, 3, 4, 500
    bk, bv = (3, 2), (4, 3)
    sk = [U.make_setup(d0, bk[0], cfg=22), U.make_setup(d - d0, bk[1], cfg=23)]
    sv = [U.make_setup(d0, bv[0], cfg=24), U.make_setup(d - d0, bv[1], cfg=25)]
    chans = gen.outlier_channels(22, groups, d)
    keys = U.to_device(np.concatenate([gen.kv_keys_chunk(22, 0, h, T, d, chans[h]) for h in range(groups)]), True)
    vals = U.to_device(np.concatenate([gen.kv_keys_chunk(22, 1, h, T, d, chans[h], scale=1.0)
                                       for h in range(groups)]), True)
    q = U.to_device(gen.kv_queries(22, 1, groups * G, d)[0], True)
    n = groups * T
    kc = [torch.zeros(n * (d0 // 32) * b, dtype=torch.int32, device=U.DEV) for b in bk]
    kn = [torch.zeros(n, device=U.DEV) for _ in range(2)]
    kg = [torch.zeros(n, device=U.DEV) for _ in range(2)]
    vc = [torch.zeros(n * (d0 // 32) * (b - 1), dtype=torch.int32, device=U.DEV) for b in bv]
    vn = [torch.zeros(n, device=U.DEV) for _ in range(2)]
    logits = torch.zeros(groups * G * T, device=U.DEV)
    out = torch.zeros(groups * G * d, device=U.DEV)
    ws_s = torch.empty(tq.tq_score_split_ws_bytes(d, d0, bk[0], bk[1], groups, G, T), dtype=torch.uint8,
                       device=U.DEV)
    ws_a = torch.empty(tq.tq_attention_split_ws_bytes(d, d0, bk[0], bk[1], groups, G, T), dtype=torch.uint8,
                       device=U.DEV)

    def step():
        tq.tq_quantize_split(sk[0].params, sk[1].params, d, d0, bk[0], bk[1], keys, kc[0], kn[0], kg[0],
                             kc[1], kn[1], kg[1])
        tq.tq_quantize_mse_split(sv[0].params, sv[1].params, d, d0, bv[0], bv[1], vals, vc[0], vn[0],
                                 vc[1], vn[1])
        tq.tq_score_ip_split(sk[0].params, sk[1].params, d, d0, bk[0], bk[1], q, kc[0], kn[0], kg[0], kc[1],
                             kn[1], kg[1], groups, G, T, tq.TQ_EST_PROD, logits, ws_s)
        tq.tq_attention_split(sk[0].params, sk[1].params, sv[0].params, sv[1].params, d, d0, bk[0], bk[1],
                              bv[0], bv[1], q, kc[0], kn[0], kg[0], kc[1], kn[1], kg[1], vc[0], vn[0], vc[1],
                              vn[1], groups, G, T, 1.0 / np.sqrt(d), tq.TQ_EST_PROD, out, ws_a)

    _replays_match(step, kc + kn + kg + vc + vn + [logits, out], [ws_s, ws_a])


def test_graph_replay_decode_attention_and_append():
    d, b, groups, G, T = 128, 4, 2, 4, 600
    sk, sv = U.make_setup(d, b, cfg=26), U.make_setup(d, b, cfg=27)
    chans = gen.outlier_channels(26, groups, d)
    keys = U.to_device(np.concatenate([gen.kv_keys_chunk(26, 0, h, T, d, chans[h]) for h in range(groups)]), True)
    vals = U.to_device(np.concatenate([gen.kv_keys_chunk(26, 1, h, T, d, chans[h], scale=1.0)
                                       for h in range(groups)]), True)
    q = U.to_device(gen.kv_queries(26, 1, groups * G, d)[0], True)
    n = groups * T
    ck = torch.zeros(n * (d // 32) * b, dtype=torch.int32, device=U.DEV)
    nk, gk = torch.zeros(n, device=U.DEV), torch.zeros(n, device=U.DEV)
    cv = torch.zeros(n * (d // 32) * (b - 1), dtype=torch.int32, device=U.DEV)
    nv = torch.zeros(n, device=U.DEV)
    out = torch.zeros(groups * G * d, device=U.DEV)
    ws = torch.empty(tq.tq_attention_ws_bytes(d, b, groups, G, T), dtype=torch.uint8, device=U.DEV)
    k_tok = keys.view(groups, T, d)[:, T - 1, :].contiguous()
    v_tok = vals.view(groups, T, d)[:, T - 1, :].contiguous()
    ws_app = torch.empty(tq.tq_append_ws_bytes(d, b, groups), dtype=torch.uint8, device=U.DEV)

    def step():
        tq.tq_quantize(sk.params, d, b, keys, ck, nk, gk)
        tq.tq_quantize_mse(sv.params, d, b, vals, cv, nv)
        tq.tq_append(sk.params, d, b, tq.TQ_EST_PROD, k_tok, T, T - 1, ck, nk, gk, ws_app)
        tq.tq_append(sv.params, d, b, tq.TQ_EST_MSE, v_tok, T, T - 1, cv, nv, None, ws_app)
        tq.tq_attention(sk.params, sv.params, d, b, b, q, ck, nk, gk, cv, nv, groups, G, T, 1.0 / np.sqrt(d),
                        tq.TQ_EST_PROD, out, ws)

    _replays_match(step, [ck, nk, gk, cv, nv, out], [ws, ws_app])
