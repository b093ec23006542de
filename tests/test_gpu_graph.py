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
