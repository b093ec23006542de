"""Out-of-bounds writes: every entry point at ragged shapes writes nothing outside its outputs.

Each output and workspace buffer is the middle of a larger allocation whose 4 KiB before and
after hold a sentinel byte; after the call (and a synchronize) both zones must still hold it.
The shapes cut every tiling of the kernels short: vector counts off the 32-vector wave tiles
and 256-vector workgroup tiles, key counts off the 16-key scan tiles and 256-key attention
blocks, query counts off the 256-query top-k tiles, head counts off the quads.  This is the
bounds check of the kernels' stores (the loads of the scan and the block kernels go through
bounded buffer resources)."""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu

GUARD = 4096
SENTINEL = 0xA5


class Guards:
    def __init__(self):
        self.bufs = []

    def new(self, numel: int, dtype=torch.float32):
        esize = torch.empty((), dtype=dtype).element_size()
        nbytes = max(numel, 1) * esize
        base = torch.full((GUARD + nbytes + GUARD,), SENTINEL, dtype=torch.uint8, device=U.DEV)
        view = base[GUARD:GUARD + nbytes].view(dtype)
        self.bufs.append((base, nbytes))
        return view

    def check(self, what: str):
        torch.cuda.synchronize()
        for i, (base, nbytes) in enumerate(self.bufs):
            head = base[:GUARD].cpu().numpy()
            tail = base[GUARD + nbytes:].cpu().numpy()
            assert np.all(head == SENTINEL), f"{what}: buffer {i} written before its start"
            assert np.all(tail == SENTINEL), f"{what}: buffer {i} written past its end ({nbytes} bytes)"


def _x(n, d, bf16, cfg):
    if bf16:
        chans = gen.outlier_channels(cfg, 1, d)
        return U.to_device(gen.kv_keys_chunk(cfg, 0, 0, n, d, chans[0]), True)
    return U.to_device(gen.unit_sphere(n, d, cfg=cfg, role=gen.ROLE_DATA) * np.float32(2.0), False)


def _encode(g: Guards, st, x):
    n = x.shape[0]
    codes = g.new(n * (st.d // 32) * st.b, torch.int32)
    nu, gamma = g.new(n), g.new(n)
    tq.tq_quantize(st.params, st.d, st.b, x, codes, nu, gamma)
    return codes, nu, gamma


@pytest.mark.parametrize("d,b,bf16,n", [(128, 4, True, 1037), (128, 3, False, 777), (128, 2, True, 33),
                                        (192, 2, False, 305), (64, 4, True, 513), (1536, 3, False, 261)])
def test_encoders_write_only_their_outputs(d, b, bf16, n):
    st = U.make_setup(d, b, cfg=90)
    x = _x(n, d, bf16, 90)
    g = Guards()
    codes, nu, gamma = _encode(g, st, x)
    u = g.new(n * d)
    tq.tq_quantize_with_rotation(st.params, d, b, x, g.new(n * (d // 32) * b, torch.int32), g.new(n), g.new(n), u)
    tq.tq_quantize_mse(st.params, d, b, x, g.new(n * (d // 32) * (b - 1), torch.int32), g.new(n))
    for mode in (tq.TQ_EST_PROD, tq.TQ_EST_MSE):
        tq.tq_dequantize(st.params, d, b, codes, nu, gamma, mode, g.new(n * d))
    g.check(f"encoders d={d} b={b} n={n}")


@pytest.mark.parametrize("d,b,groups,G,T", [(128, 4, 3, 4, 257), (128, 2, 2, 8, 33), (128, 3, 1, 4, 17),
                                            (192, 3, 2, 3, 300), (64, 4, 3, 5, 129)])
def test_scoring_writes_only_its_outputs(d, b, groups, G, T):
    st = U.make_setup(d, b, cfg=91)
    x = _x(groups * T, d, True, 91)
    q = U.to_device(gen.kv_queries(91, 1, groups * G, d).reshape(-1, d), True)
    g = Guards()
    codes, nu, gamma = _encode(g, st, x)
    ws_bytes = max(tq.tq_score_ws_bytes(d, b, groups, G, T), 256)
    for mode in (tq.TQ_EST_PROD, tq.TQ_EST_MSE):
        tq.tq_score_ip(st.params, d, b, q, codes, nu, gamma, groups, G, T, mode, g.new(groups * G * T),
                       g.new(ws_bytes, torch.uint8))
    ws = g.new(ws_bytes, torch.uint8)
    tq.tq_score_prepare(st.params, d, b, q, groups, G, ws)
    tq.tq_score_ip_prepared(st.params, d, b, codes, nu, gamma, groups, G, T, tq.TQ_EST_PROD,
                            g.new(groups * G * T), ws)
    tq.tq_score_ip_noalloc(st.params, d, b, q, codes, nu, gamma, groups, G, T, tq.TQ_EST_PROD,
                           g.new(groups * G * T))
    g.check(f"scoring d={d} b={b} groups={groups} G={G} T={T}")


@pytest.mark.parametrize("d,b,n,nq,k", [(128, 4, 1037, 37, 10), (128, 2, 700, 300, 26), (192, 3, 513, 5, 100),
                                        (128, 3, 40, 3, 40)])
def test_topk_writes_only_its_outputs(d, b, n, nq, k):
    st = U.make_setup(d, b, cfg=92)
    x = _x(n, d, False, 92)
    q = U.to_device(gen.unit_sphere(nq, d, cfg=92, role=gen.ROLE_QUERY), False)
    g = Guards()
    codes, nu, gamma = _encode(g, st, x)
    tq.tq_topk(st.params, d, b, q, codes, nu, gamma, n, k, tq.TQ_EST_PROD, g.new(nq * k, torch.int32),
               g.new(nq * k), g.new(tq.tq_topk_ws_bytes(d, b, nq, n, k), torch.uint8))
    g.check(f"top-k d={d} b={b} n={n} nq={nq} k={k}")


@pytest.mark.parametrize("d,b_k,b_v,groups,G,T", [(128, 4, 4, 3, 4, 300), (128, 3, 2, 2, 8, 65),
                                                  (192, 3, 4, 2, 3, 257), (1536, 2, 3, 1, 4, 130)])
def test_attention_and_append_write_only_their_outputs(d, b_k, b_v, groups, G, T):
    stk, stv = U.make_setup(d, b_k, cfg=93), U.make_setup(d, b_v, cfg=94)
    x = _x(groups * T, d, True, 93)
    q = U.to_device(gen.kv_queries(93, 1, groups * G, d).reshape(-1, d), True)
    g = Guards()
    ck, nk, gk = _encode(g, stk, x)
    cv, nv = g.new(groups * T * (d // 32) * (b_v - 1), torch.int32), g.new(groups * T)
    tq.tq_quantize_mse(stv.params, d, b_v, x, cv, nv)
    tq.tq_attention(stk.params, stv.params, d, b_k, b_v, q, ck, nk, gk, cv, nv, groups, G, T,
                    1.0 / np.sqrt(d), tq.TQ_EST_PROD, g.new(groups * G * d),
                    g.new(tq.tq_attention_ws_bytes(d, b_k, groups, G, T), torch.uint8))
    # one token per group appended at the last slot of both caches
    tok = x.view(groups, T, d)[:, 0, :].contiguous()
    ws = g.new(max(tq.tq_append_ws_bytes(d, b_k, groups), tq.tq_append_ws_bytes(d, b_v, groups)), torch.uint8)
    tq.tq_append(stk.params, d, b_k, tq.TQ_EST_PROD, tok, T, T - 1, ck, nk, gk, ws)
    tq.tq_append(stv.params, d, b_v, tq.TQ_EST_MSE, tok, T, T - 1, cv, nv, None, ws)
    g.check(f"attention/append d={d} groups={groups} G={G} T={T}")


@pytest.mark.parametrize("d,d0,b0,b1,groups,G,T", [(128, 64, 3, 2, 3, 4, 257), (128, 64, 4, 3, 2, 8, 33),
                                                   (192, 128, 4, 2, 2, 3, 300)])
def test_split_calls_write_only_their_outputs(d, d0, b0, b1, groups, G, T):
    sk = [U.make_setup(d0, b0, cfg=95), U.make_setup(d - d0, b1, cfg=96)]
    sv = [U.make_setup(d0, b0, cfg=97), U.make_setup(d - d0, b1, cfg=98)]
    n = groups * T
    x = _x(n, d, True, 95)
    q = U.to_device(gen.kv_queries(95, 1, groups * G, d).reshape(-1, d), True)
    g = Guards()
    k0 = (g.new(n * (d0 // 32) * b0, torch.int32), g.new(n), g.new(n))
    k1 = (g.new(n * ((d - d0) // 32) * b1, torch.int32), g.new(n), g.new(n))
    tq.tq_quantize_split(sk[0].params, sk[1].params, d, d0, b0, b1, x, *k0, *k1)
    v0 = (g.new(n * (d0 // 32) * (b0 - 1), torch.int32), g.new(n))
    v1 = (g.new(n * ((d - d0) // 32) * (b1 - 1), torch.int32), g.new(n))
    tq.tq_quantize_mse_split(sv[0].params, sv[1].params, d, d0, b0, b1, x, *v0, *v1)
    tq.tq_score_ip_split(sk[0].params, sk[1].params, d, d0, b0, b1, q, *k0, *k1, groups, G, T, tq.TQ_EST_PROD,
                         g.new(groups * G * T),
                         g.new(max(tq.tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, T), 256), torch.uint8))
    tq.tq_attention_split(sk[0].params, sk[1].params, sv[0].params, sv[1].params, d, d0, b0, b1, b0, b1, q,
                          *k0, *k1, *v0, *v1, groups, G, T, 1.0 / np.sqrt(d), tq.TQ_EST_PROD,
                          g.new(groups * G * d),
                          g.new(tq.tq_attention_split_ws_bytes(d, d0, b0, b1, groups, G, T), torch.uint8))
    g.check(f"split d={d} d0={d0} b={b0}/{b1} groups={groups} G={G} T={T}")
