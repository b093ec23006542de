"""Allocation-free decode scoring: tq_score_ip_noalloc (the library's fixed per-GPU scratch in
place of a workspace) against tq_score_ip with a caller workspace, through the C ABI.

Both run the same kernels on the same inputs, so the logits must agree bit for bit.  Two
calls in a row share the scratch, the second with a smaller input (the scratch keeps the
first call's contents); both the d = 128 kernel and the general path are covered.
"""
import numpy as np
import pytest
import torch

import kv_cache_embedding_amd as tq
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def _case(d, b, groups, G, T, cfg):
    st = U.make_setup(d, b, cfg=cfg)
    x = gen.unit_sphere(groups * T, d, cfg=cfg, role=gen.ROLE_DATA) * 3.0
    codes, nu, gamma = U.gpu_quantize(st, U.to_device(gen.f32_to_bf16_bits(x), True))
    q = U.to_device(gen.f32_to_bf16_bits(gen.unit_sphere(groups * G, d, cfg=cfg, role=gen.ROLE_QUERY)), True)
    return st, q, codes, nu, gamma


def _both(st, q, codes, nu, gamma, groups, G, T, mode):
    ref = U.gpu_score(st, q, codes, nu, gamma, groups, G, T, mode)
    out = torch.full((groups * G * T,), float("nan"), dtype=torch.float32, device=U.DEV)
    tq.tq_score_ip_noalloc(st.params, st.d, st.b, q, codes, nu, gamma, groups, G, T, mode, out)
    torch.cuda.synchronize()
    return ref, out.cpu().numpy().reshape(groups, G, T)


@pytest.mark.parametrize("d,b,G,mode", [(128, 3, 4, tq.TQ_EST_PROD), (128, 4, 8, tq.TQ_EST_MSE),
                                        (64, 3, 3, tq.TQ_EST_PROD)])
def test_noalloc_matches_workspace_call_twice(d, b, G, mode):
    big = (16, 5000)
    small = (3, 777)
    for i, (groups, T) in enumerate((big, small)):
        st, q, codes, nu, gamma = _case(d, b, groups, G, T, cfg=70 + i)
        ref, got = _both(st, q, codes, nu, gamma, groups, G, T, mode)
        print(f"[noalloc d={d} b={b} G={G} call {i + 1}: groups={groups} T={T}] "
              f"max |diff| {float(np.max(np.abs(ref - got))):.1e}", flush=True)
        assert np.array_equal(ref, got)


def test_noalloc_at_the_scratch_limit():
    # the largest group count whose workspace fits the fixed scratch, d = 128, b = 4
    d, b, G, T = 128, 4, 4, 300
    cap = tq.tq_score_noalloc_max_ws_bytes()
    groups = 1
    while tq.tq_score_ws_bytes(d, b, groups + 1, G, T) <= cap:
        groups += 1
    st, q, codes, nu, gamma = _case(d, b, groups, G, T, cfg=72)
    ref, got = _both(st, q, codes, nu, gamma, groups, G, T, tq.TQ_EST_PROD)
    assert np.array_equal(ref, got)
    with pytest.raises(tq.TQError) as e:
        tq.tq_score_ip_noalloc(st.params, d, b, torch.zeros((groups + 1) * G * d, device=U.DEV), codes, nu,
                               gamma, groups + 1, G, 1, tq.TQ_EST_PROD,
                               torch.empty((groups + 1) * G, device=U.DEV))
    assert e.value.status == tq.TQ_EUNSUPPORTED
