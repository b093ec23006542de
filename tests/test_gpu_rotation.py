"""The rotation step on its own: u = Pi x / |x| as the encoders compute it, against the
oracle's float64 rotation ([review, MSE paragraph]: random orthogonal rotation of the
normalised vector).  Tolerance: max |u_gpu - u_oracle| <= 1e-5 (u is a unit vector).

tq_quantize_with_rotation runs the encoders of tq_quantize with one extra store; its codes,
nu and gamma must equal tq_quantize's bit for bit, so the u it reports is the u the codes
were taken from.  Shapes: the fused d = 128 encoder (bf16 and float32 inputs, several tiles
and a ragged tail) and the tiled encoder (d = 64, 192, 1536, two chunks at d = 64).
"""
import numpy as np
import pytest
import torch

import oracle
from workloads import gen
import tq_testutil as U

pytestmark = pytest.mark.gpu


def _check(st, x, bf16, zero_rows=()):
    xd = U.to_device(x, bf16)
    n = xd.shape[0]
    codes, nu, gamma = U.gpu_quantize(st, xd)
    c2, nu2, ga2, u = U.gpu_quantize_rotation(st, xd)
    assert torch.equal(codes, c2) and torch.equal(nu, nu2) and torch.equal(gamma, ga2)
    x64 = U.host64(x, bf16)
    _, _, u_o = oracle.normalize_rotate(x64, st.Pi)
    u_g = u.cpu().numpy().astype(np.float64)
    err = float(np.max(np.abs(u_g - u_o)))
    rep = U.compare_codes(st, x64, U.codes_np(codes, n, st.d, st.b), nu.cpu().numpy(), gamma.cpu().numpy(),
                          u_gpu=u_g, keep=False)
    print(f"[rotation d={st.d} b={st.b} bf16={bf16} n={n}] max |u err| {err:.2e}; {U.describe(rep)}",
          flush=True)
    assert err <= U.ROTATION_TOL
    U.assert_codes_ok(rep)
    for r in zero_rows:
        assert not u_g[r].any() and nu.cpu().numpy()[r] == 0.0


@pytest.mark.parametrize("b", [2, 3, 4])
@pytest.mark.parametrize("bf16", [True, False])
def test_rotation_d128(b, bf16):
    n = 32 * 8 * 9 + 13                     # several tiles per wave and a ragged tail
    st = U.make_setup(128, b, cfg=61)
    chans = gen.outlier_channels(61, 1, 128)
    x = gen.kv_keys_chunk(61, 0, 0, n, 128, chans[0]) if bf16 else \
        gen.unit_sphere(n, 128, cfg=61, role=gen.ROLE_DATA) * 7.0
    if not bf16:
        x[[5, n - 1]] = 0.0
    _check(st, x, bf16, zero_rows=() if bf16 else (5, n - 1))


@pytest.mark.parametrize("d,b,bf16,n", [(64, 3, True, 700), (192, 4, False, 517), (1536, 2, False, 300),
                                        (1536, 4, False, 1000)])
def test_rotation_tiled(d, b, bf16, n):
    st = U.make_setup(d, b, cfg=62)
    x = gen.unit_sphere(n, d, cfg=62, role=gen.ROLE_DATA) * 0.5
    x[3] = 0.0
    if bf16:
        x = gen.f32_to_bf16_bits(x)
    _check(st, x, bf16, zero_rows=(3,))


def test_rotation_tiled_two_chunks():
    # d = 64 bf16 runs several hundred thousand vectors per pass: cross a pass boundary
    d, b = 64, 4
    st = U.make_setup(d, b, cfg=63)
    n = 1_572_864 + 301
    x = gen.f32_to_bf16_bits(gen.unit_sphere(n, d, cfg=63, role=gen.ROLE_DATA))
    xd = U.to_device(x, True)
    codes, nu, gamma = U.gpu_quantize(st, xd)
    c2, nu2, ga2, u = U.gpu_quantize_rotation(st, xd)
    assert torch.equal(codes, c2) and torch.equal(nu, nu2) and torch.equal(gamma, ga2)
    rows = np.concatenate([np.arange(0, 2000), np.arange(n - 2000, n)])
    x64 = U.host64(x[rows], True)
    _, _, u_o = oracle.normalize_rotate(x64, st.Pi)
    err = float(np.max(np.abs(u.cpu().numpy()[rows].astype(np.float64) - u_o)))
    print(f"[rotation d=64 two passes] max |u err| {err:.2e} over {rows.size} rows", flush=True)
    assert err <= U.ROTATION_TOL
