"""Host-side tests of the C ABI (no GPU): the library loads, exports every declared call,
builds the same codebook as the oracle, and rejects bad arguments before enqueuing work."""
import ctypes
import os
import re

import numpy as np
import pytest

import kv_cache_embedding_amd as tq
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "tq.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_0-9]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(tq.lib_path()):
        pytest.fail("libtq.so is not built: run __graft_entry__.build()")
    return tq.load_library()


def test_library_exports_every_declared_call(lib):
    names = declared_functions()
    assert set(names) >= {"tq_codebook_build", "tq_quantize", "tq_dequantize", "tq_score_ip",
                          "tq_topk", "tq_prepare", "tq_params_bytes", "tq_last_error"}
    raw = ctypes.CDLL(tq.lib_path())
    for name in names:
        assert hasattr(raw, name), name
        assert hasattr(tq, name), f"python binding lacks {name}"


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("d", [64, 128, 1536])
def test_codebook_matches_oracle(lib, bits, d):
    c, t = tq.tq_codebook_build(bits, d)
    co, to = oracle.codebook(bits, d)
    assert np.allclose(c, co, rtol=0, atol=1e-9 / np.sqrt(d))
    assert np.allclose(t, to, rtol=0, atol=1e-9 / np.sqrt(d))
    assert t[len(t) // 2] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
@pytest.mark.parametrize("d", [3, 64, 128, 1536])
def test_sphere_codebook_matches_oracle(lib, bits, d):
    c, t = tq.tq_codebook_build_sphere(bits, d)
    co, to = oracle.codebook_sphere(bits, d)
    assert np.allclose(c, co, rtol=0, atol=1e-10 / np.sqrt(d))
    assert np.allclose(t, to, rtol=0, atol=1e-10 / np.sqrt(d))
    assert t[len(t) // 2] == 0.0 and np.array_equal(c, -c[::-1])


def test_codebooks_at_many_levels_are_lloyd_max_fixed_points(lib):
    # 8 bits (128 cells a side) converges; the Gaussian cell means in closed form
    # (pdf difference over tail difference), checked to what that form resolves
    from scipy import stats
    c, t = tq.tq_codebook_build(8, 1)
    assert np.all(np.diff(c) > 0) and np.array_equal(c, -c[::-1])
    edges = np.concatenate([[-np.inf], t, [np.inf]])
    mean = (stats.norm.pdf(edges[:-1]) - stats.norm.pdf(edges[1:])) / (
        stats.norm.sf(edges[:-1]) - stats.norm.sf(edges[1:]))
    assert np.max(np.abs(mean - c)) < 1e-8
    cs, ts = tq.tq_codebook_build_sphere(6, 1536)
    assert np.all(np.diff(cs) > 0) and np.max(np.abs(cs * np.sqrt(1536) - tq.tq_codebook_build(6, 1)[0])) < 0.05


def test_codebook_rejects_bad_arguments(lib):
    for bad in ((0, 128), (9, 128), (3, 1)):
        with pytest.raises(tq.TQError) as e:
            tq.tq_codebook_build_sphere(*bad)
        assert e.value.status == tq.TQ_EINVAL
    with pytest.raises(tq.TQError) as e:
        tq.tq_codebook_build(0, 128)
    assert e.value.status == tq.TQ_EINVAL
    with pytest.raises(tq.TQError) as e:
        tq.tq_codebook_build(3, 0)
    assert e.value.status == tq.TQ_EINVAL


def test_params_bytes_and_workspace_helpers(lib):
    assert tq.tq_params_bytes(128, 4) > 2 * 128 * 128 * 4
    assert tq.tq_params_bytes(100, 4) == 0
    assert tq.tq_params_bytes(128, 5) == 0
    # d != 128 carries the bf16 hi/lo rows of Pi and S' (4 d^2 x 2 bytes) for the tiled encoder
    for d in (64, 192, 256):
        assert tq.tq_params_bytes(d, 4) >= 2 * d * d * 4 + 4 * d * d * 2
    assert tq.tq_score_ws_bytes(128, 4, 8, 4, 32768) % 256 == 0
    assert tq.tq_score_ws_bytes(128, 4, 8, 8, 32768) == 2 * tq.tq_score_ws_bytes(128, 4, 8, 4, 32768)
    for d, G in ((64, 4), (128, 3), (1536, 1)):
        need = 8 * G * 2 * d * 4          # Pi q and S q of every query row, float32
        assert need <= tq.tq_score_ws_bytes(d, 4, 8, G, 100) < need + 256
    assert tq.tq_score_ws_bytes(100, 4, 8, 4, 100) == 0


def _raw(lib):
    return lib


def test_invalid_arguments_return_status_without_launch(lib):
    P = ctypes.c_void_p
    fake = P(0x1000)   # never dereferenced: every call below fails validation first
    # bad d / b
    assert lib.tq_quantize(fake, 100, 4, fake, 0, 10, fake, fake, fake, None) == tq.TQ_EINVAL
    assert lib.tq_quantize(fake, 128, 5, fake, 0, 10, fake, fake, fake, None) == tq.TQ_EINVAL
    assert "shape" in tq.tq_last_error()
    # bad dtype, negative n, NULL pointers
    assert lib.tq_quantize(fake, 128, 4, fake, 7, 10, fake, fake, fake, None) == tq.TQ_EINVAL
    assert lib.tq_quantize(fake, 128, 4, fake, 0, -1, fake, fake, fake, None) == tq.TQ_EINVAL
    assert lib.tq_quantize(fake, 128, 4, None, 0, 10, fake, fake, fake, None) == tq.TQ_EINVAL
    # misaligned x
    assert lib.tq_quantize(fake, 128, 4, P(0x1002), 0, 10, fake, fake, fake, None) == tq.TQ_EINVAL
    # n == 0 is a no-op even with NULL pointers
    assert lib.tq_quantize(None, 128, 4, None, 0, 0, None, None, None, None) == tq.TQ_OK
    # every multiple of 64 in range is a valid dimension: d = 192 fails on the pointer, not the shape
    assert lib.tq_quantize(fake, 192, 4, P(0x1002), 0, 10, fake, fake, fake, None) == tq.TQ_EINVAL
    assert "misaligned" in tq.tq_last_error()
    # the rotation diagnostic validates like tq_quantize, plus its u pointer
    assert lib.tq_quantize_with_rotation(fake, 100, 4, fake, 0, 10, fake, fake, fake, fake, None) == tq.TQ_EINVAL
    assert lib.tq_quantize_with_rotation(fake, 128, 4, fake, 0, 10, fake, fake, fake, None, None) == tq.TQ_EINVAL
    assert lib.tq_quantize_with_rotation(fake, 128, 4, fake, 0, 10, fake, fake, fake, P(0x1004), None) == tq.TQ_EINVAL
    assert "misaligned" in tq.tq_last_error()
    assert lib.tq_quantize_with_rotation(None, 128, 4, None, 0, 0, None, None, None, None, None) == tq.TQ_OK
    # d = 128 MSE codes are stored 8 or 16 bytes at a time: 16-byte alignment required
    assert lib.tq_quantize_mse(fake, 128, 3, fake, 0, 10, P(0x1004), fake, None) == tq.TQ_EINVAL
    assert "misaligned" in tq.tq_last_error()
    assert lib.tq_quantize_mse_split(fake, fake, 128, 64, 3, 3, fake, 0, 10, P(0x1008), fake, fake, fake,
                                     None) == tq.TQ_EINVAL
    # allocation-free scoring: a workspace beyond the fixed scratch is refused before any
    # device call; empty sizes are a no-op
    cap = lib.tq_score_noalloc_max_ws_bytes()
    assert cap == 8 << 20
    big = 1
    while tq.tq_score_ws_bytes(128, 4, big, 4, 1024) <= cap:
        big *= 2
    assert lib.tq_score_ip_noalloc(fake, 128, 4, fake, 1, fake, fake, fake, big, 4, 1024, 0, fake,
                                   None) == tq.TQ_EUNSUPPORTED
    assert "scratch" in tq.tq_last_error()
    assert lib.tq_score_ip_noalloc(fake, 128, 4, fake, 1, fake, fake, fake, 0, 4, 1024, 0, fake, None) == tq.TQ_OK
    assert lib.tq_score_ip_noalloc(fake, 128, 4, fake, 1, fake, fake, fake, -1, 4, 1024, 0, fake,
                                   None) == tq.TQ_EINVAL
    # scoring in two phases: query prep and the prepared scan validate like tq_score_ip
    assert lib.tq_score_prepare(fake, 100, 4, fake, 1, 8, 4, fake, 1 << 20, None) == tq.TQ_EINVAL
    assert lib.tq_score_prepare(fake, 128, 4, fake, 5, 8, 4, fake, 1 << 20, None) == tq.TQ_EINVAL
    assert lib.tq_score_prepare(fake, 128, 4, None, 1, 8, 4, fake, 1 << 20, None) == tq.TQ_EINVAL
    assert lib.tq_score_prepare(fake, 128, 4, fake, 1, 8, 4, fake, 16, None) == tq.TQ_EWORKSPACE
    assert lib.tq_score_prepare(None, 128, 4, None, 1, 0, 4, None, 0, None) == tq.TQ_OK
    assert lib.tq_score_ip_prepared(fake, 128, 4, fake, fake, fake, 8, 4, 1024, 7, fake, fake, 1 << 20,
                                    None) == tq.TQ_EINVAL
    assert lib.tq_score_ip_prepared(fake, 128, 4, fake, fake, fake, 8, 4, 1024, 0, fake, fake, 16,
                                    None) == tq.TQ_EWORKSPACE
    assert lib.tq_score_ip_prepared(fake, 128, 4, P(0x1004), fake, fake, 8, 4, 1024, 0, fake, fake, 1 << 20,
                                    None) == tq.TQ_EINVAL
    assert lib.tq_score_ip_prepared(None, 128, 4, None, None, None, 8, 4, 0, 0, None, None, 0, None) == tq.TQ_OK
    # scoring: bad mode, workspace too small, unsupported G
    args = (fake, 128, 4, fake, 1, fake, fake, fake, 8, 4, 1024)
    assert lib.tq_score_ip(*args, 9, fake, fake, 1 << 30, None) == tq.TQ_EINVAL
    assert lib.tq_score_ip(*args, 0, fake, fake, 16, None) == tq.TQ_EWORKSPACE
    # G = 3 (and any d) takes the general path, whose workspace is [groups * G] x (2 d + 1) floats
    args3 = (fake, 128, 4, fake, 1, fake, fake, fake, 8, 3, 1024)
    assert lib.tq_score_ip(*args3, 0, fake, fake, 16, None) == tq.TQ_EWORKSPACE
    assert lib.tq_score_ip(fake, 128, 4, fake, 1, fake, fake, fake, 0, 4, 1024, 0, None, None, 0,
                           None) == tq.TQ_OK
    # top-k: k out of range, k > n
    assert lib.tq_topk(fake, 128, 4, fake, 0, 10, fake, fake, fake, 100, 0, 0, fake, fake, fake,
                       1 << 30, None) == tq.TQ_EINVAL
    assert lib.tq_topk(fake, 128, 4, fake, 0, 10, fake, fake, fake, 5, 10, 0, fake, fake, fake,
                       1 << 30, None) == tq.TQ_EINVAL
    # dequantize: bad mode
    assert lib.tq_dequantize(fake, 128, 4, fake, fake, fake, 10, 3, fake, None) == tq.TQ_EINVAL
    # quantize_mse: bad b, misaligned x, n == 0
    assert lib.tq_quantize_mse(fake, 128, 5, fake, 0, 10, fake, fake, None) == tq.TQ_EINVAL
    assert lib.tq_quantize_mse(fake, 128, 4, P(0x1002), 0, 10, fake, fake, None) == tq.TQ_EINVAL
    assert lib.tq_quantize_mse(None, 128, 4, None, 0, 0, None, None, None) == tq.TQ_OK
    # attention: T == 0, non-finite scale, bad mode, small workspace, empty groups
    F = ctypes.c_float
    def att(T, scale, mode, ws_bytes, groups=2, G=4):
        return lib.tq_attention(fake, fake, 128, 4, 4, fake, 1, fake, fake, fake, fake, fake,
                                groups, G, T, F(scale), mode, fake, fake, ws_bytes, None)
    assert att(0, 0.1, 0, 1 << 30) == tq.TQ_EINVAL
    assert att(100, float("nan"), 0, 1 << 30) == tq.TQ_EINVAL
    assert att(100, float("inf"), 0, 1 << 30) == tq.TQ_EINVAL
    assert att(100, 0.1, 7, 1 << 30) == tq.TQ_EINVAL
    assert att(100, 0.1, 0, 256) == tq.TQ_EWORKSPACE
    assert att(100, 0.1, 0, 0, groups=0) == tq.TQ_OK
    # d = 128 with G a multiple of 4: the block kernel scores its own keys, no logits region;
    # other shapes hold the logits too
    assert tq.tq_attention_ws_bytes(128, 4, 2, 4, 100) > tq.tq_score_ws_bytes(128, 4, 2, 4, 100)
    assert (tq.tq_attention_ws_bytes(128, 4, 2, 5, 100) - tq.tq_score_ws_bytes(128, 4, 2, 5, 100)
            >= 2 * 5 * 100 * 4 + (tq.tq_attention_ws_bytes(128, 4, 2, 4, 100) - tq.tq_score_ws_bytes(128, 4, 2, 4, 100)))
    assert tq.tq_attention_ws_bytes(64, 4, 2, 4, 100) >= 2 * 4 * 100 * 4 + tq.tq_score_ws_bytes(64, 4, 2, 4, 100)
    # append: pos outside [0, cap), bad mode, small workspace, gamma needed for keys, no groups
    def app(pos, cap=16, mode=0, ws_bytes=1 << 20, gamma=fake, groups=8):
        return lib.tq_append(fake, 128, 4, mode, fake, 1, groups, cap, pos, fake, fake, gamma, fake,
                             ws_bytes, None)
    assert app(16) == tq.TQ_EINVAL and app(-1) == tq.TQ_EINVAL
    assert app(3, mode=5) == tq.TQ_EINVAL
    assert app(3, ws_bytes=64) == tq.TQ_EWORKSPACE
    assert app(3, gamma=None) == tq.TQ_EINVAL
    assert app(3, groups=0) == tq.TQ_OK
    assert tq.tq_append_ws_bytes(128, 4, 8) >= 8 * 4 * 4 * 4 + 2 * 8 * 4


def test_prepare_rejects_bad_codebook_and_rotation(lib):
    d, b = 128, 3
    c, t = tq.tq_codebook_build(b - 1, d)
    Pi = np.eye(d, dtype=np.float32)
    S = np.ones((d, d), dtype=np.float32)
    fake = ctypes.c_void_p(0x100000)
    def call(Pi_, c_, t_):
        Pi_ = np.ascontiguousarray(Pi_, np.float32)
        c_ = np.ascontiguousarray(c_, np.float64)
        t_ = np.ascontiguousarray(t_, np.float64)
        return lib.tq_prepare(d, b, Pi_.ctypes.data, S.ctypes.data, c_.ctypes.data, t_.ctypes.data,
                              fake, None)
    assert call(Pi, c[::-1], t) == tq.TQ_EINVAL              # not ascending
    c2 = c.copy(); c2[-1] *= 1.1
    assert call(Pi, c2, t) == tq.TQ_EINVAL                   # not symmetric
    assert call(Pi * 1.01, c, t) == tq.TQ_EINVAL             # not orthogonal
    assert "orthogonal" in tq.tq_last_error()
    assert lib.tq_prepare(d, b, Pi.ctypes.data, S.ctypes.data, c.ctypes.data, t.ctypes.data,
                          ctypes.c_void_p(0x100010), None) == tq.TQ_EINVAL   # misaligned params
    # the orthogonal-QJL preparation also checks the rows of S (all ones: not orthonormal)
    assert lib.tq_prepare_orthogonal_qjl(d, b, Pi.ctypes.data, S.ctypes.data, c.ctypes.data,
                                         t.ctypes.data, fake, None) == tq.TQ_EINVAL
    assert "orthonormal" in tq.tq_last_error()
    S2 = np.ascontiguousarray(np.eye(d, dtype=np.float32) * 1.01)
    assert lib.tq_prepare_orthogonal_qjl(d, b, Pi.ctypes.data, S2.ctypes.data, c.ctypes.data,
                                         t.ctypes.data, fake, None) == tq.TQ_EINVAL


def test_split_calls_validate_without_launch(lib):
    fake = ctypes.c_void_p(0x100000)
    P = fake
    # channel groups must each be a valid d (multiple of 64, 64..4096) with bits in 2..4
    for d, d0, b0, b1 in ((128, 32, 3, 2), (128, 128, 3, 2), (128, 0, 3, 2), (192, 64, 5, 2),
                          (192, 64, 3, 1)):
        assert lib.tq_quantize_split(P, P, d, d0, b0, b1, P, tq.TQ_BF16, 10, P, P, P, P, P, P,
                                     None) == tq.TQ_EINVAL
        assert lib.tq_score_split_ws_bytes(d, d0, b0, b1, 2, 4, 100) == 0
    assert "split" in tq.tq_last_error()
    assert lib.tq_quantize_split(P, None, 128, 64, 3, 2, P, tq.TQ_BF16, 10, P, P, P, P, P, P,
                                 None) == tq.TQ_EINVAL
    assert lib.tq_quantize_split(P, P, 128, 64, 3, 2, P, tq.TQ_BF16, 0, None, None, None, None, None,
                                 None, None) == tq.TQ_OK                       # n = 0: nothing to do
    need = lib.tq_score_split_ws_bytes(128, 64, 3, 2, 2, 4, 100)
    # the larger of the general path's need (both groups' Pi q, S q operands side by side) and the
    # integer scorer's (per quad of heads: 3 + 2 operand registers of 64 lanes x 16 bytes and 8
    # float4 constants)
    assert need == max(2 * (2 * 4 * 2 * 64 * 4), 2 * ((3 + 2) * 64 * 16 + 8 * 16))
    assert lib.tq_score_split_ws_bytes(128, 64, 3, 2, 2, 3, 100) == 2 * (2 * 3 * 2 * 64 * 4)   # G % 4 != 0
    assert lib.tq_score_ip_split(P, P, 128, 64, 3, 2, P, tq.TQ_BF16, P, P, P, P, P, P, 2, 4, 100,
                                 tq.TQ_EST_PROD, P, P, need - 256, None) == tq.TQ_EWORKSPACE
    assert lib.tq_score_ip_split(P, P, 128, 64, 3, 2, P, tq.TQ_BF16, P, P, P, P, P, P, 2, 4, 100,
                                 7, P, P, need, None) == tq.TQ_EINVAL          # bad mode
    # the two phases: the same validation, workspace and size limits, nothing launched
    assert lib.tq_score_split_prepare(P, P, 128, 32, 3, 2, P, tq.TQ_BF16, 2, 4, P, need, None) == tq.TQ_EINVAL
    assert lib.tq_score_split_prepare(P, P, 128, 64, 3, 2, P, 7, 2, 4, P, need, None) == tq.TQ_EINVAL
    assert lib.tq_score_split_prepare(P, P, 128, 64, 3, 2, None, tq.TQ_BF16, 2, 4, P, need, None) == tq.TQ_EINVAL
    assert lib.tq_score_split_prepare(P, P, 128, 64, 3, 2, P, tq.TQ_BF16, 2, 4, P, need - 256,
                                      None) == tq.TQ_EWORKSPACE
    assert lib.tq_score_split_prepare(P, P, 128, 64, 3, 2, P, tq.TQ_BF16, 0, 4, None, 0, None) == tq.TQ_OK
    assert lib.tq_score_ip_split_prepared(P, P, 128, 64, 3, 2, P, P, P, P, P, P, 2, 4, 100, 7, P, P, need,
                                          None) == tq.TQ_EINVAL                # bad mode
    assert lib.tq_score_ip_split_prepared(P, P, 128, 64, 3, 2, P, P, None, P, P, P, 2, 4, 100,
                                          tq.TQ_EST_PROD, P, P, need, None) == tq.TQ_EINVAL
    assert lib.tq_score_ip_split_prepared(P, P, 128, 64, 3, 2, P, P, P, P, P, P, 2, 4, 100, tq.TQ_EST_PROD,
                                          P, P, need - 256, None) == tq.TQ_EWORKSPACE
    assert lib.tq_score_ip_split_prepared(P, P, 128, 64, 3, 2, P, P, P, P, P, P, 2, 4, 0, tq.TQ_EST_PROD,
                                          None, None, 0, None) == tq.TQ_OK     # T = 0: nothing to do
    # operands prepared for the integer scan serve keys up to 2^26 per group (buffer offsets)
    big = 1 << 26
    assert lib.tq_score_ip_split_prepared(P, P, 128, 64, 3, 2, P, P, P, P, P, P, 1, 4, big, tq.TQ_EST_PROD,
                                          P, P, need, None) == tq.TQ_EUNSUPPORTED
