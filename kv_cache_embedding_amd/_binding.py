"""ctypes marshalling for libtq.so: tensors -> (pointer, size) and torch's current stream."""
from __future__ import annotations

import ctypes
import os

import numpy as np

TQ_OK, TQ_EINVAL, TQ_EUNSUPPORTED, TQ_EHIP, TQ_EWORKSPACE = 0, 1, 2, 3, 4
TQ_F32, TQ_BF16 = 0, 1
TQ_EST_PROD, TQ_EST_MSE = 0, 1

_STATUS = {0: "TQ_OK", 1: "TQ_EINVAL", 2: "TQ_EUNSUPPORTED", 3: "TQ_EHIP", 4: "TQ_EWORKSPACE"}
_LIB = None


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_STATUS.get(status, status)}: {message}")
        self.status = status
        self.message = message


def lib_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtq.so")


def load_library():
    """Load libtq.so (after torch, so both use torch's HIP runtime). Raises if it is missing."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() (hipcc, gfx950)")
    import torch  # noqa: F401  (loads torch's libamdhip64 first)

    lib = ctypes.CDLL(path)
    P, I, I64, SZ, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_double
    sig = {
        "tq_codebook_build": (I, [I, I, ctypes.POINTER(D), ctypes.POINTER(D)]),
        "tq_params_bytes": (SZ, [I, I]),
        "tq_codebook_build_sphere": (I, [I, I, ctypes.POINTER(D), ctypes.POINTER(D)]),
        "tq_prepare": (I, [I, I, P, P, P, P, P, P]),
        "tq_prepare_orthogonal_qjl": (I, [I, I, P, P, P, P, P, P]),
        "tq_quantize": (I, [P, I, I, P, I, I64, P, P, P, P]),
        "tq_quantize_with_rotation": (I, [P, I, I, P, I, I64, P, P, P, P, P]),
        "tq_dequantize": (I, [P, I, I, P, P, P, I64, I, P, P]),
        "tq_score_ws_bytes": (SZ, [I, I, I64, I64, I64]),
        "tq_score_ip": (I, [P, I, I, P, I, P, P, P, I64, I64, I64, I, P, P, SZ, P]),
        "tq_score_ip_noalloc": (I, [P, I, I, P, I, P, P, P, I64, I64, I64, I, P, P]),
        "tq_score_prepare": (I, [P, I, I, P, I, I64, I64, P, SZ, P]),
        "tq_score_ip_prepared": (I, [P, I, I, P, P, P, I64, I64, I64, I, P, P, SZ, P]),
        "tq_score_noalloc_max_ws_bytes": (SZ, []),
        "tq_quantize_mse": (I, [P, I, I, P, I, I64, P, P, P]),
        "tq_quantize_split": (I, [P, P, I, I, I, I, P, I, I64, P, P, P, P, P, P, P]),
        "tq_score_split_ws_bytes": (SZ, [I, I, I, I, I64, I64, I64]),
        "tq_quantize_mse_split": (I, [P, P, I, I, I, I, P, I, I64, P, P, P, P, P]),
        "tq_attention_split_ws_bytes": (SZ, [I, I, I, I, I64, I64, I64]),
        "tq_attention_split": (I, [P, P, P, P, I, I, I, I, I, I, P, I, P, P, P, P, P, P, P, P, P, P, I64, I64,
                                   I64, ctypes.c_float, I, P, P, SZ, P]),
        "tq_score_ip_split": (I, [P, P, I, I, I, I, P, I, P, P, P, P, P, P, I64, I64, I64, I, P, P, SZ,
                                  P]),
        "tq_score_split_prepare": (I, [P, P, I, I, I, I, P, I, I64, I64, P, SZ, P]),
        "tq_score_ip_split_prepared": (I, [P, P, I, I, I, I, P, P, P, P, P, P, I64, I64, I64, I, P, P, SZ,
                                           P]),
        "tq_append_ws_bytes": (SZ, [I, I, I64]),
        "tq_append": (I, [P, I, I, I, P, I, I64, I64, I64, P, P, P, P, SZ, P]),
        "tq_attention_ws_bytes": (SZ, [I, I, I64, I64, I64]),
        "tq_attention": (I, [P, P, I, I, I, P, I, P, P, P, P, P, I64, I64, I64, ctypes.c_float, I,
                             P, P, SZ, P]),
        "tq_topk_ws_bytes": (SZ, [I, I, I64, I64, I]),
        "tq_topk": (I, [P, I, I, P, I, I64, P, P, P, I64, I, I, P, P, P, SZ, P]),
        "tq_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def tq_last_error() -> str:
    return load_library().tq_last_error().decode()


def _check(status: int):
    if status != TQ_OK:
        raise TQError(status, tq_last_error())


# ------------------------------------------------------------------------- helpers

def _torch():
    import torch
    return torch


def _ptr(t) -> int:
    return t.data_ptr()


def _dev(t, name: str):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _dtype_code(t, name: str) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return TQ_F32
    if t.dtype == torch.bfloat16:
        return TQ_BF16
    raise TypeError(f"{name} must be float32 or bfloat16, got {t.dtype}")


def _need(t, name: str, numel: int, dtype):
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


def _stream(stream, device) -> ctypes.c_void_p:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


# ---------------------------------------------------------------------- C calls

def _codebook_call(fn, bits_mse: int, d: int):
    L = 1 << bits_mse if 0 < bits_mse <= 8 else 2
    c = np.zeros(L, dtype=np.float64)
    t = np.zeros(max(L - 1, 1), dtype=np.float64)
    _check(fn(int(bits_mse), int(d), c.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
              t.ctypes.data_as(ctypes.POINTER(ctypes.c_double))))
    return c, t[:L - 1]


def tq_codebook_build(bits_mse: int, d: int):
    """Host float64 Lloyd-Max codebook for N(0, 1/d): (centroids[L], thresholds[L-1])."""
    return _codebook_call(load_library().tq_codebook_build, bits_mse, d)


def tq_codebook_build_sphere(bits_mse: int, d: int):
    """Host float64 Lloyd-Max codebook for the exact sphere-coordinate law in R^d."""
    return _codebook_call(load_library().tq_codebook_build_sphere, bits_mse, d)


def tq_params_bytes(d: int, b: int) -> int:
    return int(load_library().tq_params_bytes(int(d), int(b)))


def tq_prepare(d: int, b: int, Pi: np.ndarray, S: np.ndarray, centroids: np.ndarray,
               thresholds: np.ndarray, params, stream=None):
    """Fill the device parameter block `params` (uint8 tensor of tq_params_bytes(d, b))."""
    _prepare_call("tq_prepare", d, b, Pi, S, centroids, thresholds, params, stream)


def tq_prepare_orthogonal_qjl(d: int, b: int, Pi: np.ndarray, S: np.ndarray, centroids: np.ndarray,
                              thresholds: np.ndarray, params, stream=None):
    """tq_prepare for a QJL matrix S with orthonormal rows."""
    _prepare_call("tq_prepare_orthogonal_qjl", d, b, Pi, S, centroids, thresholds, params, stream)


def _prepare_call(name, d, b, Pi, S, centroids, thresholds, params, stream):
    torch = _torch()
    Pi = np.ascontiguousarray(Pi, dtype=np.float32)
    S = np.ascontiguousarray(S, dtype=np.float32)
    c = np.ascontiguousarray(centroids, dtype=np.float64)
    t = np.ascontiguousarray(thresholds, dtype=np.float64)
    if Pi.shape != (d, d) or S.shape != (d, d):
        raise ValueError("Pi and S must be d x d")
    if c.size != 1 << (b - 1) or t.size != (1 << (b - 1)) - 1:
        raise ValueError("codebook size does not match b")
    _dev(params, "params")
    _need(params, "params", tq_params_bytes(d, b), torch.uint8)
    _check(getattr(load_library(), name)(int(d), int(b), Pi.ctypes.data, S.ctypes.data, c.ctypes.data,
                                         t.ctypes.data, _ptr(params), _stream(stream, params.device)))


def tq_quantize(params, d: int, b: int, x, codes, nu, gamma, stream=None):
    """Encode x [n][d] (float32 or bfloat16) into codes [n][d/32][b] uint32, nu[n], gamma[n]."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [n][{d}]")
    n = x.shape[0]
    for tname, t in (("codes", codes), ("nu", nu), ("gamma", gamma), ("params", params)):
        _dev(t, tname)
    _need(codes, "codes", n * (d // 32) * b, torch.int32)
    _need(nu, "nu", n, torch.float32)
    _need(gamma, "gamma", n, torch.float32)
    _check(load_library().tq_quantize(_ptr(params), d, b, _ptr(x), _dtype_code(x, "x"), n,
                                      _ptr(codes), _ptr(nu), _ptr(gamma),
                                      _stream(stream, x.device)))


def tq_quantize_with_rotation(params, d: int, b: int, x, codes, nu, gamma, u, stream=None):
    """tq_quantize plus the rotated unit coordinates u [n][d] float32 the encoder computed."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [n][{d}]")
    n = x.shape[0]
    for tname, t in (("codes", codes), ("nu", nu), ("gamma", gamma), ("u", u), ("params", params)):
        _dev(t, tname)
    _need(codes, "codes", n * (d // 32) * b, torch.int32)
    _need(nu, "nu", n, torch.float32)
    _need(gamma, "gamma", n, torch.float32)
    _need(u, "u", n * d, torch.float32)
    _check(load_library().tq_quantize_with_rotation(_ptr(params), d, b, _ptr(x), _dtype_code(x, "x"), n,
                                                    _ptr(codes), _ptr(nu), _ptr(gamma), _ptr(u),
                                                    _stream(stream, x.device)))


def tq_quantize_mse(params, d: int, b: int, x, codes, nu, stream=None):
    """MSE quantizer alone: x [n][d] -> codes [n][d/32][b-1] uint32 (index planes), nu[n]."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [n][{d}]")
    n = x.shape[0]
    for tname, t in (("codes", codes), ("nu", nu), ("params", params)):
        _dev(t, tname)
    _need(codes, "codes", n * (d // 32) * (b - 1), torch.int32)
    _need(nu, "nu", n, torch.float32)
    _check(load_library().tq_quantize_mse(_ptr(params), d, b, _ptr(x), _dtype_code(x, "x"), n,
                                          _ptr(codes), _ptr(nu), _stream(stream, x.device)))


def tq_append_ws_bytes(d: int, b: int, groups: int) -> int:
    return int(load_library().tq_append_ws_bytes(d, b, groups))


def tq_append(params, d: int, b: int, mode: int, x, cap: int, pos: int, codes, nu, gamma, ws,
              stream=None):
    """Encode x [groups][d] and write vector g to slot (g, pos) of [groups][cap] caches."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [groups][{d}]")
    groups = x.shape[0]
    planes = b if mode == TQ_EST_PROD else b - 1
    for tname, t in (("codes", codes), ("nu", nu), ("ws", ws), ("params", params)):
        _dev(t, tname)
    _need(codes, "codes", groups * cap * (d // 32) * planes, torch.int32)
    _need(nu, "nu", groups * cap, torch.float32)
    if mode == TQ_EST_PROD:
        _dev(gamma, "gamma")
        _need(gamma, "gamma", groups * cap, torch.float32)
    _check(load_library().tq_append(_ptr(params), d, b, int(mode), _ptr(x), _dtype_code(x, "x"), groups,
                                    cap, pos, _ptr(codes), _ptr(nu),
                                    _ptr(gamma) if gamma is not None else None, _ptr(ws),
                                    ws.numel() * ws.element_size(), _stream(stream, x.device)))


def tq_dequantize(params, d: int, b: int, codes, nu, gamma, mode: int, xhat, stream=None):
    """Reconstruct xhat [n][d] float32 from codes/nu/gamma (n = nu.numel())."""
    torch = _torch()
    for tname, t in (("codes", codes), ("nu", nu), ("gamma", gamma), ("xhat", xhat), ("params", params)):
        _dev(t, tname)
    n = nu.numel()
    _need(codes, "codes", n * (d // 32) * b, torch.int32)
    _need(gamma, "gamma", n, torch.float32)
    _need(xhat, "xhat", n * d, torch.float32)
    _check(load_library().tq_dequantize(_ptr(params), d, b, _ptr(codes), _ptr(nu), _ptr(gamma), n,
                                        int(mode), _ptr(xhat), _stream(stream, nu.device)))


def tq_score_ws_bytes(d: int, b: int, groups: int, G: int, T: int) -> int:
    return int(load_library().tq_score_ws_bytes(d, b, groups, G, T))


def tq_score_ip(params, d: int, b: int, q, codes, nu, gamma, groups: int, G: int, T: int,
                mode: int, logits, ws, stream=None):
    """logits[groups][G][T] = estimated <q, k> for q [groups][G][d], keys codes [groups][T]."""
    torch = _torch()
    for tname, t in (("q", q), ("codes", codes), ("nu", nu), ("gamma", gamma), ("logits", logits),
                     ("ws", ws), ("params", params)):
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    _need(codes, "codes", groups * T * (d // 32) * b, torch.int32)
    _need(nu, "nu", groups * T, torch.float32)
    _need(gamma, "gamma", groups * T, torch.float32)
    _need(logits, "logits", groups * G * T, torch.float32)
    _check(load_library().tq_score_ip(_ptr(params), d, b, _ptr(q), _dtype_code(q, "q"), _ptr(codes),
                                      _ptr(nu), _ptr(gamma), groups, G, T, int(mode), _ptr(logits),
                                      _ptr(ws), ws.numel() * ws.element_size(),
                                      _stream(stream, q.device)))


def tq_score_prepare(params, d: int, b: int, q, groups: int, G: int, ws, stream=None):
    """Query operands of q [groups][G][d] into ws, for tq_score_ip_prepared."""
    for tname, t in (("q", q), ("ws", ws), ("params", params)):
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    _check(load_library().tq_score_prepare(_ptr(params), d, b, _ptr(q), _dtype_code(q, "q"), groups, G,
                                           _ptr(ws), ws.numel() * ws.element_size(), _stream(stream, q.device)))


def tq_score_ip_prepared(params, d: int, b: int, codes, nu, gamma, groups: int, G: int, T: int,
                         mode: int, logits, ws, stream=None):
    """logits[groups][G][T] from the query operands tq_score_prepare left in ws."""
    torch = _torch()
    for tname, t in (("codes", codes), ("nu", nu), ("gamma", gamma), ("logits", logits), ("ws", ws),
                     ("params", params)):
        _dev(t, tname)
    _need(codes, "codes", groups * T * (d // 32) * b, torch.int32)
    _need(nu, "nu", groups * T, torch.float32)
    _need(gamma, "gamma", groups * T, torch.float32)
    _need(logits, "logits", groups * G * T, torch.float32)
    _check(load_library().tq_score_ip_prepared(_ptr(params), d, b, _ptr(codes), _ptr(nu), _ptr(gamma), groups,
                                               G, T, int(mode), _ptr(logits), _ptr(ws),
                                               ws.numel() * ws.element_size(), _stream(stream, codes.device)))


def tq_score_noalloc_max_ws_bytes() -> int:
    return int(load_library().tq_score_noalloc_max_ws_bytes())


def tq_score_ip_noalloc(params, d: int, b: int, q, codes, nu, gamma, groups: int, G: int, T: int,
                        mode: int, logits, stream=None):
    """tq_score_ip with the library's fixed per-GPU scratch in place of a workspace."""
    torch = _torch()
    for tname, t in (("q", q), ("codes", codes), ("nu", nu), ("gamma", gamma), ("logits", logits),
                     ("params", params)):
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    _need(codes, "codes", groups * T * (d // 32) * b, torch.int32)
    _need(nu, "nu", groups * T, torch.float32)
    _need(gamma, "gamma", groups * T, torch.float32)
    _need(logits, "logits", groups * G * T, torch.float32)
    _check(load_library().tq_score_ip_noalloc(_ptr(params), d, b, _ptr(q), _dtype_code(q, "q"), _ptr(codes),
                                              _ptr(nu), _ptr(gamma), groups, G, T, int(mode), _ptr(logits),
                                              _stream(stream, q.device)))


def tq_quantize_split(params0, params1, d: int, d0: int, b0: int, b1: int, x, codes0, nu0, gamma0,
                      codes1, nu1, gamma1, stream=None):
    """Fractional rate: channels [0, d0) of x [n][d] at b0 bits (params0), [d0, d) at b1."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [n][{d}]")
    n = x.shape[0]
    for tname, t in (("codes0", codes0), ("nu0", nu0), ("gamma0", gamma0), ("codes1", codes1),
                     ("nu1", nu1), ("gamma1", gamma1), ("params0", params0), ("params1", params1)):
        _dev(t, tname)
    _need(codes0, "codes0", n * (d0 // 32) * b0, torch.int32)
    _need(codes1, "codes1", n * ((d - d0) // 32) * b1, torch.int32)
    for tname, t in (("nu0", nu0), ("gamma0", gamma0), ("nu1", nu1), ("gamma1", gamma1)):
        _need(t, tname, n, torch.float32)
    _check(load_library().tq_quantize_split(_ptr(params0), _ptr(params1), d, d0, b0, b1, _ptr(x),
                                            _dtype_code(x, "x"), n, _ptr(codes0), _ptr(nu0),
                                            _ptr(gamma0), _ptr(codes1), _ptr(nu1), _ptr(gamma1),
                                            _stream(stream, x.device)))


def tq_score_split_ws_bytes(d: int, d0: int, b0: int, b1: int, groups: int, G: int, T: int) -> int:
    return int(load_library().tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, T))


def tq_score_ip_split(params0, params1, d: int, d0: int, b0: int, b1: int, q, codes0, nu0, gamma0,
                      codes1, nu1, gamma1, groups: int, G: int, T: int, mode: int, logits, ws,
                      stream=None):
    """logits[groups][G][T] = the two channel groups' estimates summed (tq_quantize_split codes)."""
    torch = _torch()
    for tname, t in (("q", q), ("codes0", codes0), ("nu0", nu0), ("gamma0", gamma0),
                     ("codes1", codes1), ("nu1", nu1), ("gamma1", gamma1), ("logits", logits),
                     ("ws", ws), ("params0", params0), ("params1", params1)):
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    _need(codes0, "codes0", groups * T * (d0 // 32) * b0, torch.int32)
    _need(codes1, "codes1", groups * T * ((d - d0) // 32) * b1, torch.int32)
    for tname, t in (("nu0", nu0), ("gamma0", gamma0), ("nu1", nu1), ("gamma1", gamma1)):
        _need(t, tname, groups * T, torch.float32)
    _need(logits, "logits", groups * G * T, torch.float32)
    _check(load_library().tq_score_ip_split(_ptr(params0), _ptr(params1), d, d0, b0, b1, _ptr(q),
                                            _dtype_code(q, "q"), _ptr(codes0), _ptr(nu0), _ptr(gamma0),
                                            _ptr(codes1), _ptr(nu1), _ptr(gamma1), groups, G, T,
                                            int(mode), _ptr(logits), _ptr(ws),
                                            ws.numel() * ws.element_size(), _stream(stream, q.device)))


def tq_score_split_prepare(params0, params1, d: int, d0: int, b0: int, b1: int, q, groups: int, G: int,
                           ws, stream=None):
    """Both channel groups' query operands of q [groups][G][d] into ws, for tq_score_ip_split_prepared."""
    for tname, t in (("q", q), ("ws", ws), ("params0", params0), ("params1", params1)):
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    _check(load_library().tq_score_split_prepare(_ptr(params0), _ptr(params1), d, d0, b0, b1, _ptr(q),
                                                 _dtype_code(q, "q"), groups, G, _ptr(ws),
                                                 ws.numel() * ws.element_size(), _stream(stream, q.device)))


def tq_score_ip_split_prepared(params0, params1, d: int, d0: int, b0: int, b1: int, codes0, nu0, gamma0,
                               codes1, nu1, gamma1, groups: int, G: int, T: int, mode: int, logits, ws,
                               stream=None):
    """tq_score_ip_split's logits from the query operands tq_score_split_prepare left in ws."""
    torch = _torch()
    for tname, t in (("codes0", codes0), ("nu0", nu0), ("gamma0", gamma0), ("codes1", codes1), ("nu1", nu1),
                     ("gamma1", gamma1), ("logits", logits), ("ws", ws), ("params0", params0),
                     ("params1", params1)):
        _dev(t, tname)
    _need(codes0, "codes0", groups * T * (d0 // 32) * b0, torch.int32)
    _need(codes1, "codes1", groups * T * ((d - d0) // 32) * b1, torch.int32)
    for tname, t in (("nu0", nu0), ("gamma0", gamma0), ("nu1", nu1), ("gamma1", gamma1)):
        _need(t, tname, groups * T, torch.float32)
    _need(logits, "logits", groups * G * T, torch.float32)
    _check(load_library().tq_score_ip_split_prepared(_ptr(params0), _ptr(params1), d, d0, b0, b1, _ptr(codes0),
                                                     _ptr(nu0), _ptr(gamma0), _ptr(codes1), _ptr(nu1),
                                                     _ptr(gamma1), groups, G, T, int(mode), _ptr(logits),
                                                     _ptr(ws), ws.numel() * ws.element_size(),
                                                     _stream(stream, codes0.device)))


def tq_quantize_mse_split(params0, params1, d: int, d0: int, b0: int, b1: int, x, codes0, nu0, codes1,
                          nu1, stream=None):
    """Values of a fractional-rate cache: channels [0, d0) of x [n][d] by params0, the rest by params1."""
    torch = _torch()
    _dev(x, "x")
    if x.dim() != 2 or x.shape[1] != d:
        raise ValueError(f"x must be [n][{d}]")
    n = x.shape[0]
    for tname, t in (("codes0", codes0), ("nu0", nu0), ("codes1", codes1), ("nu1", nu1),
                     ("params0", params0), ("params1", params1)):
        _dev(t, tname)
    _need(codes0, "codes0", n * (d0 // 32) * (b0 - 1), torch.int32)
    _need(codes1, "codes1", n * ((d - d0) // 32) * (b1 - 1), torch.int32)
    _need(nu0, "nu0", n, torch.float32)
    _need(nu1, "nu1", n, torch.float32)
    _check(load_library().tq_quantize_mse_split(_ptr(params0), _ptr(params1), d, d0, b0, b1, _ptr(x),
                                                _dtype_code(x, "x"), n, _ptr(codes0), _ptr(nu0),
                                                _ptr(codes1), _ptr(nu1), _stream(stream, x.device)))


def tq_attention_split_ws_bytes(d: int, d0: int, bk0: int, bk1: int, groups: int, G: int, T: int) -> int:
    return int(load_library().tq_attention_split_ws_bytes(d, d0, bk0, bk1, groups, G, T))


def tq_attention_split(params_k0, params_k1, params_v0, params_v1, d: int, d0: int, bk0: int, bk1: int,
                       bv0: int, bv1: int, q, codes_k0, nu_k0, gamma_k0, codes_k1, nu_k1, gamma_k1,
                       codes_v0, nu_v0, codes_v1, nu_v1, groups: int, G: int, T: int, scale: float,
                       mode: int, out, ws, stream=None):
    """Decode attention over a fractional-rate KV cache -> out [groups][G][d] float32."""
    torch = _torch()
    named = (("q", q), ("codes_k0", codes_k0), ("nu_k0", nu_k0), ("gamma_k0", gamma_k0),
             ("codes_k1", codes_k1), ("nu_k1", nu_k1), ("gamma_k1", gamma_k1), ("codes_v0", codes_v0),
             ("nu_v0", nu_v0), ("codes_v1", codes_v1), ("nu_v1", nu_v1), ("out", out), ("ws", ws),
             ("params_k0", params_k0), ("params_k1", params_k1), ("params_v0", params_v0),
             ("params_v1", params_v1))
    for tname, t in named:
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    n = groups * T
    _need(codes_k0, "codes_k0", n * (d0 // 32) * bk0, torch.int32)
    _need(codes_k1, "codes_k1", n * ((d - d0) // 32) * bk1, torch.int32)
    _need(codes_v0, "codes_v0", n * (d0 // 32) * (bv0 - 1), torch.int32)
    _need(codes_v1, "codes_v1", n * ((d - d0) // 32) * (bv1 - 1), torch.int32)
    for tname, t in (("nu_k0", nu_k0), ("gamma_k0", gamma_k0), ("nu_k1", nu_k1), ("gamma_k1", gamma_k1),
                     ("nu_v0", nu_v0), ("nu_v1", nu_v1)):
        _need(t, tname, n, torch.float32)
    _need(out, "out", groups * G * d, torch.float32)
    _check(load_library().tq_attention_split(
        _ptr(params_k0), _ptr(params_k1), _ptr(params_v0), _ptr(params_v1), d, d0, bk0, bk1, bv0, bv1,
        _ptr(q), _dtype_code(q, "q"), _ptr(codes_k0), _ptr(nu_k0), _ptr(gamma_k0), _ptr(codes_k1),
        _ptr(nu_k1), _ptr(gamma_k1), _ptr(codes_v0), _ptr(nu_v0), _ptr(codes_v1), _ptr(nu_v1), groups, G, T,
        float(scale), int(mode), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
        _stream(stream, q.device)))


def tq_attention_ws_bytes(d: int, b_k: int, groups: int, G: int, T: int) -> int:
    return int(load_library().tq_attention_ws_bytes(d, b_k, groups, G, T))


def tq_attention(params_k, params_v, d: int, b_k: int, b_v: int, q, codes_k, nu_k, gamma_k,
                 codes_v, nu_v, groups: int, G: int, T: int, scale: float, mode: int, out, ws,
                 stream=None):
    """out[groups][G][d] = softmax(scale * estimated logits) times the MSE-reconstructed values."""
    torch = _torch()
    for tname, t in (("q", q), ("codes_k", codes_k), ("nu_k", nu_k), ("gamma_k", gamma_k),
                     ("codes_v", codes_v), ("nu_v", nu_v), ("out", out), ("ws", ws),
                     ("params_k", params_k), ("params_v", params_v)):
        _dev(t, tname)
    if q.numel() < groups * G * d:
        raise ValueError("q holds fewer than groups*G*d elements")
    _need(codes_k, "codes_k", groups * T * (d // 32) * b_k, torch.int32)
    _need(nu_k, "nu_k", groups * T, torch.float32)
    _need(gamma_k, "gamma_k", groups * T, torch.float32)
    _need(codes_v, "codes_v", groups * T * (d // 32) * (b_v - 1), torch.int32)
    _need(nu_v, "nu_v", groups * T, torch.float32)
    _need(out, "out", groups * G * d, torch.float32)
    _check(load_library().tq_attention(_ptr(params_k), _ptr(params_v), d, b_k, b_v, _ptr(q),
                                       _dtype_code(q, "q"), _ptr(codes_k), _ptr(nu_k), _ptr(gamma_k),
                                       _ptr(codes_v), _ptr(nu_v), groups, G, T, float(scale),
                                       int(mode), _ptr(out), _ptr(ws), ws.numel() * ws.element_size(),
                                       _stream(stream, q.device)))


def tq_topk_ws_bytes(d: int, b: int, nq: int, n: int, k: int) -> int:
    return int(load_library().tq_topk_ws_bytes(d, b, nq, n, k))


def tq_topk(params, d: int, b: int, q, codes, nu, gamma, n: int, k: int, mode: int, idx, score,
            ws, stream=None):
    """Top-k keys by estimated inner product for each query row of q [nq][d]."""
    torch = _torch()
    for tname, t in (("q", q), ("codes", codes), ("nu", nu), ("gamma", gamma), ("idx", idx),
                     ("score", score), ("ws", ws), ("params", params)):
        _dev(t, tname)
    if q.dim() != 2 or q.shape[1] != d:
        raise ValueError(f"q must be [nq][{d}]")
    nq = q.shape[0]
    _need(codes, "codes", n * (d // 32) * b, torch.int32)
    _need(nu, "nu", n, torch.float32)
    _need(gamma, "gamma", n, torch.float32)
    _need(idx, "idx", nq * k, torch.int32)
    _need(score, "score", nq * k, torch.float32)
    _check(load_library().tq_topk(_ptr(params), d, b, _ptr(q), _dtype_code(q, "q"), nq, _ptr(codes),
                                  _ptr(nu), _ptr(gamma), n, int(k), int(mode), _ptr(idx), _ptr(score),
                                  _ptr(ws), ws.numel() * ws.element_size(),
                                  _stream(stream, q.device)))
