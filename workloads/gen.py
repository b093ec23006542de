"""Seeded input generators for the TurboQuant quantize / inner-product path.

Every array is drawn from NumPy's PCG64 seeded by ``SeedSequence([cfg, role, *extra])``
so that any chunk of any workload can be regenerated on its own, on any host.
Draws are taken in float64 (``standard_normal``); float32 inputs are the float64 draws
rounded to nearest; bf16 inputs are those float32 values rounded to nearest-even.

The random rotation and the random projection are *inputs* of the method (the pages
draw them once, independently of the data): they are drawn here, once per
(configuration, repetition), and handed to both sides as float32 arrays.

Nothing here quantizes, rotates or estimates anything.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = [
    "ROLE_DATA", "ROLE_QUERY", "ROLE_PI", "ROLE_S", "ROLE_OUTLIER", "ROLE_BASIS",
    "rng", "haar_orthogonal", "gaussian_matrix", "f32_to_bf16_bits", "bf16_bits_to_f32",
    "unit_sphere", "outlier_channels", "kv_keys_chunk", "kv_queries", "kv_keys",
    "lowrank_basis", "lowrank_block", "lowrank_vectors", "lowrank_queries",
    "KVConfig", "SearchConfig", "TOY", "DECODE_LAYER", "DECODE_BATCH16", "EMBED_SEARCH",
    "LONG_CONTEXT", "CONFIGS", "LOWRANK_BLOCK",
]

ROLE_DATA, ROLE_QUERY, ROLE_PI, ROLE_S, ROLE_OUTLIER, ROLE_BASIS = range(6)

#: vectors per independently seeded block of the low-rank embedding workload
LOWRANK_BLOCK = 16384


def rng(cfg: int, role: int, *extra: int) -> np.random.Generator:
    """PCG64 generator for (configuration, role, extra counters)."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([cfg, role, *extra])))


# ----------------------------------------------------------------------------- dtypes

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the raw uint16 bits.

    NaN payloads are kept quiet (0x7FC0) so that rounding never turns a NaN into Inf.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of raw bfloat16 bits (uint16) to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ method parameters

def haar_orthogonal(d: int, cfg: int, rep: int = 0, role: int = ROLE_PI) -> np.ndarray:
    """Random orthogonal d x d matrix, Haar distributed, as float32.

    Drawn as the Q factor of a QR factorisation of a standard Gaussian matrix, with each
    column multiplied by the sign of the matching diagonal entry of R (this sign fix is
    what makes the distribution uniform over the orthogonal group).  ``role`` picks the
    random stream (ROLE_S for an orthogonal QJL matrix).
    """
    g = rng(cfg, role, rep).standard_normal((d, d))
    q, r = np.linalg.qr(g)
    q = q * np.sign(np.diag(r))[None, :]
    return np.ascontiguousarray(q.astype(np.float32))


def gaussian_matrix(m: int, d: int, cfg: int, rep: int = 0) -> np.ndarray:
    """m x d matrix of independent N(0, 1) entries, as float32."""
    return np.ascontiguousarray(rng(cfg, ROLE_S, rep).standard_normal((m, d)).astype(np.float32))


# ------------------------------------------------------------------------- workloads

def unit_sphere(n: int, d: int, cfg: int, role: int, rep: int = 0) -> np.ndarray:
    """n float32 vectors drawn N(0, I_d) and scaled to unit length (in float64)."""
    x = rng(cfg, role, rep).standard_normal((n, d))
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return np.ascontiguousarray(x.astype(np.float32))


def outlier_channels(cfg: int, n_heads: int, d: int, per_head: int = 4) -> np.ndarray:
    """For each KV head, ``per_head`` distinct channels (sorted) that carry outliers."""
    g = rng(cfg, ROLE_OUTLIER, 0)
    return np.stack([np.sort(g.choice(d, size=per_head, replace=False)) for _ in range(n_heads)])


def kv_keys_chunk(cfg: int, seq: int, head: int, T: int, d: int, channels: np.ndarray,
                  scale: float = 20.0, rep: int = 0) -> np.ndarray:
    """Keys of one (sequence, KV head): [T][d] bf16 bits.

    N(0, 1) entries, the head's outlier channels multiplied by ``scale`` on every token,
    then float64 -> float32 -> bf16 (round to nearest even).
    """
    k = rng(cfg, ROLE_DATA, rep, seq, head).standard_normal((T, d))
    k[:, channels] *= scale
    return f32_to_bf16_bits(k.astype(np.float32))


def kv_keys(cfg: int, n_seq: int, n_kv: int, T: int, d: int, rep: int = 0,
            channels: np.ndarray | None = None) -> np.ndarray:
    """Whole key cache [n_seq * n_kv][T][d] bf16 bits (group g = seq * n_kv + head)."""
    if channels is None:
        channels = outlier_channels(cfg, n_kv, d)
    out = np.empty((n_seq * n_kv, T, d), dtype=np.uint16)
    for s in range(n_seq):
        for h in range(n_kv):
            out[s * n_kv + h] = kv_keys_chunk(cfg, s, h, T, d, channels[h], rep=rep)
    return out


def kv_queries(cfg: int, n_seq: int, n_q_heads: int, d: int, rep: int = 0) -> np.ndarray:
    """Decode-step queries [n_seq][n_q_heads][d] bf16 bits, N(0, 1), no outliers.

    Query head j of a sequence attends with KV head j // (n_q_heads // n_kv): GQA groups of
    consecutive query heads, so [n_seq][n_q_heads][d] is already [groups][G][d].
    """
    q = rng(cfg, ROLE_QUERY, rep).standard_normal((n_seq, n_q_heads, d))
    return f32_to_bf16_bits(q.astype(np.float32))


def lowrank_basis(d: int, rank: int, cfg: int) -> np.ndarray:
    """Shared low-rank basis B ~ N(0, 1)^{d x rank} (float64)."""
    return rng(cfg, ROLE_BASIS, 0).standard_normal((d, rank))


def _lowrank_draw(g: np.random.Generator, n: int, basis: np.ndarray, snr: float) -> np.ndarray:
    d, rank = basis.shape
    w = g.standard_normal((n, rank))
    noise_var = rank / snr  # E|Bw|^2 = d*rank, E|eps|^2 = d*rank/snr
    eps = g.standard_normal((n, d)) * math.sqrt(noise_var)
    x = w @ basis.T + eps
    x /= np.linalg.norm(x, axis=1, keepdims=True)
    return x.astype(np.float32)


def lowrank_block(block: int, d: int, rank: int, snr: float, cfg: int, rep: int = 0,
                  basis: np.ndarray | None = None, n_total: int | None = None) -> np.ndarray:
    """Vectors [block*LOWRANK_BLOCK, ...) of the low-rank-plus-noise embedding set (float32, unit)."""
    if basis is None:
        basis = lowrank_basis(d, rank, cfg)
    n = LOWRANK_BLOCK
    if n_total is not None:
        n = min(n, n_total - block * LOWRANK_BLOCK)
    return _lowrank_draw(rng(cfg, ROLE_DATA, rep, block), n, basis, snr)


def lowrank_vectors(n: int, d: int, rank: int, snr: float, cfg: int, rep: int = 0) -> np.ndarray:
    """The first n vectors of the low-rank embedding set (block-seeded, so prefixes agree)."""
    basis = lowrank_basis(d, rank, cfg)
    out = np.empty((n, d), dtype=np.float32)
    for blk in range((n + LOWRANK_BLOCK - 1) // LOWRANK_BLOCK):
        lo = blk * LOWRANK_BLOCK
        out[lo:lo + LOWRANK_BLOCK] = lowrank_block(blk, d, rank, snr, cfg, rep, basis, n_total=n)
    return out


def lowrank_queries(nq: int, d: int, rank: int, snr: float, cfg: int, rep: int = 0) -> np.ndarray:
    """Queries drawn from the same low-rank law as the embedding set (float32, unit)."""
    return _lowrank_draw(rng(cfg, ROLE_QUERY, rep), nq, lowrank_basis(d, rank, cfg), snr)


# ---------------------------------------------------------------------- config table

@dataclasses.dataclass(frozen=True)
class KVConfig:
    """A quantized key cache scored by one decode step (GQA)."""
    cfg: int
    name: str
    n_seq: int
    n_kv: int
    T: int
    d: int
    bits: tuple
    n_q_heads: int          # per sequence
    dtype: str = "bf16"

    @property
    def G(self) -> int:
        return self.n_q_heads // self.n_kv

    @property
    def groups(self) -> int:
        return self.n_seq * self.n_kv

    @property
    def n_keys(self) -> int:
        return self.groups * self.T


@dataclasses.dataclass(frozen=True)
class SearchConfig:
    """Unit vectors quantized once, then scored against a batch of queries (flat scan)."""
    cfg: int
    name: str
    n: int
    d: int
    bits: tuple
    nq: int
    k: int = 10
    dtype: str = "f32"
    lowrank: tuple | None = None   # (rank, snr) or None for the isotropic unit sphere


TOY = SearchConfig(0, "toy", n=4096, d=128, bits=(4,), nq=64, k=10)
DECODE_LAYER = KVConfig(1, "decode_layer", n_seq=1, n_kv=8, T=32768, d=128, bits=(4,), n_q_heads=32)
DECODE_BATCH16 = KVConfig(2, "decode_batch16", n_seq=16, n_kv=8, T=8192, d=128, bits=(2, 3),
                          n_q_heads=32)
EMBED_SEARCH = SearchConfig(3, "embedding_search", n=1_000_000, d=1536, bits=(2, 4), nq=1000, k=10,
                            lowrank=(64, 3.0))
LONG_CONTEXT = KVConfig(4, "long_context", n_seq=16, n_kv=8, T=131072, d=128, bits=(3,),
                        n_q_heads=32)

CONFIGS = {c.cfg: c for c in (TOY, DECODE_LAYER, DECODE_BATCH16, EMBED_SEARCH, LONG_CONTEXT)}
