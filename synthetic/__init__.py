"""Seeded synthetic workloads for the Slim-Attention decode path.

This module only draws random numbers and lays them out in the storage
formats the decode path consumes.  It holds none of the attention
arithmetic: no scores, no softmax, no W_KV, no value recovery.  Both the
float64 oracle (``oracle/``) and the HIP library are fed from here, and
neither imports the other.

Workload recipe (the five decode configurations of this project, plus the
8K uniform-length point of the 7B shape):

* ``W_Q, W_V ~ N(0, 1/d)`` (second parameter is the variance).
* ``W_K = Qo . diag(s) . Ro`` with ``Qo, Ro`` Haar-random orthogonal
  (sign-fixed QR of a Gaussian matrix) and ``s ~ U[0.5, 2]`` i.i.d., so
  W_K is square and invertible with condition number at most 4, the
  precondition of Slim Attention ("K-Cache is All You Need" section of the
  Slim Attention article: W_K and W_V square, W_K invertible).
* Context rows ``X_b ~ N(0, 1)`` drawn in float32; the new token
  ``x_b ~ N(0, 1)``; the query handed to decode is ``q_b = fp32(x_b . W_Q)``.
* The K cache the decode path reads is ``cache_round(fp32(X_b . W_K))``
  with the product taken in float32 (numpy sgemm) and ``cache_round`` the
  identity for float32 caches and round-to-nearest-even to bfloat16 for
  bf16 caches.  Rows at or beyond ``len_b`` hold ``fill`` (0 by default).
* Configurations whose weights are stored in bf16 (the Whisper-shaped
  cross-attention one) round W_K to bf16 once, here, so that every
  consumer sees the same bf16-representable matrix.

Streams: every role draws from its own ``numpy.random.SeedSequence``
child keyed by ``(seed, role, ...)`` so that any block of rows can be
regenerated alone (row blocks of ``ROW_BLOCK`` tokens per sequence).
"""
from __future__ import annotations

from dataclasses import dataclass, field
import math

import numpy as np

ROW_BLOCK = 1024

# role ids for SeedSequence spawn keys
_R_WEIGHTS, _R_LENGTHS, _R_X, _R_XNEW = 1, 2, 3, 4


@dataclass(frozen=True)
class Config:
    name: str
    d: int
    H: int
    dh: int
    B: int
    T_max: int
    len_lo: int          # lengths ~ U[len_lo, len_hi] (integers, inclusive)
    len_hi: int
    cache: str           # "f32" | "bf16"   K cache storage
    wkv: str             # "f32" | "bf16"   device copy of W_KV
    seed: int
    prefill: bool = False        # K cache written on device from X and W_K
    weights_bf16: bool = False   # W_K stored in bf16
    desc: str = ""

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dh)

    @property
    def ragged(self) -> bool:
        return self.len_lo != self.len_hi


CONFIGS = {
    "tiny_f32": Config("tiny_f32", d=64, H=4, dh=16, B=1, T_max=32, len_lo=32, len_hi=32,
                 cache="f32", wkv="f32", seed=0,
                 desc="tiny MHA decode, fp32: d=64 H=4 dh=16 B=1 T=32"),
    "gpt2_small": Config("gpt2_small", d=768, H=12, dh=64, B=8, T_max=2048, len_lo=2048, len_hi=2048,
                 cache="bf16", wkv="bf16", seed=1,
                 desc="GPT-2-small-shaped layer decode: d=768 H=12 dh=64 B=8 T=2048, bf16 K"),
    "7b_ragged": Config("7b_ragged", d=4096, H=32, dh=128, B=16, T_max=8192, len_lo=1024, len_hi=8192,
                 cache="bf16", wkv="bf16", seed=2,
                 desc="7B-shaped layer decode: d=4096 H=32 dh=128 B=16 T~U[1024,8192], bf16 K and W_KV"),
    "7b_8k": Config("7b_8k", d=4096, H=32, dh=128, B=16, T_max=8192, len_lo=8192, len_hi=8192,
                    cache="bf16", wkv="bf16", seed=2,
                    desc="7B-shaped layer decode at uniform T=8192: d=4096 H=32 dh=128 B=16"),
    "long_128k": Config("long_128k", d=4096, H=32, dh=128, B=1, T_max=131072, len_lo=131072, len_hi=131072,
                 cache="bf16", wkv="bf16", seed=3,
                 desc="long-context single-stream decode: d=4096 H=32 dh=128 B=1 T=131072, bf16 K"),
    "whisper_large": Config("whisper_large", d=1280, H=20, dh=64, B=64, T_max=1500, len_lo=1500, len_hi=1500,
                 cache="bf16", wkv="bf16", seed=4, prefill=True, weights_bf16=True,
                 desc="Whisper-large-shaped cross-attention decode: d=1280 H=20 dh=64 B=64 "
                      "encoder T=1500 written by prefill from X, bf16"),
}


def shrink(cfg: Config, **kw) -> Config:
    """Same recipe and seed with some sizes replaced (parity cases at reduced size)."""
    vals = dict(cfg.__dict__)
    vals.update(kw)
    if "T_max" in kw and "len_hi" not in kw:
        vals["len_hi"] = min(vals["len_hi"], vals["T_max"])
        vals["len_lo"] = min(vals["len_lo"], vals["len_hi"])
    return Config(**vals)


def _rng(cfg: Config, *key: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(cfg.seed, spawn_key=tuple(key)))


# ----------------------------------------------------------------------------
# storage-format helpers (bit layout only)

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)
    r = np.where(nan, (u >> np.uint32(16)) | np.uint32(0x40), r)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# draws

@dataclass
class Weights:
    W_Q: np.ndarray      # [d, d] float64
    W_K: np.ndarray      # [d, d] float64 (bf16-representable when cfg.weights_bf16)
    W_V: np.ndarray      # [d, d] float64
    Qo: np.ndarray       # factors of W_K before any bf16 rounding
    Ro: np.ndarray
    s: np.ndarray


def haar_orthogonal(rng: np.random.Generator, n: int) -> np.ndarray:
    g = rng.standard_normal((n, n))
    q, r = np.linalg.qr(g)
    return q * np.sign(np.diag(r))[None, :]


def weights(cfg: Config) -> Weights:
    d = cfg.d
    rng = _rng(cfg, _R_WEIGHTS)
    W_Q = rng.standard_normal((d, d)) / math.sqrt(d)
    Qo = haar_orthogonal(rng, d)
    Ro = haar_orthogonal(rng, d)
    s = rng.uniform(0.5, 2.0, size=d)
    W_V = rng.standard_normal((d, d)) / math.sqrt(d)
    W_K = (Qo * s[None, :]) @ Ro
    if cfg.weights_bf16:
        W_K = bf16_bits_to_f32(f32_to_bf16_bits(W_K.astype(np.float32))).astype(np.float64)
    return Weights(W_Q=W_Q, W_K=W_K, W_V=W_V, Qo=Qo, Ro=Ro, s=s)


def lengths(cfg: Config) -> np.ndarray:
    if not cfg.ragged:
        return np.full(cfg.B, cfg.len_hi, dtype=np.int32)
    rng = _rng(cfg, _R_LENGTHS)
    return rng.integers(cfg.len_lo, cfg.len_hi, endpoint=True, size=cfg.B).astype(np.int32)


def x_rows(cfg: Config, b: int, t0: int, t1: int) -> np.ndarray:
    """Context rows X_b[t0:t1] (float32), regenerated from per-block streams."""
    out = np.empty((max(t1 - t0, 0), cfg.d), dtype=np.float32)
    blk0, blk1 = t0 // ROW_BLOCK, (t1 + ROW_BLOCK - 1) // ROW_BLOCK
    for blk in range(blk0, blk1):
        lo, hi = blk * ROW_BLOCK, (blk + 1) * ROW_BLOCK
        a, z = max(lo, t0), min(hi, t1)
        if a >= z:
            continue
        rows = _rng(cfg, _R_X, b, blk).standard_normal((z - lo, cfg.d), dtype=np.float32)
        out[a - t0:z - t0] = rows[a - lo:]
    return out


def x_new(cfg: Config) -> np.ndarray:
    return _rng(cfg, _R_XNEW).standard_normal((cfg.B, cfg.d), dtype=np.float32)


def queries(cfg: Config, w: Weights) -> np.ndarray:
    """q_b = fp32(x_b . W_Q), [B, d] float32."""
    return (x_new(cfg).astype(np.float64) @ w.W_Q).astype(np.float32)


def k_rows(cfg: Config, w: Weights, b: int, t0: int, t1: int,
           WK32: np.ndarray | None = None) -> np.ndarray:
    """Cache rows for X_b[t0:t1]: float32 array, or uint16 bf16 bits for bf16 caches."""
    if WK32 is None:
        WK32 = w.W_K.astype(np.float32)
    k = x_rows(cfg, b, t0, t1) @ WK32
    return f32_to_bf16_bits(k) if cfg.cache == "bf16" else k.astype(np.float32)


def k_cache(cfg: Config, w: Weights, lens: np.ndarray, fill: float = 0.0,
            T_alloc: int | None = None) -> np.ndarray:
    """K cache [B, T_alloc, d] in storage dtype; rows >= len_b hold ``fill``."""
    return _proj_cache(cfg, w.W_K, lens, fill, T_alloc)


def v_cache(cfg: Config, w: Weights, lens: np.ndarray, fill: float = 0.0,
            T_alloc: int | None = None) -> np.ndarray:
    """Value cache of standard MHA, cache_round(fp32(X_b . W_V)), same layout
    as ``k_cache``; only the K+V comparator reads it."""
    return _proj_cache(cfg, w.W_V, lens, fill, T_alloc)


def _proj_cache(cfg: Config, W: np.ndarray, lens: np.ndarray, fill: float,
                T_alloc: int | None) -> np.ndarray:
    T_alloc = cfg.T_max if T_alloc is None else T_alloc
    WK32 = W.astype(np.float32)
    if cfg.cache == "bf16":
        fillbits = f32_to_bf16_bits(np.array([fill], dtype=np.float32))[0]
        out = np.full((cfg.B, T_alloc, cfg.d), fillbits, dtype=np.uint16)
    else:
        out = np.full((cfg.B, T_alloc, cfg.d), fill, dtype=np.float32)
    step = 8 * ROW_BLOCK
    for b in range(cfg.B):
        n = int(min(lens[b], T_alloc))
        for t0 in range(0, n, step):
            t1 = min(n, t0 + step)
            k = x_rows(cfg, b, t0, t1) @ WK32
            out[b, t0:t1] = f32_to_bf16_bits(k) if cfg.cache == "bf16" else k
    return out


def prefill_inputs(cfg: Config, w: Weights, n: int | None = None):
    """Inputs of the prefill step: X [B, n, d] and W_K [d, d], both in the
    cache storage format (float32, or uint16 bf16 bits)."""
    n = cfg.T_max if n is None else n
    X = np.stack([x_rows(cfg, b, 0, n) for b in range(cfg.B)])
    if cfg.cache == "bf16":
        return f32_to_bf16_bits(X), f32_to_bf16_bits(w.W_K.astype(np.float32))
    return X, w.W_K.astype(np.float32)


@dataclass
class Workload:
    cfg: Config
    w: Weights
    lengths: np.ndarray
    q: np.ndarray
    K: np.ndarray | None = field(default=None)


def make(cfg: Config | str, with_cache: bool = True, fill: float = 0.0) -> Workload:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    w = weights(cfg)
    lens = lengths(cfg)
    q = queries(cfg, w)
    K = k_cache(cfg, w, lens, fill=fill) if with_cache else None
    return Workload(cfg=cfg, w=w, lengths=lens, q=q, K=K)
