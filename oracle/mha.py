"""Float64 reference arithmetic (test infrastructure only; see package docstring).

Notation follows the Slim Attention article (localbendi.com), section
"K-Cache is All You Need": row-vector convention, Q = X.W_Q, K = X.W_K,
V = X.W_V; W_KV = W_K^-1 . W_V; V = K . W_KV.  A head h owns the columns
[h*dh, (h+1)*dh) of q, K and V.  Scores are scaled by ``scale`` (1/sqrt(dh)
for standard MHA, which the pages leave implicit).
"""
from __future__ import annotations

import math

import numpy as np


# ----------------------------------------------------------------------------
# storage formats

def bf16_decode(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 (round to nearest even) -> bfloat16 (round to nearest
    even), returned as float64 values."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    rest = u & np.uint64(0xFFFF)
    up = (rest > 0x8000) | ((rest == 0x8000) & ((keep & np.uint64(1)) == 1))
    keep = keep + up.astype(np.uint64)
    out = (keep << np.uint64(16)).astype(np.uint32).view(np.float32).astype(np.float64)
    return np.where(np.isfinite(f), out, f.astype(np.float64))


def cache_to_f64(K: np.ndarray) -> np.ndarray:
    """A cache in storage dtype (float32, or uint16 bf16 bits) as float64."""
    if K.dtype == np.uint16:
        return bf16_decode(K)
    return np.asarray(K, dtype=np.float64)


def _clamp_len(n, T):
    return int(min(max(int(n), 0), T))


# ----------------------------------------------------------------------------
# standard MHA decode: the definition the GPU path must reproduce

def mha_decode(q, K, V, lengths, H: int, dh: int, scale: float) -> np.ndarray:
    """Standard multi-head attention for one new query per sequence.

    q [B, H*dh]; K, V [B, T, H*dh] (explicit caches); lengths [B].
    Sequence b attends over its first len_b rows (clamped to [0, T]); a
    sequence with no rows yields zeros.  Returns o [B, H, dh] float64.
    For head h:  s_t = scale * q_h . K[t, h]   (the attention scores),
    p = softmax(s),  o_h = sum_t p_t V[t, h]   (standard MHA, the baseline the
    Slim Attention article rewrites).
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, T = K.shape[0], K.shape[1]
    o = np.zeros((B, H, dh))
    for b in range(B):
        n = _clamp_len(lengths[b], T)
        if n == 0:
            continue
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = scale * (K[b, :n, c] @ q[b, c])
            e = np.exp(s - s.max())
            p = e / e.sum()
            o[b, h] = p @ V[b, :n, c]
    return o


def mha_decode_loop(q, K, V, lengths, H: int, dh: int, scale: float) -> np.ndarray:
    """The same definition written as scalar loops (O(T*d) per sequence).
    Only for tiny inputs; used to pin the matrix form above."""
    B, T = len(K), len(K[0])
    o = np.zeros((B, H, dh))
    for b in range(B):
        n = _clamp_len(lengths[b], T)
        for h in range(H):
            if n == 0:
                continue
            scores = []
            for t in range(n):
                acc = 0.0
                for j in range(dh):
                    acc += float(q[b][h * dh + j]) * float(K[b][t][h * dh + j])
                scores.append(scale * acc)
            m = max(scores)
            weights = [math.exp(x - m) for x in scores]
            z = sum(weights)
            for j in range(dh):
                num = 0.0
                for t in range(n):
                    num += weights[t] * float(V[b][t][h * dh + j])
                o[b, h, j] = num / z
    return o


def explicit_values(K, W_K, W_V, cols=None, block: int = 8192) -> np.ndarray:
    """Explicit value cache for a K cache, built without W_KV.

    The K rows the device reads are K~ = round(X.W_K).  The context that
    produced exactly these rows is X~ = K~ . W_K^-1 (float64 linear solve of
    X~ W_K = K~), and its MHA value rows are V = X~ . W_V.  ``cols`` selects
    columns of V (default: all).  K may be [T, d] or [B, T, d], in storage
    dtype or float64; rows are processed in blocks of ``block``.
    """
    K = np.asarray(K)
    W_K = np.asarray(W_K, dtype=np.float64)
    W_V = np.asarray(W_V, dtype=np.float64)
    Wv = W_V if cols is None else W_V[:, cols]
    shape = K.shape
    flat = K.reshape(-1, shape[-1])
    out = np.empty((flat.shape[0], Wv.shape[1]))
    WKt = W_K.T
    for r0 in range(0, flat.shape[0], block):
        r1 = min(flat.shape[0], r0 + block)
        Kb = cache_to_f64(flat[r0:r1])
        Xt = np.linalg.solve(WKt, Kb.T).T          # X~ W_K = K~
        out[r0:r1] = Xt @ Wv
    return out.reshape(shape[:-1] + (Wv.shape[1],))


def value_map(W_K, W_V, cols=None) -> np.ndarray:
    """M = W_K^-1 . W_V[:, cols] by float64 solve of W_K . M = W_V[:, cols]:
    the map from cache rows to the value columns ``cols`` of the context that
    produced them (V[:, cols] = K~ . M), for ``explicit_values_cols``."""
    W_V = np.asarray(W_V, dtype=np.float64)
    return np.linalg.solve(np.asarray(W_K, dtype=np.float64), W_V if cols is None else W_V[:, cols])


def explicit_values_cols(K, W_K, W_V, cols, block: int = 16384, M=None) -> np.ndarray:
    """V[..., cols] of ``explicit_values``, with the float64 product
    associated the other way: K~ . (W_K^-1 . W_V[:, cols]) instead of
    (K~ . W_K^-1) . W_V[:, cols].  Same definition, one d x d solve instead of
    one per row block; used for the full-size caches and pinned against
    ``explicit_values`` on small inputs.  ``M`` may pass ``value_map(W_K, W_V,
    cols)`` computed once for many calls (W_K and W_V are then not used)."""
    K = np.asarray(K)
    Y = value_map(W_K, W_V, cols) if M is None else np.asarray(M, dtype=np.float64)
    shape = K.shape
    flat = K.reshape(-1, shape[-1])
    out = np.empty((flat.shape[0], Y.shape[1]))
    for r0 in range(0, flat.shape[0], block):
        r1 = min(flat.shape[0], r0 + block)
        out[r0:r1] = cache_to_f64(flat[r0:r1]) @ Y
    return out.reshape(shape[:-1] + (Y.shape[1],))


# ----------------------------------------------------------------------------
# the Slim forms (pinned against the definition; not used as GPU reference)

def wkv(W_K, W_V) -> np.ndarray:
    """W_KV = W_K^-1 . W_V (Slim Attention article, section "K-Cache is All You
    Need", the new parameter matrix), by float64 LU solve of W_K . W_KV = W_V."""
    return np.linalg.solve(np.asarray(W_K, dtype=np.float64), np.asarray(W_V, dtype=np.float64))


def slim_decode_opt1(q, K, W_KV, lengths, H: int, dh: int, scale: float) -> np.ndarray:
    """Generation step, first option of the article: compute V = K . W_KV
    from the K cache, then multiply the softmax result by V."""
    K = cache_to_f64(np.asarray(K))
    V = K @ np.asarray(W_KV, dtype=np.float64)
    return mha_decode(q, K, V, lengths, H, dh, scale)


def slim_decode_opt2(q, K, W_KV, lengths, H: int, dh: int, scale: float) -> np.ndarray:
    """Generation step, second option of the article (better for long
    sequences): multiply the softmax result by K first, then by W_KV.
    Head h's value columns are K (all d columns) . W_KV[:, h*dh:(h+1)*dh], so
    the softmax row of head h multiplies every column of K."""
    q = np.asarray(q, dtype=np.float64)
    K = cache_to_f64(np.asarray(K))
    W_KV = np.asarray(W_KV, dtype=np.float64)
    B, T = K.shape[0], K.shape[1]
    o = np.zeros((B, H, dh))
    for b in range(B):
        n = _clamp_len(lengths[b], T)
        if n == 0:
            continue
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = scale * (K[b, :n, c] @ q[b, c])
            e = np.exp(s - s.max())
            p = e / e.sum()
            u = p @ K[b, :n, :]                    # [d]
            o[b, h] = u @ W_KV[:, c]
    return o


# ----------------------------------------------------------------------------
# prompt phase: the K cache write

def prefill(X, W_K, cache: str) -> np.ndarray:
    """K = X . W_K in float64, rounded to the cache format ("f32": to float32;
    "bf16": to float32 then bfloat16, both round-to-nearest-even).  The prompt
    phase computes K for all tokens and caches it (article section "K-Cache is
    All You Need", prompt phase).  X [..., d] and W_K [d, d] are taken as
    float64 values of whatever the device is given."""
    Kf = np.asarray(X, dtype=np.float64) @ np.asarray(W_K, dtype=np.float64)
    if cache == "bf16":
        return round_bf16(Kf)
    return Kf.astype(np.float32).astype(np.float64)


def prefill_loop(X, W_K, cache: str) -> np.ndarray:
    """Scalar-loop form of ``prefill`` for tiny inputs."""
    X = np.asarray(X, dtype=np.float64)
    W = np.asarray(W_K, dtype=np.float64)
    n, d = X.shape
    out = np.zeros((n, d))
    for i in range(n):
        for j in range(d):
            acc = 0.0
            for k in range(d):
                acc += X[i, k] * W[k, j]
            out[i, j] = acc
    if cache == "bf16":
        return round_bf16(out)
    return out.astype(np.float32).astype(np.float64)


def err_rel(o, o_ref) -> float:
    """The parity metric: max |o - o_ref| / max |o_ref|, both maxima over the
    whole output (every sequence, head and column), i.e. the max-abs error
    relative to the reference output's L-infinity norm.  When the reference
    is zero everywhere the metric is the absolute max |o - o_ref|.  A NaN
    anywhere makes the result NaN, which fails every `err <= tol` gate."""
    o = np.asarray(o, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    den = np.abs(o_ref).max()
    num = np.abs(o - o_ref).max()
    return float(num / den) if den > 0 else float(num)


# ----------------------------------------------------------------------------
# the whole generation step

def generate_step(x, W_Q, W_K, W_V, K_cache, lengths, H: int, dh: int, scale: float,
                  cache: str):
    """One generation step in the order the Slim Attention article gives
    (section "K-Cache is All You Need", generation phase): first the query of
    the new token, q = x . W_Q; then its scores against the K rows cached at
    earlier steps, their softmax and the attention output (here by the plain
    definition over explicit values, ``mha_decode``); last, the new token's
    key k = x . W_K is appended to the cache for the next step.

    x [B, d]; W_Q, W_K, W_V [d, d] (float64 values of whatever the device is
    given); K_cache [B, T, d] in storage dtype; lengths [B].
    Returns (o [B, H, dh], k_new [B, d] rounded to the cache format as in
    ``prefill``, lengths_next [B]).  Sequence b's new row goes to row
    len_b (clamped to [0, T]); a full cache (len_b = T) takes no new row and
    keeps its length."""
    x = np.asarray(x, dtype=np.float64)
    q = x @ np.asarray(W_Q, dtype=np.float64)
    K = cache_to_f64(np.asarray(K_cache))
    V = explicit_values(K_cache, W_K, W_V)
    o = mha_decode(q, K, V, lengths, H, dh, scale)
    k_new = prefill(x, W_K, cache)
    T = K.shape[1]
    lens = np.array([_clamp_len(n, T) for n in lengths], dtype=np.int64)
    lengths_next = np.where(lens < T, lens + 1, T)
    return o, k_new, lengths_next


def append_rows(K_cache, k_new, lengths):
    """The cache after a generation step: row len_b of sequence b replaced by
    k_new[b] where len_b < T (storage dtype kept; bf16 rows are stored as
    their bit patterns)."""
    K = np.array(K_cache, copy=True)
    T = K.shape[1]
    for b in range(K.shape[0]):
        n = _clamp_len(lengths[b], T)
        if n < T:
            if K.dtype == np.uint16:
                v = np.asarray(k_new[b], dtype=np.float64).astype(np.float32).view(np.uint32)
                K[b, n] = (v >> np.uint32(16)).astype(np.uint16)  # exact: already bf16 values
            else:
                K[b, n] = k_new[b]
    return K


# ----------------------------------------------------------------------------
# many queries over one context: shared-context cross-attention, prompt phase

def multi_query_attention(Q, K, V, limits, H: int, dh: int, scale: float) -> np.ndarray:
    """Standard multi-head attention of n queries over ONE key/value context.

    Q [n, H*dh]; K, V [T, H*dh] explicit (float64 values); limits [n] or
    None: query i attends rows [0, limit_i) (clamped to [0, T]; None = all
    T rows).  A query with no rows yields zeros.  Returns [n, H, dh].
    With every limit T this is cross-attention of n decoder queries over one
    shared encoder context; with limit_i = t0 + i + 1 it is the causal
    attention of a prompt's tokens (each token sees itself and all earlier
    rows), the prompt phase of the Slim Attention article (section "K-Cache
    is All You Need": queries and keys of all prompt tokens computed in
    parallel)."""
    Q = np.asarray(Q, dtype=np.float64)
    K = cache_to_f64(np.asarray(K))
    V = np.asarray(V, dtype=np.float64)
    n, T = Q.shape[0], K.shape[0]
    lim = np.full(n, T) if limits is None else np.asarray(limits)
    o = np.zeros((n, H, dh))
    for i in range(n):
        r = _clamp_len(lim[i], T)
        if r == 0:
            continue
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = scale * (K[:r, c] @ Q[i, c])
            e = np.exp(s - s.max())
            o[i, h] = (e / e.sum()) @ V[:r, c]
    return o


def multi_query_cost(n: int, H: int, T: int, d: int) -> dict:
    """Multiply-accumulate counts of the two generation options of the Slim
    Attention article (section "K-Cache is All You Need") for n queries over
    a T-row context, projections included: option 1 forms V = K.W_KV
    (T d^2) and multiplies the softmax by it (n T d); option 2 multiplies the
    softmax of every head by all d columns of K (n H T d) and the n H rows by
    W_KV's head slices (n d^2)."""
    return {"opt1": T * d * d + n * T * d, "opt2": n * H * T * d + n * d * d}
