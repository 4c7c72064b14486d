"""Pins for the float64 oracle (CPU only).

Every oracle function is checked against something other than itself: values
worked by hand (tests/golden/hand_*.json), closed forms, scalar-loop brute
force, textbook special cases and a library routine.  The planted-mistake
tests at the end show that the pins catch the plausible slips (a dropped
term, a wrong sign or index, a transposed operand).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synthetic as syn

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


def _rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.abs(a - b).max() / max(np.abs(b).max(), 1e-300))


def _small_case(seed, B=2, T=9, H=2, dh=4, lens=None):
    rng = np.random.default_rng(seed)
    d = H * dh
    q = rng.standard_normal((B, d))
    K = rng.standard_normal((B, T, d))
    V = rng.standard_normal((B, T, d))
    if lens is None:
        lens = rng.integers(1, T + 1, size=B)
    return q, K, V, np.asarray(lens), H, dh, 1.0 / math.sqrt(dh)


# ---------------------------------------------------------------------------
# hand-derived values

def test_hand_two_heads_all_forms():
    g = _load("hand_two_heads.json")
    q = np.array([g["q"]])
    K = np.array([g["K"]])
    V = np.array([g["V"]])
    W = np.array(g["W_KV"])
    o_ref = np.array([g["o"]])
    lens = [2]
    args = (g["H"], g["dh"], g["scale"])
    assert np.abs(oracle.mha_decode(q, K, V, lens, *args) - o_ref).max() < 1e-14
    assert np.abs(oracle.mha_decode_loop(q, K, V, lens, *args) - o_ref).max() < 1e-14
    assert np.abs(oracle.slim_decode_opt1(q, K, W, lens, *args) - o_ref).max() < 1e-13
    assert np.abs(oracle.slim_decode_opt2(q, K, W, lens, *args) - o_ref).max() < 1e-13
    # V = K . W_KV, worked by hand
    assert np.abs(K[0] @ W - V[0]).max() < 1e-14


def test_hand_wkv_and_prefill():
    g = _load("hand_wkv.json")
    W_K, W_V = np.array(g["W_K"]), np.array(g["W_V"])
    assert np.abs(oracle.wkv(W_K, W_V) - np.array(g["W_KV"])).max() < 1e-15
    assert np.abs(np.linalg.inv(W_K) - np.array(g["W_K_inv"])).max() < 1e-15
    X = np.array(g["X"])
    assert np.abs(oracle.prefill(X, W_K, "f32") - np.array(g["K"])).max() == 0
    assert np.abs(oracle.explicit_values(np.array(g["K"]), W_K, W_V) - np.array(g["V"])).max() < 1e-15


# ---------------------------------------------------------------------------
# closed forms and the rewrite identity

@pytest.mark.parametrize("name", ["tiny_f32", "gpt2_small"])
def test_wkv_closed_form(name):
    """W_K = Qo diag(s) Ro  =>  W_K^-1 = Ro^T diag(1/s) Qo^T, so
    W_KV = Ro^T diag(1/s) Qo^T W_V exactly."""
    cfg = syn.CONFIGS[name]
    w = syn.weights(cfg)
    closed = (w.Ro.T / w.s[None, :]) @ (w.Qo.T @ w.W_V)
    assert _rel(oracle.wkv(w.W_K, w.W_V), closed) < 1e-12


def test_eq2_rewrite_tiny_f32():
    """V = X.W_V = (X.W_K).W_KV in float64 to 1e-10 (the identity of the
    article's "K-Cache is All You Need" section)."""
    cfg = syn.CONFIGS["tiny_f32"]
    w = syn.weights(cfg)
    X = syn.x_rows(cfg, 0, 0, cfg.T_max).astype(np.float64)
    V = X @ w.W_V
    V2 = (X @ w.W_K) @ oracle.wkv(w.W_K, w.W_V)
    assert _rel(V2, V) < 1e-10


def test_explicit_values_matches_unrounded_mha_tiny_f32():
    """For an fp32 cache, X~ = K~ W_K^-1 recovers X to fp32 rounding and the
    explicit V tracks X.W_V to the same order."""
    cfg = syn.CONFIGS["tiny_f32"]
    w = syn.weights(cfg)
    lens = syn.lengths(cfg)
    K = syn.k_cache(cfg, w, lens)
    V = oracle.explicit_values(K, w.W_K, w.W_V)
    X = syn.x_rows(cfg, 0, 0, cfg.T_max).astype(np.float64)
    assert _rel(V[0], X @ w.W_V) < 1e-5


def test_explicit_values_cols_matches_full():
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], T_max=96, B=2)
    wl = syn.make(cfg)
    cols = np.r_[64:128, 640:704]
    full = oracle.explicit_values(wl.K, wl.w.W_K, wl.w.W_V)[..., cols]
    part = oracle.explicit_values_cols(wl.K, wl.w.W_K, wl.w.W_V, cols)
    assert _rel(part, full) < 1e-12
    once = oracle.explicit_values_cols(wl.K, None, None, cols, M=oracle.value_map(wl.w.W_K, wl.w.W_V)[:, cols])
    assert _rel(once, full) < 1e-12


def test_value_map_closed_form():
    """value_map = W_K^-1 W_V[:, cols] = Ro^T diag(1/s) Qo^T W_V[:, cols]."""
    cfg = syn.CONFIGS["gpt2_small"]
    w = syn.weights(cfg)
    cols = np.r_[0:64, 700:768]
    closed = (w.Ro.T / w.s[None, :]) @ (w.Qo.T @ w.W_V[:, cols])
    assert _rel(oracle.value_map(w.W_K, w.W_V, cols), closed) < 1e-12


def test_whole_output_reference_helper():
    """The head-group-by-head-group reference of the full-size GPU tests
    equals the plain definition over explicit_values on a ragged case."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from gpu_common import oracle_decode_full
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], d=256, H=4, dh=64, B=4, T_max=40, len_lo=0, len_hi=40)
    wl = syn.make(cfg)
    lens = np.array([40, 0, 1, 23], dtype=np.int32)
    K = syn.k_cache(cfg, wl.w, lens)
    want = oracle.mha_decode(wl.q, oracle.cache_to_f64(K), oracle.explicit_values(K, wl.w.W_K, wl.w.W_V),
                             lens, cfg.H, cfg.dh, cfg.scale)
    got = oracle_decode_full(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V, head_group=3)
    assert _rel(got, want) < 1e-12
    assert np.abs(got[1]).max() == 0


# ---------------------------------------------------------------------------
# brute force

@pytest.mark.parametrize("seed,T,H,dh", [(1, 1, 1, 4), (2, 5, 2, 4), (3, 17, 4, 2), (4, 64, 2, 8)])
def test_loop_vs_matrix(seed, T, H, dh):
    q, K, V, lens, H, dh, scale = _small_case(seed, B=3, T=T, H=H, dh=dh)
    a = oracle.mha_decode(q, K, V, lens, H, dh, scale)
    b = oracle.mha_decode_loop(q, K, V, lens, H, dh, scale)
    assert _rel(a, b) < 1e-12


def test_loop_vs_matrix_tiny_f32():
    cfg = syn.CONFIGS["tiny_f32"]
    wl = syn.make(cfg)
    K = oracle.cache_to_f64(wl.K)
    V = oracle.explicit_values(wl.K, wl.w.W_K, wl.w.W_V)
    a = oracle.mha_decode(wl.q, K, V, wl.lengths, cfg.H, cfg.dh, cfg.scale)
    b = oracle.mha_decode_loop(wl.q, K, V, wl.lengths, cfg.H, cfg.dh, cfg.scale)
    assert _rel(a, b) < 1e-12


def test_prefill_vs_loop():
    rng = np.random.default_rng(7)
    X = rng.standard_normal((3, 8))
    W = rng.standard_normal((8, 8))
    for cache in ("f32", "bf16"):
        assert np.array_equal(oracle.prefill(X, W, cache), oracle.prefill_loop(X, W, cache))


# ---------------------------------------------------------------------------
# textbook special cases

def test_len_one_returns_first_value_row():
    q, K, V, _, H, dh, scale = _small_case(11, B=2, T=6, H=3, dh=4)
    o = oracle.mha_decode(q, K, V, [1, 1], H, dh, scale)
    assert np.abs(o - V[:, 0, :].reshape(2, H, dh)).max() < 1e-15


def test_zero_query_is_mean_of_values():
    q, K, V, _, H, dh, scale = _small_case(12, B=2, T=7, H=2, dh=4)
    lens = [7, 3]
    o = oracle.mha_decode(np.zeros_like(q), K, V, lens, H, dh, scale)
    for b, n in enumerate(lens):
        assert _rel(o[b], V[b, :n].mean(axis=0).reshape(H, dh)) < 1e-14


def test_sharp_query_selects_row():
    q, K, V, _, H, dh, scale = _small_case(13, B=1, T=8, H=2, dh=4)
    for h in range(H):
        c = slice(h * dh, (h + 1) * dh)
        ts = int(np.argmax(np.linalg.norm(K[0, :, c], axis=1)))
        q[0, c] = 1e4 * K[0, ts, c]
        o = oracle.mha_decode(q, K, V, [8], H, dh, scale)
        assert np.abs(o[0, h] - V[0, ts, c]).max() < 1e-9


def test_permutation_invariance():
    q, K, V, _, H, dh, scale = _small_case(14, B=1, T=10, H=2, dh=4)
    perm = np.random.default_rng(0).permutation(10)
    a = oracle.mha_decode(q, K, V, [10], H, dh, scale)
    b = oracle.mha_decode(q, K[:, perm], V[:, perm], [10], H, dh, scale)
    assert _rel(a, b) < 1e-13


def test_duplicated_tokens_invariance():
    q, K, V, _, H, dh, scale = _small_case(15, B=1, T=6, H=2, dh=4)
    a = oracle.mha_decode(q, K, V, [6], H, dh, scale)
    b = oracle.mha_decode(q, np.concatenate([K, K], 1), np.concatenate([V, V], 1), [12], H, dh, scale)
    assert _rel(a, b) < 1e-13


def test_linearity_in_values():
    q, K, V, lens, H, dh, scale = _small_case(16, B=2, T=6, H=2, dh=4)
    V2 = np.random.default_rng(1).standard_normal(V.shape)
    a = oracle.mha_decode(q, K, V + 2.0 * V2, lens, H, dh, scale)
    b = oracle.mha_decode(q, K, V, lens, H, dh, scale) + 2.0 * oracle.mha_decode(q, K, V2, lens, H, dh, scale)
    assert _rel(a, b) < 1e-13


def test_empty_and_clamped_lengths():
    q, K, V, _, H, dh, scale = _small_case(17, B=2, T=5, H=2, dh=4)
    o = oracle.mha_decode(q, K, V, [0, 99], H, dh, scale)
    assert np.all(o[0] == 0)
    assert _rel(o[1], oracle.mha_decode(q, K, V, [0, 5], H, dh, scale)[1]) == 0


def test_identity_wk_gives_wv():
    rng = np.random.default_rng(18)
    W_V = rng.standard_normal((6, 6))
    assert np.array_equal(oracle.wkv(np.eye(6), W_V), W_V)


# ---------------------------------------------------------------------------
# the Slim forms agree with explicit-V MHA

@pytest.mark.parametrize("name,T,B", [("tiny_f32", None, None), ("gpt2_small", 64, 2)])
def test_opt1_opt2_explicit_agree(name, T, B):
    cfg = syn.CONFIGS[name]
    if T is not None:
        cfg = syn.shrink(cfg, T_max=T, B=B)
    wl = syn.make(cfg)
    K = oracle.cache_to_f64(wl.K)
    V = oracle.explicit_values(wl.K, wl.w.W_K, wl.w.W_V)
    W = oracle.wkv(wl.w.W_K, wl.w.W_V)
    args = (wl.lengths, cfg.H, cfg.dh, cfg.scale)
    ref = oracle.mha_decode(wl.q, K, V, *args)
    assert _rel(oracle.slim_decode_opt1(wl.q, wl.K, W, *args), ref) < 1e-10
    assert _rel(oracle.slim_decode_opt2(wl.q, wl.K, W, *args), ref) < 1e-10


# ---------------------------------------------------------------------------
# storage formats, pinned to a library routine

def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(19)
    x = np.concatenate([
        rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
        # exact bf16 ties (lower 16 bits 0x8000) with even and odd kept bits
        (np.arange(1, 2001, dtype=np.uint32) << 16 | 0x8000).view(np.float32).astype(np.float64),
        np.array([0.0, -0.0, 1.0, -1.5, 3.0e38, -3.0e38]),
    ])
    ours = oracle.round_bf16(x)
    ref = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    # the generator's storage rounding follows the same rule
    bits = syn.f32_to_bf16_bits(x.astype(np.float32))
    assert np.array_equal(oracle.bf16_decode(bits), ref)


def test_generator_row_blocks_are_stable():
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], T_max=3000, B=1)
    a = syn.x_rows(cfg, 0, 0, 3000)
    b = syn.x_rows(cfg, 0, 500, 2100)
    c = syn.x_rows(cfg, 0, 0, 700)
    assert np.array_equal(a[500:2100], b)
    assert np.array_equal(a[:700], c)


def test_generator_wk_conditioning():
    for name in ("tiny_f32", "gpt2_small", "whisper_large"):
        w = syn.weights(syn.CONFIGS[name])
        assert np.linalg.cond(w.W_K) <= 4.0 * 1.01


def test_memory_halving():
    """K-only cache bytes are exactly half of K+V cache bytes at equal dtype
    (the article's 2x context-memory claim)."""
    for cfg in syn.CONFIGS.values():
        per = 4 if cfg.cache == "f32" else 2
        k_only = cfg.B * cfg.T_max * cfg.d * per
        kv = 2 * cfg.B * cfg.T_max * cfg.d * per
        assert k_only * 2 == kv


def test_golden_tiny_f32_regression():
    """Guards the oracle against drift: output written by
    tests/golden/make_golden.py (which calls only oracle/ and synthetic/)."""
    g = _load("tiny_f32_oracle.json")
    cfg = syn.CONFIGS["tiny_f32"]
    wl = syn.make(cfg)
    K = oracle.cache_to_f64(wl.K)
    V = oracle.explicit_values(wl.K, wl.w.W_K, wl.w.W_V)
    o = oracle.mha_decode(wl.q, K, V, wl.lengths, cfg.H, cfg.dh, cfg.scale)
    assert _rel(o, np.array(g["o"])) < 1e-12


# ---------------------------------------------------------------------------
# planted mistakes: each mutant of the decode definition must fail a pin

def _mut_no_scale(q, K, V, lens, H, dh, scale):
    return oracle.mha_decode(q, K, V, lens, H, dh, 1.0)


def _mut_no_normalise(q, K, V, lens, H, dh, scale):
    B, T = K.shape[:2]
    o = np.zeros((B, H, dh))
    for b in range(B):
        n = min(int(lens[b]), T)
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = scale * (K[b, :n, c] @ q[b, c])
            o[b, h] = np.exp(s - s.max()) @ V[b, :n, c]
    return o


def _mut_wrong_value_head(q, K, V, lens, H, dh, scale):
    V2 = np.roll(V.reshape(V.shape[0], V.shape[1], H, dh), 1, axis=2).reshape(V.shape)
    return oracle.mha_decode(q, K, V2, lens, H, dh, scale)


def _mut_sign(q, K, V, lens, H, dh, scale):
    return oracle.mha_decode(-np.asarray(q), K, V, lens, H, dh, scale)


def _mut_off_by_one(q, K, V, lens, H, dh, scale):
    return oracle.mha_decode(q, K, V, np.maximum(np.asarray(lens) - 1, 1), H, dh, scale)


def _mut_transposed_head_block(q, K, V, lens, H, dh, scale):
    # scores from K with each head's block transposed (a common layout slip)
    if dh == 1:
        K2 = K[:, :, ::-1]
    else:
        K2 = K.reshape(K.shape[0], K.shape[1], H, dh)[..., ::-1].reshape(K.shape)
    return oracle.mha_decode(q, K2, V, lens, H, dh, scale)


def _pins_pass(f):
    g = _load("hand_two_heads.json")
    ok = np.abs(f(np.array([g["q"]]), np.array([g["K"]]), np.array([g["V"]]), [2],
                  g["H"], g["dh"], g["scale"]) - np.array([g["o"]])).max() < 1e-12
    for seed in (1, 2, 3):
        q, K, V, lens, H, dh, scale = _small_case(seed, B=3, T=7, H=2, dh=4)
        ok &= _rel(f(q, K, V, lens, H, dh, scale),
                   oracle.mha_decode_loop(q, K, V, lens, H, dh, scale)) < 1e-12
    return bool(ok)


@pytest.mark.parametrize("mutant", [_mut_no_scale, _mut_no_normalise, _mut_wrong_value_head,
                                    _mut_sign, _mut_off_by_one, _mut_transposed_head_block])
def test_pins_catch_planted_mistakes(mutant):
    assert _pins_pass(oracle.mha_decode)
    assert not _pins_pass(mutant)


def test_pins_catch_transposed_wkv():
    g = _load("hand_two_heads.json")
    args = (np.array([g["q"]]), np.array([g["K"]]), np.array(g["W_KV"]).T, [2], g["H"], g["dh"], g["scale"])
    assert np.abs(oracle.slim_decode_opt2(*args) - np.array([g["o"]])).max() > 1e-3


# ---------------------------------------------------------------------------
# the generation step: attend over the rows cached at earlier steps, then append

def _step_weights(seed, d):
    rng = np.random.default_rng(seed)
    Qo, _ = np.linalg.qr(rng.standard_normal((d, d)))
    Ro, _ = np.linalg.qr(rng.standard_normal((d, d)))
    W_K = (Qo * rng.uniform(0.5, 2.0, size=d)[None, :]) @ Ro
    return rng.standard_normal((d, d)) / math.sqrt(d), W_K, rng.standard_normal((d, d)) / math.sqrt(d)


def _causal_excl_loop(X, W_Q, W_K, W_V, H, dh, scale):
    """Textbook attention of token i over tokens t < i (no self term), pure
    float64 loops on unrounded K = X W_K and V = X W_V; token 0 gets zeros."""
    n, d = X.shape
    Q, K, V = X @ W_Q, X @ W_K, X @ W_V
    out = np.zeros((n, H, dh))
    for i in range(1, n):
        for h in range(H):
            s = []
            for t in range(i):
                s.append(scale * sum(Q[i, h * dh + j] * K[t, h * dh + j] for j in range(dh)))
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for j in range(dh):
                out[i, h, j] = sum(e[t] * V[t, h * dh + j] for t in range(i)) / z
    return out


def _run_steps(step_fn, X, W_Q, W_K, W_V, H, dh, T):
    """Feeds the rows of X one per step into an initially empty float32 cache."""
    d = X.shape[1]
    K = np.zeros((1, T, d), dtype=np.float32)
    lens = np.array([0])
    outs = []
    for i in range(X.shape[0]):
        o, k_new, lens_next = step_fn(X[i:i + 1], W_Q, W_K, W_V, K, lens, H, dh, 1 / math.sqrt(dh), "f32")
        K = oracle.append_rows(K, k_new, lens)
        lens = lens_next
        outs.append(o[0])
    return np.stack(outs), K, lens


def test_step_sequence_is_strictly_causal_attention():
    H, dh, n = 2, 4, 7
    d = H * dh
    W_Q, W_K, W_V = _step_weights(11, d)
    X = np.random.default_rng(12).standard_normal((n, d))
    got, K, lens = _run_steps(oracle.generate_step, X, W_Q, W_K, W_V, H, dh, T=n + 2)
    want = _causal_excl_loop(X, W_Q, W_K, W_V, H, dh, 1 / math.sqrt(dh))
    assert np.abs(got[0]).max() == 0                       # nothing cached yet
    assert _rel(got, want) < 1e-5                          # float32 cache rounding only
    assert int(lens[0]) == n
    assert np.abs(K[0, :n] - (X @ W_K)).max() < 1e-5 * np.abs(X @ W_K).max()
    assert np.all(K[0, n:] == 0)


def test_step_full_and_bf16_cache():
    H, dh, T = 2, 4, 5
    d = H * dh
    W_Q, W_K, W_V = _step_weights(13, d)
    rng = np.random.default_rng(14)
    X = rng.standard_normal((3, T, d))
    K = np.stack([syn.f32_to_bf16_bits((X[b] @ W_K).astype(np.float32)) for b in range(3)])
    lens = np.array([T, 2, 0])
    x = rng.standard_normal((3, d))
    o, k_new, nxt = oracle.generate_step(x, W_Q, W_K, W_V, K, lens, H, dh, 0.5, "bf16")
    assert list(nxt) == [T, 3, 1]
    assert np.abs(o[2]).max() == 0
    assert np.abs(k_new - oracle.round_bf16(x @ W_K)).max() == 0
    K2 = oracle.append_rows(K, k_new, lens)
    assert np.array_equal(K2[0], K[0])                       # full: untouched
    assert np.array_equal(oracle.bf16_decode(K2[1, 2]), k_new[1])
    assert np.array_equal(oracle.bf16_decode(K2[2, 0]), k_new[2])
    assert np.array_equal(np.delete(K2[1], 2, axis=0), np.delete(K[1], 2, axis=0))


def _mut_step_append_first(x, W_Q, W_K, W_V, K_cache, lengths, H, dh, scale, cache):
    k_new = oracle.prefill(x, W_K, cache)
    K2 = oracle.append_rows(K_cache, k_new, lengths)
    T = K2.shape[1]
    lens = np.minimum(np.asarray(lengths) + 1, T)
    q = np.asarray(x, dtype=np.float64) @ W_Q
    o = oracle.mha_decode(q, oracle.cache_to_f64(K2), oracle.explicit_values(K2, W_K, W_V), lens, H, dh, scale)
    return o, k_new, lens


def _mut_step_query_from_wk(x, W_Q, W_K, W_V, K_cache, lengths, H, dh, scale, cache):
    return oracle.generate_step(x, W_K, W_K, W_V, K_cache, lengths, H, dh, scale, cache)


@pytest.mark.parametrize("mutant", [_mut_step_append_first, _mut_step_query_from_wk])
def test_step_pin_catches_planted_mistakes(mutant):
    H, dh, n = 2, 4, 6
    d = H * dh
    W_Q, W_K, W_V = _step_weights(15, d)
    X = np.random.default_rng(16).standard_normal((n, d))
    want = _causal_excl_loop(X, W_Q, W_K, W_V, H, dh, 1 / math.sqrt(dh))
    got, _, _ = _run_steps(mutant, X, W_Q, W_K, W_V, H, dh, T=n + 1)
    assert _rel(got, want) > 1e-3


# ---------------------------------------------------------------------------
# many queries over one context

def _causal_incl_loop(Q, K, V, H, dh, scale, t0=0):
    """Prompt token i (absolute row t0 + i) attends rows 0..t0+i, scalar loops."""
    n = Q.shape[0]
    out = np.zeros((n, H, dh))
    for i in range(n):
        r = t0 + i + 1
        for h in range(H):
            s = [scale * sum(Q[i, h * dh + j] * K[t, h * dh + j] for j in range(dh)) for t in range(r)]
            m = max(s)
            e = [math.exp(v - m) for v in s]
            z = sum(e)
            for j in range(dh):
                out[i, h, j] = sum(e[t] * V[t, h * dh + j] for t in range(r)) / z
    return out


def test_multi_query_causal_matches_loop():
    rng = np.random.default_rng(21)
    H, dh, T, t0 = 2, 3, 9, 4
    d = H * dh
    Q = rng.standard_normal((T - t0, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    lim = t0 + np.arange(T - t0) + 1
    got = oracle.multi_query_attention(Q, K, V, lim, H, dh, 0.7)
    assert _rel(got, _causal_incl_loop(Q, K, V, H, dh, 0.7, t0)) < 1e-12


def test_multi_query_shared_context_is_decode_with_broadcast_cache():
    rng = np.random.default_rng(22)
    H, dh, T, n = 3, 4, 11, 5
    d = H * dh
    Q = rng.standard_normal((n, d))
    K = rng.standard_normal((T, d))
    V = rng.standard_normal((T, d))
    lim = np.array([11, 0, 3, 20, 1])
    got = oracle.multi_query_attention(Q, K, V, lim, H, dh, 0.5)
    want = oracle.mha_decode_loop(Q, np.broadcast_to(K, (n, T, d)), np.broadcast_to(V, (n, T, d)), lim,
                                  H, dh, 0.5)
    assert _rel(got, want) < 1e-12
    assert np.abs(got[1]).max() == 0
    assert np.abs(got[4] - V[0].reshape(H, dh)).max() < 1e-14       # one row: its value row
    full = oracle.multi_query_attention(Q, K, V, None, H, dh, 0.5)
    assert np.array_equal(full[0], got[0])


def test_multi_query_options_agree():
    """Both Slim options (V = K W_KV materialised, or softmax times K then
    W_KV) reproduce the explicit-V definition for many queries."""
    rng = np.random.default_rng(23)
    H, dh, T, n = 2, 4, 10, 6
    d = H * dh
    W_K, W_V = _step_weights(24, d)[1], rng.standard_normal((d, d)) / math.sqrt(d)
    X = rng.standard_normal((T, d))
    K = X @ W_K
    Q = rng.standard_normal((n, d))
    lim = np.array([10, 4, 7, 1, 10, 9])
    want = oracle.multi_query_attention(Q, K, X @ W_V, lim, H, dh, 0.5)
    Wkv = oracle.wkv(W_K, W_V)
    opt1 = oracle.multi_query_attention(Q, K, K @ Wkv, lim, H, dh, 0.5)
    # option 2 written out: per head, softmax over all d columns of K, then the head slice of W_KV
    opt2 = np.zeros_like(want)
    for i in range(n):
        for h in range(H):
            c = slice(h * dh, (h + 1) * dh)
            s = 0.5 * (K[:lim[i], c] @ Q[i, c])
            p = np.exp(s - s.max())
            opt2[i, h] = (p / p.sum()) @ K[:lim[i]] @ Wkv[:, c]
    assert _rel(opt1, want) < 1e-10 and _rel(opt2, want) < 1e-10


def test_multi_query_cost_model():
    c = oracle.multi_query_cost(1, 32, 131072, 4096)                 # one decode query: option 2
    assert c["opt2"] < c["opt1"]
    c = oracle.multi_query_cost(2048, 12, 2048, 768)                 # a whole prompt: option 1
    assert c["opt1"] < c["opt2"]


def test_multi_query_cost_hand_worked():
    """Exact counts worked by hand (tests/golden/multi_query_cost_worked.json).
    Every term of both counts is non-zero there, so dropping any one of the
    four terms changes a value."""
    for c in _load("multi_query_cost_worked.json")["cases"]:
        got = oracle.multi_query_cost(c["n"], c["H"], c["T"], c["d"])
        assert got == {"opt1": c["opt1"], "opt2": c["opt2"]}, c


def _counted_options(Q, K, Wkv, H, dh, scale):
    """Both generation options written as scalar loops that count their
    multiply-accumulates (the scores, common to both, are not counted).
    Returns (out1, macs1, out2, macs2)."""
    n, d = Q.shape
    T = K.shape[0]
    p = np.zeros((n, H, T))
    for i in range(n):
        for h in range(H):
            s = np.array([scale * sum(Q[i, h * dh + j] * K[t, h * dh + j] for j in range(dh)) for t in range(T)])
            e = np.exp(s - s.max())
            p[i, h] = e / e.sum()
    macs1 = 0
    V = np.zeros((T, d))                                   # option 1: V = K . W_KV ...
    for t in range(T):
        for c in range(d):
            for k in range(d):
                V[t, c] += K[t, k] * Wkv[k, c]
                macs1 += 1
    out1 = np.zeros((n, H, dh))                            # ... then softmax times V
    for i in range(n):
        for h in range(H):
            for j in range(dh):
                for t in range(T):
                    out1[i, h, j] += p[i, h, t] * V[t, h * dh + j]
                    macs1 += 1
    macs2 = 0
    out2 = np.zeros((n, H, dh))
    for i in range(n):
        for h in range(H):
            u = np.zeros(d)                                # option 2: softmax times all d columns of K ...
            for c in range(d):
                for t in range(T):
                    u[c] += p[i, h, t] * K[t, c]
                    macs2 += 1
            for j in range(dh):                            # ... then the head's columns of W_KV
                for c in range(d):
                    out2[i, h, j] += u[c] * Wkv[c, h * dh + j]
                    macs2 += 1
    return out1, macs1, out2, macs2


@pytest.mark.parametrize("n,H,dh,T", [(3, 2, 2, 5), (1, 2, 2, 5), (2, 3, 1, 4)])
def test_multi_query_cost_counts_the_loops(n, H, dh, T):
    """The cost model equals the multiply-accumulates that brute-force loops of
    the two options perform, and those loops reproduce the explicit-V
    definition (so they are the options, not just counters)."""
    rng = np.random.default_rng(31 + n + T)
    d = H * dh
    Q, K, Wkv = rng.standard_normal((n, d)), rng.standard_normal((T, d)), rng.standard_normal((d, d))
    out1, m1, out2, m2 = _counted_options(Q, K, Wkv, H, dh, 0.6)
    want = oracle.multi_query_attention(Q, K, K @ Wkv, None, H, dh, 0.6)
    assert _rel(out1, want) < 1e-12 and _rel(out2, want) < 1e-12
    assert oracle.multi_query_cost(n, H, T, d) == {"opt1": m1, "opt2": m2}


@pytest.mark.parametrize("drop", range(4))
def test_multi_query_cost_pin_catches_a_dropped_term(drop):
    def mutant(n, H, T, d):
        t = [T * d * d, n * T * d, n * H * T * d, n * d * d]
        t[drop] = 0
        return {"opt1": t[0] + t[1], "opt2": t[2] + t[3]}
    cases = _load("multi_query_cost_worked.json")["cases"]
    assert any(mutant(c["n"], c["H"], c["T"], c["d"]) != {"opt1": c["opt1"], "opt2": c["opt2"]} for c in cases)
    _, m1, _, m2 = _counted_options(*(np.ones((3, 4)), np.ones((5, 4)), np.ones((4, 4))), 2, 2, 1.0)
    assert mutant(3, 2, 5, 4) != {"opt1": m1, "opt2": m2}


# ---------------------------------------------------------------------------
# the parity metric

def test_err_rel_hand_worked():
    """max|o - o_ref| / max|o_ref| over the whole output, worked by hand
    (tests/golden/err_rel_worked.json): the error's and the reference's maxima
    at different indexes, a negative largest difference, 3-D outputs, the
    all-zero reference (absolute error), and a case where one sequence alone
    would give a different value."""
    for c in _load("err_rel_worked.json")["cases"]:
        assert abs(oracle.err_rel(np.array(c["o"]), np.array(c["o_ref"])) - c["err"]) < 1e-12, c["name"]


def test_err_rel_nan_fails_every_gate():
    o = np.array([[np.nan, 1.0]])
    assert not (oracle.err_rel(o, np.array([[1.0, 1.0]])) <= 1.0)
    assert not (oracle.err_rel(np.array([[1.0, 1.0]]), o) <= 1.0)


def _err_mutants():
    a = lambda x: np.asarray(x, dtype=np.float64)
    return [
        lambda o, r: float(np.abs(a(o) - a(r)).mean() / np.abs(a(r)).max()),          # mean for max
        lambda o, r: float((a(o) - a(r)).max() / np.abs(a(r)).max()),                 # no abs on the error
        lambda o, r: float(np.abs(a(o) - a(r)).max() / a(r).max()),                   # signed max of ref
        lambda o, r: float(np.abs(a(o) - a(r)).max() / np.abs(a(o)).max()),          # max of o, not ref
        lambda o, r: float((np.abs(a(o) - a(r)) / np.maximum(np.abs(a(r)), 1e-300)).max()),  # elementwise
        lambda o, r: max(float(np.abs(a(o)[b] - a(r)[b]).max() / max(np.abs(a(r)[b]).max(), 1e-300))
                         for b in range(a(r).shape[0])),                               # per sequence
        lambda o, r: 0.0 if np.abs(a(r)).max() == 0 else float(
            np.abs(a(o) - a(r)).max() / np.abs(a(r)).max()),                          # zero ref read as exact
    ]


@pytest.mark.parametrize("k", range(7))
def test_err_rel_pin_catches_planted_mistakes(k):
    f = _err_mutants()[k]
    cases = _load("err_rel_worked.json")["cases"]
    with np.errstate(divide="ignore", invalid="ignore"):
        bad = [c["name"] for c in cases
               if not abs(f(np.array(c["o"]), np.array(c["o_ref"])) - c["err"]) < 1e-12]
    assert bad, "a planted mistake in the metric passed every worked case"
