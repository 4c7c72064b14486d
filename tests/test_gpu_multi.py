"""GPU parity of many queries over one context (slim_multi_query through the
C ABI): cross-attention of n decoder queries over one shared encoder K, and
the causal prompt phase, with both generation options of the method.  Against
the float64 oracle (standard attention over explicit values rebuilt from the
bf16 K without W_KV) on the same seeded inputs; tolerance
max|o - o_ref| / max|o_ref| <= 2e-2 (bf16 K)."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import TOL, bf16_bits, check_prefill_bf16, log, to_dev

pytestmark = pytest.mark.gpu


def _context(cfg, T):
    """One context of T rows (sequence 0 of the config's recipe): K in bf16
    bits, float64 values of the weights, W_KV on the device."""
    import kv_cache_reduction_amd as slim
    w = syn.weights(cfg)
    K = syn.k_cache(syn.shrink(cfg, B=1), w, np.array([T]), T_alloc=T)[0]
    Wkv = to_dev(slim.wkv(w.W_K, w.W_V, cfg.wkv))
    return w, K, Wkv


def _run(name, cfg, Q, K, Wkv, w, limits, option, tol=TOL["bf16"]):
    import torch
    import kv_cache_reduction_amd as slim
    n, d = Q.shape
    T = K.shape[0]
    out = torch.full((n, cfg.H, cfg.dh), float("nan"), dtype=torch.float32, device="cuda")
    lim_d = None if limits is None else to_dev(np.asarray(limits, dtype=np.int32))
    log(f"[multi] {name}: n={n} T={T} d={d} H={cfg.H} option={option} "
        f"(auto picks {slim.multi_query_option(n, cfg.H, cfg.dh, T)})")
    slim.multi_query(to_dev(Q.astype(np.float32)), to_dev(K), Wkv, out, cfg.H, cfg.dh, limits=lim_d,
                     scale=cfg.scale, option=option)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    V = oracle.explicit_values(K, w.W_K, w.W_V)
    ref = oracle.multi_query_attention(Q.astype(np.float64), K, V, limits, cfg.H, cfg.dh, cfg.scale)
    err = oracle.err_rel(o, ref)
    log(f"[multi] {name} option {option}: err={err:.3e} max|ref|={np.abs(ref).max():.3e}")
    assert np.isfinite(o).all()
    assert err <= tol
    if limits is not None:
        empty = np.clip(np.asarray(limits), 0, T) == 0
        assert np.all(o[empty] == 0)
    return o


@pytest.mark.parametrize("option", [1, 2])
def test_shared_context_whisper_large_shape(option):
    cfg = syn.shrink(syn.CONFIGS["whisper_large"], B=64, T_max=200, len_lo=200, len_hi=200)
    w, K, Wkv = _context(cfg, 200)
    Q = syn.queries(cfg, w)                       # 64 decoder queries, one encoder context
    _run("shared whisper_large-shaped", cfg, Q, K, Wkv, w, None, option)


@pytest.mark.parametrize("option", [1, 2])
def test_ragged_limits_dh128(option):
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=40, T_max=300, len_lo=300, len_hi=300)
    w, K, Wkv = _context(cfg, 300)
    Q = syn.queries(cfg, w)                       # 40 queries: a ragged last block of 32
    lim = (np.arange(40) * 37) % 331 - 10         # negative, zero, partial tiles, beyond T
    _run("ragged limits dh=128", cfg, Q, K, Wkv, w, lim, option)


@pytest.mark.parametrize("option", [1, 2])
def test_prompt_phase_causal(option):
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], B=1, T_max=230, len_lo=230, len_hi=230)
    w, K, Wkv = _context(cfg, 230)
    t0 = 37                                       # the prompt continues a cached prefix
    X = syn.x_rows(cfg, 0, t0, 230).astype(np.float64)
    Q = (X @ w.W_Q).astype(np.float32)
    lim = t0 + np.arange(230 - t0) + 1
    _run("prompt causal gpt2_small-shaped", cfg, Q, K, Wkv, w, lim, option)


def test_options_agree_and_one_query_is_decode():
    import torch
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS["whisper_large"], B=3, T_max=161, len_lo=161, len_hi=161)
    w, K, Wkv = _context(cfg, 161)
    Q = syn.queries(cfg, w)
    o1 = _run("agree", cfg, Q, K, Wkv, w, None, 1)
    o2 = _run("agree", cfg, Q, K, Wkv, w, None, 2)
    assert oracle.err_rel(o1, o2) <= TOL["bf16"]
    # one query over the context is the decode step of a one-sequence batch
    out = torch.empty((1, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    Kd = to_dev(K[None])
    slim.decode(to_dev(Q[:1]), Kd, to_dev(np.array([161], dtype=np.int32)), Wkv, out, cfg.H, cfg.dh, cfg.scale)
    torch.cuda.synchronize()
    assert oracle.err_rel(out.cpu().numpy()[0], o2[0]) <= TOL["bf16"]


@pytest.mark.parametrize("option", [0, 1, 2])
def test_whisper_large_full_shared_encoder_context(option):
    """Whisper-large-shaped cross-attention at full size with one shared
    encoder context: 64 decoder queries, T=1500, d=1280, K written by the
    device prefill from bf16 X and W_K."""
    import torch
    import kv_cache_reduction_amd as slim
    cfg = syn.CONFIGS["whisper_large"]
    w = syn.weights(cfg)
    Xb, Wb = syn.prefill_inputs(syn.shrink(cfg, B=1), w)
    Kd = torch.zeros((1, cfg.T_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    slim.prefill(to_dev(Xb), to_dev(Wb), Kd)
    torch.cuda.synchronize()
    K = bf16_bits(Kd)[0]
    X64, W64 = oracle.bf16_decode(Xb[0]), oracle.bf16_decode(Wb)
    check_prefill_bf16(K, X64, W64, "whisper_large shared context")
    Wkv = to_dev(slim.wkv(w.W_K, w.W_V, cfg.wkv))
    Q = syn.queries(cfg, w)
    _run("whisper_large full shared context", cfg, Q, K, Wkv, w, None, option)


def test_rejects_bad_arguments():
    import torch
    import kv_cache_reduction_amd as slim
    Q = torch.zeros((4, 128), dtype=torch.float32, device="cuda")
    K = torch.zeros((16, 128), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((128, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((4, 2, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(slim.SlimError):
        slim.multi_query(Q, K, W, out, 2, 64, option=3)
    with pytest.raises(slim.SlimError):      # option 1 forms V with the bf16 product only
        slim.multi_query(Q, K, W.float(), out, 2, 64, option=1)
    out2 = torch.empty((4, 4, 32), dtype=torch.float32, device="cuda")
    with pytest.raises(slim.SlimError):      # dh = 32 is not built
        slim.multi_query(Q, K, W, out2, 4, 32, option=2)


@pytest.mark.parametrize("T,n,option", [(1, 1, 1), (1, 5, 2), (33, 1, 1), (33, 70, 2), (95, 130, 0)])
def test_small_contexts_and_query_counts(T, n, option):
    """Contexts shorter than one tile, a single query, query counts that
    leave partial query blocks, in both options."""
    cfg = syn.shrink(syn.CONFIGS["whisper_large"], B=n, T_max=T, len_lo=T, len_hi=T)
    w, K, Wkv = _context(cfg, T)
    Q = syn.queries(cfg, w)
    _run(f"small T={T} n={n}", cfg, Q, K, Wkv, w, None, option)


def test_all_limits_zero_gives_zeros():
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], B=9, T_max=40, len_lo=40, len_hi=40)
    w, K, Wkv = _context(cfg, 40)
    Q = syn.queries(cfg, w)
    for option in (1, 2):
        import torch
        import kv_cache_reduction_amd as slim
        out = torch.full((9, cfg.H, cfg.dh), 7.0, dtype=torch.float32, device="cuda")
        slim.multi_query(to_dev(Q), to_dev(K), Wkv, out, cfg.H, cfg.dh,
                         limits=to_dev(np.zeros(9, dtype=np.int32)), scale=cfg.scale, option=option)
        torch.cuda.synchronize()
        assert torch.count_nonzero(out).item() == 0
