"""Seeded sweep of shapes the fixed cases do not reach: random head counts,
head widths, batch sizes, cache sizes and ragged lengths (zeros and clamped
values included), for the decode step (bf16 and fp32 caches), many queries
over one context (both options, with limits) and the whole generation step.
Every case is checked against the float64 oracle at the decode tolerance."""
import math

import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import TOL, gpu_decode, log, oracle_decode, to_dev

pytestmark = pytest.mark.gpu


def _cfg(rng, cache, dhs, hmax, bmax, tmax):
    dh = int(rng.choice(dhs))
    H = int(rng.integers(1, hmax + 1))
    while cache == "bf16" and (H * dh) % 8 != 0:
        H += 1
    B = int(rng.integers(1, bmax + 1))
    T = int(rng.integers(1, tmax + 1))
    return syn.Config(f"rand-{cache}", d=H * dh, H=H, dh=dh, B=B, T_max=T, len_lo=0, len_hi=T,
                      cache=cache, wkv=cache, seed=int(rng.integers(100, 10 ** 6)))


def _lengths(rng, B, T):
    lens = rng.integers(0, T + 1, size=B)
    if B > 2:
        lens[0] = 0
        lens[1] = T + 5          # clamped to T
    return lens.astype(np.int32)


@pytest.mark.parametrize("seed", range(6))
def test_random_decode_bf16(seed):
    rng = np.random.default_rng(1000 + seed)
    cfg = _cfg(rng, "bf16", [32, 64, 128], 32, 12, 700)
    wl = syn.make(syn.shrink(cfg, len_lo=cfg.T_max, len_hi=cfg.T_max), with_cache=False)
    lens = _lengths(rng, cfg.B, cfg.T_max)
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    log(f"[random] bf16 decode: B={cfg.B} H={cfg.H} dh={cfg.dh} T={cfg.T_max} lens={lens.tolist()}")
    Wd = to_dev(__import__("kv_cache_reduction_amd").wkv(wl.w.W_K, wl.w.W_V, "bf16"))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, Wd)
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    err = oracle.err_rel(o, ref)
    log(f"[random] err={err:.3e}")
    assert np.isfinite(o).all() and err <= TOL["bf16"]
    assert np.all(o[np.minimum(lens, cfg.T_max) == 0] == 0)


@pytest.mark.parametrize("seed", range(4))
def test_random_decode_fp32(seed):
    rng = np.random.default_rng(2000 + seed)
    cfg = _cfg(rng, "f32", [1, 2, 4, 8, 16, 32, 64, 128, 256], 24, 6, 300)
    wl = syn.make(syn.shrink(cfg, len_lo=cfg.T_max, len_hi=cfg.T_max), with_cache=False)
    lens = _lengths(rng, cfg.B, cfg.T_max)
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    log(f"[random] f32 decode: B={cfg.B} H={cfg.H} dh={cfg.dh} T={cfg.T_max} lens={lens.tolist()}")
    Wd = to_dev(__import__("kv_cache_reduction_amd").wkv(wl.w.W_K, wl.w.W_V, "f32"))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, Wd)
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    err = oracle.err_rel(o, ref)
    log(f"[random] err={err:.3e}")
    assert np.isfinite(o).all() and err <= TOL["f32"]


@pytest.mark.parametrize("H", [1, 4, 5, 8, 9, 16, 17, 32, 33, 64])
def test_decode_fp32_head_bucket_edges(H):
    """The fp32 attend kernel is compiled for at most 4, 8, 16, 32 or 64
    heads; head counts on both sides of each bound."""
    rng = np.random.default_rng(5000 + H)
    cfg = syn.Config("f32-heads", d=H * 16, H=H, dh=16, B=3, T_max=70, len_lo=0, len_hi=70,
                     cache="f32", wkv="f32", seed=7000 + H)
    wl = syn.make(syn.shrink(cfg, len_lo=cfg.T_max, len_hi=cfg.T_max), with_cache=False)
    lens = _lengths(rng, cfg.B, cfg.T_max)
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    log(f"[random] f32 heads: B={cfg.B} H={H} dh=16 T={cfg.T_max} lens={lens.tolist()}")
    Wd = to_dev(__import__("kv_cache_reduction_amd").wkv(wl.w.W_K, wl.w.W_V, "f32"))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, Wd)
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    err = oracle.err_rel(o, ref)
    log(f"[random] err={err:.3e}")
    assert np.isfinite(o).all() and err <= TOL["f32"]
    assert np.all(o[np.minimum(lens, cfg.T_max) == 0] == 0)


@pytest.mark.parametrize("seed", range(4))
def test_random_multi_query(seed):
    import torch
    import kv_cache_reduction_amd as slim
    rng = np.random.default_rng(3000 + seed)
    dh = int(rng.choice([64, 128]))
    H = int(rng.choice([2, 4, 6, 8, 10]))
    if (H * dh) % 128:
        H += 1
    n = int(rng.integers(1, 150))
    T = int(rng.integers(1, 400))
    cfg = syn.Config("rand-mq", d=H * dh, H=H, dh=dh, B=n, T_max=T, len_lo=T, len_hi=T, cache="bf16",
                     wkv="bf16", seed=int(rng.integers(100, 10 ** 6)))
    w = syn.weights(cfg)
    K = syn.k_cache(syn.shrink(cfg, B=1), w, np.array([T]), T_alloc=T)[0]
    Q = syn.queries(cfg, w)
    lim = rng.integers(-3, T + 4, size=n).astype(np.int32)
    V = oracle.explicit_values(K, w.W_K, w.W_V)
    ref = oracle.multi_query_attention(Q.astype(np.float64), K, V, lim, H, dh, cfg.scale)
    Wkv = to_dev(slim.wkv(w.W_K, w.W_V, "bf16"))
    for option in (1, 2):
        out = torch.full((n, H, dh), float("nan"), dtype=torch.float32, device="cuda")
        slim.multi_query(to_dev(Q), to_dev(K), Wkv, out, H, dh, limits=to_dev(lim), scale=cfg.scale, option=option)
        torch.cuda.synchronize()
        o = out.cpu().numpy().astype(np.float64)
        err = oracle.err_rel(o, ref)
        log(f"[random] multi n={n} H={H} dh={dh} T={T} option {option}: err={err:.3e}")
        assert np.isfinite(o).all() and err <= TOL["bf16"]


@pytest.mark.parametrize("seed", range(3))
def test_random_generation_step(seed):
    import torch
    import kv_cache_reduction_amd as slim
    rng = np.random.default_rng(4000 + seed)
    cfg = _cfg(rng, "bf16", [32, 64, 128], 16, 40, 300)
    w = syn.weights(cfg)
    lens = _lengths(rng, cfg.B, cfg.T_max)
    K = syn.k_cache(cfg, w, np.minimum(lens, cfg.T_max))
    x = rng.standard_normal((cfg.B, cfg.d)).astype(np.float32)
    WQb = syn.f32_to_bf16_bits(w.W_Q.astype(np.float32))
    WKb = syn.f32_to_bf16_bits(w.W_K.astype(np.float32))
    WQ64, WK64 = oracle.bf16_decode(WQb), oracle.bf16_decode(WKb)
    Wkv = to_dev(slim.wkv(WK64, w.W_V, "bf16"))
    Kd = to_dev(K)
    out = torch.empty((cfg.B, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    nxt = torch.zeros(cfg.B, dtype=torch.int32, device="cuda")
    log(f"[random] step: B={cfg.B} H={cfg.H} dh={cfg.dh} T={cfg.T_max} lens={lens.tolist()}")
    slim.step(to_dev(x), to_dev(WQb), to_dev(WKb), Kd, to_dev(lens), nxt, Wkv, out, cfg.H, cfg.dh, cfg.scale)
    torch.cuda.synchronize()
    o_ref, k_ref, nxt_ref = oracle.generate_step(x.astype(np.float64), WQ64, WK64, w.W_V, K, lens,
                                                 cfg.H, cfg.dh, cfg.scale, "bf16")
    err = oracle.err_rel(out.cpu().numpy(), o_ref)
    log(f"[random] step err={err:.3e}")
    assert err <= TOL["bf16"]
    assert np.array_equal(nxt.cpu().numpy(), nxt_ref)
