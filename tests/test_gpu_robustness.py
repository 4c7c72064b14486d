"""GPU tests of the decode path's failure reporting, graph replay and wide
fp32 rows, through the C ABI:
 * an exchange wait that runs out of its bound marks the affected outputs
   NaN and is reported by slim_decode_status (forced from the host: a small
   spin bound and a tag skew that keeps one column group's entries from
   matching, so every kernel still exits);
 * the status word is cleared by each call, whatever the workspace held;
 * slim_decode captured in a HIP graph and replayed with new queries equals
   the eager call bit for bit (the exchange mailboxes are reset per replay);
 * fp32 caches with d = 16384 (64 heads of 256), whose attend needs more
   than 64 KB of LDS."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import TOL, dev_wkv, gpu_decode, log, oracle_decode, report_err, to_dev

pytestmark = pytest.mark.gpu


def _xchg_case(B=2, T=700):
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=B, T_max=T, len_lo=1, len_hi=T)
    wl = syn.make(cfg)
    return cfg, wl


def test_exchange_timeout_is_reported(monkeypatch):
    import torch
    import kv_cache_reduction_amd as slim
    cfg, wl = _xchg_case()
    Kd, Wd = to_dev(wl.K), dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    ws = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, Kd.dtype))
    monkeypatch.setenv("SLIM_XCHG_SPIN", "64")
    monkeypatch.setenv("SLIM_XCHG_SKEW", "1")
    log("[robust] exchange with skewed tags and a 64-poll bound")
    o = gpu_decode(cfg, wl.q, Kd, wl.lengths, Wd, ws=ws)
    assert slim.decode_status(ws) == slim.TIMEOUT
    assert np.isnan(o).all()
    monkeypatch.delenv("SLIM_XCHG_SKEW")
    monkeypatch.delenv("SLIM_XCHG_SPIN")
    o = gpu_decode(cfg, wl.q, Kd, wl.lengths, Wd, ws=ws)
    assert slim.decode_status(ws) == 0
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    assert report_err("after a timeout, normal call", o, ref) <= TOL["bf16"]


def test_step_timeout_is_reported(monkeypatch):
    import torch
    import kv_cache_reduction_amd as slim
    cfg, wl = _xchg_case(B=3, T=300)
    WQ = to_dev(syn.f32_to_bf16_bits(wl.w.W_Q.astype(np.float32)))
    WK = to_dev(syn.f32_to_bf16_bits(wl.w.W_K.astype(np.float32)))
    Kd, Wd = to_dev(wl.K), dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    lens = to_dev(np.minimum(wl.lengths, cfg.T_max - 1).astype(np.int32))
    nxt = torch.empty_like(lens)
    out = torch.empty((cfg.B, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    ws = slim.workspace(slim.step_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, Kd.dtype))
    x = to_dev(syn.x_new(cfg))
    monkeypatch.setenv("SLIM_XCHG_SPIN", "16")
    monkeypatch.setenv("SLIM_XCHG_SKEW", "1")
    slim.step(x, WQ, WK, Kd, lens, nxt, Wd, out, cfg.H, cfg.dh, cfg.scale, ws)
    assert slim.decode_status(ws) == slim.TIMEOUT
    assert torch.isnan(out).all()


def test_status_cleared_whatever_the_workspace_held():
    import torch
    import kv_cache_reduction_amd as slim
    for name, kw in (("gpt2_small", dict(B=2, T_max=300)), ("7b_ragged", dict(B=2, T_max=300)),
                     ("tiny_f32", {})):
        cfg = syn.shrink(syn.CONFIGS[name], **kw)
        wl = syn.make(cfg)
        Kd = to_dev(wl.K)
        ws = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, Kd.dtype))
        ws.fill_(0xFF)
        gpu_decode(cfg, wl.q, Kd, wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V), ws=ws)
        assert slim.decode_status(ws) == 0, name


def test_decode_graph_replay_with_new_queries():
    """B = 1, T = 8192, d = 4096: 64-token chunks, so every mailbox ring slot
    is used once per launch and a replay with the previous replay's tags
    would find them already there.  Each replay, with a new q copied into the
    captured buffer and eager work between replays, must equal the eager
    call bit for bit."""
    import torch
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS["long_128k"], T_max=8192, len_lo=8192, len_hi=8192)
    wl = syn.make(cfg)
    Kd, Wd = to_dev(wl.K), dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    ld = to_dev(wl.lengths.astype(np.int32))
    ws = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, Kd.dtype))
    ws_eager = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, Kd.dtype))
    q_static = to_dev(wl.q.astype(np.float32))
    out_g = torch.zeros((1, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    out_e = torch.zeros_like(out_g)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            slim.decode(q_static, Kd, ld, Wd, out_g, cfg.H, cfg.dh, cfg.scale, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        slim.decode(q_static, Kd, ld, Wd, out_g, cfg.H, cfg.dh, cfg.scale, ws)
    rng = np.random.default_rng(5)
    for r in range(4):
        q_new = (wl.q * (1.0 if r == 0 else rng.uniform(0.5, 2.0))).astype(np.float32)
        if r >= 2:
            q_new = rng.standard_normal(q_new.shape).astype(np.float32)
        q_static.copy_(to_dev(q_new))
        out_g.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        slim.decode(to_dev(q_new), Kd, ld, Wd, out_e, cfg.H, cfg.dh, cfg.scale, ws_eager)
        torch.cuda.synchronize()
        assert slim.decode_status(ws) == 0
        same = torch.equal(out_g, out_e)
        log(f"[robust] graph replay {r}: bit-identical to eager = {same}")
        assert same
        if r in (0, 3):
            ref = oracle_decode(cfg, q_new, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
            assert report_err(f"graph replay {r}", out_g.cpu().numpy().astype(np.float64), ref) <= TOL["bf16"]


def test_f32_wide_rows_over_64k_lds():
    """fp32 cache with H = 64, dh = 256 (d = 16384): the attend stages a whole
    row in LDS (66 KB).  W_K = I, so the value rows are K . W_V and the
    oracle's first Slim form (pinned against the definition) applies with
    W_KV = W_V."""
    import torch
    import kv_cache_reduction_amd as slim
    H, dh, B, T = 64, 256, 2, 40
    d = H * dh
    rng = np.random.default_rng(64)
    K = rng.standard_normal((B, T, d)).astype(np.float32)
    q = rng.standard_normal((B, d)).astype(np.float32)
    W = (rng.standard_normal((d, d), dtype=np.float32) / np.float32(np.sqrt(d))).astype(np.float32)
    lens = np.array([40, 13], dtype=np.int32)
    cfg = syn.Config("f32_wide", d=d, H=H, dh=dh, B=B, T_max=T, len_lo=1, len_hi=T, cache="f32", wkv="f32",
                     seed=0)
    o = gpu_decode(cfg, q, to_dev(K), lens, to_dev(W))
    ref = oracle.slim_decode_opt1(q, K, W.astype(np.float64), lens, H, dh, cfg.scale)
    assert np.isfinite(o).all()
    assert report_err("f32 d=16384", o, ref) <= TOL["f32"]
