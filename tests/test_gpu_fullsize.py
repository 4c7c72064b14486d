"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default plan).  The device computes every output and the
float64 oracle recomputes every output: all (sequence, head) pairs, with the
metric max|o - o_ref| / max|o_ref| taken over the whole [B, H, dh] output."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import (TOL, bf16_bits, check_prefill_bf16, dev_wkv, gpu_decode, log, oracle_decode_full,
                        report_err, to_dev)

pytestmark = pytest.mark.gpu


def _check(name, o, ref):
    assert o.shape == ref.shape
    assert np.isfinite(o).all()
    err = report_err(name, o, ref)
    assert err <= TOL["bf16"]


def test_7b_ragged_full_size_whole_output():
    cfg = syn.CONFIGS["7b_ragged"]
    log(f"[fullsize] 7b_ragged: generating {cfg.desc}")
    wl = syn.make(cfg)
    log(f"[fullsize] 7b_ragged lengths: {wl.lengths.tolist()}")
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    log("[fullsize] 7b_ragged: oracle over all 16 x 32 (sequence, head) pairs")
    ref = oracle_decode_full(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("7b_ragged", o, ref)


def test_7b_8k_full_size_whole_output():
    cfg = syn.CONFIGS["7b_8k"]
    log(f"[fullsize] 7b_8k: generating {cfg.desc}")
    wl = syn.make(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    log("[fullsize] 7b_8k: oracle over all 16 x 32 (sequence, head) pairs")
    ref = oracle_decode_full(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("7b_8k", o, ref)


def test_long_128k_full_131072_whole_output():
    cfg = syn.CONFIGS["long_128k"]
    log(f"[fullsize] long_128k: generating {cfg.desc}")
    wl = syn.make(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    log("[fullsize] long_128k: oracle over all 32 heads")
    ref = oracle_decode_full(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("long_128k", o, ref)


def test_whisper_large_full_prefill_and_decode_whole_output():
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    cfg = syn.CONFIGS["whisper_large"]
    log(f"[fullsize] whisper_large: generating {cfg.desc}")
    wl = syn.make(cfg, with_cache=False)
    Xb, Wb = syn.prefill_inputs(cfg, wl.w)
    Kd = torch.zeros((cfg.B, cfg.T_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    slim.prefill(to_dev(Xb), to_dev(Wb), Kd)
    o = gpu_decode(cfg, wl.q, Kd, wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    Kbits = bf16_bits(Kd)
    W64 = oracle.bf16_decode(Wb)
    # the oracle's own cache, from the same bf16 X and W_K; the device's
    # prefill is checked against it for all 64 sequences
    X64 = oracle.bf16_decode(Xb.reshape(-1, cfg.d))
    K_ref = oracle.prefill(X64, W64, "bf16").reshape(cfg.B, cfg.T_max, cfg.d)
    check_prefill_bf16(Kbits.reshape(-1, cfg.d), X64, W64, "whisper_large, all 64 sequences")
    log("[fullsize] whisper_large: oracle over all 64 x 20 (sequence, head) pairs")
    ref = oracle_decode_full(cfg, wl.q, K_ref, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("whisper_large", o, ref)
