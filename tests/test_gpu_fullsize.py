"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default plan).  The device computes every output; the
float64 oracle recomputes sampled sequences and heads one by one."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import (TOL, bf16_bits, check_prefill_bf16, dev_wkv, gpu_decode, log, oracle_decode,
                        to_dev)

pytestmark = pytest.mark.gpu


def _check(name, o, ref):
    err = oracle.err_rel(o, ref)
    log(f"[fullsize] {name}: err={err:.3e} max|ref|={np.abs(ref).max():.3e}")
    assert np.isfinite(o).all()
    assert err <= TOL["bf16"]


def test_7b_ragged_full_size_sampled():
    cfg = syn.CONFIGS["7b_ragged"]
    log(f"[fullsize] 7b_ragged: generating {cfg.desc}")
    wl = syn.make(cfg)
    log(f"[fullsize] 7b_ragged lengths: {wl.lengths.tolist()}")
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    assert np.isfinite(o).all()
    seqs, heads = [0, 7, 15], [0, 13, 31]
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V, seqs=seqs, heads=heads)
    _check("7b_ragged", o[np.ix_(seqs, heads)], ref)


def test_long_128k_full_131072_sampled_heads():
    cfg = syn.CONFIGS["long_128k"]
    log(f"[fullsize] long_128k: generating {cfg.desc}")
    wl = syn.make(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    assert np.isfinite(o).all()
    heads = [0, 17, 31]
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V, heads=heads, reassociate=True)
    _check("long_128k", o[:, heads], ref)


def test_whisper_large_full_prefill_and_decode_sampled():
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    cfg = syn.CONFIGS["whisper_large"]
    log(f"[fullsize] whisper_large: generating {cfg.desc}")
    wl = syn.make(cfg, with_cache=False)
    Xb, Wb = syn.prefill_inputs(cfg, wl.w)
    Kd = torch.zeros((cfg.B, cfg.T_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    slim.prefill(to_dev(Xb), to_dev(Wb), Kd)
    o = gpu_decode(cfg, wl.q, Kd, wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    assert np.isfinite(o).all()
    seqs = [0, 31, 63]
    Kbits = bf16_bits(Kd)
    W64 = oracle.bf16_decode(Wb)
    K_ref = np.zeros((cfg.B, cfg.T_max, cfg.d))
    for b in seqs:
        X64 = oracle.bf16_decode(Xb[b])
        K_ref[b] = oracle.prefill(X64, W64, "bf16")
        check_prefill_bf16(Kbits[b], X64, W64, f"whisper_large seq {b}")
    ref = oracle_decode(cfg, wl.q, K_ref, wl.lengths, wl.w.W_K, wl.w.W_V, seqs=seqs)
    _check("whisper_large", o[seqs], ref)
