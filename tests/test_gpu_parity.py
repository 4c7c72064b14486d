"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs, element by element, at sizes the oracle finishes in
seconds (several chunks, ragged tails, empty sequences), plus the invariants
of the method.  Tolerance: max|o - o_ref| / max|o_ref| <= 1e-4 for fp32 caches
and <= 2e-2 for bf16 caches."""
import json
import os

import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import (TOL, bf16_bits, check_prefill_bf16, dev_wkv, gpu_decode, log, oracle_decode,
                        to_dev)

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def _check(name, o, ref, tol):
    err = oracle.err_rel(o, ref)
    log(f"[parity] {name}: err={err:.3e} tol={tol:.0e} max|ref|={np.abs(ref).max():.3e}")
    assert np.isfinite(o).all()
    assert err <= tol, f"{name}: err {err:.3e} > {tol}"
    return err


def _workload(cfg, fill=0.0):
    wl = syn.make(cfg, fill=fill)
    return wl


def test_hand_example_fp32_path():
    g = json.load(open(os.path.join(HERE, "golden", "hand_two_heads.json")))
    cfg = syn.Config("hand", d=2, H=2, dh=1, B=1, T_max=2, len_lo=2, len_hi=2, cache="f32",
                     wkv="f32", seed=0)
    K = np.array([g["K"]], dtype=np.float32)
    W = to_dev(np.array(g["W_KV"], dtype=np.float32))
    o = gpu_decode(syn.Config(**{**cfg.__dict__}), np.array([g["q"]], dtype=np.float32), to_dev(K),
                   np.array([2]), W)
    # the fixture's scale is 1, the config's is 1/sqrt(1) = 1
    _check("hand", o, np.array([g["o"]]), 1e-5)


def test_tiny_f32():
    cfg = syn.CONFIGS["tiny_f32"]
    wl = _workload(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("tiny_f32", o, ref, TOL["f32"])


def test_tiny_f32_ragged():
    cfg = syn.shrink(syn.CONFIGS["tiny_f32"], B=5, T_max=45, len_lo=0, len_hi=45)
    wl = _workload(cfg)
    lens = np.array([0, 1, 45, 17, 60], dtype=np.int32)  # empty, single row, full, ragged, clamped
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    assert np.all(o[0] == 0)
    _check("tiny_f32-ragged", o, ref, TOL["f32"])


def test_gpt2_small_bf16_full():
    cfg = syn.CONFIGS["gpt2_small"]
    wl = _workload(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("gpt2_small", o, ref, TOL["bf16"])


def test_7b_ragged_shape_small():
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=6, T_max=1200, len_lo=1, len_hi=1200)
    wl = _workload(cfg)
    lens = wl.lengths.copy()
    lens[1] = 0
    lens[3] = 5000  # clamped to T_max
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    assert np.all(o[1] == 0)
    _check("7b_ragged-small", o, ref, TOL["bf16"])


def test_long_128k_shape_16k():
    cfg = syn.shrink(syn.CONFIGS["long_128k"], T_max=16384)
    wl = _workload(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("long_128k-16k", o, ref, TOL["bf16"])


def test_whisper_large_prefill_then_decode_small():
    """Whisper-shaped cross-attention: the K cache is written on the device
    by slim_prefill from X and W_K; the oracle builds its own cache from the
    same bf16 X and W_K in float64."""
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS["whisper_large"], B=6)
    wl = syn.make(cfg, with_cache=False)
    Xb, Wb = syn.prefill_inputs(cfg, wl.w)
    Kd = torch.zeros((cfg.B, cfg.T_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    slim.prefill(to_dev(Xb), to_dev(Wb), Kd)
    o = gpu_decode(cfg, wl.q, Kd, wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    K_ref = oracle.prefill(oracle.bf16_decode(Xb), oracle.bf16_decode(Wb), "bf16")
    ref = oracle_decode(cfg, wl.q, K_ref, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("whisper_large-small", o, ref, TOL["bf16"])


# ---------------------------------------------------------------------------
# prefill

def test_prefill_bf16_matches_oracle():
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS["whisper_large"], B=3, T_max=300)
    w = syn.weights(cfg)
    Xb, Wb = syn.prefill_inputs(cfg, w, n=300)
    Kd = torch.zeros((cfg.B, cfg.T_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    slim.prefill(to_dev(Xb), to_dev(Wb), Kd)
    torch.cuda.synchronize()
    check_prefill_bf16(bf16_bits(Kd), oracle.bf16_decode(Xb), oracle.bf16_decode(Wb), "whisper_large-shape")


@pytest.mark.parametrize("B,n,d", [(3, 37, 72), (2, 70, 200), (1, 300, 1032), (1, 1000, 4096)])
def test_prefill_bf16_ragged_tiles(B, n, d):
    """bf16 prefill where the last k block, the last column tile and the last
    row tile are all partial (d not a multiple of 64 or 128, B*n not a
    multiple of 64), and the k-block count is not a multiple of the
    prefetch depth; appended at row offsets with the rows past T_max
    skipped.  The shapes reach the 64x64 tiles and (1000 x 4096) the
    64x128 ones."""
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    rng = np.random.default_rng(d)
    Xb = syn.f32_to_bf16_bits(rng.standard_normal((B, n, d)).astype(np.float32))
    Wb = syn.f32_to_bf16_bits((rng.standard_normal((d, d)) / np.sqrt(d)).astype(np.float32))
    T = n + 9
    t0 = np.array([(5 * b) % 12 for b in range(B)], dtype=np.int32)
    Kd = torch.zeros((B, T, d), dtype=torch.bfloat16, device="cuda")
    slim.prefill(to_dev(Xb), to_dev(Wb), Kd, t0=to_dev(t0))
    torch.cuda.synchronize()
    bits = bf16_bits(Kd)
    X64, W64 = oracle.bf16_decode(Xb), oracle.bf16_decode(Wb)
    rows, xs = [], []
    for b in range(B):
        for i in range(n):
            if t0[b] + i < T:
                rows.append(bits[b, t0[b] + i])
                xs.append(X64[b, i])
        skipped = [t for t in range(T) if not (t0[b] <= t < t0[b] + n)]
        assert np.all(bits[b, skipped] == 0)
    check_prefill_bf16(np.array(rows), np.array(xs), W64, f"ragged tiles B={B} n={n} d={d}")


def test_prefill_append_offsets_and_fp32():
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    rng = np.random.default_rng(5)
    B, n, d, T = 3, 5, 72, 16
    X = rng.standard_normal((B, n, d)).astype(np.float32)
    W = rng.standard_normal((d, d)).astype(np.float32)
    t0 = np.array([0, 7, 13], dtype=np.int32)  # the last one runs past T_max: rows >= T are skipped
    Kd = torch.full((B, T, d), -7.0, dtype=torch.float32, device="cuda")
    slim.prefill(to_dev(X), to_dev(W), Kd, t0=to_dev(t0))
    torch.cuda.synchronize()
    got = Kd.cpu().numpy()
    ref = oracle.prefill(X, W, "f32")
    for b in range(B):
        for i in range(n):
            t = t0[b] + i
            if t < T:
                assert np.abs(got[b, t] - ref[b, i]).max() <= 1e-5 * np.abs(ref).max()
        untouched = [t for t in range(T) if not (t0[b] <= t < t0[b] + n)]
        assert np.all(got[b, untouched] == -7.0)


# ---------------------------------------------------------------------------
# comparator (explicit K and V)

@pytest.mark.parametrize("name,kw", [("gpt2_small", {}), ("7b_ragged", dict(B=5, T_max=900, len_lo=1, len_hi=900)),
                                     ("whisper_large", dict(B=4))])
def test_comparator_matches_oracle(name, kw):
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS[name], **kw) if kw else syn.CONFIGS[name]
    cfg = syn.Config(**{**cfg.__dict__, "prefill": False})
    wl = syn.make(cfg)
    V = syn.v_cache(cfg, wl.w, wl.lengths)
    out = torch.empty((cfg.B, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    slim.mha_decode_kv(to_dev(wl.q), to_dev(wl.K), to_dev(V), to_dev(wl.lengths), out, cfg.H, cfg.dh,
                       cfg.scale)
    torch.cuda.synchronize()
    ref = oracle.mha_decode(wl.q, oracle.cache_to_f64(wl.K), oracle.cache_to_f64(V), wl.lengths,
                            cfg.H, cfg.dh, cfg.scale)
    _check(f"kv-{name}", out.cpu().numpy(), ref, 1e-3)


# ---------------------------------------------------------------------------
# invariants

def test_rows_beyond_length_are_never_read():
    """NaN garbage past len_b must not change a single output bit."""
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=4, T_max=700, len_lo=100, len_hi=650)
    wl0 = syn.make(cfg, fill=0.0)
    wln = syn.make(cfg, fill=float("nan"))
    W = dev_wkv(cfg, wl0.w.W_K, wl0.w.W_V)
    a = gpu_decode(cfg, wl0.q, to_dev(wl0.K), wl0.lengths, W)
    b = gpu_decode(cfg, wln.q, to_dev(wln.K), wln.lengths, W)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("chunks", ["1", "3", "37", "200"])
def test_chunk_count_invariance(monkeypatch, chunks):
    """Any split of the token stream gives the same attention: every plan
    meets the oracle bound, and plans differ from each other only by the
    bf16 rounding of the softmax weights (taken against per-chunk maxima)."""
    cfg = syn.shrink(syn.CONFIGS["long_128k"], T_max=3000)
    wl = syn.make(cfg)
    W = dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    base = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, W)
    import kv_cache_reduction_amd as slim
    monkeypatch.setenv("SLIM_CHUNKS", chunks)
    ws = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, 1))
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, W, ws=ws)
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    diff = oracle.err_rel(o, base)
    log(f"[parity] chunks={chunks}: rel diff vs default plan {diff:.2e}")
    _check(f"chunks={chunks}", o, ref, TOL["bf16"])
    assert diff < 1e-2


def test_phases_equal_full_call_and_deterministic():
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], B=3, T_max=700)
    wl = syn.make(cfg)
    W = dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    Kd = to_dev(wl.K)
    a = gpu_decode(cfg, wl.q, Kd, wl.lengths, W)
    b = gpu_decode(cfg, wl.q, Kd, wl.lengths, W, phases=True)
    c = gpu_decode(cfg, wl.q, Kd, wl.lengths, W)
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_single_row_returns_value_row():
    """len = 1: softmax is 1, so o_h = V[0, h] = (K[0] . W_KV)[h]."""
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=3, T_max=16, len_lo=1, len_hi=1)
    wl = syn.make(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    V0 = oracle.explicit_values(wl.K[:, 0], wl.w.W_K, wl.w.W_V).reshape(cfg.B, cfg.H, cfg.dh)
    _check("len1", o, V0, TOL["bf16"])


def test_all_lengths_zero():
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], B=2, T_max=64)
    wl = syn.make(cfg)
    o = gpu_decode(cfg, wl.q, to_dev(wl.K), np.zeros(2, np.int32), dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    assert np.all(o == 0)


def test_workspace_too_small_is_rejected():
    torch = pytest.importorskip("torch")
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS["gpt2_small"], B=2, T_max=64)
    wl = syn.make(cfg)
    need = slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, 1)
    ws = slim.workspace(need - 256)
    with pytest.raises(slim.SlimError) as e:
        gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V), ws=ws[:need - 256])
    assert e.value.status == 3


def test_two_column_groups_ragged_with_empty_sequence():
    """Two-column-group attend kernel (d > 2048) on a ragged 7B-shaped batch
    with an empty sequence and many pieces per chunk."""
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=5, T_max=2000, len_lo=1, len_hi=2000)
    wl = syn.make(cfg)
    lens = wl.lengths.copy()
    lens[2] = 0
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    assert np.all(o[2] == 0)
    _check("two column groups", o, ref, TOL["bf16"])


@pytest.mark.parametrize("xchg", ["1", "0"])
def test_score_exchange_and_fallback(monkeypatch, xchg):
    """The exchange kernel (each column group forms its own heads' scores and
    the pair swaps them) and the kernel that forms all scores in both
    workgroups, on a 7B-shaped ragged batch with several pieces per chunk."""
    monkeypatch.setenv("SLIM_XCHG", xchg)
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=6, T_max=3000, len_lo=1, len_hi=3000)
    wl = syn.make(cfg)
    lens = wl.lengths.copy()
    lens[3] = 0
    lens[4] = 1
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    assert np.all(o[3] == 0)
    _check(f"xchg={xchg}", o, ref, TOL["bf16"])


def test_exchange_shape_with_q_4_byte_aligned():
    """q only 4-byte aligned (a view one float into a buffer) on the
    exchange kernel's shape: q reaches LDS by 4-byte DMA, so the result
    matches the oracle and equals, to the bf16 tolerance, the call with an
    aligned q."""
    import torch
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS["7b_ragged"], B=3, T_max=700, len_lo=1, len_hi=700)
    wl = syn.make(cfg)
    K = syn.k_cache(cfg, wl.w, np.minimum(wl.lengths, cfg.T_max))
    Kd, Wd = to_dev(K), dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    flat = torch.zeros(cfg.B * cfg.d + 4, dtype=torch.float32, device="cuda")
    qv = flat[1:1 + cfg.B * cfg.d].view(cfg.B, cfg.d)
    qv.copy_(to_dev(wl.q.astype(np.float32)))
    assert qv.data_ptr() % 16 == 4
    out = torch.empty((cfg.B, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    slim.decode(qv, Kd, to_dev(wl.lengths.astype(np.int32)), Wd, out, cfg.H, cfg.dh, cfg.scale)
    torch.cuda.synchronize()
    o = out.cpu().numpy().astype(np.float64)
    ref = oracle_decode(cfg, wl.q, K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check("q at a 4-byte offset", o, ref, TOL["bf16"])
    o16 = gpu_decode(cfg, wl.q, Kd, wl.lengths, Wd)
    assert oracle.err_rel(o, o16) <= TOL["bf16"]


@pytest.mark.parametrize("H,dh,B,T", [(20, 64, 4, 150), (20, 64, 19, 150), (32, 128, 17, 96), (32, 32, 6, 200)])
def test_finish_mfma_projection_group_tails(H, dh, B, T):
    """The finish's W_KV projection on MFMA (bf16 W_KV, at least 4 sequences
    per workgroup): B = 4 at the threshold, a last sequence group of 3
    (B = 19, 8 per group) and of 1 (B = 17 at d = 4096, 16 per group), and
    dh = 32 (two 16-column tiles, only two of the four waves hold tiles);
    ragged lengths with an empty sequence."""
    cfg = syn.Config(f"tails-{B}", d=H * dh, H=H, dh=dh, B=B, T_max=T, len_lo=1, len_hi=T,
                     cache="bf16", wkv="bf16", seed=700 + B)
    wl = syn.make(cfg, with_cache=False)
    lens = wl.lengths.copy()
    lens[B // 2] = 0
    K = syn.k_cache(cfg, wl.w, np.minimum(lens, cfg.T_max))
    o = gpu_decode(cfg, wl.q, to_dev(K), lens, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, K, lens, wl.w.W_K, wl.w.W_V)
    assert np.all(o[B // 2] == 0)
    _check(f"MFMA projection tails H={H} dh={dh} B={B}", o, ref, TOL["bf16"])


@pytest.mark.parametrize("H,dh", [(6, 16), (3, 256)])
def test_finish_mfma_projection_f32_cache_bf16_wkv(H, dh):
    """fp32 cache with bf16 W_KV at head widths the bf16-cache path does not
    take: dh = 16 (one 16-column tile, one wave holds it) and dh = 256
    (64-row blocks, four tiles per wave), with 5 sequences so that the
    projection runs on MFMA.  W_KV in bf16 bounds the error, so the bf16
    tolerance applies."""
    cfg = syn.Config(f"f32c-bf16w-{dh}", d=H * dh, H=H, dh=dh, B=5, T_max=90, len_lo=1, len_hi=90,
                     cache="f32", wkv="bf16", seed=900 + dh)
    wl = syn.make(cfg, with_cache=False)
    K = syn.k_cache(cfg, wl.w, np.minimum(wl.lengths, cfg.T_max))
    o = gpu_decode(cfg, wl.q, to_dev(K), wl.lengths, dev_wkv(cfg, wl.w.W_K, wl.w.W_V))
    ref = oracle_decode(cfg, wl.q, K, wl.lengths, wl.w.W_K, wl.w.W_V)
    _check(f"f32 cache, bf16 W_KV, dh={dh}", o, ref, TOL["bf16"])


@pytest.mark.parametrize("name,kw", [("7b_ragged", dict(B=5, T_max=2000, len_lo=1, len_hi=2000)),
                                     ("long_128k", dict(T_max=8192)), ("whisper_large", dict(B=5, T_max=700))])
def test_partials_bf16_and_f32(monkeypatch, name, kw):
    """bf16 caches keep their chunk partials in bf16 by default (rounded once
    from the fp32 accumulator); SLIM_PARTIALS=f32 keeps them in fp32.  Both
    meet the oracle bound, and they differ by about the bf16 rounding of one
    partial."""
    import kv_cache_reduction_amd as slim
    cfg = syn.shrink(syn.CONFIGS[name], **kw)
    wl = syn.make(cfg)
    W = dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    o16 = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, W)
    monkeypatch.setenv("SLIM_PARTIALS", "f32")
    ws = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, 1))
    o32 = gpu_decode(cfg, wl.q, to_dev(wl.K), wl.lengths, W, ws=ws)
    e16 = _check(f"{name} bf16 partials", o16, ref, TOL["bf16"])
    e32 = _check(f"{name} fp32 partials", o32, ref, TOL["bf16"])
    diff = oracle.err_rel(o16, o32)
    log(f"[parity] {name}: bf16 vs fp32 partials differ by {diff:.2e} (errors {e16:.2e} / {e32:.2e})")
    assert diff <= 2.0 ** -7
