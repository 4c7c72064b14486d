"""slim_decode_noalloc (the decode call that allocates nothing; its
workspace is the library's own device array) against slim_decode with a
caller workspace, through the C ABI: two calls in a row on the same device
array, the second with a smaller input, each equal to slim_decode's output
bit for bit (same kernels and plan) and within the bf16 tolerance of the
float64 oracle; a shape whose workspace exceeds the array is rejected
before anything is enqueued."""
import numpy as np
import pytest

import oracle
import synthetic as syn
from gpu_common import TOL, dev_wkv, log, oracle_decode, report_err, to_dev

pytestmark = pytest.mark.gpu


def _run(cfg, wl):
    import torch
    import kv_cache_reduction_amd as slim
    Kd, Wd = to_dev(wl.K), dev_wkv(cfg, wl.w.W_K, wl.w.W_V)
    qd, ld = to_dev(wl.q.astype(np.float32)), to_dev(wl.lengths.astype(np.int32))
    need = slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, Kd.dtype)
    assert 0 < need <= slim.NOALLOC_SCRATCH_BYTES
    out_n = torch.full((cfg.B, cfg.H, cfg.dh), float("nan"), dtype=torch.float32, device="cuda")
    out_w = torch.full_like(out_n, float("nan"))
    slim.decode_noalloc(qd, Kd, ld, Wd, out_n, cfg.H, cfg.dh, cfg.scale)
    torch.cuda.synchronize()
    slim.decode(qd, Kd, ld, Wd, out_w, cfg.H, cfg.dh, cfg.scale)
    torch.cuda.synchronize()
    o = out_n.cpu().numpy().astype(np.float64)
    same = torch.equal(out_n, out_w)
    log(f"[noalloc] {cfg.name} B={cfg.B} T={cfg.T_max}: workspace {need} bytes, equal to slim_decode: {same}")
    assert same
    ref = oracle_decode(cfg, wl.q, wl.K, wl.lengths, wl.w.W_K, wl.w.W_V)
    assert report_err(f"noalloc {cfg.name}", o, ref) <= TOL["bf16"]


def test_noalloc_two_calls_second_smaller():
    big = syn.shrink(syn.CONFIGS["7b_ragged"], B=5, T_max=2000, len_lo=1, len_hi=2000)
    _run(big, syn.make(big))                     # exchange kernel, two column groups
    small = syn.shrink(syn.CONFIGS["gpt2_small"], B=2, T_max=300)
    _run(small, syn.make(small))                 # one column group, fewer chunks


def test_noalloc_rejects_a_workspace_over_the_array():
    import torch
    import kv_cache_reduction_amd as slim
    B, H, dh, T = 512, 32, 128, 8192
    need = slim.decode_workspace_bytes(B, H, dh, T, torch.bfloat16)
    assert need > slim.NOALLOC_SCRATCH_BYTES
    d = H * dh
    q = torch.zeros((B, d), dtype=torch.float32, device="cuda")
    K = torch.zeros((B, 8, d), dtype=torch.bfloat16, device="cuda")   # shape check only: never read
    lens = torch.zeros(B, dtype=torch.int32, device="cuda")
    W = torch.zeros((d, d), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((B, H, dh), dtype=torch.float32, device="cuda")
    st = slim.lib.slim_decode_noalloc(q.data_ptr(), K.data_ptr(), slim.BF16, lens.data_ptr(), W.data_ptr(),
                                      slim.BF16, out.data_ptr(), B, H, dh, T, 0.1,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 3   # SLIM_ERR_WORKSPACE
