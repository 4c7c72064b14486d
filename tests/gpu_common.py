"""Shared helpers of the GPU parity tests: move seeded inputs to the device,
run the HIP path through the C ABI, and build the float64 references."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synthetic as syn

TOL = {"f32": 1e-4, "bf16": 2e-2}   # max|o - o_ref| / max|o_ref|


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def slim_mod():
    import kv_cache_reduction_amd as slim
    return slim


def to_dev(a: np.ndarray):
    """numpy storage (float32, int32, or uint16 bf16 bits) -> device tensor."""
    torch = torch_mod()
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to("cuda").view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def bf16_bits(t) -> np.ndarray:
    torch = torch_mod()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev_wkv(cfg: syn.Config, W_K: np.ndarray, W_V: np.ndarray):
    """W_KV from the library's host solver, on the device in the config's dtype."""
    return to_dev(slim_mod().wkv(W_K, W_V, cfg.wkv))


def gpu_decode(cfg: syn.Config, q: np.ndarray, Kdev, lens: np.ndarray, Wdev, ws=None,
               phases: bool = False) -> np.ndarray:
    torch = torch_mod()
    slim = slim_mod()
    B = q.shape[0]
    out = torch.empty((B, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
    qd = to_dev(q.astype(np.float32))
    ld = to_dev(np.asarray(lens, dtype=np.int32))
    if ws is None:
        ws = slim.workspace(slim.decode_workspace_bytes(B, cfg.H, cfg.dh, Kdev.shape[1], Kdev.dtype))
    if phases:
        slim.decode_attend(qd, Kdev, ld, Wdev, out, cfg.H, cfg.dh, cfg.scale, ws)
        slim.decode_finish(qd, Kdev, ld, Wdev, out, cfg.H, cfg.dh, cfg.scale, ws)
    else:
        slim.decode(qd, Kdev, ld, Wdev, out, cfg.H, cfg.dh, cfg.scale, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def head_cols(heads, dh) -> np.ndarray:
    return np.concatenate([np.arange(h * dh, (h + 1) * dh) for h in heads])


def oracle_decode(cfg: syn.Config, q: np.ndarray, K: np.ndarray, lens: np.ndarray,
                  W_K: np.ndarray, W_V: np.ndarray, seqs=None, heads=None,
                  reassociate: bool = False) -> np.ndarray:
    """Float64 standard MHA over explicit K and V for the given sequences and
    heads.  K is the cache the device read (storage dtype or float64); V is
    rebuilt from it without W_KV.  Returns [len(seqs), len(heads), dh]."""
    seqs = list(range(q.shape[0])) if seqs is None else list(seqs)
    heads = list(range(cfg.H)) if heads is None else list(heads)
    cols = head_cols(heads, cfg.dh)
    out = np.zeros((len(seqs), len(heads), cfg.dh))
    for i, b in enumerate(seqs):
        n = int(min(max(int(lens[b]), 0), K.shape[1]))
        if n == 0:
            continue
        Kb = K[b, :n]
        if reassociate:
            V = oracle.explicit_values_cols(Kb, W_K, W_V, cols)
        else:
            V = oracle.explicit_values(Kb, W_K, W_V, cols=cols)
        Kc = oracle.cache_to_f64(Kb)[:, cols]
        out[i] = oracle.mha_decode(q[b:b + 1, cols], Kc[None], V[None], [n], len(heads), cfg.dh,
                                   cfg.scale)[0]
    return out


def check_prefill_bf16(got_bits: np.ndarray, X: np.ndarray, W: np.ndarray, name: str) -> None:
    """Device prefill output against the float64 product of the same bf16 X
    and W.  Each element is within one bf16 ulp of the rounded exact product
    plus the worst-case float32 summation error n * 2^-24 * sum_k |x_k w_k|
    (near-cancelling sums can round differently); and at least 99.9% of the
    elements are bit-identical to the correctly rounded product."""
    ref = oracle.prefill(X, W, "bf16")
    got = oracle.bf16_decode(got_bits)
    absprod = np.abs(X) @ np.abs(W)
    n = X.shape[-1]
    mag = np.maximum(np.abs(ref), 2.0 ** -126)
    ulp = 2.0 ** (np.floor(np.log2(mag)) - 7)
    bound = ulp + n * 2.0 ** -24 * absprod
    diff = np.abs(got - ref)
    exact = float(np.mean(diff == 0))
    log(f"[parity] prefill {name}: exact {exact:.5f}, max diff/bound {float((diff / bound).max()):.3f}")
    assert np.all(diff <= bound)
    assert exact >= 0.999


def oracle_decode_full(cfg: syn.Config, q: np.ndarray, K: np.ndarray, lens: np.ndarray,
                       W_K: np.ndarray, W_V: np.ndarray, head_group: int = 8) -> np.ndarray:
    """The whole [B, H, dh] float64 reference, built head group by head group
    so that host memory stays bounded at the long-context size: for each
    sequence and group of heads, V[:, cols] = K~ . (W_K^-1 W_V[:, cols])
    (``explicit_values_cols``, pinned against the full form; the solve is
    done once), then standard MHA over those heads."""
    B = q.shape[0]
    M = oracle.value_map(W_K, W_V)
    out = np.zeros((B, cfg.H, cfg.dh))
    for b in range(B):
        n = int(min(max(int(lens[b]), 0), K.shape[1]))
        if n == 0:
            continue
        Kb = K[b, :n]
        for h0 in range(0, cfg.H, head_group):
            heads = list(range(h0, min(cfg.H, h0 + head_group)))
            cols = head_cols(heads, cfg.dh)
            V = oracle.explicit_values_cols(Kb, None, None, cols, M=M[:, cols])
            Kc = oracle.cache_to_f64(Kb[:, cols])
            out[b, heads] = oracle.mha_decode(q[b:b + 1, cols], Kc[None], V[None], [n], len(heads), cfg.dh,
                                              cfg.scale)[0]
    return out


def report_err(name: str, o: np.ndarray, ref: np.ndarray) -> float:
    """Logs the whole-output metric and the largest per-sequence value (not
    gated) and returns the whole-output metric."""
    err = oracle.err_rel(o, ref)
    per_seq = max(oracle.err_rel(o[b], ref[b]) for b in range(ref.shape[0]))
    log(f"[parity] {name}: whole-output err={err:.3e} max|ref|={np.abs(ref).max():.3e} "
        f"worst sequence err={per_seq:.3e} elements={ref.size}")
    return err
