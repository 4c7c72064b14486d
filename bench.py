"""Benchmark: Slim-Attention K-cache-only decode on one MI355X.

One step = one pass of the decode path (attend: scores, online softmax and
softmax-times-K over the whole K cache; finish: chunk merge and W_KV
projection) for one new token per sequence.  W_KV (host, once per layer) and
the K cache write (prefill) happen before the timed region.

Default workload: long-context single-stream decode, d=4096, H=32, dh=128,
B=1, T=131072, bf16 K cache and W_KV.  Inputs are synthetic and seeded; the
K cache is written on the device by slim_prefill from bf16 X and W_K, and two
copies are rotated so the 256 MB Infinity Cache cannot serve a step from the
previous one.

Prints one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode tokens/s and K-cache GB/s (% HBM peak) at T=8K/128K, 1 MI355X"
HBM_PEAK_GBPS = 8000.0
ATTEND_SOURCES = ["kv_cache_reduction_amd/csrc/attend_bf16.hip", "kv_cache_reduction_amd/csrc/common.hpp",
                  "kv_cache_reduction_amd/csrc/internal.hpp"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", default="long_128k", choices=["gpt2_small", "7b_ragged", "7b_8k", "long_128k", "whisper_large"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="skip comparator, T=8K point, probe")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# device workload

def bf16_dev(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def build_cache(cfg, w, W, lens, torch, slim):
    """Cache rows round(X_b . W) for every sequence, written on the device by
    slim_prefill from bf16 X (seeded rows) and bf16 W."""
    import synthetic as syn
    K = torch.zeros((cfg.B, cfg.T_max, cfg.d), dtype=torch.bfloat16, device="cuda")
    Wd = bf16_dev(syn.f32_to_bf16_bits(W.astype(np.float32)))
    blk = 8192
    for b in range(cfg.B):
        n = int(lens[b])
        for t0 in range(0, n, blk):
            t1 = min(n, t0 + blk)
            X = bf16_dev(syn.f32_to_bf16_bits(syn.x_rows(cfg, b, t0, t1)))[None]
            t0d = torch.tensor([t0], dtype=torch.int32, device="cuda")
            slim.prefill(X, Wd, K[b:b + 1], t0=t0d)
    torch.cuda.synchronize()
    return K


class Workload:
    def __init__(self, name, torch, slim, with_v=False, rotate=2):
        import synthetic as syn
        self.cfg = cfg = syn.CONFIGS[name]
        t = time.time()
        w = syn.weights(cfg)
        # the device K cache is built from bf16 W_K, so W_KV comes from the same matrix
        WK = syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(w.W_K.astype(np.float32))).astype(np.float64)
        self.lens = syn.lengths(cfg)
        self.w, self.WK = w, WK
        self.q = torch.from_numpy(syn.queries(cfg, w)).cuda()
        self.ld = torch.from_numpy(self.lens).cuda()
        log(f"[bench] {name}: weights {time.time() - t:.1f}s")
        t = time.time()
        W = slim.wkv(WK, w.W_V, cfg.wkv)
        self.W = bf16_dev(W) if cfg.wkv == "bf16" else torch.from_numpy(W).cuda()
        log(f"[bench] {name}: W_KV (host LU, d={cfg.d}) {time.time() - t:.1f}s")
        t = time.time()
        K0 = build_cache(cfg, w, WK, self.lens, torch, slim)
        self.K = [K0] + [K0.clone() for _ in range(rotate - 1)]
        self.V = None
        if with_v:
            V0 = build_cache(cfg, w, w.W_V, self.lens, torch, slim)
            self.V = [V0] + [V0.clone() for _ in range(rotate - 1)]
        log(f"[bench] {name}: caches via prefill {time.time() - t:.1f}s")
        self.out = torch.empty((cfg.B, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
        self.ws = slim.workspace(slim.decode_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, slim.BF16))
        self.kv_ws = slim.workspace(slim.mha_kv_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, slim.BF16))
        self.k_bytes = int(self.lens.astype(np.int64).sum()) * cfg.d * 2


def time_slim(wl, torch, slim, steps, warmup):
    """Step time: `steps` slim_decode calls back to back between two events.
    Attend time (for the roofline): a second loop with an event pair around
    each attend launch; those events sit between kernels, so this loop is
    not used for the step time."""
    cfg = wl.cfg
    args = lambda i: (wl.q, wl.K[i % len(wl.K)], wl.ld, wl.W, wl.out, cfg.H, cfg.dh, cfg.scale, wl.ws)
    for i in range(warmup):
        slim.decode(*args(i))
    torch.cuda.synchronize()
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    start.record()
    for i in range(steps):
        slim.decode(*args(i))
    stop.record()
    torch.cuda.synchronize()
    ms_step = start.elapsed_time(stop) / steps
    a0 = [E(enable_timing=True) for _ in range(steps)]
    a1 = [E(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        a0[i].record()
        slim.decode_attend(*args(i))
        a1[i].record()
        slim.decode_finish(*args(i))
    torch.cuda.synchronize()
    attend = np.array([a0[i].elapsed_time(a1[i]) for i in range(steps)])
    return ms_step, attend


def time_step(wl, torch, slim, steps, warmup):
    """The whole generation step (slim_step): q and k from the new token's x
    by bf16 W_Q and W_K, attention over len_b - 1 cached rows, k appended at
    row len_b - 1 (the same row every step, so the cache never fills)."""
    import synthetic as syn
    cfg = wl.cfg
    WQ = bf16_dev(syn.f32_to_bf16_bits(wl.w.W_Q.astype(np.float32)))
    WK = bf16_dev(syn.f32_to_bf16_bits(wl.WK.astype(np.float32)))
    x = torch.from_numpy(syn.x_new(cfg)).cuda()
    lens = torch.from_numpy(np.maximum(wl.lens - 1, 0).astype(np.int32)).cuda()
    nxt = torch.empty_like(lens)
    ws = slim.workspace(slim.step_workspace_bytes(cfg.B, cfg.H, cfg.dh, cfg.T_max, slim.BF16))
    args = lambda i: (x, WQ, WK, wl.K[i % len(wl.K)], lens, nxt, wl.W, wl.out, cfg.H, cfg.dh, cfg.scale, ws)
    for i in range(warmup):
        slim.step(*args(i))
    torch.cuda.synchronize()
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    start.record()
    for i in range(steps):
        slim.step(*args(i))
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def _event_ms(torch, fn, steps, warmup):
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    start.record()
    for _ in range(steps):
        fn()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def _graph_ms(torch, fn, out, steps):
    """Device time of one call: the call captured once in a graph and
    replayed `steps` times between events (a call of a few tens of us is
    otherwise bound by the host's launch rate).  Every replay's output must
    equal the eager call's bit for bit."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    ref = out.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for _ in range(3):
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        if not torch.equal(out, ref):
            raise RuntimeError("graph replay differs from the eager call")
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    start.record()
    for _ in range(steps):
        g.replay()
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def multi_query_flops(n, H, dh, T, limits, option):
    """Algorithmic flops of n queries over one context: scores 2 L d, the
    softmax times K on all d columns per head 2 H L d and the projection
    2 n d^2 (option 2), or V = K.W_KV 2 T d^2 and the softmax times V 2 L d
    (option 1), with L the summed rows the queries attend."""
    d = H * dh
    L = float(np.sum(np.clip(limits, 0, T))) if limits is not None else float(n) * T
    if option == 1:
        return 2.0 * T * d * d + 2.0 * L * d + 2.0 * L * d
    return 2.0 * L * d + 2.0 * H * L * d + 2.0 * n * d * d


def time_multi(torch, slim, steps):
    """Many queries over one context: Whisper-large-shaped cross-attention of
    64 decoder queries over one shared encoder context (T=1500, d=1280), and
    a GPT-2-small-shaped prompt of 2048 tokens attending causally over itself
    (d=768).  K written by slim_prefill from bf16 X and W_K; bf16 W_KV.
    Device time per call by graph replay."""
    import synthetic as syn
    out = {}
    cases = [("shared_context", syn.CONFIGS["whisper_large"], 64, False), ("prompt", syn.CONFIGS["gpt2_small"], 2048, True)]
    for name, cfg, n, causal in cases:
        w = syn.weights(cfg)
        T = cfg.T_max
        one = syn.shrink(cfg, B=1)
        Xb = syn.f32_to_bf16_bits(syn.x_rows(one, 0, 0, T))
        K = torch.zeros((1, T, cfg.d), dtype=torch.bfloat16, device="cuda")
        slim.prefill(bf16_dev(Xb)[None], bf16_dev(syn.f32_to_bf16_bits(w.W_K.astype(np.float32))), K)
        K = K[0]
        Wkv = bf16_dev(slim.wkv(syn.bf16_bits_to_f32(syn.f32_to_bf16_bits(w.W_K.astype(np.float32))).astype(
            np.float64), w.W_V, "bf16"))
        if causal:
            X = syn.x_rows(one, 0, T - n, T).astype(np.float64)
            Q = torch.from_numpy((X @ w.W_Q).astype(np.float32)).cuda()
            lim_np = (T - n) + np.arange(n, dtype=np.int32) + 1
            lim = torch.from_numpy(lim_np).cuda()
        else:
            Q = torch.from_numpy(syn.queries(cfg, w)[:n]).cuda()
            lim_np, lim = None, None
        o = torch.empty((n, cfg.H, cfg.dh), dtype=torch.float32, device="cuda")
        rec = {"workload": (f"{n} queries over one context of {T} rows, d={cfg.d} H={cfg.H} dh={cfg.dh}"
                            + (", causal (prompt phase)" if causal else ", shared (cross-attention)")),
               "auto_option": slim.multi_query_option(n, cfg.H, cfg.dh, T)}
        for opt in (1, 2):
            ws = slim.workspace(slim.multi_query_workspace_bytes(n, cfg.H, cfg.dh, T, torch.bfloat16, opt))
            ms = _graph_ms(torch, lambda: slim.multi_query(Q, K, Wkv, o, cfg.H, cfg.dh, limits=lim,
                                                           scale=cfg.scale, option=opt, ws=ws), o, steps)
            fl = multi_query_flops(n, cfg.H, cfg.dh, T, lim_np, opt)
            rec[f"option{opt}"] = {"us": ms * 1e3, "tokens_s": n / (ms * 1e-3), "tflops": fl / (ms * 1e-3) / 1e12,
                                   "mfma_bf16_frac": fl / (ms * 1e-3) / 2.5e15}
            log(f"[bench] {name}: option {opt}: {ms * 1e3:.1f} us, {fl / (ms * 1e-3) / 1e12:.1f} TFLOP/s")
        out[name] = rec
    return out


def time_kv(wl, torch, slim, steps, warmup):
    cfg = wl.cfg
    args = lambda i: (wl.q, wl.K[i % len(wl.K)], wl.V[i % len(wl.V)], wl.ld, wl.out, cfg.H, cfg.dh,
                      cfg.scale, wl.kv_ws)
    for i in range(warmup):
        slim.mha_decode_kv(*args(i))
    torch.cuda.synchronize()
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    start.record()
    for i in range(steps):
        slim.mha_decode_kv(*args(i))
    stop.record()
    torch.cuda.synchronize()
    return start.elapsed_time(stop) / steps


def probe_copy_gbps(torch, slim, dst, src):
    """Plain copy of a known size (read + write); its counter readings
    calibrate FETCH_SIZE / WRITE_SIZE."""
    for _ in range(2):
        slim.probe_copy(dst, src)
    torch.cuda.synchronize()
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    n = 5
    start.record()
    for _ in range(n):
        slim.probe_copy(dst, src)
    stop.record()
    torch.cuda.synchronize()
    return 2 * src.numel() * src.element_size() / (start.elapsed_time(stop) / n * 1e-3) / 1e9


def measured_traffic(kernel_sources):
    """HBM bytes per attend launch from the committed counter summary, if the
    counters were taken on the current kernel source; otherwise None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "attend_bf16_long_128k_counters.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    h = hashlib.sha256()
    for f in kernel_sources:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if rec.get("kernel_source_sha256") != h.hexdigest():
        return None
    return rec.get("hbm_bytes_per_launch")


def attend_kernel_name(cfg):
    """The attend kernel the library picks for this shape: the score
    exchange between the two column groups for d = 2*dc with dh = 128 (d a
    multiple of 512 above 2048), the one-workgroup-per-column-group kernel
    otherwise."""
    xchg = (cfg.dh == 128 and cfg.d > 2048 and cfg.d % 512 == 0
            and os.environ.get("SLIM_XCHG", "1") != "0")
    return "slim::attend_xchg_kernel<4>" if xchg else "slim::attend_bf16_kernel"


def probe_read_gbps(torch, slim, src):
    sink = torch.empty(slim.probe_sink_floats(), dtype=torch.float32, device="cuda")
    for _ in range(3):
        slim.probe_read(src, sink)
    torch.cuda.synchronize()
    E = torch.cuda.Event
    start, stop = E(enable_timing=True), E(enable_timing=True)
    n = 10
    start.record()
    for _ in range(n):
        slim.probe_read(src, sink)
    stop.record()
    torch.cuda.synchronize()
    return src.numel() * src.element_size() / (start.elapsed_time(stop) / n * 1e-3) / 1e9


# ---------------------------------------------------------------------------
# CPU baseline: the float64 oracle on a bounded sample of the same workload

def cpu_baseline(name, T_sample=16384, min_seconds=10.0):
    import oracle
    import synthetic as syn
    cfg = syn.shrink(syn.CONFIGS[name], B=1, T_max=T_sample, len_lo=T_sample, len_hi=T_sample)
    full = syn.CONFIGS[name]
    wl = syn.make(cfg)
    K = oracle.cache_to_f64(wl.K)
    V = oracle.explicit_values(wl.K, wl.w.W_K, wl.w.W_V)  # plays the role of the prefill: untimed
    threads = None
    try:
        from threadpoolctl import threadpool_info
        threads = max((i.get("num_threads") or 1) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:
        threads = None
    times = []
    t_all = time.time()
    while time.time() - t_all < min_seconds or len(times) < 3:
        t = time.perf_counter()
        oracle.mha_decode(wl.q, K, V, wl.lengths, cfg.H, cfg.dh, cfg.scale)
        times.append(time.perf_counter() - t)
    t_med = float(np.median(times))
    # the oracle's decode work is linear in the live tokens: scale to the full workload
    full_tokens = int(syn.lengths(full).astype(np.int64).sum())
    t_step = t_med * full_tokens / T_sample
    cpu_model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {
        "value": full.B / t_step,
        "unit": "tokens/s",
        "cores": threads if threads else os.cpu_count(),
        "kind": "oracle",
        "sample": (f"float64 numpy oracle (standard MHA over explicit K and V) on one sequence of "
                   f"{T_sample} tokens of the {name} shape (d={full.d}, H={full.H}, dh={full.dh}), "
                   f"median of {len(times)} runs ({t_med * 1e3:.1f} ms), scaled linearly to "
                   f"{full_tokens} tokens; V construction untimed"),
        "host_cpus": os.cpu_count(),
        "cpu_model": cpu_model,
    }


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}): the path's sharding over "
              f"several GPUs is a design, not built or run here", file=sys.stderr)
        sys.exit(2)
    import torch
    import kv_cache_reduction_amd as slim
    assert torch.cuda.is_available(), "no GPU visible"
    props = torch.cuda.get_device_properties(0)
    log(f"[bench] device {props.name} {getattr(props, 'gcnArchName', '')} CUs={props.multi_processor_count}")

    name = args.config
    wl = Workload(name, torch, slim, with_v=not args.no_extras)
    cfg = wl.cfg
    log(f"[bench] timing {name}: {args.warmup} warmup + {args.steps} steps")
    ms_step, attend = time_slim(wl, torch, slim, args.steps, args.warmup)
    att_ms = float(attend.mean())
    tokens_s = cfg.B / (ms_step * 1e-3)
    k_gbps_step = wl.k_bytes / (ms_step * 1e-3) / 1e9
    k_gbps_attend = wl.k_bytes / (att_ms * 1e-3) / 1e9
    log(f"[bench] {name}: {ms_step * 1e3:.1f} us/step, attend {att_ms * 1e3:.1f} us "
        f"({k_gbps_attend:.0f} GB/s), step K-rate {k_gbps_step:.0f} GB/s, {tokens_s:.1f} tokens/s")

    res = {
        "metric": METRIC,
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.desc, "d": cfg.d, "H": cfg.H, "dh": cfg.dh, "batch": cfg.B,
                   "T": cfg.T_max, "k_cache": "bf16", "w_kv": cfg.wkv,
                   "arith": "fp32 scores/softmax/accumulate, bf16 softmax-times-K on MFMA"},
        "k_cache_gbps": k_gbps_step,
        "k_cache_hbm_frac": k_gbps_step / HBM_PEAK_GBPS,
        "roofline": {"bound": "hbm", "achieved": k_gbps_attend, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": k_gbps_attend / HBM_PEAK_GBPS,
                     "traffic": measured_traffic(ATTEND_SOURCES) if name == "long_128k" else None,
                     "kernel": attend_kernel_name(cfg), "kernel_us": att_ms * 1e3,
                     "algorithmic_bytes": wl.k_bytes},
    }

    if not args.no_extras:
        ms_gen = time_step(wl, torch, slim, max(10, args.steps // 2), 3)
        wbytes = 2 * cfg.d * cfg.d * 2
        res["generation_step"] = {
            "what": ("slim_step: q = x.W_Q and k = x.W_K (bf16 weights, fp32 accumulate), attention "
                     "over len_b - 1 cached rows, k appended at row len_b - 1"),
            "tokens_s": cfg.B / (ms_gen * 1e-3), "ms_per_step": ms_gen,
            "over_decode_us": (ms_gen - ms_step) * 1e3,
            "projection_weight_bytes": wbytes}
        log(f"[bench] generation step: {ms_gen * 1e3:.1f} us/step "
            f"({(ms_gen - ms_step) * 1e3:.1f} us over the decode)")
        res["multi_query"] = time_multi(torch, slim, max(10, args.steps // 2))
        ms_kv = time_kv(wl, torch, slim, max(10, args.steps // 2), 3)
        res["comparator"] = {"what": "standard MHA decode over explicit bf16 K and V caches (same box)",
                             "tokens_s": cfg.B / (ms_kv * 1e-3), "ms_per_step": ms_kv,
                             "kv_gbps": 2 * wl.k_bytes / (ms_kv * 1e-3) / 1e9,
                             "slim_speedup": ms_kv / ms_step}
        log(f"[bench] comparator: {ms_kv * 1e3:.1f} us/step, slim speedup {ms_kv / ms_step:.2f}x")
        res["probe_read_gbps"] = probe_read_gbps(torch, slim, wl.K[0])
        log(f"[bench] HBM read probe: {res['probe_read_gbps']:.0f} GB/s")
        res["probe_copy_gbps"] = probe_copy_gbps(torch, slim, wl.K[1], wl.K[0])
        log(f"[bench] HBM copy probe (read+write): {res['probe_copy_gbps']:.0f} GB/s")
        del wl
        torch.cuda.empty_cache()
        if name == "long_128k":
            w2 = Workload("7b_8k", torch, slim, with_v=False)
            ms2, att2 = time_slim(w2, torch, slim, max(10, args.steps // 2), 3)
            res["secondary"] = {"workload": w2.cfg.desc, "tokens_s": w2.cfg.B / (ms2 * 1e-3),
                                "ms_per_step": ms2, "k_cache_gbps": w2.k_bytes / (ms2 * 1e-3) / 1e9,
                                "attend_gbps": w2.k_bytes / (att2.mean() * 1e-3) / 1e9}
            log(f"[bench] 7b_8k: {ms2 * 1e3:.1f} us/step, {res['secondary']['k_cache_gbps']:.0f} GB/s")
            del w2
            torch.cuda.empty_cache()

    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle) ...")
        res["cpu_baseline"] = cpu_baseline(name)
        log(f"[bench] cpu baseline: {res['cpu_baseline']['value']:.3f} tokens/s")
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
