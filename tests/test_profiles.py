"""The committed measurement records agree with each other and with the
sources they describe: the bench's JSON line carries the roofline and CPU
baseline objects, its `traffic` is the HBM figure of the counter summary,
and that summary was taken on the attend kernel as it is now (its source
hash matches), so a kernel edit without new counters fails here."""
import hashlib
import json
import os

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def _load(name):
    with open(os.path.join(PROFILES, name)) as f:
        return json.load(f)


def test_bench_record_has_the_contract_fields():
    b = _load("bench_long_128k_decode.json")
    for k in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step", "higher_is_better",
              "scaling", "vs_baseline", "dtype", "data", "config", "roofline", "cpu_baseline"):
        assert k in b, k
    r = b["roofline"]
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac"] - r["achieved"] / r["peak"]) < 1e-9
    # achieved = algorithmic bytes per launch over the kernel's mean duration
    assert abs(r["achieved"] - r["algorithmic_bytes"] / (r["kernel_us"] * 1e-6) / 1e9) < 1e-6 * r["achieved"]
    assert r["algorithmic_bytes"] == 131072 * 4096 * 2
    assert abs(b["value"] - 1.0 / (b["ms_per_step"] * 1e-3)) < 1e-6 * b["value"]   # B = 1 token per step
    c = b["cpu_baseline"]
    assert c["kind"] == "oracle" and c["cores"] >= 1 and c["value"] > 0


def test_bench_traffic_is_the_counter_summary_of_the_current_kernel():
    b = _load("bench_long_128k_decode.json")
    rec = _load("attend_bf16_long_128k_counters.json")
    assert b["roofline"]["traffic"] == rec["hbm_bytes_per_launch"]
    cal = rec["calibration"]
    want = round(rec["fetch_size_kib_per_dispatch_median"] * 1024 * cal["fetch_factor"]
                 + rec["write_size_kib_per_dispatch_median"] * 1024 * cal["write_factor"])
    assert abs(rec["hbm_bytes_per_launch"] - want) <= 1
    h = hashlib.sha256()
    for f in rec["kernel_sources"]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    assert rec["kernel_source_sha256"] == h.hexdigest(), "attend sources changed since the counters were taken"
