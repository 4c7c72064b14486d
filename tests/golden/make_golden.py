"""Writes tests/golden/tiny_f32_oracle.json: the float64 oracle's output on the
seeded tiny_f32 workload (d=64, H=4, dh=16, B=1, T=32, fp32 cache).

It calls only ``oracle`` and ``synthetic``; nothing here touches the HIP
library.  Rerun after a deliberate change to the oracle or the generator:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
import synthetic as syn  # noqa: E402


def main():
    cfg = syn.CONFIGS["tiny_f32"]
    wl = syn.make(cfg)
    K = oracle.cache_to_f64(wl.K)
    V = oracle.explicit_values(wl.K, wl.w.W_K, wl.w.W_V)
    o = oracle.mha_decode(wl.q, K, V, wl.lengths, cfg.H, cfg.dh, cfg.scale)
    out = {
        "what": "float64 oracle output o[B,H,dh] for the seeded tiny_f32 workload",
        "config": cfg.desc,
        "seed": cfg.seed,
        "writer": "tests/golden/make_golden.py (calls oracle/ and synthetic/ only)",
        "o": o.tolist(),
    }
    with open(os.path.join(HERE, "tiny_f32_oracle.json"), "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
