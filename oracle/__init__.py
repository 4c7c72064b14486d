"""Float64 CPU oracle for the Slim-Attention K-cache-only decode step.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The
product path (``kv_cache_reduction_amd``) never does, and shares no code with
this package: the two meet only through the seeded inputs of ``synthetic``.

What it computes.  Slim Attention is an exact rewrite of standard multi-head
attention (Slim Attention article, localbendi.com, section "K-Cache is All
You Need": the rewrite is mathematically exact, so accuracy is unchanged;
the pulseaugur.com summary of "Slim attention: cut your context memory in
half without loss" says the same).  The reference for the decode step is
therefore the plain definition: standard MHA decode over explicit K and V
caches, in float64 (``mha.mha_decode``).  Its value cache is rebuilt from the
K cache the device reads, without W_KV (``mha.explicit_values``).

The Slim forms themselves (``mha.wkv``, ``mha.slim_decode_opt1``,
``mha.slim_decode_opt2``) are here only so tests can pin them against the
definition; the GPU parity tests compare against ``mha_decode``.

Pins (tests/test_oracle.py, run with ``-m "not gpu"``): a hand-derived
two-token example, closed forms, brute-force loops, textbook special cases,
a library routine for bf16 rounding, and planted mistakes that the pins must
catch.  No function here is "parity unpinned".
"""
from .mha import (  # noqa: F401
    bf16_decode,
    round_bf16,
    cache_to_f64,
    mha_decode,
    mha_decode_loop,
    explicit_values,
    explicit_values_cols,
    value_map,
    wkv,
    slim_decode_opt1,
    slim_decode_opt2,
    prefill,
    prefill_loop,
    generate_step,
    append_rows,
    multi_query_attention,
    multi_query_cost,
    err_rel,
)
