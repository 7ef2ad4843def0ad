"""CPU oracle for MiniKV-style compressed-KV attention.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product path
(``bit_quantized_attention_two_amd``) never does, and this package never
imports the product path.  The arithmetic lives in ``minikv_oracle.c`` (plain
C, fp64 attention, step-by-step fp32 codec); this package builds it with gcc
and wraps it for numpy arrays.
"""
from .build_oracle import build, lib_path  # noqa: F401
from .api import (  # noqa: F401
    h2d, f2h_rne, quant_group, dequant, budgets, prefill_rows, prefill_unit,
    select, pack_unit, decode_unit, cache_bytes, OracleCache,
    quant_group_bits, pack_unit_bits, dequant_unit, attend, complement,
    diffkv_score, diffkv_tiers, OracleMixedCache,
)
