"""CPU oracle for paged-attention decode — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The library (``include/pa.h`` and
``paged_attention_decode_block_amd``) never imports, calls or links it, and it
shares no code with the library: not a kernel, header, helper or table.

It is a plain, slow, obviously correct NumPy implementation in float64:

  codecs     bf16 <-> float64 (round to nearest even) and the OCP E4M3FN decode
             and encode (round to nearest even)
  attention  block-table gather, dequantisation, decode attention over the
             gathered pages (with the causal mask of the appended tokens), the
             same attention restricted to a token range (split-KV partials) and
             the log-sum-exp merge of partials
  plan       the persistent work-list rule, written as a direct simulation
  cache      the KV-cache append (the write side): new tokens' K/V through the
             block table into their pages, quantised to fp8 per token and head
             or per tensor

The pages (hw-native-sys/simpler issue #998, Ascend/RecSDK issue #1281 and
ROCm/FlyDSL PR #910) name paged-attention decode, its block table, split-KV
partitions with a reducer and per-token or per-tensor fp8 KV scales, but print
no formula and no worked example; each function below states the plainest
reading it implements. Parity status of every function is pinned by the
``-m "not gpu"`` tests (brute force, library routines, closed forms and
invariants); none is "parity unpinned".
"""
from .codecs import (bf16_bits_to_f64, f64_to_bf16_bits, round_to_bf16, e4m3fn_to_f64,
                     e4m3fn_encode)
from . import cache
from .attention import (gather_rows, dequant_rows, decode, attend_range,
                        decode_split, merge_partials)
from .plan import plan, Plan

__all__ = [
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_to_bf16", "e4m3fn_to_f64", "e4m3fn_encode",
    "cache",
    "gather_rows", "dequant_rows", "decode", "attend_range", "decode_split",
    "merge_partials", "plan", "Plan",
]
