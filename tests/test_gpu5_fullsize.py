"""Full-size workloads in the launch configuration bench.py times.

Every output must be finite and the device status clean, and every sequence
is compared with the CPU oracle element by element, each sequence attended on
its own (the oracle takes well under a second per sequence, 65,536-token ones
included, on a 16-thread host).
"""
import numpy as np
import pytest

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import run, say, to_f64, tol
from tests.helpers import assert_close

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

FULL = ["C1_tiny", "C2_single_seq", "C3_batched_gqa", "C4_fp8_q1_per_token",
        "C4_fp8_q4_per_token", "C4_fp8_q1_per_tensor", "C4_fp8_q4_per_tensor",
        "C5_long_ctx_d256"]


def _check_every_sequence(w, got, label):
    spec = w.spec
    worst = 0.0
    for b in range(spec.batch):
        want, _ = oracle.decode(w.q[b:b + 1], w.k_cache, w.v_cache, w.block_table[b:b + 1],
                                w.context_lens[b:b + 1], spec.q_len, spec.scale, spec.page_size,
                                spec.kv_dtype, spec.kv_scale_mode, w.kv_scales)
        err = assert_close(got[b:b + 1], want, tol(spec), f"{label} sequence {b}")
        worst = max(worst, err)
        if b % 8 == 0 or b == spec.batch - 1:
            say(f"[{label}] sequence {b} (ctx {int(w.context_lens[b])}): max abs err {err:.2e}")
    say(f"[{label}] all {spec.batch} sequences: max abs err {worst:.2e}")


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", FULL)
def test_full_size_parity(name):
    spec = W.CONFIGS[name]
    w = W.generate(spec, 2026)
    say(f"[full] {name}: {spec.batch} sequences, {int(w.context_lens.sum())} tokens")
    out, plan = run(w)
    assert pa.pa_plan_status(plan) == 0
    got = to_f64(out)
    assert np.isfinite(got).all()
    _check_every_sequence(w, got, f"full {name}")


# twice the context lengths of three workloads (the largest shapes bench.py's
# scale sweep times): up to 16384 tokens at C3, 65536 tokens (64 pages of 1024)
# at C4
DOUBLED = ["C3_batched_gqa", "C4_fp8_q1_per_token", "C4_fp8_q4_per_token"]


@pytest.mark.timeout(300)
@pytest.mark.parametrize("name", DOUBLED)
def test_doubled_contexts_parity(name):
    base = W.CONFIGS[name]
    spec = W.scaled(base, ctx_lo=2 * base.ctx_lo, ctx_hi=2 * base.ctx_hi, max_ctx=0)
    w = W.generate(spec, 2029)
    say(f"[full x2] {name}: {spec.batch} sequences, {int(w.context_lens.sum())} tokens, "
        f"max {int(w.context_lens.max())}")
    out, plan = run(w)
    assert pa.pa_plan_status(plan) == 0
    got = to_f64(out)
    assert np.isfinite(got).all()
    _check_every_sequence(w, got, f"full x2 {name}")
