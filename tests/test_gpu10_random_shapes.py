"""Random shapes: every axis the decode supports, drawn together.

The other decode tests vary one axis at a time around the benchmark's
workloads. Each of these 96 seeded cases draws all of them at once: batch,
q_len, kv heads and GQA group, head_dim, page size, KV dtype and scale mode,
block-table capacity, partition size, grid multiplier and reduce mode (the
tuned choice, separate, or fused), with ragged context lengths that include
the extremes (q_len itself and the full capacity). The decode must match the
oracle within the dtype's tolerance, with a clean device status.
"""
import random

import pytest

import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import check, run, say

pytestmark = pytest.mark.gpu

CASES = 96


def _draw(i):
    r = random.Random(7000 + i)
    hkv = r.choice([1, 2, 4, 8])
    group = r.choice([1, 2, 4, 8, 16])
    d = r.choice([128, 256])
    q_len = r.choice([1, 1, 2, 3, 4, 8])
    ps = r.choice([16, 32, 64, 128, 256, 512, 1024])
    fp8 = r.random() < 0.5
    mode = r.choice([W.SCALE_PER_TOKEN_HEAD, W.SCALE_PER_TENSOR]) if fp8 else W.SCALE_NONE
    batch = r.randint(1, 6)
    pages = r.randint(1, max(1, 4096 // ps))
    cap = max(pages * ps, q_len)
    ctx = [r.choice([q_len, cap, r.randint(q_len, cap), r.randint(q_len, cap)]) for _ in range(batch)]
    spec = W.Spec(f"rand{i}", batch, q_len, hkv * group, hkv, d, ps, min(ctx), max(ctx),
                  kv_dtype=W.KV_FP8 if fp8 else W.KV_BF16, kv_scale_mode=mode, max_ctx=cap)
    partition = r.choice([16, 32, 64, 128, 256, 1024])
    mult = r.choice([0, 1, 2])
    flags = r.choice([0, pa.PA_FLAG_SEPARATE_REDUCE, pa.PA_FLAG_FUSED_REDUCE])
    return spec, ctx, partition, mult, flags


@pytest.mark.parametrize("i", range(CASES))
def test_random_shape(i):
    spec, ctx, partition, mult, flags = _draw(i)
    w = W.generate(spec, 2026 + i, context_lens=ctx)
    say(f"[random {i}] B={spec.batch} q_len={spec.q_len} Hq={spec.num_q_heads} "
        f"Hkv={spec.num_kv_heads} D={spec.head_dim} page={spec.page_size} {spec.kv_dtype}/"
        f"{spec.kv_scale_mode} cap={spec.max_ctx} ctx={ctx} P={partition} mult={mult} flags={flags}")
    out, plan = run(w, partition=partition, grid_multiplier=mult, flags=flags)
    assert pa.pa_plan_status(plan) == 0
    check(w, out, f"random case {i}")
