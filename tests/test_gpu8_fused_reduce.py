"""The fused reduce (PA_FLAG_FUSED_REDUCE) and the tuned choices.

With the fused reduce the partition pass merges each split pair itself: the
last of the pair's workgroups to finish (per-pair arrival counters) runs the
reduce kernel's arithmetic in slot order. Its output must be bitwise the
separate reduce's, launch after launch on one plan (the counters reset
themselves), under graph replay, with query blocks, with the plan reused
while contexts grow, and with a pair split over every workgroup; and it must
match the oracle. Every setting the tuning table can choose is run against
the oracle too.
"""
import pytest
import torch

import paged_attention_decode_block_amd as pa
import workloads as W
from paged_attention_decode_block_amd import tuning
from tests.gpu_util import DEV, MODE_CODE, check, dims_for, say, upload

pytestmark = pytest.mark.gpu

FUSED, SEPARATE = pa.PA_FLAG_FUSED_REDUCE, pa.PA_FLAG_SEPARATE_REDUCE

SPECS = {
    "bf16_gqa": W.scaled(W.C3, batch=5, ctx_lo=100, ctx_hi=1200, max_ctx=1280),
    "fp8_tok_q1": W.scaled(W.C4_Q1_TOK, batch=3, ctx_lo=300, ctx_hi=3000, max_ctx=3072),
    "fp8_tok_q4": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=300, ctx_hi=3000, max_ctx=3072),
    "fp8_ten_q4": W.scaled(W.C4_Q4_TEN, batch=3, ctx_lo=4, ctx_hi=3000, max_ctx=3072),
    "d256_q8": W.scaled(W.C5, batch=2, ctx_lo=300, ctx_hi=1500, max_ctx=1536, pool_slack=0.2),
    "fp8_tok_d256": W.scaled(W.C5, batch=2, ctx_lo=300, ctx_hi=1500, max_ctx=1536,
                             pool_slack=0.2, kv_dtype=W.KV_FP8,
                             kv_scale_mode=W.SCALE_PER_TOKEN_HEAD),
    # 192 rows per kv head: the shared-tile instantiation of 8 waves per chunk
    "bf16_q24_g8": W.Spec("bf16_q24_g8", 3, 24, 8, 1, 128, 32, 24, 1500, max_ctx=2048),
}


def _decode(w, d, flags, partition=None, mult=0, plan=None, reps=1, ctx=None):
    s = w.spec
    ctx = d.context_lens if ctx is None else ctx
    if plan is None:
        plan = pa.pa_plan(dims_for(w, partition, mult, flags), ctx)
    outs = []
    for _ in range(reps):
        out = torch.full_like(d.q, float("nan"))
        pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, ctx, s.q_len, s.scale,
                     MODE_CODE[s.kv_scale_mode], d.kv_scales, out)
        outs.append(out)
    return outs, plan


def _same(a, b):
    return torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("partition,mult", [(256, 0), (32, 4), (16, 1)])
@pytest.mark.parametrize("name", sorted(SPECS))
def test_fused_equals_separate(name, partition, mult):
    w = W.generate(SPECS[name], 2029)
    d = upload(w)
    (sep,), plan_s = _decode(w, d, SEPARATE, partition, mult)
    fused, plan_f = _decode(w, d, FUSED, partition, mult, reps=3)
    assert plan_f.c.dims.flags & FUSED and plan_s.c.dims.flags & SEPARATE
    split = sum(1 for n in plan_f.region("nseg", plan_f.c.num_pairs).cpu().tolist() if n > 1)
    say(f"[fused] {name} P={partition} mult={mult}: {split} split pairs")
    assert pa.pa_plan_status(plan_f) == 0 and pa.pa_plan_status(plan_s) == 0
    for i, f in enumerate(fused):
        assert _same(f, sep), f"{name}: launch {i} on one plan"
    # every arrival counter is back at zero for the next launch
    assert (plan_f.region("counters", plan_f.c.num_pairs) == 0).all()
    check(w, fused[0], f"fused {name} P={partition}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_tok"])
def test_fused_one_pair_over_every_workgroup(kv):
    """A 16384-token pair at partition 16: 1024 items, a segment on every
    workgroup, so the last arrival merges as many partials as there are
    workgroups."""
    base = {"bf16": W.Spec("one_pair_bf16", 1, 4, 16, 1, 128, 16, 16384, 16384, max_ctx=16384),
            "fp8_tok": W.Spec("one_pair_fp8", 1, 4, 16, 1, 128, 1024, 16384, 16384,
                              kv_dtype=W.KV_FP8, kv_scale_mode=W.SCALE_PER_TOKEN_HEAD,
                              max_ctx=16384)}[kv]
    w = W.generate(base, 2026)
    d = upload(w)
    say(f"[fused] one pair over every workgroup {kv}")
    (sep,), _ = _decode(w, d, SEPARATE, 16)
    fused, plan = _decode(w, d, FUSED, 16, reps=2)
    assert int(plan.region("nseg", 1).item()) == plan.c.grid
    assert all(_same(f, sep) for f in fused)
    check(w, fused[0], f"fused one pair {kv}")


def test_fused_with_query_blocks():
    """q_len 20 x 16 rows: two query blocks (16 + 4 queries), each with its own
    counters."""
    spec = W.Spec("long_q_fused", 4, 20, 16, 1, 128, 1024, 20, 1500, kv_dtype=W.KV_FP8,
                  kv_scale_mode=W.SCALE_PER_TENSOR, max_ctx=2048)
    w = W.generate(spec, 2029, context_lens=[20, 21, 700, 1500])
    d = upload(w)
    (sep,), _ = _decode(w, d, SEPARATE, 64)
    fused, plan = _decode(w, d, FUSED, 64, reps=2)
    assert plan.c.q_block < spec.q_len
    assert all(_same(f, sep) for f in fused)
    check(w, fused[0], "fused query blocks")


def test_fused_graph_replay_and_reused_plan():
    """One fused plan and one separate-reduce plan, both at the start lengths:
    the contexts grow by one token per step (the caches hold the grown tokens
    already; 32-token partitions, so some pairs cross a partition boundary),
    and each step decodes on the same plans: the fused one inside a replayed
    graph, the separate one eagerly. Every replay is bitwise the separate
    decode on its plan (different plans split differently, so only the same
    plan's outputs are bitwise equal) and matches the oracle."""
    spec = W.scaled(W.C3, batch=4, ctx_lo=240, ctx_hi=1100, max_ctx=1280)
    final = W.generate(spec, 2039)
    d = upload(final)
    steps = 5
    start = d.context_lens - steps
    ctx = start.clone()
    plan = pa.pa_plan(dims_for(final, 32, 0, FUSED), start.clone())
    plan_s = pa.pa_plan(dims_for(final, 32, 0, SEPARATE), start.clone())
    out = torch.zeros_like(d.q)
    s = spec

    def body():
        ctx.add_(1)
        pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, ctx, 1, s.scale,
                     pa.PA_SCALE_NONE, None, out)

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            body()
    torch.cuda.current_stream().wait_stream(stream)
    ctx.copy_(start)
    for i in range(steps):
        graph.replay()
        torch.cuda.synchronize()
        (want,), _ = _decode(final, d, SEPARATE, plan=plan_s, ctx=ctx.clone())
        torch.cuda.synchronize()
        assert _same(out, want), f"step {i}"
        wi = W.Workload(spec, final.seed, final.q, final.k_cache, final.v_cache,
                        final.block_table, ctx.cpu(), final.kv_scales, final.num_pages)
        check(wi, out, f"fused reused plan, step {i}")
    assert pa.pa_plan_status(plan) == 0 and pa.pa_plan_status(plan_s) == 0


def _tuned_settings():
    vals = sorted({e.value for e in tuning.read_table()})
    return vals or [(1, 256, 0)]


@pytest.mark.parametrize("mult,partition,fused", _tuned_settings())
@pytest.mark.parametrize("name", ["bf16_gqa", "fp8_tok_q4", "d256_q8"])
def test_every_tuned_setting_matches_the_oracle(name, mult, partition, fused):
    w = W.generate(SPECS[name], 2026)
    d = upload(w)
    say(f"[tuned] {name} mult={mult} P={partition} fused={fused}")
    (out,), plan = _decode(w, d, FUSED if fused else SEPARATE, partition, mult)
    assert pa.pa_plan_status(plan) == 0
    check(w, out, f"tuned setting {name} ({mult}, {partition}, {fused})")
