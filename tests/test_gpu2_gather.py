"""The decode's own page loader reads exactly the cache rows the block table
names (bitwise).

pa_debug_gather runs the partition pass's loader (block-table entries, then
16-byte buffer loads sized to a segment's live rows) of the plan's own
decode instantiation over every chunk of every segment, and writes the
registers back out in the order the math reads them. Every row of every
pair must equal the oracle's gather of the same cache byte for byte, every
per-token scale bit for bit, and every row a chunk holds past its segment's
end must load as zeros (else PA_DEV_DEBUG_DEAD_ROW).

Cases choose the loader variants by their shapes: per-block entries (page
16, chunks of two blocks spanning two pages) and one page per chunk (pages
of 128 and 1024), bf16 and fp8 with both scale modes, head_dim 128 and 256,
the shared-tile loader of 64-row fp8 pairs, partitions of 16 tokens (a
segment ends inside a 32-token chunk, so a whole block is dead), ragged
context ends, and contexts grown after the plan was built.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import DEV, dims_for, say, upload

pytestmark = pytest.mark.gpu

# name: (spec, partition or None)
CASES = {
    # per-block entries: page 16 < a 32-token chunk
    "bf16 D128 page 16": (W.scaled(W.C3, batch=5, ctx_lo=1, ctx_hi=300, max_ctx=512), None),
    "bf16 D128 page 16, partition 16": (W.scaled(W.C3, batch=3, ctx_lo=1, ctx_hi=200,
                                                 max_ctx=256), 16),
    # one page per chunk
    "bf16 D128 page 128": (W.scaled(W.C2, batch=3, ctx_lo=1, ctx_hi=600, max_ctx=640,
                                    pool_pages=0, pool_slack=0.3), None),
    "fp8 per-token q1 page 1024": (W.scaled(W.C4_Q1_TOK, batch=3, ctx_lo=4, ctx_hi=2500,
                                            max_ctx=3072), None),
    "fp8 per-tensor q1 page 16": (W.scaled(W.C4_Q1_TEN, batch=4, page_size=16, ctx_lo=1,
                                           ctx_hi=700, max_ctx=768), None),
    # shared tiles (64-row fp8 pairs): one wave loads K, the other V
    "fp8 per-token q4 page 1024 shared": (W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=4, ctx_hi=2500,
                                                   max_ctx=3072), None),
    "fp8 per-tensor q4 page 16 shared": (W.scaled(W.C4_Q4_TEN, batch=3, page_size=16, ctx_lo=4,
                                                  ctx_hi=700, max_ctx=768), None),
    "fp8 per-token q4 page 32 partition 48": (W.scaled(W.C4_Q4_TOK, batch=3, page_size=32,
                                                       ctx_lo=4, ctx_hi=500, max_ctx=512), 48),
    # shared tiles for long queries: 4 or 8 waves share each chunk (bf16 and fp8)
    "bf16 D128 page 16, 128 rows shared": (W.scaled(W.C3, batch=3, q_len=32, ctx_lo=32,
                                                    ctx_hi=400, max_ctx=512), None),
    "bf16 D128 page 128, 256 rows shared": (W.scaled(W.C2, batch=3, q_len=16, ctx_lo=16,
                                                     ctx_hi=600, max_ctx=640, pool_pages=0,
                                                     pool_slack=0.3), None),
    "fp8 per-token q16 page 1024, 256 rows shared": (W.scaled(W.C4_Q4_TOK, batch=2, q_len=16,
                                                              ctx_lo=16, ctx_hi=2500,
                                                              max_ctx=3072), None),
    "bf16 D256 page 32, 64 rows shared": (W.scaled(W.C5, batch=2, q_len=4, ctx_lo=8, ctx_hi=700,
                                                   max_ctx=1024, pool_slack=0.2), None),
    # head_dim 256
    "bf16 D256 page 32": (W.scaled(W.C5, batch=2, ctx_lo=8, ctx_hi=700, max_ctx=1024,
                                   pool_slack=0.2), None),
    "fp8 per-token D256 page 32": (W.scaled(W.C5, batch=2, ctx_lo=8, ctx_hi=700, max_ctx=1024,
                                            pool_slack=0.2, kv_dtype=W.KV_FP8,
                                            kv_scale_mode=W.SCALE_PER_TOKEN_HEAD), None),
}


def _bytes(cache: torch.Tensor) -> torch.Tensor:
    """[pages, Hkv, ps, D] cache -> [pages, Hkv, ps, row bytes] uint8 (CPU)."""
    c = cache.cpu().contiguous()
    return c.view(torch.uint8).view(*c.shape[:3], c.shape[3] * c.element_size())


def _gather(w: W.Workload, d, ctx_dev, partition=None):
    s = w.spec
    plan = pa.pa_plan(dims_for(w, partition), d.context_lens)
    cap = s.max_pages_per_seq * s.page_size
    pairs = s.batch * s.num_kv_heads
    k_out = torch.zeros(pairs, cap, s.head_dim, dtype=d.k_cache.dtype, device=DEV)
    v_out = torch.zeros_like(k_out)
    per_tok = s.kv_scale_mode == W.SCALE_PER_TOKEN_HEAD
    s_out = torch.zeros(2, pairs, cap, dtype=torch.float32, device=DEV) if per_tok else None
    pa.pa_debug_gather(plan, d.k_cache, d.v_cache, d.block_table, ctx_dev, k_out, v_out,
                       kv_scales=d.kv_scales, scales_out=s_out)
    status = pa.pa_plan_status(plan)
    return status, k_out, v_out, s_out


def _compare(w: W.Workload, ctxs, k_out, v_out, s_out, what):
    s = w.spec
    kb, vb = _bytes(w.k_cache), _bytes(w.v_cache)
    ko = k_out.cpu().view(torch.uint8).numpy()
    vo = v_out.cpu().view(torch.uint8).numpy()
    so = None if s_out is None else s_out.cpu().numpy().view(np.uint32)
    for b in range(s.batch):
        c = int(ctxs[b])
        for g in range(s.num_kv_heads):
            p = b * s.num_kv_heads + g
            np.testing.assert_array_equal(
                ko[p, :c], oracle.gather_rows(kb, w.block_table, b, g, c, s.page_size),
                err_msg=f"{what}: K rows of pair {p}")
            np.testing.assert_array_equal(
                vo[p, :c], oracle.gather_rows(vb, w.block_table, b, g, c, s.page_size),
                err_msg=f"{what}: V rows of pair {p}")
            assert (ko[p, c:] == 0).all() and (vo[p, c:] == 0).all(), f"{what}: rows past ctx"
            if so is not None:
                for which in (0, 1):
                    sc = w.kv_scales[which].numpy()[..., None]
                    want = oracle.gather_rows(sc, w.block_table, b, g, c, s.page_size)[:, 0]
                    np.testing.assert_array_equal(so[which, p, :c], want.view(np.uint32),
                                                  err_msg=f"{what}: scales {which} pair {p}")
                    assert (so[which, p, c:] == 0).all()


@pytest.mark.parametrize("name", sorted(CASES))
def test_loader_bitwise(name):
    spec, partition = CASES[name]
    w = W.generate(spec, 2026)
    say(f"[gather] {name} ctx={w.context_lens.tolist()} partition={partition}")
    d = upload(w)
    status, k_out, v_out, s_out = _gather(w, d, d.context_lens, partition)
    assert status == 0, f"device status {status}"
    _compare(w, w.context_lens.tolist(), k_out, v_out, s_out, name)


def _random_spec(i):
    import random
    r = random.Random(8100 + i)
    hkv = r.choice([1, 2, 4, 8])
    group = r.choice([1, 2, 4, 8, 16])
    q_len = r.choice([1, 1, 2, 4, 8])
    ps = r.choice([16, 32, 64, 128, 256, 512, 1024])
    fp8 = r.random() < 0.5
    mode = r.choice([W.SCALE_PER_TOKEN_HEAD, W.SCALE_PER_TENSOR]) if fp8 else W.SCALE_NONE
    batch = r.randint(1, 5)
    cap = max(r.randint(1, max(1, 3072 // ps)) * ps, q_len)
    ctx = [r.choice([q_len, cap, r.randint(q_len, cap)]) for _ in range(batch)]
    spec = W.Spec(f"loader_rand{i}", batch, q_len, hkv * group, hkv, r.choice([128, 256]), ps,
                  min(ctx), max(ctx), kv_dtype=W.KV_FP8 if fp8 else W.KV_BF16,
                  kv_scale_mode=mode, max_ctx=cap)
    return spec, ctx, r.choice([16, 32, 48, 64, 256, 1024])


@pytest.mark.parametrize("i", range(32))
def test_loader_random_shapes_bitwise(i):
    """Seeded random shapes (kv heads, group, q_len, head_dim, page size,
    capacity, dtype and scale mode, partition size drawn together): whichever
    instantiation the decode picks, its loader reads exactly the oracle's
    rows and scales."""
    spec, ctx, partition = _random_spec(i)
    w = W.generate(spec, 4100 + i, context_lens=ctx)
    say(f"[gather random {i}] B={spec.batch} q_len={spec.q_len} Hq={spec.num_q_heads} "
        f"Hkv={spec.num_kv_heads} D={spec.head_dim} page={spec.page_size} {spec.kv_dtype}/"
        f"{spec.kv_scale_mode} cap={spec.max_ctx} ctx={ctx} P={partition}")
    d = upload(w)
    status, k_out, v_out, s_out = _gather(w, d, d.context_lens, partition)
    assert status == 0, f"device status {status}"
    _compare(w, ctx, k_out, v_out, s_out, f"random case {i}")


@pytest.mark.parametrize("name", ["bf16 D128 page 16", "fp8 per-token q1 page 1024",
                                  "fp8 per-token q4 page 1024 shared"])
def test_loader_reads_live_context_lengths(name):
    """A plan built at shorter contexts; the loader (like the decode) runs each
    pair's last segment to the live length, across page and partition
    boundaries."""
    spec, partition = CASES[name]
    grow = 37 * spec.q_len
    w_final = W.generate(spec, 2029)
    final = w_final.context_lens.clone()
    start = torch.clamp(final - grow, min=spec.q_len)
    w = W.Workload(spec, 2029, w_final.q, w_final.k_cache, w_final.v_cache, w_final.block_table,
                   start, w_final.kv_scales, w_final.num_pages)
    say(f"[gather] {name}: plan at {start.tolist()}, live {final.tolist()}")
    d = upload(w)
    plan_ctx = d.context_lens.clone()
    live = final.to(torch.int32).to(DEV)
    s = w.spec
    plan = pa.pa_plan(dims_for(w, partition), plan_ctx)
    cap = s.max_pages_per_seq * s.page_size
    pairs = s.batch * s.num_kv_heads
    k_out = torch.zeros(pairs, cap, s.head_dim, dtype=d.k_cache.dtype, device=DEV)
    v_out = torch.zeros_like(k_out)
    per_tok = s.kv_scale_mode == W.SCALE_PER_TOKEN_HEAD
    s_out = torch.zeros(2, pairs, cap, dtype=torch.float32, device=DEV) if per_tok else None
    pa.pa_debug_gather(plan, d.k_cache, d.v_cache, d.block_table, live, k_out, v_out,
                       kv_scales=d.kv_scales, scales_out=s_out)
    assert pa.pa_plan_status(plan) == 0
    _compare(w, final.tolist(), k_out, v_out, s_out, f"{name} grown")


def test_debug_bounds_flags_bad_page():
    spec = W.scaled(W.C3, batch=2, ctx_lo=40, ctx_hi=60, max_ctx=64)
    w = W.generate(spec, 2029)
    w.block_table[1, 1] = w.num_pages + 5          # out of range on purpose
    d = upload(w)
    plan = pa.pa_plan(dims_for(w, flags=pa.PA_FLAG_DEBUG_BOUNDS), d.context_lens)
    cap = spec.max_pages_per_seq * spec.page_size
    k_out = torch.zeros(spec.batch * spec.num_kv_heads, cap, spec.head_dim, dtype=torch.bfloat16,
                        device=DEV)
    v_out = torch.zeros_like(k_out)
    pa.pa_debug_gather(plan, d.k_cache, d.v_cache, d.block_table, d.context_lens, k_out, v_out)
    st = pa.pa_plan_status(plan)
    assert st & pa.PA_DEV_BAD_PAGE and not st & pa.PA_DEV_DEBUG_DEAD_ROW
    # tokens of the bad page load as zeros; the others are the cache's rows
    bad = slice(spec.page_size, 2 * spec.page_size)
    ko = k_out.cpu().view(torch.int16)
    for g in range(spec.num_kv_heads):
        assert (ko[spec.num_kv_heads + g, bad] == 0).all()
    # the decode kernel checks the same way and reads such tokens as zeros
    plan = pa.pa_plan(dims_for(w, flags=pa.PA_FLAG_DEBUG_BOUNDS), d.context_lens)
    out = torch.empty_like(d.q)
    pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens, 1, spec.scale,
                 pa.PA_SCALE_NONE, None, out)
    assert pa.pa_plan_status(plan) & pa.PA_DEV_BAD_PAGE
    assert torch.isfinite(out.float()).all()
