"""Decode parity: the HIP path vs the CPU oracle, element by element.

Tolerance |gpu - oracle| <= tol + tol * |oracle| with tol = 8e-3 for bf16 KV
and 2e-2 for fp8 KV (the oracle decodes the same fp8 bytes). Inputs are the
seeded workloads (unused pages and dead slots poisoned with NaN), at sizes
the float64 oracle finishes in seconds but that still span several pages,
partitions and a ragged tail.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from oracle import cache
from tests.gpu_util import DEV, MODE_CODE, check, dims_for, run, say, to_f64, tol, upload
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu

SMALL = {
    # the two same-shape cases of the Ascend issue, full size
    "C1": W.C1,
    "C2": W.C2,
    # reduced versions of the batched / fp8 / long-context workloads
    "C3r": W.scaled(W.C3, batch=6, ctx_lo=1, ctx_hi=900, max_ctx=1024),
    "C4r_q1_tok": W.scaled(W.C4_Q1_TOK, batch=3, ctx_lo=1, ctx_hi=2500, max_ctx=3072),
    "C4r_q4_tok": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=4, ctx_hi=2500, max_ctx=3072),
    "C4r_q1_ten": W.scaled(W.C4_Q1_TEN, batch=3, ctx_lo=1, ctx_hi=2500, max_ctx=3072),
    "C4r_q4_ten": W.scaled(W.C4_Q4_TEN, batch=3, ctx_lo=4, ctx_hi=2500, max_ctx=3072),
    "C5r": W.scaled(W.C5, batch=2, ctx_lo=8, ctx_hi=1500, max_ctx=2048, pool_slack=0.1),
}


@pytest.mark.parametrize("seed", W.SEEDS)
@pytest.mark.parametrize("name", list(SMALL))
def test_decode_parity(name, seed):
    w = W.generate(SMALL[name], seed)
    say(f"[decode] {name} seed={seed} ctx={w.context_lens.tolist()}")
    out, plan = run(w)
    err = check(w, out, f"{name}/{seed}")
    assert pa.pa_plan_status(plan) == 0
    say(f"[decode] {name} seed={seed} max abs err {err:.3e}")


@pytest.mark.parametrize("P", [16, 32, 64, 4096])
def test_partition_sizes(P):
    # P = 16 with many sequences gives more items than workgroups, so segments
    # span several items and pairs split over several workgroups
    spec = W.scaled(W.C3, batch=12, ctx_lo=100, ctx_hi=1500, max_ctx=2048)
    w = W.generate(spec, 2039)
    say(f"[decode] partition {P}")
    out, _ = run(w, partition=P)
    check(w, out, f"P={P}")


@pytest.mark.parametrize("mult", [1, 2, 4])
def test_grid_multiplier(mult):
    spec = W.scaled(W.C4_Q4_TOK, batch=4, ctx_lo=3000, ctx_hi=9000, max_ctx=9216)
    w = W.generate(spec, 2026)
    say(f"[decode] grid multiplier {mult}")
    out, plan = run(w, grid_multiplier=mult)
    assert plan.c.grid == plan.c.num_cus * mult
    check(w, out, f"mult={mult}")


@pytest.mark.parametrize("ps", [16, 32, 64, 128, 256, 512, 1024])
def test_page_sizes(ps):
    spec = W.scaled(W.C3, batch=3, ctx_lo=1, ctx_hi=1100, page_size=ps, max_ctx=2048)
    w = W.generate(spec, 2029)
    say(f"[decode] page size {ps}")
    out, _ = run(w)
    check(w, out, f"ps={ps}")


@pytest.mark.parametrize("q_len,hq,hkv,d", [(1, 8, 8, 128), (2, 8, 2, 128), (3, 16, 1, 128),
                                            (1, 32, 1, 128), (2, 32, 1, 128), (4, 12, 1, 128),
                                            (8, 4, 4, 256), (2, 16, 2, 256), (4, 8, 1, 256),
                                            (3, 10, 1, 256),
                                            # shared-tile instantiations: 65..256 rows at
                                            # head_dim 128, 33..64 at 256, one pass
                                            (5, 16, 1, 128), (8, 16, 1, 128), (12, 16, 1, 128),
                                            (16, 16, 1, 128), (9, 20, 2, 128), (5, 8, 1, 256),
                                            (16, 4, 1, 256)])
def test_row_shapes(q_len, hq, hkv, d):
    # rows per kv head R = q_len * hq / hkv from 1 to 256: one to sixteen 16-row
    # tiles, all in one kernel
    spec = W.Spec(f"rows_{q_len}x{hq}/{hkv}_d{d}", 3, q_len, hq, hkv, d, 32, q_len, 700,
                  max_ctx=1024)
    w = W.generate(spec, 2026)
    say(f"[decode] {spec.name} ctx={w.context_lens.tolist()}")
    out, plan = run(w)
    assert plan.c.q_block == q_len
    check(w, out, spec.name)


@pytest.mark.parametrize("mode", [W.SCALE_PER_TOKEN_HEAD, W.SCALE_PER_TENSOR])
@pytest.mark.parametrize("q_len,hq,hkv", [(8, 16, 16), (1, 16, 1), (2, 16, 1)])
def test_fp8_head_dim_256(q_len, hq, hkv, mode):
    # fp8 KV at head_dim 256: rows per kv head 8, 16 and 32 (one and two
    # 16-row tiles), both scale modes
    spec = W.Spec(f"fp8_d256_{q_len}x{hq}/{hkv}_{mode}", 3, q_len, hq, hkv, 256, 32, q_len, 900,
                  kv_dtype=W.KV_FP8, kv_scale_mode=mode, max_ctx=1024)
    w = W.generate(spec, 2039)
    say(f"[decode] {spec.name} ctx={w.context_lens.tolist()}")
    out, _ = run(w)
    check(w, out, spec.name)


@pytest.mark.parametrize("kv", ["bf16", "fp8_tok", "fp8_ten"])
def test_edge_contexts(kv):
    base = {"bf16": W.scaled(W.C5, batch=6, q_len=4, num_q_heads=8, num_kv_heads=2, head_dim=128),
            "fp8_tok": W.scaled(W.C4_Q4_TOK, batch=6),
            "fp8_ten": W.scaled(W.C4_Q4_TEN, batch=6)}[kv]
    ps = base.page_size
    # minimum (ctx = q_len), a single page, a page + 1, a partition + 1, a
    # multiple of the partition, and the block-table capacity
    cap = -(-max(600, ps + 1) // ps) * ps
    ctxs = [4, ps, ps + 1, 257, 512, cap]
    spec = W.scaled(base, batch=len(ctxs), ctx_lo=min(ctxs), ctx_hi=max(ctxs), max_ctx=cap,
                    pool_slack=0.5)
    w = W.generate(spec, 2026, context_lens=ctxs)
    say(f"[decode] edges {kv} ctx={ctxs}")
    out, plan = run(w)
    check(w, out, f"edges/{kv}")
    assert pa.pa_plan_status(plan) == 0


def test_bad_context_reports_and_writes_nothing():
    spec = W.scaled(W.C3, batch=2, ctx_lo=30, ctx_hi=40, max_ctx=64)
    w = W.generate(spec, 2026)
    w.context_lens[1] = 65                          # past capacity
    out, plan = run(w)
    assert pa.pa_plan_status(plan) == pa.PA_DEV_BAD_CONTEXT


@pytest.mark.parametrize("scale", [-0.2, 0.0, 1.5])
@pytest.mark.parametrize("kv", ["bf16", "fp8_tok", "fp8_ten_q4", "fp8_tok_q4"])
def test_softmax_scales(kv, scale):
    # a negative scale (the max tracks the most negative dot product), zero
    # (uniform weights over the visible keys) and a large one (scores spread
    # over tens of exp2 units, so the lazy rescale moves the running max often).
    # The q_len-4 fp8 kernels share K/V tiles and take their row sums from a
    # PV tile of ones; per-token, from the probabilities before the V scale.
    spec = {"bf16": W.scaled(W.C3, batch=4, ctx_lo=1, ctx_hi=900, max_ctx=1024),
            "fp8_tok": W.scaled(W.C4_Q1_TOK, batch=3, ctx_lo=1, ctx_hi=2500, max_ctx=3072),
            "fp8_ten_q4": W.scaled(W.C4_Q4_TEN, batch=3, ctx_lo=4, ctx_hi=2500, max_ctx=3072),
            "fp8_tok_q4": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=4, ctx_hi=2500, max_ctx=3072)}[kv]
    w = W.generate(spec, 2029)
    say(f"[decode] scale {scale} {kv} ctx={w.context_lens.tolist()}")
    d = upload(w)
    plan = pa.pa_plan(dims_for(w), d.context_lens)
    out = torch.empty_like(d.q)
    pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens, spec.q_len, scale,
                 MODE_CODE[spec.kv_scale_mode], d.kv_scales, out)
    want, _ = oracle.decode(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, spec.q_len,
                            scale, spec.page_size, spec.kv_dtype, spec.kv_scale_mode, w.kv_scales)
    err = assert_close(to_f64(out), want, tol(spec), f"scale {scale} {kv}")
    assert pa.pa_plan_status(plan) == 0
    say(f"[decode] scale {scale} {kv}: max abs err {err:.3e}")


@pytest.mark.parametrize("kv", ["bf16", "fp8_tok"])
def test_pages_beyond_4_gib(kv):
    """A pool larger than 4 GiB per cache with the workload's pages placed
    past the first 4 GiB: byte offsets of K, V and per-token scales exceed
    32 bits. The output equals the oracle's on the compact pool (the result
    does not depend on where pages sit), and an append through the same
    table writes the oracle's bytes at those pages."""
    spec = {"bf16": W.scaled(W.C3, batch=3, ctx_lo=100, ctx_hi=700, max_ctx=1024),
            "fp8_tok": W.scaled(W.C4_Q4_TOK, batch=2, ctx_lo=900, ctx_hi=2500, max_ctx=3072)}[kv]
    w = W.generate(spec, 2026)
    page_bytes = w.k_cache[0].numel() * w.k_cache.element_size()
    base = (1 << 32) // page_bytes + 17                  # first page past 4 GiB
    big = base + w.num_pages
    say(f"[decode] {kv}: {big} pages of {page_bytes} B ({big * page_bytes / 2**30:.1f} GiB per cache)")
    k_big = torch.empty((big,) + tuple(w.k_cache.shape[1:]), dtype=w.k_cache.dtype, device=DEV)
    v_big = torch.empty_like(k_big)
    k_big[base:] = w.k_cache.to(DEV)
    v_big[base:] = w.v_cache.to(DEV)
    sc_big = None
    if w.kv_scales is not None:
        sc_big = torch.empty((2, big) + tuple(w.kv_scales.shape[2:]), dtype=torch.float32, device=DEV)
        sc_big[:, base:] = w.kv_scales.to(DEV)
    bt = torch.where(w.block_table >= 0, w.block_table + base, w.block_table).to(DEV)
    ctx = w.context_lens.to(DEV)
    dims = pa.make_dims(batch=spec.batch, q_len=spec.q_len, num_q_heads=spec.num_q_heads,
                        num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim,
                        page_size=spec.page_size, num_pages=big,
                        max_pages_per_seq=spec.max_pages_per_seq,
                        kv_dtype=dims_for(w).kv_dtype, kv_scale_mode=dims_for(w).kv_scale_mode)
    plan = pa.pa_plan(dims, ctx)
    q = w.q.to(DEV)
    out = torch.empty_like(q)
    pa.pa_decode(plan, q, k_big, v_big, bt, ctx, spec.q_len, spec.scale,
                 MODE_CODE[spec.kv_scale_mode], sc_big, out)
    assert pa.pa_plan_status(plan) == 0
    check(w, out, f"beyond 4 GiB {kv}")
    # the append writes its rows through the same table
    r = np.random.default_rng(4)
    nk = torch.from_numpy(r.standard_normal((spec.batch, spec.q_len, spec.num_kv_heads,
                                             spec.head_dim), dtype=np.float32)).to(torch.bfloat16)
    nv = torch.from_numpy(r.standard_normal(nk.shape, dtype=np.float32)).to(torch.bfloat16)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.pa_cache_append(dims, nk.to(DEV), nv.to(DEV), bt, ctx, k_big, v_big, sc_big, status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    fp8 = spec.kv_dtype == W.KV_FP8
    bf16_bits = lambda t: t.view(torch.int16).numpy().view(np.uint16)
    bits = (lambda t: t.numpy()) if fp8 else bf16_bits
    wk, wv, ws, wst = cache.append(bf16_bits(nk), bf16_bits(nv), w.block_table.numpy(), w.context_lens.numpy(),
                                   spec.q_len, spec.page_size, bits(w.k_cache), bits(w.v_cache), fp8,
                                   spec.kv_scale_mode == W.SCALE_PER_TOKEN_HEAD,
                                   None if w.kv_scales is None else w.kv_scales.numpy())
    assert wst == 0
    assert np.array_equal(bits(k_big[base:].cpu()), wk) and np.array_equal(bits(v_big[base:].cpu()), wv)
    if ws is not None:
        assert np.array_equal(sc_big[:, base:].cpu().numpy().view(np.uint32), ws.view(np.uint32))


LONG_Q = {
    # name: (q_len, Hq, Hkv, D, kv dtype, scale mode); rows = q_len * Hq / Hkv. Up to
    # 256 rows (64 at head_dim 256) one kernel reads each chunk once for all of
    # them; past that the queries go in blocks.
    "q5_g16_d128": (5, 16, 1, 128, W.KV_BF16, W.SCALE_NONE),           # 80 rows: one pass
    "q24_g8_d128": (24, 8, 1, 128, W.KV_BF16, W.SCALE_NONE),           # 192 rows: one pass
    "q40_g1_d256": (40, 4, 4, 256, W.KV_BF16, W.SCALE_NONE),           # 40 rows: one pass
    "q8_g16_fp8_tok": (8, 16, 1, 128, W.KV_FP8, W.SCALE_PER_TOKEN_HEAD),  # 128 rows: one pass
    "q9_g16_fp8_ten": (9, 16, 1, 128, W.KV_FP8, W.SCALE_PER_TENSOR),      # 144 rows: one pass
    "q20_g16_d128": (20, 16, 1, 128, W.KV_BF16, W.SCALE_NONE),         # 320 rows: 16 + 4 queries
    "q33_g8_fp8_tok": (33, 8, 1, 128, W.KV_FP8, W.SCALE_PER_TOKEN_HEAD),  # 264 rows: 32 + 1
    "q40_g4_d256": (40, 8, 2, 256, W.KV_BF16, W.SCALE_NONE),           # 160 rows: 4 blocks of 16 + 8
}


@pytest.mark.parametrize("name", list(LONG_Q))
def test_long_queries(name):
    """Many query rows per kv head (chunked prefill of q_len tokens): one
    kernel serves up to 256 rows (64 at head_dim 256), its waves sharing each
    K/V chunk through LDS; past that the queries are decoded in blocks, each
    with the keys up to its own last query. Contexts include the shortest,
    ctx = q_len."""
    q_len, hq, hkv, d, kvd, mode = LONG_Q[name]
    ps = 1024 if kvd == W.KV_FP8 else 32
    spec = W.Spec(name, 4, q_len, hq, hkv, d, ps, q_len, 1500, kv_dtype=kvd, kv_scale_mode=mode,
                  max_ctx=2048)
    ctxs = [q_len, q_len + 1, 700, 1500]
    w = W.generate(spec, 2029, context_lens=ctxs)
    rows = q_len * hq // hkv
    say(f"[decode] long q {name} ({rows} rows) ctx={ctxs}")
    out, plan = run(w)
    fits = rows <= (256 if d == 128 else 64)
    assert (plan.c.q_block == q_len) == fits, (plan.c.q_block, q_len)
    assert pa.pa_plan_status(plan) == 0
    check(w, out, name)


def test_long_queries_past_the_plan_lds_tables():
    """Query blocks over a batch whose plan tables do not fit in LDS (more
    than 8192 sequences): each block's work list comes from the table kernel
    and the items kernel. A sample of sequences is compared with the oracle."""
    spec = W.Spec("long_q_8200", 8200, 20, 16, 1, 128, 32, 20, 64, max_ctx=64, pool_slack=0.0)
    w = W.generate(spec, 2039)
    say(f"[decode] long q, {spec.batch} sequences, {int(w.context_lens.sum())} tokens")
    out, plan = run(w)
    assert plan.c.q_block < spec.q_len
    assert pa.pa_plan_status(plan) == 0
    got = to_f64(out)
    assert np.isfinite(got).all()
    ctx = w.context_lens.tolist()
    for b in sorted({0, 1, 4095, 4096, 8191, 8192, spec.batch - 1, int(np.argmin(ctx)),
                     int(np.argmax(ctx))}):
        want, _ = oracle.decode(w.q[b:b + 1], w.k_cache, w.v_cache, w.block_table[b:b + 1],
                                w.context_lens[b:b + 1], spec.q_len, spec.scale, spec.page_size,
                                spec.kv_dtype, spec.kv_scale_mode, w.kv_scales)
        assert_close(got[b:b + 1], want, tol(spec), f"long q sequence {b}")


def test_long_queries_bad_context_reports():
    spec = W.Spec("long_q_bad", 2, 20, 16, 1, 128, 32, 20, 300, max_ctx=512)
    w = W.generate(spec, 2026, context_lens=[20, 300])
    w.context_lens[0] = 19                           # shorter than q_len
    out, plan = run(w)
    assert plan.c.q_block < spec.q_len
    assert pa.pa_plan_status(plan) == pa.PA_DEV_BAD_CONTEXT


@pytest.mark.parametrize("P", [16, 256])
@pytest.mark.parametrize("kv", ["bf16", "fp8_tok"])
def test_one_sequence_over_every_workgroup(kv, P):
    """One long sequence and one kv head: its pair is split over every
    workgroup (P = 16: 1024 items, four per workgroup, 256 segments; P = 256:
    64 single-item segments), so the reduce merges that many partials."""
    base = {"bf16": W.Spec("one_pair_bf16", 1, 4, 16, 1, 128, 16, 16384, 16384, max_ctx=16384),
            "fp8_tok": W.Spec("one_pair_fp8", 1, 4, 16, 1, 128, 1024, 16384, 16384, kv_dtype=W.KV_FP8,
                              kv_scale_mode=W.SCALE_PER_TOKEN_HEAD, max_ctx=16384)}[kv]
    w = W.generate(base, 2026)
    say(f"[decode] one pair over every workgroup {kv} P={P}")
    out, plan = run(w, partition=P)
    assert pa.pa_plan_status(plan) == 0
    check(w, out, f"one pair {kv} P={P}")
