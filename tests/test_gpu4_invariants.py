"""Invariants of the GPU path, and the split-KV partials themselves."""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import DEV, MODE_CODE, Dev, check, dims_for, run, say, tol, to_f64, upload
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu

SPECS = {
    "bf16": W.scaled(W.C3, batch=5, ctx_lo=100, ctx_hi=1200, max_ctx=1280),
    "fp8_tok_q4": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=300, ctx_hi=3000, max_ctx=3072),
    "d256_q8": W.scaled(W.C5, batch=2, ctx_lo=300, ctx_hi=1500, max_ctx=1536, pool_slack=0.2),
}


def _repage(w: W.Workload, seed: int) -> W.Workload:
    """Same logical cache, pages moved to other physical slots."""
    perm = torch.from_numpy(np.random.default_rng(seed).permutation(w.num_pages)).long()
    k = torch.empty_like(w.k_cache)
    v = torch.empty_like(w.v_cache)
    k[perm] = w.k_cache
    v[perm] = w.v_cache
    sc = w.kv_scales
    if sc is not None and sc.dim() == 4:
        sc = torch.empty_like(w.kv_scales)
        sc[:, perm] = w.kv_scales
    bt = torch.where(w.block_table >= 0, perm[w.block_table.clamp(min=0).long()].int(),
                     w.block_table)
    return W.Workload(w.spec, w.seed, w.q, k, v, bt, w.context_lens, sc, w.num_pages)


@pytest.mark.parametrize("name", sorted(SPECS))
def test_page_placement_is_bitwise_invariant(name):
    w = W.generate(SPECS[name], 2029)
    say(f"[inv] placement {name}")
    a, _ = run(w)
    b, _ = run(_repage(w, 7))
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("name", sorted(SPECS))
def test_repeat_and_graph_replay_are_bitwise_equal(name):
    w = W.generate(SPECS[name], 2039)
    say(f"[inv] determinism + graph {name}")
    d = upload(w)
    ref, _ = run(w, d)
    again, _ = run(w, d)
    assert torch.equal(ref.view(torch.int16), again.view(torch.int16))

    s = w.spec
    dims = dims_for(w)
    ws = torch.empty(pa.pa_workspace_bytes(dims, pa.pa_query_device(0)), dtype=torch.uint8,
                     device=DEV)
    out = torch.zeros_like(d.q)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            plan = pa.pa_plan(dims, d.context_lens, workspace=ws)
            pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens, s.q_len,
                         s.scale, MODE_CODE[s.kv_scale_mode], d.kv_scales, out)
    torch.cuda.current_stream().wait_stream(stream)
    for rep in range(3):
        out.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        # eager work between replays
        run(w, d)
        torch.cuda.synchronize()


def test_constant_values_return_the_constant():
    spec = SPECS["bf16"]
    w = W.generate(spec, 2026)
    w.v_cache.fill_(0.8125)
    out, _ = run(w)
    got = to_f64(out)
    assert np.abs(got - 0.8125).max() <= 8e-3 * 0.8125 + 1e-6


@pytest.mark.parametrize("name", ["fp8_tok_q4", "d256_q8"])
def test_causal_equals_sequential_single_token_decode(name):
    spec = SPECS[name]
    w = W.generate(spec, 2026)
    say(f"[inv] causal vs sequential {name}")
    d = upload(w)
    full, _ = run(w, d)
    full = to_f64(full)
    s1 = W.scaled(spec, q_len=1)
    for i in range(spec.q_len):
        ctx_i = w.context_lens - spec.q_len + i + 1
        wi = W.Workload(s1, w.seed, w.q[:, i:i + 1].contiguous(), w.k_cache, w.v_cache,
                        w.block_table, ctx_i, w.kv_scales, w.num_pages)
        di = Dev(wi.q.to(DEV), d.k_cache, d.v_cache, d.block_table, ctx_i.to(DEV), d.kv_scales)
        step, _ = run(wi, di)
        assert_close(full[:, i], to_f64(step)[:, 0], 2 * tol(spec), f"{name} query {i}")


@pytest.mark.parametrize("name", sorted(SPECS))
def test_split_partials_match_oracle_ranges(name):
    """Each split segment's partial O and log-sum-exp equal the oracle's
    attention over that segment's token range; unsplit pairs' rows equal the
    oracle's output."""
    spec = SPECS[name]
    w = W.generate(spec, 2026)
    d = upload(w)
    plan = pa.pa_plan(dims_for(w, partition=64), d.context_lens)
    out = torch.zeros_like(d.q)
    s = spec
    pa.pa_decode_partition(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens,
                           s.q_len, s.scale, MODE_CODE[s.kv_scale_mode], d.kv_scales, out)
    torch.cuda.synchronize()
    S = int(plan.region("status", 4)[2])
    segs = plan.region("segs", 4 * S).view(-1, 4).cpu().tolist()
    nseg = plan.region("nseg", plan.c.num_pairs).cpu().tolist()
    R, D = plan.c.rows, s.head_dim
    slots = max(sg[3] for sg in segs) + 1 if any(sg[3] >= 0 for sg in segs) else 0
    po = plan.region("partial_o", slots * R * D, torch.float32).view(slots, R, D).cpu().numpy()
    pl = plan.region("partial_lse", slots * R, torch.float32).view(slots, R).cpu().numpy()
    say(f"[inv] partials {name}: {S} segments, {slots} slots")
    want_full = None
    checked = 0
    for pair, t0, t1, slot in segs:
        b, g = divmod(pair, s.num_kv_heads)
        if slot < 0:
            assert nseg[pair] == 1
            if want_full is None:
                want_full = oracle.decode(w.q, w.k_cache, w.v_cache, w.block_table,
                                          w.context_lens, s.q_len, s.scale, s.page_size,
                                          s.kv_dtype, s.kv_scale_mode, w.kv_scales)[0]
            grp = s.group
            got = to_f64(out)[b, :, g * grp:(g + 1) * grp].reshape(R, D)
            assert_close(got, want_full[b, :, g * grp:(g + 1) * grp].reshape(R, D), tol(s))
            continue
        o, lse = oracle.attend_range(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens,
                                     s.q_len, s.scale, s.page_size, b, g, t0, t1, s.kv_dtype,
                                     s.kv_scale_mode, w.kv_scales)
        fin = np.isfinite(lse)
        assert (np.isfinite(pl[slot]) == fin).all(), "empty rows must have lse = -inf"
        assert_close(po[slot][fin], o[fin], tol(s), f"partial O slot {slot}")
        assert_close(pl[slot][fin], lse[fin], tol(s), f"partial lse slot {slot}")
        assert (po[slot][~fin] == 0).all()
        checked += 1
    assert checked > 0


@pytest.mark.parametrize("name", ["bf16", "fp8_tok_q4"])
def test_page_size_does_not_change_output_bitwise(name):
    """The same logical cache in 16-token pages (a chunk spans pages: one
    block-table entry per 16-token block) and in 64-token pages (a chunk lies
    in one page: one entry and one descriptor per chunk) gives bit-identical
    output: the addressing changes, the arithmetic does not."""
    spec16 = W.scaled(SPECS[name], page_size=16)
    spec64 = W.scaled(SPECS[name], page_size=64)
    w16 = W.generate(spec16, 2031)
    w64 = _same_cache(w16, spec64)
    say(f"[inv] page size 16 vs 64 {name}")
    a, _ = run(w16)
    b, _ = run(w64)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    check(w64, b, f"{name} page 64")


def _same_cache(w: W.Workload, spec: W.Spec) -> W.Workload:
    """w's logical K/V (and scales) re-laid out in pages of spec.page_size, in
    order: sequence b's pages come one after another."""
    ps0, ps = w.spec.page_size, spec.page_size
    B, Hkv, D = w.spec.batch, w.spec.num_kv_heads, w.spec.head_dim
    ctx = w.context_lens.tolist()
    pages = [-(-c // ps) for c in ctx]
    npool = sum(pages)
    k = torch.zeros((npool, Hkv, ps, D), dtype=w.k_cache.dtype)
    v = torch.zeros_like(k)
    per_tok = w.kv_scales is not None and w.kv_scales.dim() == 4
    sc = torch.zeros((2, npool, Hkv, ps), dtype=torch.float32) if per_tok else w.kv_scales
    maxp = spec.max_pages_per_seq
    bt = torch.full((B, maxp), -1, dtype=torch.int32)
    nxt = 0
    for b in range(B):
        for pg in range(pages[b]):
            bt[b, pg] = nxt + pg
        for t in range(ctx[b]):
            src = int(w.block_table[b, t // ps0])
            dst = nxt + t // ps
            k[dst, :, t % ps] = w.k_cache[src, :, t % ps0]
            v[dst, :, t % ps] = w.v_cache[src, :, t % ps0]
            if per_tok:
                sc[:, dst, :, t % ps] = w.kv_scales[:, src, :, t % ps0]
        nxt += pages[b]
    return W.Workload(spec, w.seed, w.q, k, v, bt, w.context_lens, sc, npool)


def test_decodes_on_concurrent_streams_match_sequential_ones():
    """Plans and decodes of three workloads issued on three streams at once,
    each with its own workspace and output, several rounds without a sync in
    between: every output is bitwise the one the same call gives alone on
    the default stream. (The library keeps no state between calls but the
    caller's workspaces, so nothing may leak across streams.)"""
    names = sorted(SPECS)
    ws_, ds, refs = {}, {}, {}
    for name in names:
        w = W.generate(SPECS[name], 2039)
        d = upload(w)
        ref, _ = run(w, d)
        ws_[name], ds[name], refs[name] = w, d, ref
    torch.cuda.synchronize()
    streams = {name: torch.cuda.Stream() for name in names}
    outs = {name: [] for name in names}
    say("[inv] three streams at once")
    for st in streams.values():
        st.wait_stream(torch.cuda.current_stream())
    for rnd in range(4):
        for name in names:
            w, d, s = ws_[name], ds[name], ws_[name].spec
            with torch.cuda.stream(streams[name]):
                plan = pa.pa_plan(dims_for(w), d.context_lens, stream=streams[name])
                out = torch.full_like(d.q, float("nan"))
                pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens,
                             s.q_len, s.scale, MODE_CODE[s.kv_scale_mode], d.kv_scales, out,
                             stream=streams[name])
                outs[name].append((out, plan))
    torch.cuda.synchronize()
    for name in names:
        for rnd, (out, plan) in enumerate(outs[name]):
            assert pa.pa_plan_status(plan) == 0
            assert torch.equal(out.view(torch.int16), refs[name].view(torch.int16)), \
                f"{name}, round {rnd}"
