"""Decode steps back to back, captured in a graph.

One decode step of a serving loop: the context lengths grow by q_len on the
device, the new tokens' K/V are appended to the paged cache
(pa_cache_append), the work list is rebuilt from the grown lengths (pa_plan)
and the step decodes (pa_decode). Every call is asynchronous on the caller's
stream and allocates nothing, so the whole step is captured once and
replayed: one step per replay, and several steps unrolled in one graph.

Checks: every replay's output is bitwise equal to the same calls made
eagerly; the cache (bytes and scales) after the last step equals the
oracle's appends bit for bit; each step's output matches the oracle's decode
of that step's cache within the decode tolerance. The loops cross page and
partition boundaries and one starts at a context of q_len tokens.
"""
import numpy as np
import pytest
import torch

import paged_attention_decode_block_amd as pa
import workloads as W
from oracle import cache
from tests.gpu_util import DEV, MODE_CODE, check, dims_for, say, upload

pytestmark = pytest.mark.gpu

STEPS = 4

# (spec, final context lengths); start = final - STEPS * q_len
LOOPS = {
    "bf16_gqa_q1": (W.scaled(W.C3, batch=4, ctx_lo=5, ctx_hi=900, max_ctx=1024),
                    [258, 515, 5, 700]),
    "fp8_tok_q1": (W.scaled(W.C4_Q1_TOK, batch=3, ctx_lo=1026, ctx_hi=2050, max_ctx=3072),
                   [1026, 2050, 1500]),
    "fp8_ten_q4": (W.scaled(W.C4_Q4_TEN, batch=3, ctx_lo=1030, ctx_hi=2060, max_ctx=3072),
                   [1030, 2060, 1800]),
    "d256_q8": (W.scaled(W.C5, batch=2, ctx_lo=300, ctx_hi=520, max_ctx=1024, pool_slack=0.2),
                [300, 520]),
}


class State:
    """Device copies of one loop's mutable state (cache, scales, lengths)."""

    def __init__(self, loop: W.DecodeLoop):
        self.d = upload(loop.start)
        self.status = torch.zeros(1, dtype=torch.int32, device=DEV)

    def reset(self, other: "State") -> None:
        for name in ("k_cache", "v_cache", "context_lens", "kv_scales"):
            dst = getattr(self.d, name)
            if dst is not None:
                dst.copy_(getattr(other.d, name))
        self.status.zero_()


def _step(loop, dims, st: State, ws, q, nk, nv, out):
    s = loop.start.spec
    d = st.d
    d.context_lens.add_(s.q_len)
    pa.pa_cache_append(dims, nk, nv, d.block_table, d.context_lens, d.k_cache, d.v_cache,
                       d.kv_scales, st.status)
    plan = pa.pa_plan(dims, d.context_lens, workspace=ws)
    pa.pa_decode(plan, q, d.k_cache, d.v_cache, d.block_table, d.context_lens, s.q_len, s.scale,
                 MODE_CODE[s.kv_scale_mode], d.kv_scales, out)
    return plan


def _workspace(dims):
    return torch.empty(pa.pa_workspace_bytes(dims, pa.pa_query_device(0)), dtype=torch.uint8,
                       device=DEV)


def _capture(fn):
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            fn()
    torch.cuda.current_stream().wait_stream(stream)
    return graph


def _bits(t: torch.Tensor) -> np.ndarray:
    t = t.cpu()
    return t.view(torch.int16).numpy().view(np.uint16) if t.dtype == torch.bfloat16 else t.numpy()


def _oracle_states(loop: W.DecodeLoop):
    """Cache state after each step's append, by the oracle's rule."""
    s, w = loop.start.spec, loop.start
    fp8 = s.kv_dtype == W.KV_FP8
    per_tok = s.kv_scale_mode == W.SCALE_PER_TOKEN_HEAD
    kc, vc = _bits(w.k_cache), _bits(w.v_cache)
    sc = None if w.kv_scales is None else w.kv_scales.numpy()
    bt = w.block_table.numpy()
    states = []
    for i in range(loop.steps):
        ctx = loop.context_lens_at(i).numpy()
        kc, vc, sc, status = cache.append(_bits(loop.new_k[i]), _bits(loop.new_v[i]), bt, ctx,
                                          s.q_len, s.page_size, kc, vc, fp8, per_tok, sc)
        assert status == 0
        states.append((kc, vc, sc))
    return states


def _as_cache(a: np.ndarray, fp8: bool) -> torch.Tensor:
    return torch.from_numpy(a) if fp8 else torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("name", list(LOOPS))
def test_graph_captured_decode_loop(name):
    spec, final = LOOPS[name]
    loop = W.decode_loop(spec, 2026, STEPS, final)
    s = spec
    say(f"[loop] {name} start ctx={loop.start.context_lens.tolist()} steps={STEPS}")
    dims = dims_for(loop.start)
    q = loop.q.to(DEV)
    nk, nv = loop.new_k.to(DEV), loop.new_v.to(DEV)

    # eager reference
    eager = State(loop)
    ws_e = _workspace(dims)
    outs = torch.zeros(STEPS, *q.shape[1:], dtype=torch.bfloat16, device=DEV)
    for i in range(STEPS):
        plan_e = _step(loop, dims, eager, ws_e, q[i], nk[i], nv[i], outs[i])
    torch.cuda.synchronize()
    assert int(eager.status.item()) == 0 and pa.pa_plan_status(plan_e) == 0

    # one step per replay, inputs copied into static buffers between replays
    g1 = State(loop)
    ws1 = _workspace(dims)
    q_in, nk_in, nv_in = q[0].clone(), nk[0].clone(), nv[0].clone()
    out1 = torch.zeros_like(q[0])
    holder = {}
    graph = _capture(lambda: holder.update(plan=_step(loop, dims, g1, ws1, q_in, nk_in, nv_in,
                                                      out1)))
    for i in range(STEPS):
        q_in.copy_(q[i])
        nk_in.copy_(nk[i])
        nv_in.copy_(nv[i])
        out1.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out1.view(torch.int16), outs[i].view(torch.int16)), f"replay {i}"
    assert int(g1.status.item()) == 0 and pa.pa_plan_status(holder["plan"]) == 0
    for t in ("k_cache", "v_cache", "kv_scales", "context_lens"):
        a, b = getattr(g1.d, t), getattr(eager.d, t)
        if a is not None:
            assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), t

    # all steps unrolled in one graph, replayed twice from the start state
    gs = State(loop)
    start = State(loop)
    ws_s = _workspace(dims)
    out_all = torch.zeros_like(outs)

    def steps():
        for i in range(STEPS):
            _step(loop, dims, gs, ws_s, q[i], nk[i], nv[i], out_all[i])

    graph_all = _capture(steps)
    for rep in range(2):
        gs.reset(start)
        out_all.zero_()
        graph_all.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_all.view(torch.int16), outs.view(torch.int16)), f"unrolled {rep}"
        assert int(gs.status.item()) == 0
        # eager work between replays
        _step(loop, dims, State(loop), _workspace(dims), q[0], nk[0], nv[0], torch.empty_like(q[0]))
        torch.cuda.synchronize()

    # the oracle: cache bytes after the last append, and every step's output
    states = _oracle_states(loop)
    fp8 = s.kv_dtype == W.KV_FP8
    kc, vc, sc = states[-1]
    assert np.array_equal(_bits(eager.d.k_cache), kc) and np.array_equal(_bits(eager.d.v_cache), vc)
    if sc is not None:
        assert np.array_equal(eager.d.kv_scales.cpu().numpy().view(np.uint32), sc.view(np.uint32))
    for i in range(STEPS):
        kc, vc, sc = states[i]
        wi = W.Workload(s, 2026, loop.q[i], _as_cache(kc, fp8), _as_cache(vc, fp8),
                        loop.start.block_table, loop.context_lens_at(i),
                        None if sc is None else torch.from_numpy(sc), loop.start.num_pages)
        check(wi, outs[i], f"{name} step {i}")
    say(f"[loop] {name} ok")


@pytest.mark.parametrize("name", list(LOOPS))
def test_plan_reused_across_steps(name):
    """One plan, built at the loop's start lengths, serves every step: each
    step grows context_lens by q_len, appends its tokens and decodes on the
    same plan, whose pairs' last segments then run to the live lengths
    (across page and partition boundaries: 254 -> 258 at page 16 and
    partition 256, 1022 -> 1026 and 1014 -> 1030 at page and partition 1024,
    488 -> 520 at partition 512). Every step matches the oracle; the same
    steps replayed from one captured graph (no plan inside) are bitwise
    equal to the eager ones."""
    spec, final = LOOPS[name]
    loop = W.decode_loop(spec, 2026, STEPS, final)
    s = spec
    say(f"[reuse] {name} start ctx={loop.start.context_lens.tolist()} steps={STEPS}")
    dims = dims_for(loop.start)
    q = loop.q.to(DEV)
    nk, nv = loop.new_k.to(DEV), loop.new_v.to(DEV)
    mode = MODE_CODE[s.kv_scale_mode]

    def step(st: State, plan, qi, nki, nvi, out):
        d = st.d
        d.context_lens.add_(s.q_len)
        pa.pa_cache_append(dims, nki, nvi, d.block_table, d.context_lens, d.k_cache, d.v_cache,
                           d.kv_scales, st.status)
        pa.pa_decode(plan, qi, d.k_cache, d.v_cache, d.block_table, d.context_lens, s.q_len,
                     s.scale, mode, d.kv_scales, out)

    eager = State(loop)
    plan = pa.pa_plan(dims, eager.d.context_lens.clone(), workspace=_workspace(dims))
    outs = torch.zeros(STEPS, *q.shape[1:], dtype=torch.bfloat16, device=DEV)
    for i in range(STEPS):
        step(eager, plan, q[i], nk[i], nv[i], outs[i])
    torch.cuda.synchronize()
    assert int(eager.status.item()) == 0 and pa.pa_plan_status(plan) == 0

    g = State(loop)
    plan_g = pa.pa_plan(dims, g.d.context_lens.clone(), workspace=_workspace(dims))
    q_in, nk_in, nv_in = q[0].clone(), nk[0].clone(), nv[0].clone()
    out_g = torch.zeros_like(q[0])
    graph = _capture(lambda: step(g, plan_g, q_in, nk_in, nv_in, out_g))
    for i in range(STEPS):
        q_in.copy_(q[i])
        nk_in.copy_(nk[i])
        nv_in.copy_(nv[i])
        out_g.zero_()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g.view(torch.int16), outs[i].view(torch.int16)), f"replay {i}"
    assert pa.pa_plan_status(plan_g) == 0

    states = _oracle_states(loop)
    fp8 = s.kv_dtype == W.KV_FP8
    for i in range(STEPS):
        kc, vc, sc = states[i]
        wi = W.Workload(s, 2026, loop.q[i], _as_cache(kc, fp8), _as_cache(vc, fp8),
                        loop.start.block_table, loop.context_lens_at(i),
                        None if sc is None else torch.from_numpy(sc), loop.start.num_pages)
        check(wi, outs[i], f"{name} reused plan, step {i}")
    say(f"[reuse] {name} ok")


def test_stale_plan_is_reported():
    """Context lengths below the plan's, or past the block table's capacity,
    set PA_DEV_BAD_CONTEXT, and those sequences are decoded over the plan's
    lengths: bitwise the output of a decode at the plan's lengths."""
    spec = W.scaled(W.C3, batch=3, ctx_lo=100, ctx_hi=900, max_ctx=1024)
    w = W.generate(spec, 2039)
    d = upload(w)
    dims = dims_for(w)
    want = torch.empty_like(d.q)
    plan = pa.pa_plan(dims, d.context_lens)
    pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens, 1, spec.scale,
                 pa.PA_SCALE_NONE, None, want)
    assert pa.pa_plan_status(plan) == 0
    cap = spec.max_pages_per_seq * spec.page_size
    for label, change in (("shrunk", lambda c: c - 5), ("past capacity", lambda c: c * 0 + cap + 3)):
        live = d.context_lens.clone()
        live[1] = change(live[1])
        say(f"[reuse] stale plan: {label}, ctx {d.context_lens.tolist()} -> {live.tolist()}")
        plan = pa.pa_plan(dims, d.context_lens)
        out = torch.empty_like(d.q)
        pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, live, 1, spec.scale,
                     pa.PA_SCALE_NONE, None, out)
        assert pa.pa_plan_status(plan) == pa.PA_DEV_BAD_CONTEXT, label
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), label
