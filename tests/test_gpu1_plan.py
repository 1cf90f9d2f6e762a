"""pa_plan's work list on the GPU equals the oracle's rule bit for bit."""
import random

import pytest
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import DEV, plan_arrays, say

pytestmark = pytest.mark.gpu


def _plan_case(ctxs, Hkv, P, q_len, ps, maxp, mult=0, name=""):
    say(f"[plan] {name} B={len(ctxs)} Hkv={Hkv} P={P} q_len={q_len} ps={ps} maxp={maxp} mult={mult}")
    dims = pa.make_dims(batch=len(ctxs), q_len=q_len, num_q_heads=Hkv, num_kv_heads=Hkv,
                        head_dim=128, page_size=ps, num_pages=1, max_pages_per_seq=maxp,
                        partition_size=P, grid_multiplier=mult)
    ctx = torch.tensor(ctxs, dtype=torch.int32, device=DEV)
    plan = pa.pa_plan(dims, ctx)
    got = plan_arrays(plan, len(ctxs))
    want = oracle.plan(ctxs, Hkv, P, plan.c.grid, q_len, ps, maxp)
    assert got["status"] == want.status
    assert got["num_items"] == want.num_items
    assert got["wg_begin"] == want.wg_begin
    assert got["nseg"] == want.nseg
    assert got["seg_base"] == want.seg_base
    assert got["items"] == [tuple(i) for i in want.items]
    assert got["num_segs"] == len(want.segs)
    assert got["segs"] == [tuple(s) for s in want.segs]
    assert got["wg_seg_begin"] == want.wg_seg_begin
    assert got["pseg_base"] == want.pseg_base
    assert got["batch_base"] == want.batch_base
    # the decode's records: each segment with its sequence, kv head and
    # context length; each workgroup's segment range and first record
    want_info = [(p // Hkv, p % Hkv, t0, t1, slot, ctxs[p // Hkv], p, 0)
                 for p, t0, t1, slot in want.segs]
    assert got["seg_info"] == want_info
    G = plan.c.grid
    for w in range(G):
        s0, s1 = want.wg_seg_begin[w], want.wg_seg_begin[w + 1]
        head = got["wg_head"][w]
        if want.status:
            assert head == (0,) * 16
            continue
        assert (head[0], head[8]) == (s0, s1), f"workgroup {w}"
        if s0 < s1:
            assert head[1:8] == want_info[s0][:7], f"workgroup {w}"
        assert head[9:] == (0,) * 7
    assert pa.pa_plan_status(plan) == want.status


@pytest.mark.parametrize("seed", range(24))
def test_plan_random(seed):
    r = random.Random(1000 + seed)
    B = r.randint(1, 70)
    Hkv = r.choice([1, 2, 8, 16])
    P = r.choice([16, 32, 256, 1024])
    q_len = r.choice([1, 4, 8])
    ps = r.choice([16, 32, 1024])
    maxp = r.randint(1, 64)
    ctxs = [r.randint(q_len, maxp * ps) for _ in range(B)]
    _plan_case(ctxs, Hkv, P, q_len, ps, maxp, mult=r.choice([0, 1, 2, 4]), name=f"seed{seed}")


@pytest.mark.parametrize("name", sorted(W.CONFIGS))
def test_plan_configs(name):
    s = W.CONFIGS[name]
    for seed in W.SEEDS:
        ctxs = [int(c) for c in W.draw_context_lens(s, seed)]
        _plan_case(ctxs, s.num_kv_heads, s.partition_size, s.q_len, s.page_size,
                   s.max_pages_per_seq, name=f"{name}/{seed}")


def test_plan_tables_past_lds():
    # more sequences (8192) or pairs (16336) than the plan kernel keeps in LDS:
    # the tables live in the workspace and one workgroup builds the list
    r = random.Random(7)
    _plan_case([r.randint(1, 64) for _ in range(8193)], 1, 16, 1, 16, 4, name="8193 sequences")
    _plan_case([r.randint(1, 64) for _ in range(2043)], 8, 16, 1, 16, 4, name="16344 pairs")


def test_plan_many_pairs_in_lds():
    # the larger LDS tables (up to 8192 sequences and 16336 pairs; context
    # lengths reread, segment counts recomputed; up to 256 workgroups writing
    # the list) and a batch of 1024 sequences x 8 kv heads
    r = random.Random(8)
    _plan_case([r.randint(1, 64) for _ in range(2042)], 8, 16, 1, 16, 4, name="16336 pairs")
    _plan_case([r.randint(1, 64) for _ in range(8192)], 1, 16, 1, 16, 4, name="8192 sequences")
    _plan_case([r.randint(1, 64) for _ in range(5000)], 2, 16, 4, 16, 4, name="5000 sequences, q_len 4")
    _plan_case([r.randint(1, 300) for _ in range(600)], 8, 32, 1, 16, 20, name="4800 pairs")
    _plan_case([r.randint(512, 8192) for _ in range(1024)], 8, 256, 1, 16, 512,
               name="1024 sequences x 8 kv heads")


def test_plan_edges():
    _plan_case([1], 1, 256, 1, 16, 1, name="one token")
    _plan_case([16] * 300, 1, 16, 1, 16, 1, name="one item per pair, N > G")
    _plan_case([4096], 1, 16, 1, 1024, 4, name="one pair over every workgroup")
    _plan_case([1024 * 4] * 3, 4, 1024, 8, 1024, 4, name="full capacity")
    _plan_case([5, 3], 1, 256, 4, 16, 1, name="bad context (3 < q_len 4)")
    _plan_case([17], 1, 256, 1, 16, 1, name="bad context (past capacity)")
