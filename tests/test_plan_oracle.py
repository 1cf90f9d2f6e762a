"""Pins of the oracle's work-list rule by closed forms and counting (no GPU)."""
import bisect
import random

import pytest

import oracle


def _check(pl, ctxs, Hkv, P, G):
    pairs = len(ctxs) * Hkv
    # N = Hkv * sum ceil(ctx / P)
    N = Hkv * sum(-(-c // P) for c in ctxs)
    assert pl.num_items == N == len(pl.items)
    # ranges: G + 1 monotone bounds from 0 to N, sizes floor or ceil of N / G
    wb = pl.wg_begin
    assert len(wb) == G + 1 and wb[0] == 0 and wb[-1] == N
    sizes = [wb[w + 1] - wb[w] for w in range(G)]
    assert all(s in (N // G, -(-N // G)) for s in sizes)
    # every token of every pair covered exactly once, in order
    cover = {}
    for p, t0, t1, _ in pl.items:
        cover.setdefault(p, []).append((t0, t1))
    assert sorted(cover) == list(range(pairs))
    for p, spans in cover.items():
        ctx = ctxs[p // Hkv]
        assert spans[0][0] == 0 and spans[-1][1] == ctx
        for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
            assert a1 == b0
        for t0, t1 in spans:
            assert t0 % P == 0 and 0 < t1 - t0 <= P
    # nseg = number of distinct workgroups owning some item of the pair
    owners = {}
    for x, (p, *_rest) in enumerate(pl.items):
        w = bisect.bisect_right(wb, x) - 1
        while wb[w] == wb[w + 1]:      # skip empty ranges sharing the bound
            w += 1
        owners.setdefault(p, set()).add(w)
    assert pl.nseg == [len(owners[p]) for p in range(pairs)]
    assert sum(pl.nseg) <= G + pairs - 1
    # slots: split pairs own seg_base[p] .. seg_base[p] + nseg - 1, all distinct
    total = pl.seg_base[-1]
    assert total == sum(n for n in pl.nseg if n > 1)
    used = {}
    for x, (p, t0, t1, slot) in enumerate(pl.items):
        if pl.nseg[p] == 1:
            assert slot == -1
        else:
            assert pl.seg_base[p] <= slot < pl.seg_base[p] + pl.nseg[p]
            w = bisect.bisect_right(wb, x) - 1
            while wb[w] == wb[w + 1]:
                w += 1
            used.setdefault(slot, set()).add((p, w))
    assert sorted(used) == list(range(total))
    assert all(len(v) == 1 for v in used.values())
    # batch_base[b]: the index of sequence b's first item, read off the item
    # list (pair // Hkv is the sequence); B + 1 entries ending at N
    B = len(ctxs)
    first = [None] * B
    for x, (p, *_rest) in enumerate(pl.items):
        first[p // Hkv] = x if first[p // Hkv] is None else first[p // Hkv]
    assert pl.batch_base == first + [N]
    for b in range(B):
        assert pl.batch_base[b + 1] - pl.batch_base[b] == Hkv * -(-ctxs[b] // P)
    # pseg_base[p]: segments of pairs before p, counted in the segment list
    # (workgroup order is pair order); consecutive differences are nseg
    assert pl.pseg_base == [sum(1 for s in pl.segs if s[0] < p) for p in range(pairs + 1)]
    assert all(pl.pseg_base[p + 1] - pl.pseg_base[p] == pl.nseg[p] for p in range(pairs))
    # segments: one per (workgroup, pair) run, tokens contiguous, slots as items
    assert len(pl.segs) == sum(pl.nseg) == pl.pseg_base[-1]
    assert pl.wg_seg_begin[0] == 0 and pl.wg_seg_begin[-1] == len(pl.segs)
    for w in range(G):
        runs = []
        for x in range(wb[w], wb[w + 1]):
            p, t0, t1, slot = pl.items[x]
            if runs and runs[-1][0] == p:
                runs[-1][2] = t1
            else:
                runs.append([p, t0, t1, slot])
        assert [list(s) for s in pl.segs[pl.wg_seg_begin[w]:pl.wg_seg_begin[w + 1]]] == runs


@pytest.mark.parametrize("seed", range(40))
def test_plan_closed_forms_random(seed):
    r = random.Random(seed)
    B = r.randint(1, 9)
    Hkv = r.choice([1, 2, 8])
    P = r.choice([32, 64, 256, 1024])
    G = r.choice([1, 3, 8, 80, 256, 512])
    q_len = r.choice([1, 4, 8])
    ps = r.choice([16, 32, 1024])
    maxp = r.randint(1, 40)
    ctxs = [r.randint(q_len, maxp * ps) for _ in range(B)]
    pl = oracle.plan(ctxs, Hkv, P, G, q_len, ps, maxp)
    assert pl.status == 0
    _check(pl, ctxs, Hkv, P, G)


def test_plan_one_workgroup_never_splits():
    pl = oracle.plan([5000, 1, 300], 4, 256, 1, 1, 16, 400)
    assert pl.nseg == [1] * 12 and pl.seg_base[-1] == 0
    assert all(it[3] == -1 for it in pl.items)


def test_plan_bad_context_is_reported_and_empty():
    for ctxs, q_len in (([0], 1), ([3], 4), ([65], 1)):
        pl = oracle.plan(ctxs, 1, 256, 4, q_len, 16, 4)
        assert pl.status == 1 and pl.num_items == 0 and pl.items == []
        assert pl.wg_begin == [0] * 5
