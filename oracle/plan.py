"""Persistent work-list rule, as a direct simulation (test infrastructure only).

The pages describe the metadata scheduler only by what it does: it builds the
metadata a persistent decode kernel walks, on a grid of CU count x a grid
multiplier ("num_sm = base_cu * _PA_METADATA_GRID_OVERSUB", default one grid
per CU), with a split reducer combining the pieces ("[Kernel][Perf] Optimize
paged-attention metadata decode", ROCm/FlyDSL PR #910, "Pull request
overview", the code excerpt, "Summary" and "Motivation"). The list format is
not on the pages; this library fixes it as follows, and the GPU plan kernel
must reproduce it bit for bit:

  items      for b ascending, then kv head g, then partition k: item
             (pair = b * Hkv + g, tok_begin = k * P, tok_end = min((k+1) * P,
             ctx_b)) for k < ceil(ctx_b / P)
  ranges     workgroup w of G owns items [floor(w N / G), floor((w+1) N / G))
  segments   a maximal run of same-pair items inside one workgroup's range
  nseg[p]    number of segments of pair p; 1 means the pair is finished by
             one workgroup, which writes the output itself
  seg_base   slots for split pairs only: seg_base[p] = sum of nseg[p'] over
             earlier pairs p' with nseg[p'] > 1
  slot       of an item: -1 for a pair with nseg = 1, else seg_base[p] + the
             index of its segment among the pair's segments, in item order
  segs       one (pair, tok_begin, tok_end, slot) per segment, in workgroup
             order; wg_seg_begin[w] = index of workgroup w's first segment
  pseg_base  exclusive prefix sum of nseg over all pairs
  batch_base index of the first item of sequence b (B + 1 entries)
  status     1 if some ctx_b is outside [max(1, q_len), max_pages * page_size];
             then the plan is empty (N = 0, every range empty, nseg = 0)

This module computes these by walking the ranges one item at a time; the GPU
computes them with prefix sums and a closed form, so the two share no method.
"""
from __future__ import annotations

import dataclasses
from typing import List

STATUS_OK = 0
STATUS_BAD_CONTEXT = 1


@dataclasses.dataclass
class Plan:
    num_items: int
    items: List[tuple]          # (pair, tok_begin, tok_end, slot)
    wg_begin: List[int]         # G + 1 entries
    nseg: List[int]             # per pair
    seg_base: List[int]         # per pair + 1 (last = total slots)
    status: int
    segs: List[tuple] = dataclasses.field(default_factory=list)
    wg_seg_begin: List[int] = dataclasses.field(default_factory=list)
    pseg_base: List[int] = dataclasses.field(default_factory=list)
    batch_base: List[int] = dataclasses.field(default_factory=list)


def plan(context_lens, num_kv_heads: int, partition: int, grid: int, q_len: int,
         page_size: int, max_pages_per_seq: int) -> Plan:
    ctxs = [int(c) for c in context_lens]
    B = len(ctxs)
    pairs = B * num_kv_heads
    cap = max_pages_per_seq * page_size
    if any(c < max(1, q_len) or c > cap for c in ctxs):
        return Plan(0, [], [0] * (grid + 1), [0] * pairs, [0] * (pairs + 1), STATUS_BAD_CONTEXT,
                    [], [0] * (grid + 1), [0] * (pairs + 1), [0] * (B + 1))

    raw = []
    for b, c in enumerate(ctxs):
        for g in range(num_kv_heads):
            k = 0
            while k * partition < c:
                raw.append((b * num_kv_heads + g, k * partition, min((k + 1) * partition, c)))
                k += 1
    N = len(raw)
    wg_begin = [w * N // grid for w in range(grid + 1)]

    # Walk every workgroup's range; each change of pair inside it, and the
    # start of the range, opens a new segment.
    seg_of_item = [None] * N       # (pair, index of the segment within its pair)
    nseg = [0] * pairs
    for w in range(grid):
        prev = None
        for x in range(wg_begin[w], wg_begin[w + 1]):
            p = raw[x][0]
            if p != prev:
                nseg[p] += 1
                prev = p
            seg_of_item[x] = (p, nseg[p] - 1)

    seg_base = [0] * (pairs + 1)
    for p in range(pairs):
        seg_base[p + 1] = seg_base[p] + (nseg[p] if nseg[p] > 1 else 0)

    items = []
    for x, (p, t0, t1) in enumerate(raw):
        _, j = seg_of_item[x]
        slot = -1 if nseg[p] == 1 else seg_base[p] + j
        items.append((p, t0, t1, slot))

    # Segments in workgroup order, each spanning its run of items.
    segs = []
    wg_seg_begin = []
    for w in range(grid):
        wg_seg_begin.append(len(segs))
        for x in range(wg_begin[w], wg_begin[w + 1]):
            p, t0, t1, slot = items[x]
            if x == wg_begin[w] or items[x - 1][0] != p:
                segs.append([p, t0, t1, slot])
            else:
                segs[-1][2] = t1
    wg_seg_begin.append(len(segs))
    pseg_base = [0] * (pairs + 1)
    for p in range(pairs):
        pseg_base[p + 1] = pseg_base[p] + nseg[p]
    batch_base = [0]
    for c in ctxs:
        batch_base.append(batch_base[-1] + num_kv_heads * -(-c // partition))
    return Plan(N, items, wg_begin, nseg, seg_base, STATUS_OK, [tuple(x) for x in segs],
                wg_seg_begin, pseg_base, batch_base)
