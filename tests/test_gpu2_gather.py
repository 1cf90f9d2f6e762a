"""The decode kernel's page addressing, exposed by pa_debug_gather, reads
exactly the cache rows the block table names (bitwise)."""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import DEV, dims_for, say, upload

pytestmark = pytest.mark.gpu

CASES = {
    "C3-like bf16 page 16": W.scaled(W.C3, batch=5, ctx_lo=1, ctx_hi=300, max_ctx=512),
    "C4-like fp8 page 1024": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=4, ctx_hi=2500, max_ctx=3072),
    "C5-like bf16 D256 page 32": W.scaled(W.C5, batch=2, ctx_lo=8, ctx_hi=700, max_ctx=1024,
                                          pool_slack=0.2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gather_bitwise(name):
    spec = CASES[name]
    w = W.generate(spec, 2026)
    say(f"[gather] {name} ctx={w.context_lens.tolist()}")
    d = upload(w)
    plan = pa.pa_plan(dims_for(w), d.context_lens)
    cap = spec.max_pages_per_seq * spec.page_size
    pairs = spec.batch * spec.num_kv_heads
    row = w.k_cache.shape[-1] * w.k_cache.element_size()
    k_out = torch.zeros(pairs, cap, row, dtype=torch.uint8, device=DEV)
    v_out = torch.zeros_like(k_out)
    pa.pa_debug_gather(plan, d.k_cache, d.v_cache, d.block_table, d.context_lens, k_out, v_out)
    k_out, v_out = k_out.cpu().numpy(), v_out.cpu().numpy()
    kb = w.k_cache.view(torch.uint8).view(*w.k_cache.shape[:3], row)
    vb = w.v_cache.view(torch.uint8).view(*w.v_cache.shape[:3], row)
    for b in range(spec.batch):
        c = int(w.context_lens[b])
        for g in range(spec.num_kv_heads):
            p = b * spec.num_kv_heads + g
            np.testing.assert_array_equal(
                k_out[p, :c], oracle.gather_rows(kb, w.block_table, b, g, c, spec.page_size))
            np.testing.assert_array_equal(
                v_out[p, :c], oracle.gather_rows(vb, w.block_table, b, g, c, spec.page_size))
            assert (k_out[p, c:] == 0).all() and (v_out[p, c:] == 0).all()
    assert pa.pa_plan_status(plan) == 0


def test_debug_bounds_flags_bad_page():
    spec = W.scaled(W.C3, batch=2, ctx_lo=40, ctx_hi=60, max_ctx=64)
    w = W.generate(spec, 2029)
    w.block_table[1, 1] = w.num_pages + 5          # out of range on purpose
    d = upload(w)
    plan = pa.pa_plan(dims_for(w, flags=pa.PA_FLAG_DEBUG_BOUNDS), d.context_lens)
    row = spec.head_dim * 2
    cap = spec.max_pages_per_seq * spec.page_size
    k_out = torch.zeros(spec.batch * spec.num_kv_heads, cap, row, dtype=torch.uint8, device=DEV)
    v_out = torch.zeros_like(k_out)
    pa.pa_debug_gather(plan, d.k_cache, d.v_cache, d.block_table, d.context_lens, k_out, v_out)
    assert pa.pa_plan_status(plan) & pa.PA_DEV_BAD_PAGE
    # the decode kernel checks the same way and reads such tokens as zeros
    plan = pa.pa_plan(dims_for(w, flags=pa.PA_FLAG_DEBUG_BOUNDS), d.context_lens)
    out = torch.empty_like(d.q)
    pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens, 1, spec.scale,
                 pa.PA_SCALE_NONE, None, out)
    assert pa.pa_plan_status(plan) & pa.PA_DEV_BAD_PAGE
    assert torch.isfinite(out.float()).all()
