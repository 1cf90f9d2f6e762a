"""The seeded input generator: shapes, determinism, poisoning (no GPU)."""
import math

import numpy as np
import torch

import workloads as W


def test_shapes_and_determinism():
    a = W.generate(W.C2, 2026)
    b = W.generate(W.C2, 2026)
    c = W.generate(W.C2, 2029)
    assert a.q.shape == (1, 1, 16, 128) and a.q.dtype == torch.bfloat16
    assert a.k_cache.shape == (64, 1, 128, 128)
    assert a.block_table.shape == (1, 4) and a.context_lens.tolist() == [512]
    for x, y in ((a.q, b.q), (a.k_cache, b.k_cache), (a.v_cache, b.v_cache)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert not torch.equal(a.k_cache.view(torch.int16), c.k_cache.view(torch.int16))
    assert sorted(a.block_table[0].tolist()) == sorted(set(a.block_table[0].tolist()))


def test_poisoning_marks_only_dead_data():
    spec = W.scaled(W.C3, batch=6, ctx_lo=20, ctx_hi=70)
    w = W.generate(spec, 2039)
    bt = w.block_table
    live = torch.zeros(w.num_pages, spec.page_size, dtype=torch.bool)
    for b in range(spec.batch):
        c = int(w.context_lens[b])
        for t in range(c):
            live[int(bt[b, t // spec.page_size]), t % spec.page_size] = True
        assert (bt[b, -(-c // spec.page_size):] == -1).all()
    k = w.k_cache.float()
    nan = torch.isnan(k).all(dim=-1).all(dim=1)     # [pages, slots]
    assert torch.equal(nan, ~live)
    assert torch.isfinite(k[live.unsqueeze(1).expand(-1, spec.num_kv_heads, -1)]).all()


def test_fp8_quantiser_per_token_and_per_tensor():
    for mode in (W.SCALE_PER_TOKEN_HEAD, W.SCALE_PER_TENSOR):
        spec = W.scaled(W.C4_Q4_TOK, batch=2, ctx_lo=1500, ctx_hi=2100, page_size=256,
                        kv_scale_mode=mode, max_ctx=4096)
        w = W.generate(spec, 2026, poison=False)
        codes = w.k_cache
        assert codes.dtype == torch.uint8
        vals = codes.view(torch.float8_e4m3fn).float()
        assert torch.isfinite(vals).all() and vals.abs().max() <= 448
        if mode == W.SCALE_PER_TOKEN_HEAD:
            assert w.kv_scales.shape == (2, w.num_pages, 1, 256)
            # each row reaches the top of the range after scaling
            assert (vals.abs().amax(dim=-1) == 448).float().mean() > 0.99
        else:
            assert w.kv_scales.shape == (2,)
            assert vals.abs().max() == 448


def test_kv_bytes_counts_payload():
    w = W.generate(W.C1, 2026)
    assert w.kv_bytes() == 2 * 128 * 1 * 128 * 2
    spec = W.scaled(W.C4_Q1_TOK, batch=2, ctx_lo=1000, ctx_hi=1000, max_ctx=2048)
    w = W.generate(spec, 2026)
    assert w.kv_bytes() == 2 * 2000 * 128 + 2 * 2000 * 4


def test_decode_loop_poisons_exactly_the_slots_its_steps_fill():
    spec = W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=1030, ctx_hi=2060, max_ctx=3072)
    steps = 3
    loop = W.decode_loop(spec, 2026, steps, [1030, 2060, 1800])
    ref = W.generate(spec, 2026, context_lens=[1030, 2060, 1800])
    start = loop.start.context_lens.tolist()
    assert start == [1030 - 12, 2060 - 12, 1800 - 12]
    assert loop.context_lens_at(steps - 1).tolist() == [1030, 2060, 1800]
    assert loop.q.shape == (steps, 3, 4, 16, 128) and loop.new_k.shape == (steps, 3, 4, 1, 128)
    assert torch.equal(loop.q[0].view(torch.int16), loop.start.q.view(torch.int16))
    bt = loop.start.block_table
    changed = (loop.start.k_cache != ref.k_cache).any(dim=-1)       # [pages, Hkv, ps]
    want = torch.zeros_like(changed)
    for b in range(spec.batch):
        for t in range(start[b], start[b] + steps * spec.q_len):
            want[int(bt[b, t // spec.page_size]), :, t % spec.page_size] = True
    assert torch.equal(changed, want)
    assert (loop.start.k_cache[want] == 0x7F).all()
    assert torch.isnan(loop.start.kv_scales[:, want]).all()
    again = W.decode_loop(spec, 2026, steps, [1030, 2060, 1800])
    for x, y in ((loop.q, again.q), (loop.new_k, again.new_k), (loop.new_v, again.new_v)):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))
