"""Planted mistakes in the oracle must fail its pins (no GPU).

Each case patches one plausible slip into a copy of an oracle function — a
wrong head grouping, an off-by-one causal mask, a dropped scale, a transposed
page index, a wrong subnormal exponent, unnormalised merge weights, a segment
counter that ignores the pair — and checks that at least one pin test raises.
The patches live only here, on the CPU; the oracle itself is unchanged.
"""
import numpy as np
import pytest

import oracle
import oracle.attention as att
import oracle.codecs as codecs
from tests import test_oracle as T
from tests import test_plan_oracle as TP


def _pins():
    T.test_worked_example_attention()
    T.test_decode_matches_brute_force(3, [3, 17], 4)
    T.test_decode_matches_torch_sdpa()
    T.test_split_equals_unsplit(64)
    T.test_fp8_decode_matches_brute_force_on_dequantised_values("per_token_head")


def _interleaved_groups(q, k_cache, v_cache, block_table, context_lens, b, g, q_len, kv_dtype,
                        scale_mode, kv_scales, page_size):
    ctx = int(att._np(context_lens)[b])
    qn = att._np(q)
    Hq, Hkv = qn.shape[2], att._np(k_cache).shape[1]
    group = Hq // Hkv
    K = att.dequant_rows(att.gather_rows(k_cache, block_table, b, g, ctx, page_size), kv_dtype,
                         scale_mode, kv_scales, 0, block_table, b, g, ctx, page_size)
    V = att.dequant_rows(att.gather_rows(v_cache, block_table, b, g, ctx, page_size), kv_dtype,
                         scale_mode, kv_scales, 1, block_table, b, g, ctx, page_size)
    heads = list(range(g, Hq, Hkv))                       # slip: h % Hkv grouping
    Q = codecs.bf16_bits_to_f64(qn[b][:, heads, :]).reshape(q_len * group, -1)
    return ctx, group, Q, K, V


def _mask_off_by_one(ctx, q_len, group, t0, t1):
    i = np.arange(q_len * group) // group
    t = np.arange(t0, t1)
    return t[None, :] < (ctx - q_len + i)[:, None] + (i[:, None] == 0)   # slip for i > 0


def _page_index_swapped(cache, block_table, b, g, ctx, page_size):
    cache = att._np(cache)
    bt = att._np(block_table)
    t = np.arange(ctx)
    return cache[bt[b, t % bt.shape[1]].astype(np.int64), g, t % page_size, :]   # slip


def _subnormal_exp(codes):
    c = np.asarray(codes).astype(np.uint8).astype(np.int64)
    s, e, m = (c >> 7) & 1, (c >> 3) & 0xF, c & 7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -7, (1.0 + m / 8.0) * np.exp2(e - 7.0))  # slip
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


def _merge_unnormalised(os_, lses):
    os_ = np.asarray(os_)
    lses = np.asarray(lses)
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - lses.max(axis=0)[None, :]))
    return (w[:, :, None] * os_).sum(axis=0)        # slip: no division by sum w


MUTATIONS = {
    "interleaved head groups": (att, "_pair_inputs", _interleaved_groups),
    "causal mask off by one": (att, "_visible", _mask_off_by_one),
    "page index from t % maxp": (att, "gather_rows", _page_index_swapped),
    "subnormal exponent -7": (att, "e4m3fn_to_f64", _subnormal_exp),
    "merge without normalising": (att, "merge_partials", _merge_unnormalised),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_attention_mistake_is_caught(name, monkeypatch):
    mod, attr, fn = MUTATIONS[name]
    monkeypatch.setattr(mod, attr, fn)
    with pytest.raises(AssertionError):
        _pins()


def test_planted_scale_mistake_is_caught(monkeypatch):
    real = att.decode

    def no_scale(q, k, v, bt, ctx, q_len, scale, *a, **kw):
        return real(q, k, v, bt, ctx, q_len, 1.0, *a, **kw)      # slip: scale dropped
    monkeypatch.setattr(oracle, "decode", no_scale)
    with pytest.raises(AssertionError):
        _pins()


def test_planted_plan_mistake_is_caught(monkeypatch):
    real = oracle.plan

    def global_segment_index(*a, **kw):
        pl = real(*a, **kw)
        # slip: slots numbered by item order over all split items, not per segment
        k = 0
        items = []
        for p, t0, t1, slot in pl.items:
            if slot >= 0:
                items.append((p, t0, t1, k))
                k += 1
            else:
                items.append((p, t0, t1, slot))
        pl.items = items
        return pl
    monkeypatch.setattr(oracle, "plan", global_segment_index)
    with pytest.raises(AssertionError):
        T.test_worked_example_plans()
    with pytest.raises(AssertionError):
        for s in range(40):
            TP.test_plan_closed_forms_random(s)


def _tables_batch_base_per_head(pl, Hkv):
    # slip: first item of each sequence counted for one kv head only
    bb = [0]
    for b in range(len(pl.batch_base) - 1):
        bb.append(bb[-1] + (pl.batch_base[b + 1] - pl.batch_base[b]) // Hkv)
    pl.batch_base = bb


def _tables_pseg_inclusive(pl, Hkv):
    # slip: inclusive instead of exclusive prefix sum of the segment counts
    run, out = 0, []
    for n in pl.nseg:
        run += n
        out.append(run)
    pl.pseg_base = out + [run]


@pytest.mark.parametrize("slip", [_tables_batch_base_per_head, _tables_pseg_inclusive])
def test_planted_plan_table_mistake_is_caught(slip, monkeypatch):
    real = oracle.plan

    def mutated(context_lens, num_kv_heads, *a, **kw):
        pl = real(context_lens, num_kv_heads, *a, **kw)
        slip(pl, num_kv_heads)
        return pl
    monkeypatch.setattr(oracle, "plan", mutated)
    with pytest.raises(AssertionError):
        T.test_worked_example_plans()
    with pytest.raises(AssertionError):
        for s in range(40):
            TP.test_plan_closed_forms_random(s)


def _encode_ties_away(x):
    # slip: ties rounded away from zero instead of to the even code
    x = np.asarray(x, dtype=np.float64)
    vals = codecs._e4m3fn_nonneg_values()
    a = np.abs(x)
    hi = np.minimum(np.searchsorted(vals, a, side="left"), len(vals) - 1)
    lo = np.maximum(hi - 1, 0)
    code = np.where(vals[hi] - a <= a - vals[lo], hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _encode_truncating(x):
    # slip: rounds toward zero
    x = np.asarray(x, dtype=np.float64)
    vals = codecs._e4m3fn_nonneg_values()
    a = np.abs(x)
    code = (np.searchsorted(vals, a, side="right") - 1).astype(np.uint8)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _cache_pins():
    from tests import test_oracle_cache as TC
    TC.test_encode_matches_torch_cast_on_every_bf16_value_and_every_midpoint()
    TC.test_encode_ties_go_to_the_even_code()
    TC.test_per_token_append_scale_and_codes()
    TC.test_per_tensor_append_uses_the_given_scales_and_clamps()
    TC.test_generator_quantiser_agrees_with_the_oracle_rule()


@pytest.mark.parametrize("slip", ["ties away", "truncation", "scale / 240", "multiply by scale"])
def test_planted_cache_mistake_is_caught(slip, monkeypatch):
    from oracle import cache
    if slip == "ties away":
        monkeypatch.setattr(cache, "e4m3fn_encode", _encode_ties_away)
        monkeypatch.setattr(codecs, "e4m3fn_encode", _encode_ties_away)
        monkeypatch.setattr(oracle, "e4m3fn_encode", _encode_ties_away)
    elif slip == "truncation":
        monkeypatch.setattr(cache, "e4m3fn_encode", _encode_truncating)
        monkeypatch.setattr(oracle, "e4m3fn_encode", _encode_truncating)
    elif slip == "scale / 240":
        monkeypatch.setattr(cache, "E4M3FN_MAX", np.float32(240.0))   # the FNUZ maximum
    else:
        real_quant = cache.quantise_row

        def times_scale(x_f32, scale):
            return real_quant(x_f32, np.float32(1.0) / (np.float32(scale) ** 2))   # slip: x * s
        monkeypatch.setattr(cache, "quantise_row", times_scale)
    with pytest.raises(AssertionError):
        _cache_pins()
