"""Planted mistakes in the oracle must fail its pins (no GPU).

Each case patches one plausible slip into a copy of an oracle function — a
wrong head grouping, an off-by-one or top-left causal mask, a dropped scale,
a transposed page index, a wrong subnormal exponent, unnormalised merge
weights, a log-sum-exp in the wrong log base or over unshifted exponentials,
swapped or logically-paged per-token scales, bf16 ties rounded away from zero
or rounded twice, a segment counter that ignores the pair, an unclipped last
partition, ranges rounded up — and checks that at least one pin test raises.
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


# --------------------------------------------------------------------------- more slips

def _attend_range_with(lse_of, l_of):
    """attend_range with its log-sum-exp or its normaliser replaced."""
    def fn(q, k_cache, v_cache, block_table, context_lens, q_len, scale, page_size, b, g, t0, t1,
           kv_dtype=att.KV_BF16, scale_mode=att.SCALE_NONE, kv_scales=None):
        ctx, group, Q, K, V = att._pair_inputs(q, k_cache, v_cache, block_table, context_lens, b, g,
                                               q_len, kv_dtype, scale_mode, kv_scales, page_size)
        R, D = Q.shape
        t1 = min(t1, ctx)
        o = np.zeros((R, D))
        lse = np.full(R, -np.inf)
        if t1 <= t0:
            return o, lse
        s = scale * (Q @ K[t0:t1].T)
        vis = att._visible(ctx, q_len, group, t0, t1)
        for r in range(R):
            sr = s[r][vis[r]]
            if sr.size == 0:
                continue
            m = sr.max()
            w = np.exp(sr - m)
            l = l_of(sr, m, w)
            o[r] = (w @ V[t0:t1][vis[r]]) / l
            lse[r] = lse_of(m, l)
        return o, lse
    return fn


def _visible_top_left(ctx, q_len, group, t0, t1):
    i = np.arange(q_len * group) // group
    t = np.arange(t0, t1)
    return t[None, :] <= i[:, None]                 # slip: query i aligned to key i, not ctx - q_len + i


def _scales_k_v_swapped(kv_scales, which, block_table, b, g, ctx, page_size):
    sc = att._np(kv_scales)
    bt = att._np(block_table)
    t = np.arange(ctx)
    return sc[1 - which, bt[b, t // page_size].astype(np.int64), g, t % page_size].astype(np.float64)


def _scales_logical_page(kv_scales, which, block_table, b, g, ctx, page_size):
    sc = att._np(kv_scales)
    t = np.arange(ctx)
    return sc[which, t // page_size, g, t % page_size].astype(np.float64)   # slip: no block table


MORE_ATTENTION = {
    "lse in the log2 domain": (att, "attend_range",
                               _attend_range_with(lambda m, l: m + np.log2(l), lambda sr, m, w: w.sum())),
    "partial normalised by the unshifted sum": (att, "attend_range",
                                                _attend_range_with(lambda m, l: m + np.log(l),
                                                                   lambda sr, m, w: np.exp(sr).sum())),
    "causal mask aligned top-left": (att, "_visible", _visible_top_left),
    "K and V scales swapped": (att, "_gather_scales", _scales_k_v_swapped),
    "scale page taken from the logical page": (att, "_gather_scales", _scales_logical_page),
}


@pytest.mark.parametrize("name", sorted(MORE_ATTENTION))
def test_more_planted_attention_mistakes_are_caught(name, monkeypatch):
    mod, attr, fn = MORE_ATTENTION[name]
    monkeypatch.setattr(mod, attr, fn)
    if attr == "attend_range":
        monkeypatch.setattr(oracle, "attend_range", fn)
    with pytest.raises(AssertionError):
        _pins()


def _round_bf16_ties_away(x):
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x) & (x != 0)
    _, e = np.frexp(x[fin])
    ulp_exp = np.maximum(e, -125) - 8
    y = np.ldexp(x[fin], -ulp_exp)
    out[fin] = np.ldexp(np.trunc(y + np.copysign(0.5, y)), ulp_exp)   # slip: ties away from zero
    return out


def _round_bf16_via_float32(x):
    x = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)   # slip: rounds twice
    return _real_round_bf16(x)


_real_round_bf16 = codecs.round_to_bf16


@pytest.mark.parametrize("slip", [_round_bf16_ties_away, _round_bf16_via_float32])
def test_planted_bf16_rounding_mistake_is_caught(slip, monkeypatch):
    monkeypatch.setattr(codecs, "round_to_bf16", slip)
    monkeypatch.setattr(oracle, "round_to_bf16", slip)
    with pytest.raises(AssertionError):
        T.test_code_points()


def _last_item_not_clipped(pl):
    # slip: every item spans a whole partition, the last one past the context
    P = None
    for p, t0, t1, slot in pl.items:
        if P is None or t1 - t0 > P:
            P = t1 - t0
    pl.items = [(p, t0, t0 + P, slot) for p, t0, t1, slot in pl.items]


def _ranges_rounded_up(pl):
    # slip: workgroup w starts at ceil(w N / G)
    G = len(pl.wg_begin) - 1
    pl.wg_begin = [-(-w * pl.num_items // G) for w in range(G + 1)]


@pytest.mark.parametrize("slip", [_last_item_not_clipped, _ranges_rounded_up])
def test_planted_plan_range_mistake_is_caught(slip, monkeypatch):
    real = oracle.plan

    def mutated(*a, **kw):
        pl = real(*a, **kw)
        slip(pl)
        return pl
    monkeypatch.setattr(oracle, "plan", mutated)
    with pytest.raises(AssertionError):
        T.test_worked_example_plans()
    with pytest.raises(AssertionError):
        for s in range(40):
            TP.test_plan_closed_forms_random(s)
