"""Pins of the CPU oracle against things other than itself (no GPU).

* hand-derived worked examples (tests/golden/*.json)
* brute force: plain loops over a contiguous cache, no paging
* a library routine: torch's scaled_dot_product_attention in float64
* closed forms: one key, zero keys, constant values, one dominant key
* invariants: page placement, split vs unsplit, causal vs sequential decode
* the number codecs against their format definitions and torch's casts
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.attention import KV_BF16, KV_FP8, SCALE_NONE, SCALE_PER_TENSOR, SCALE_PER_TOKEN_HEAD
from tests.helpers import brute_force, to_paged

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bits(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16).view(torch.int16)


def _f64(x: torch.Tensor) -> np.ndarray:
    return x.to(torch.bfloat16).to(torch.float64).numpy()


def _random_case(seed, B, q_len, Hq, Hkv, D, ctxs, page_size, slack=3):
    g = torch.Generator().manual_seed(seed)
    T = max(ctxs)
    Q = torch.randn(B, q_len, Hq, D, generator=g).to(torch.bfloat16)
    K = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    V = torch.randn(B, Hkv, T, D, generator=g).to(torch.bfloat16)
    need = sum(-(-c // page_size) for c in ctxs)
    rng = np.random.default_rng(seed)
    kc, bt = to_paged(K, ctxs, page_size, need + slack, rng)
    rng = np.random.default_rng(seed)
    vc, _ = to_paged(V, ctxs, page_size, need + slack, rng)
    return Q, K, V, kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32)


# --------------------------------------------------------------------------- golden

def test_worked_example_attention():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_attention.json")))
    p = ex["params"]
    ps, D, Hkv = p["page_size"], p["head_dim"], p["num_kv_heads"]
    kc = torch.zeros(p["num_pages"], Hkv, ps, D)
    vc = torch.zeros(p["num_pages"], Hkv, ps, D)
    bt = torch.tensor(p["block_table"], dtype=torch.int32)
    for t, (k, v) in enumerate(zip(ex["keys_by_token"], ex["values_by_token"])):
        pg = int(bt[0, t // ps])
        kc[pg, 0, t % ps] = torch.tensor(k, dtype=torch.float32)
        vc[pg, 0, t % ps] = torch.tensor(v, dtype=torch.float32)
    q = torch.tensor(ex["q"], dtype=torch.float32).unsqueeze(0)
    out, _ = oracle.decode(_bits(q), _bits(kc), _bits(vc), bt,
                           torch.tensor([p["context_len"]], dtype=torch.int32), p["q_len"],
                           p["scale"], ps)
    np.testing.assert_allclose(out[0], np.array(ex["expected_out"]), rtol=0, atol=1e-15)


def test_worked_example_plans():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_plan.json")))
    for c in ex["cases"]:
        pl = oracle.plan(c["context_lens"], c["num_kv_heads"], c["partition"], c["grid"],
                         c["q_len"], c["page_size"], c["max_pages_per_seq"])
        assert [list(i) for i in pl.items] == c["items"], c["name"]
        assert pl.wg_begin == c["wg_begin"], c["name"]
        assert pl.nseg == c["nseg"], c["name"]
        assert pl.seg_base == c["seg_base"], c["name"]
        assert pl.status == c["status"], c["name"]
        assert [list(x) for x in pl.segs] == c["segs"], c["name"]
        assert pl.wg_seg_begin == c["wg_seg_begin"], c["name"]
        assert pl.pseg_base == c["pseg_base"], c["name"]
        assert pl.batch_base == c["batch_base"], c["name"]


def test_code_points():
    ex = json.load(open(os.path.join(GOLDEN, "code_points.json")))
    for code, val, _ in ex["e4m3fn"]:
        got = float(oracle.e4m3fn_to_f64([code])[0])
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), (code, got, val)
    for x, bits, _ in ex["bf16_round"]:
        assert int(oracle.f64_to_bf16_bits([x])[0]) == bits, (x, bits)


# --------------------------------------------------------------------------- codecs

def test_e4m3fn_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3fn_to_f64(codes.numpy())
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert nan.sum() == 2 and set(np.nonzero(nan)[0]) == {0x7F, 0xFF}
    np.testing.assert_array_equal(got[~nan], ref[~nan])
    assert np.nanmax(got) == 448.0
    # every finite code is exactly a bf16 value (decode to bf16 loses nothing)
    assert (oracle.round_to_bf16(got[~nan]) == got[~nan]).all()


def test_bf16_round_matches_torch_on_float32_inputs():
    g = torch.Generator().manual_seed(7)
    x = torch.cat([torch.randn(20000, generator=g) * 10 ** torch.randint(-30, 30, (20000,), generator=g),
                   torch.tensor([0.0, -0.0, 1.0, 65504.0, 1e-40, -3e-39])]).to(torch.float32)
    ref = x.to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    got = oracle.f64_to_bf16_bits(x.to(torch.float64).numpy())
    np.testing.assert_array_equal(got, ref)
    back = oracle.bf16_bits_to_f64(ref)
    np.testing.assert_array_equal(back, x.to(torch.bfloat16).to(torch.float64).numpy())


# --------------------------------------------------------------------------- brute force

@pytest.mark.parametrize("q_len,ctxs,ps", [(1, [5, 13], 4), (3, [3, 17], 4), (2, [9, 2], 1),
                                           (1, [1, 1], 2), (4, [7, 31], 8)])
def test_decode_matches_brute_force(q_len, ctxs, ps):
    B, Hq, Hkv, D = 2, 4, 2, 8
    Q, K, V, kc, vc, bt, ctx = _random_case(11 + q_len, B, q_len, Hq, Hkv, D, ctxs, ps)
    out, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 0.37, ps)
    ref = brute_force(_f64(Q), _f64(K), _f64(V), ctxs, q_len, 0.37)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_decode_matches_torch_sdpa():
    B, q_len, Hq, Hkv, D, ps = 2, 4, 8, 2, 128, 16
    ctxs = [70, 33]
    Q, K, V, kc, vc, bt, ctx = _random_case(5, B, q_len, Hq, Hkv, D, ctxs, ps)
    out, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 1 / math.sqrt(D), ps)
    grp = Hq // Hkv
    for b in range(B):
        c = ctxs[b]
        q = torch.from_numpy(_f64(Q[b])).permute(1, 0, 2)                   # [Hq, q_len, D]
        k = torch.from_numpy(_f64(K[b, :, :c])).repeat_interleave(grp, 0)  # [Hq, c, D]
        v = torch.from_numpy(_f64(V[b, :, :c])).repeat_interleave(grp, 0)
        i = torch.arange(q_len)[:, None]
        t = torch.arange(c)[None, :]
        mask = t <= (c - q_len + i)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask,
                                                                scale=1 / math.sqrt(D))
        np.testing.assert_allclose(out[b], ref.permute(1, 0, 2).numpy(), rtol=1e-11, atol=1e-12)


# --------------------------------------------------------------------------- closed forms

def test_single_key_returns_its_value():
    Q, K, V, kc, vc, bt, ctx = _random_case(3, 2, 1, 4, 1, 16, [1, 1], 4)
    out, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, 1, 0.25, 4)
    for b in range(2):
        np.testing.assert_array_equal(out[b, 0], np.repeat(_f64(V[b, :, 0]), 4, axis=0))


def test_zero_keys_give_mean_of_visible_values():
    q_len, ctxs, ps = 3, [6, 11], 4
    Q, K, V, kc, vc, bt, ctx = _random_case(4, 2, q_len, 2, 2, 8, ctxs, ps)
    kc = torch.zeros_like(kc)
    out, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 0.5, ps)
    for b, c in enumerate(ctxs):
        for i in range(q_len):
            for h in range(2):
                want = _f64(V[b, h, :c - q_len + i + 1]).mean(axis=0)
                np.testing.assert_allclose(out[b, i, h], want, rtol=1e-13, atol=1e-14)


def test_constant_values_return_the_constant():
    Q, K, V, kc, vc, bt, ctx = _random_case(6, 2, 2, 4, 2, 32, [40, 9], 8)
    vc = torch.full_like(vc, 0.8125)
    out, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, 2, 0.3, 8)
    np.testing.assert_allclose(out, 0.8125, rtol=0, atol=1e-14)


def test_one_dominant_key():
    D, ps, c = 16, 4, 10
    Q, K, V, kc, vc, bt, ctx = _random_case(8, 1, 1, 1, 1, D, [c], ps)
    # make key 6 parallel to q and large: its weight is ~1
    K2 = K.clone()
    K2[0, 0, 6] = Q[0, 0, 0].to(torch.float32) * 30
    kc2, bt2 = to_paged(K2.to(torch.bfloat16), [c], ps, 6, np.random.default_rng(0))
    vc2, _ = to_paged(V, [c], ps, 6, np.random.default_rng(0))
    out, _ = oracle.decode(_bits(Q), _bits(kc2), _bits(vc2), bt2, ctx, 1, 1.0, ps)
    np.testing.assert_allclose(out[0, 0, 0], _f64(V[0, 0, 6]), rtol=0, atol=1e-12)


# --------------------------------------------------------------------------- invariants

def test_page_placement_does_not_change_output():
    q_len, ctxs, ps = 2, [37, 64, 5], 8
    g = torch.Generator().manual_seed(9)
    Q = torch.randn(3, q_len, 4, 16, generator=g)
    K = torch.randn(3, 2, 64, 16, generator=g).to(torch.bfloat16)
    V = torch.randn(3, 2, 64, 16, generator=g).to(torch.bfloat16)
    outs = []
    for s in (1, 2, 3):
        kc, bt = to_paged(K, ctxs, ps, 30, np.random.default_rng(s))
        vc, _ = to_paged(V, ctxs, ps, 30, np.random.default_rng(s))
        outs.append(oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt,
                                  torch.tensor(ctxs, dtype=torch.int32), q_len, 0.25, ps)[0])
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


@pytest.mark.parametrize("P", [16, 32, 64, 256, 4096])
def test_split_equals_unsplit(P):
    q_len, ctxs, ps = 4, [300, 33, 257], 16
    Q, K, V, kc, vc, bt, ctx = _random_case(10, 3, q_len, 4, 1, 32, ctxs, ps)
    ref, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 0.2, ps)
    got = oracle.decode_split(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 0.2, ps, P)
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


def test_split_row_with_no_visible_key_has_zero_weight():
    # q_len 4, ctx 258, P 256: partition [256, 258) is invisible to queries 0 and 1
    q_len, ps = 4, 16
    Q, K, V, kc, vc, bt, ctx = _random_case(12, 1, q_len, 2, 1, 16, [258], ps)
    o, lse = oracle.attend_range(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 0.3, ps,
                                 0, 0, 256, 512)
    rows_q0_q1 = slice(0, 2 * 2)
    assert np.isneginf(lse[rows_q0_q1]).all() and (o[rows_q0_q1] == 0).all()
    assert np.isfinite(lse[4:]).all()


def test_causal_equals_sequential_single_token_decode():
    q_len, ctxs, ps = 5, [12, 40], 4
    Q, K, V, kc, vc, bt, ctx = _random_case(13, 2, q_len, 6, 3, 16, ctxs, ps)
    out, _ = oracle.decode(_bits(Q), _bits(kc), _bits(vc), bt, ctx, q_len, 0.4, ps)
    for i in range(q_len):
        ctx_i = torch.tensor([c - q_len + i + 1 for c in ctxs], dtype=torch.int32)
        step, _ = oracle.decode(_bits(Q[:, i:i + 1]), _bits(kc), _bits(vc), bt, ctx_i, 1, 0.4, ps)
        # equal up to the summation order of the matrix products (masked keys add exact zeros)
        np.testing.assert_allclose(out[:, i], step[:, 0], rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- fp8 KV

@pytest.mark.parametrize("mode", [SCALE_PER_TENSOR, SCALE_PER_TOKEN_HEAD])
def test_fp8_decode_matches_brute_force_on_dequantised_values(mode):
    B, q_len, Hq, Hkv, D, ps = 2, 2, 4, 1, 8, 4
    ctxs = [9, 14]
    g = torch.Generator().manual_seed(21)
    T = max(ctxs)
    Q = torch.randn(B, q_len, Hq, D, generator=g).to(torch.bfloat16)
    codes = torch.randint(0, 256, (B, Hkv, T, D), generator=g, dtype=torch.int32).to(torch.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x10          # no NaN codes in live data
    vcodes = torch.randint(0, 256, (B, Hkv, T, D), generator=g, dtype=torch.int32).to(torch.uint8)
    vcodes[(vcodes & 0x7F) == 0x7F] = 0x22
    if mode == SCALE_PER_TENSOR:
        ksc = torch.full((B, Hkv, T), 0.0123)
        vsc = torch.full((B, Hkv, T), 3.5)
    else:
        ksc = torch.rand(B, Hkv, T, generator=g) * 0.05 + 1e-3
        vsc = torch.rand(B, Hkv, T, generator=g) * 2 + 0.1
    # dequantised reference values via torch's own fp8 cast
    Kd = codes.view(torch.float8_e4m3fn).to(torch.float64) * ksc[..., None].to(torch.float64)
    Vd = vcodes.view(torch.float8_e4m3fn).to(torch.float64) * vsc[..., None].to(torch.float64)
    need = sum(-(-c // ps) for c in ctxs)
    kc, bt = to_paged(codes, ctxs, ps, need + 2, np.random.default_rng(1), fill=0x7F)
    vc, _ = to_paged(vcodes, ctxs, ps, need + 2, np.random.default_rng(1), fill=0x7F)
    if mode == SCALE_PER_TENSOR:
        scales = torch.tensor([0.0123, 3.5], dtype=torch.float32)
        Kd = codes.view(torch.float8_e4m3fn).to(torch.float64) * float(scales[0])
        Vd = vcodes.view(torch.float8_e4m3fn).to(torch.float64) * float(scales[1])
    else:
        kp, _ = to_paged(ksc.unsqueeze(-1), ctxs, ps, need + 2, np.random.default_rng(1))
        vp, _ = to_paged(vsc.unsqueeze(-1), ctxs, ps, need + 2, np.random.default_rng(1))
        scales = torch.stack([kp[..., 0], vp[..., 0]]).contiguous()
        Kd = codes.view(torch.float8_e4m3fn).to(torch.float64) * ksc.to(torch.float64)[..., None]
        Vd = vcodes.view(torch.float8_e4m3fn).to(torch.float64) * vsc.to(torch.float64)[..., None]
    out, _ = oracle.decode(_bits(Q), kc, vc, bt, torch.tensor(ctxs, dtype=torch.int32), q_len,
                           0.35, ps, KV_FP8, mode, scales)
    ref = brute_force(_f64(Q), Kd.numpy(), Vd.numpy(), ctxs, q_len, 0.35)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)


def test_gather_matches_fancy_index():
    Q, K, V, kc, vc, bt, ctx = _random_case(14, 2, 1, 2, 2, 8, [19, 7], 4)
    for b, c in enumerate([19, 7]):
        for g in range(2):
            rows = oracle.gather_rows(_bits(kc), bt, b, g, c, 4)
            np.testing.assert_array_equal(rows, _bits(K[b, g, :c]).numpy())
