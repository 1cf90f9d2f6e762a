"""Pins of the oracle's E4M3FN encoder and KV-cache append (no GPU)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import cache


def _bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().astype(np.uint16)


def _bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def test_encode_round_trips_every_finite_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = oracle.e4m3fn_to_f64(codes)
    assert np.array_equal(oracle.e4m3fn_encode(vals), codes)


def test_encode_matches_torch_cast_on_every_bf16_value_and_every_midpoint():
    # a library routine: torch's float -> float8_e4m3fn cast rounds to
    # nearest even; it is compared on all bf16 values in range and on the
    # exact midpoints between neighbouring codes (the ties)
    allbits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):   # the NaN patterns among them
        x = _bits_to_f32(allbits).astype(np.float64)
    x = x[np.isfinite(x) & (np.abs(x) <= 448)]
    vals = oracle.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3fn_encode(x), want)


def test_encode_ties_go_to_the_even_code():
    # 1.0625 lies halfway between 1 (0x38) and 1.125 (0x39); 232 between 224
    # (0x76) and 240 (0x77); 2^-10 between 0 and the smallest subnormal
    assert oracle.e4m3fn_encode([1.0625, 1.1875, 232.0, 2.0 ** -10, -1.0625]).tolist() == \
        [0x38, 0x3A, 0x76, 0x00, 0xB8]
    with pytest.raises(ValueError):
        oracle.e4m3fn_encode([449.0])


def _case(fp8, per_token, q_len=3, B=2, Hkv=2, D=16, ps=4, maxp=4, seed=0):
    r = np.random.default_rng(seed)
    num_pages = B * maxp + 2
    ctx = np.array([q_len + 2, maxp * ps], dtype=np.int32)[:B]
    bt = np.full((B, maxp), -1, dtype=np.int32)
    perm = r.permutation(num_pages)
    for b in range(B):
        for p in range(-(-int(ctx[b]) // ps)):
            bt[b, p] = perm[b * maxp + p]
    nk = _bf16_bits(r.standard_normal((B, q_len, Hkv, D)) * 3)
    nv = _bf16_bits(r.standard_normal((B, q_len, Hkv, D)))
    shape = (num_pages, Hkv, ps, D)
    if fp8:
        kc = r.integers(0, 0x7E, size=shape, dtype=np.uint8)
        vc = r.integers(0, 0x7E, size=shape, dtype=np.uint8)
        sc = (r.random((2, num_pages, Hkv, ps)).astype(np.float32) if per_token
              else np.array([0.02, 0.005], dtype=np.float32))
    else:
        kc = r.integers(0, 0x3F80, size=shape, dtype=np.uint16)
        vc = r.integers(0, 0x3F80, size=shape, dtype=np.uint16)
        sc = None
    return nk, nv, bt, ctx, q_len, ps, kc, vc, sc


def _positions(bt, ctx, q_len, ps):
    for b in range(len(ctx)):
        for i in range(q_len):
            t = int(ctx[b]) - q_len + i
            yield b, i, int(bt[b, t // ps]), t % ps


def test_bf16_append_writes_exactly_the_new_rows():
    nk, nv, bt, ctx, q_len, ps, kc, vc, sc = _case(False, False)
    k2, v2, _, st = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, False, False)
    assert st == 0
    touched = np.zeros(kc.shape[:3], dtype=bool)
    for b, i, page, slot in _positions(bt, ctx, q_len, ps):
        assert np.array_equal(k2[page, :, slot], nk[b, i])
        assert np.array_equal(v2[page, :, slot], nv[b, i])
        touched[page, :, slot] = True
    assert np.array_equal(k2[~touched], kc[~touched]) and np.array_equal(v2[~touched], vc[~touched])
    # read back through the oracle's own gather: the last q_len tokens
    for b in range(len(ctx)):
        for g in range(nk.shape[2]):
            got = oracle.gather_rows(k2, bt, b, g, int(ctx[b]), ps)
            assert np.array_equal(got[int(ctx[b]) - q_len:], nk[b, :, g])


def test_per_token_append_scale_and_codes():
    nk, nv, bt, ctx, q_len, ps, kc, vc, sc = _case(True, True)
    nk[0, 0, 1] = 0  # an all-zero row
    k2, v2, s2, st = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, True, True, sc)
    assert st == 0
    for b, i, page, slot in _positions(bt, ctx, q_len, ps):
        for which, (src, dst) in enumerate(((nk, k2), (nv, v2))):
            for g in range(src.shape[2]):
                x = _bits_to_f32(src[b, i, g]).astype(np.float64)
                s = s2[which, page, g, slot]
                deq = oracle.e4m3fn_to_f64(dst[page, g, slot])
                if not x.any():
                    assert s == 1 and not deq.any()
                    continue
                # closed forms: scale = max|x| / 448 in float32; the largest
                # element lands on the largest code
                assert s == np.float32(np.float32(np.abs(x).max()) / np.float32(448))
                assert np.abs(deq).max() == 448
                # error bound of a 3-bit-mantissa rounding: half a unit in the
                # last place, 2^-4 relative for normals, 2^-10 absolute below
                err = np.abs(deq * s - x)
                assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * s) * (1 + 1e-6))


def test_per_tensor_append_uses_the_given_scales_and_clamps():
    nk, nv, bt, ctx, q_len, ps, kc, vc, sc = _case(True, False)
    k2, v2, s2, st = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, True, False, sc)
    assert st == 0 and np.array_equal(s2, sc)
    for b, i, page, slot in _positions(bt, ctx, q_len, ps):
        x = _bits_to_f32(nk[b, i]).astype(np.float64)   # |x| up to ~10: x / 0.02 > 448 clamps
        deq = oracle.e4m3fn_to_f64(k2[page, :, slot])
        big = np.abs(x / 0.02) >= 448
        assert np.all(np.abs(deq[big]) == 448)
        assert np.array_equal(np.sign(deq[x != 0]), np.sign(x[x != 0]))


def test_bad_context_and_bad_page_are_skipped_and_reported():
    nk, nv, bt, ctx, q_len, ps, kc, vc, sc = _case(False, False)
    ctx_bad = ctx.copy()
    ctx_bad[0] = q_len - 1
    k2, v2, _, st = cache.append(nk, nv, bt, ctx_bad, q_len, ps, kc, vc, False, False)
    assert st == cache.BAD_CONTEXT
    for b, i, page, slot in _positions(bt, ctx, q_len, ps):
        if b == 0:
            assert np.array_equal(k2[page, :, slot], kc[page, :, slot])
    bt_bad = bt.copy()
    t = int(ctx[1]) - 1
    bt_bad[1, t // ps] = kc.shape[0]          # past the pool
    k3, _, _, st = cache.append(nk, nv, bt_bad, ctx, q_len, ps, kc, vc, False, False)
    assert st == cache.BAD_PAGE


def test_generator_quantiser_agrees_with_the_oracle_rule():
    # the seeded workloads quantise their float32 draws with torch's cast;
    # the oracle's rule gives the same bytes for the same scale
    r = np.random.default_rng(5)
    x = (r.standard_normal((64, 128)) * 2).astype(np.float32)
    amax = np.abs(x).max(axis=1)
    s = (amax / np.float32(448)).astype(np.float32)
    got = W.quantise_e4m3fn(torch.from_numpy(x), torch.from_numpy(s).unsqueeze(-1)).numpy()
    want = np.stack([cache.quantise_row(x[i], s[i]) for i in range(64)])
    assert np.array_equal(got, want)
