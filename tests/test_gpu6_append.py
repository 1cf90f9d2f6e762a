"""KV-cache append on the GPU vs the oracle's rule: cache bytes and scales bit
for bit, every bf16 value through the fp8 encode, bad rows reported and left
alone, and append followed by decode."""
import numpy as np
import pytest
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from oracle import cache
from tests.gpu_util import DEV, KV_CODE, MODE_CODE, Dev, check, run, say, to_f64
from tests.helpers import assert_close

pytestmark = pytest.mark.gpu


def _dims(B, q_len, Hkv, D, ps, num_pages, maxp, fp8, mode):
    return pa.make_dims(batch=B, q_len=q_len, num_q_heads=Hkv, num_kv_heads=Hkv, head_dim=D,
                        page_size=ps, num_pages=num_pages, max_pages_per_seq=maxp,
                        kv_dtype=pa.PA_KV_FP8_E4M3FN if fp8 else pa.PA_KV_BF16,
                        kv_scale_mode=mode)


def _bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().astype(np.uint16)


def _draw(seed, B, q_len, Hkv, D, ps, maxp, fp8, mode):
    """New tokens (a mix of scales, an all-zero row and a one-hot row), context
    lengths that put some tokens across a page boundary, a shuffled block
    table and caches / scales full of noise."""
    r = np.random.default_rng(seed)
    num_pages = B * maxp + 3
    ctx = r.integers(q_len, maxp * ps + 1, size=B).astype(np.int32)
    ctx[0] = q_len                      # the first tokens of a sequence
    if B > 1:
        ctx[1] = min(maxp * ps, ps + q_len // 2 + 1)   # straddles pages 0 and 1
    bt = np.full((B, maxp), -1, dtype=np.int32)
    perm = r.permutation(num_pages)
    for b in range(B):
        n = -(-int(ctx[b]) // ps)
        bt[b, :n] = perm[b * maxp:b * maxp + n]
    mag = np.exp(r.uniform(-6, 6, size=(B, q_len, Hkv, 1)))
    nk = r.standard_normal((B, q_len, Hkv, D)) * mag
    nv = r.standard_normal((B, q_len, Hkv, D)) * mag[::-1]
    nk[0, 0, 0] = 0.0
    nv[-1, -1, -1] = 0.0
    nv[-1, -1, -1, 3] = -2.5
    nk, nv = _bf16_bits(nk), _bf16_bits(nv)
    shape = (num_pages, Hkv, ps, D)
    if fp8:
        kc = r.integers(0, 0x7E, size=shape, dtype=np.uint8)
        vc = r.integers(0, 0x7E, size=shape, dtype=np.uint8)
        sc = (r.random((2, num_pages, Hkv, ps)).astype(np.float32)
              if mode == pa.PA_SCALE_PER_TOKEN_HEAD else np.array([0.03, 0.011], dtype=np.float32))
    else:
        kc = r.integers(0, 0x3F80, size=shape, dtype=np.uint16)
        vc = r.integers(0, 0x3F80, size=shape, dtype=np.uint16)
        sc = None
    return nk, nv, bt, ctx, kc, vc, sc, num_pages


def _dev(x, dtype):
    return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).view(dtype).to(DEV)


def _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc):
    cdt = torch.uint8 if kc.dtype == np.uint8 else torch.int16
    k = _dev(kc.view(np.int16) if cdt == torch.int16 else kc, cdt)
    v = _dev(vc.view(np.int16) if cdt == torch.int16 else vc, cdt)
    s = _dev(sc, torch.float32)
    st = torch.zeros(1, dtype=torch.int32, device=DEV)
    pa.pa_cache_append(dims, _dev(nk.view(np.int16), torch.int16), _dev(nv.view(np.int16), torch.int16),
                       _dev(bt, torch.int32), _dev(ctx, torch.int32), k, v, s, st)
    torch.cuda.synchronize()
    back = lambda t, npdt: t.cpu().numpy().view(npdt)
    npdt = np.uint8 if cdt == torch.uint8 else np.uint16
    return back(k, npdt), back(v, npdt), None if s is None else s.cpu().numpy(), int(st.item())


CASES = {
    # name: (B, q_len, Hkv, D, page size, max pages, fp8, scale mode)
    "bf16_c3_like": (6, 1, 8, 128, 16, 8, False, pa.PA_SCALE_NONE),
    "bf16_c5_like": (2, 8, 16, 256, 32, 4, False, pa.PA_SCALE_NONE),
    "fp8_tok_q4": (5, 4, 1, 128, 1024, 2, True, pa.PA_SCALE_PER_TOKEN_HEAD),
    "fp8_ten_q4": (5, 4, 1, 128, 1024, 2, True, pa.PA_SCALE_PER_TENSOR),
    "fp8_tok_d256": (3, 8, 4, 256, 16, 4, True, pa.PA_SCALE_PER_TOKEN_HEAD),
    "fp8_ten_d256": (3, 8, 4, 256, 16, 4, True, pa.PA_SCALE_PER_TENSOR),
}


def _random_case(i):
    import random
    r = random.Random(9100 + i)
    ps = r.choice([16, 32, 64, 128, 256, 512, 1024])
    q_len = r.choice([1, 1, 2, 3, 4, 8, 16])
    maxp = max(r.randint(1, 6), -(-q_len // ps))
    fp8 = r.random() < 0.6
    mode = (r.choice([pa.PA_SCALE_PER_TOKEN_HEAD, pa.PA_SCALE_PER_TENSOR]) if fp8
            else pa.PA_SCALE_NONE)
    return (r.randint(1, 7), q_len, r.choice([1, 2, 4, 8, 16]), r.choice([128, 256]), ps, maxp,
            fp8, mode)


@pytest.mark.parametrize("i", range(32))
def test_append_random_shapes_bitwise(i):
    """Seeded random shapes (batch, q_len, kv heads, head_dim, page size,
    capacity, dtype and scale mode drawn together), cache bytes and scales
    bit for bit against the oracle."""
    B, q_len, Hkv, D, ps, maxp, fp8, mode = _random_case(i)
    nk, nv, bt, ctx, kc, vc, sc, num_pages = _draw(300 + i, B, q_len, Hkv, D, ps, maxp, fp8, mode)
    say(f"[append random {i}] B={B} q_len={q_len} Hkv={Hkv} D={D} page={ps} maxp={maxp} "
        f"fp8={fp8} mode={mode} ctx={ctx.tolist()}")
    dims = _dims(B, q_len, Hkv, D, ps, num_pages, maxp, fp8, mode)
    gk, gv, gs, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    wk, wv, ws, wst = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, fp8,
                                   mode == pa.PA_SCALE_PER_TOKEN_HEAD, sc)
    assert st == wst == 0
    assert np.array_equal(gk, wk) and np.array_equal(gv, wv)
    if ws is not None:
        assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("name", list(CASES))
def test_append_matches_oracle_bitwise(name):
    B, q_len, Hkv, D, ps, maxp, fp8, mode = CASES[name]
    nk, nv, bt, ctx, kc, vc, sc, num_pages = _draw(11, B, q_len, Hkv, D, ps, maxp, fp8, mode)
    say(f"[append] {name} ctx={ctx.tolist()}")
    dims = _dims(B, q_len, Hkv, D, ps, num_pages, maxp, fp8, mode)
    gk, gv, gs, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    wk, wv, ws, wst = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, fp8,
                                   mode == pa.PA_SCALE_PER_TOKEN_HEAD, sc)
    assert st == wst == 0
    assert np.array_equal(gk, wk) and np.array_equal(gv, wv)
    if ws is not None:
        assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))


def test_every_bf16_value_encodes_like_the_oracle():
    """Per-tensor scale 1: the kernel's fp8 encode of every finite bf16 value
    (the +-448 clamp included; all E4M3FN midpoints are bf16 values) equals
    the oracle's round-to-nearest-even encoder."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    with np.errstate(invalid="ignore"):
        x = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    bits = bits[np.isfinite(x)]
    D, Hkv, q_len, ps = 128, 1, 8, 16
    rows = -(-len(bits) // D)
    B = -(-rows // q_len)
    flat = np.zeros(B * q_len * D, dtype=np.uint16)
    flat[:len(bits)] = bits
    nk = flat.reshape(B, q_len, Hkv, D)
    nv = nk[::-1].copy()
    ctx = np.full(B, q_len, dtype=np.int32)
    bt = np.arange(B, dtype=np.int32).reshape(B, 1)
    kc = np.zeros((B, Hkv, ps, D), dtype=np.uint8)
    vc = np.zeros_like(kc)
    sc = np.array([1.0, 1.0], dtype=np.float32)
    say(f"[append] exhaustive encode over {len(bits)} bf16 values")
    dims = _dims(B, q_len, Hkv, D, ps, B, 1, True, pa.PA_SCALE_PER_TENSOR)
    gk, gv, _, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    assert st == 0
    x = (nk.astype(np.uint32) << np.uint32(16)).view(np.float32).reshape(B, q_len, D)
    want = oracle.e4m3fn_encode(np.clip(x, -448, 448))
    assert np.array_equal(gk[:, 0, :q_len], want)


def test_bad_context_and_bad_page_are_reported_and_not_written():
    B, q_len, Hkv, D, ps, maxp = 3, 2, 2, 128, 16, 3
    nk, nv, bt, ctx, kc, vc, sc, num_pages = _draw(5, B, q_len, Hkv, D, ps, maxp, True,
                                                    pa.PA_SCALE_PER_TOKEN_HEAD)
    ctx = ctx.copy()
    ctx[0] = q_len - 1                        # shorter than the appended tokens
    bt = bt.copy()
    t = int(ctx[2]) - 1
    bt[2, t // ps] = num_pages + 5            # past the pool
    say("[append] bad context + bad page")
    dims = _dims(B, q_len, Hkv, D, ps, num_pages, maxp, True, pa.PA_SCALE_PER_TOKEN_HEAD)
    gk, gv, gs, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    wk, wv, ws, wst = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, True, True, sc)
    assert st == wst == pa.PA_DEV_BAD_CONTEXT | pa.PA_DEV_BAD_PAGE
    assert np.array_equal(gk, wk) and np.array_equal(gv, wv)
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))


@pytest.mark.parametrize("name", ["fp8_tok_q4", "bf16_c5_like"])
def test_append_then_decode(name):
    """A seeded workload whose last q_len tokens are written by the append
    kernel decodes like the oracle on the oracle-appended cache."""
    base = {"fp8_tok_q4": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=300, ctx_hi=2500, max_ctx=3072),
            "bf16_c5_like": W.scaled(W.C5, batch=2, ctx_lo=100, ctx_hi=1200, max_ctx=1280,
                                     pool_slack=0.2)}[name]
    w = W.generate(base, 2026)
    s = w.spec
    fp8 = s.kv_dtype == W.KV_FP8
    per_tok = s.kv_scale_mode == W.SCALE_PER_TOKEN_HEAD
    r = np.random.default_rng(3)
    nk = _bf16_bits(r.standard_normal((s.batch, s.q_len, s.num_kv_heads, s.head_dim)))
    nv = _bf16_bits(r.standard_normal((s.batch, s.q_len, s.num_kv_heads, s.head_dim)))
    bt = w.block_table.numpy()
    ctx = w.context_lens.numpy()
    kc = w.k_cache.numpy() if fp8 else w.k_cache.view(torch.int16).numpy().view(np.uint16)
    vc = w.v_cache.numpy() if fp8 else w.v_cache.view(torch.int16).numpy().view(np.uint16)
    sc = None if w.kv_scales is None else w.kv_scales.numpy()
    say(f"[append] append + decode {name}")
    dims = pa.make_dims(batch=s.batch, q_len=s.q_len, num_q_heads=s.num_q_heads,
                        num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, page_size=s.page_size,
                        num_pages=w.num_pages, max_pages_per_seq=s.max_pages_per_seq,
                        kv_dtype=KV_CODE[s.kv_dtype], kv_scale_mode=MODE_CODE[s.kv_scale_mode])
    gk, gv, gs, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    wk, wv, ws, _ = cache.append(nk, nv, bt, ctx, s.q_len, s.page_size, kc, vc, fp8, per_tok, sc)
    assert st == 0 and np.array_equal(gk, wk) and np.array_equal(gv, wv)
    to_t = (lambda a: torch.from_numpy(a)) if fp8 else (lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16))
    w2 = W.Workload(s, w.seed, w.q, to_t(gk), to_t(gv), w.block_table, w.context_lens,
                    None if gs is None else torch.from_numpy(gs), w.num_pages)
    out, _ = run(w2)
    check(w2, out, f"append + decode {name}")


def test_quotients_near_code_boundaries_encode_like_the_oracle():
    """Per-tensor scales that are not powers of two, applied to values at and
    around every E4M3FN midpoint times the scale (the f32 quotient then
    decides the code), and per-token rows over a wide range of magnitudes:
    bytes and scales equal the oracle's bit for bit."""
    vals = oracle.e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
    mids = (vals[1:] + vals[:-1]) / 2
    D, q_len, ps = 128, 8, 16
    r = np.random.default_rng(9)
    for scale in (0.0173, 0.3, 1.7, 3.0e-3, 1.0 / 3.0, 91.0):
        x = np.concatenate([mids, -mids, mids * (1 + 2.0 ** -9), mids * (1 - 2.0 ** -9)]) * scale
        x = np.concatenate([x, r.standard_normal(2 * D * q_len * 4) * scale * 100])
        n = -(-len(x) // (D * q_len)) * D * q_len
        x = np.pad(x, (0, n - len(x)))
        B = n // (D * q_len)
        nk = _bf16_bits(x.reshape(B, q_len, 1, D))
        nv = _bf16_bits(-x[::-1].reshape(B, q_len, 1, D))
        ctx = np.full(B, q_len, dtype=np.int32)
        bt = np.arange(B, dtype=np.int32).reshape(B, 1)
        kc = np.zeros((B, 1, ps, D), dtype=np.uint8)
        vc = np.zeros_like(kc)
        sc = np.array([scale, scale * 0.77], dtype=np.float32)
        dims = _dims(B, q_len, 1, D, ps, B, 1, True, pa.PA_SCALE_PER_TENSOR)
        gk, gv, _, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
        wk, wv, _, _ = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, True, False, sc)
        assert st == 0 and np.array_equal(gk, wk) and np.array_equal(gv, wv), f"scale {scale}"
    # per token: magnitudes from 1e-30 to 1e30 across rows
    B, q_len, Hkv = 16, 8, 2
    mag = 10.0 ** r.uniform(-30, 30, size=(B, q_len, Hkv, 1))
    nk = _bf16_bits(r.standard_normal((B, q_len, Hkv, D)) * mag)
    nv = _bf16_bits(r.standard_normal((B, q_len, Hkv, D)) * mag[:, ::-1])
    ctx = np.full(B, q_len, dtype=np.int32)
    bt = np.arange(B, dtype=np.int32).reshape(B, 1)
    kc = np.zeros((B, Hkv, ps, D), dtype=np.uint8)
    vc = np.zeros_like(kc)
    sc = np.zeros((2, B, Hkv, ps), dtype=np.float32)
    dims = _dims(B, q_len, Hkv, D, ps, B, 1, True, pa.PA_SCALE_PER_TOKEN_HEAD)
    gk, gv, gs, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    wk, wv, ws, _ = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, True, True, sc)
    assert st == 0 and np.array_equal(gk, wk) and np.array_equal(gv, wv)
    assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))


def _rows_case(nk_rows, nv_rows, per_token, sc=None):
    """Rows [n, D] of bf16 bits appended one per sequence (q_len 1, one kv
    head, page 16): GPU bytes and scales vs the oracle, bit for bit."""
    n, D = nk_rows.shape
    q_len, ps = 1, 16
    nk = nk_rows.reshape(n, q_len, 1, D)
    nv = nv_rows.reshape(n, q_len, 1, D)
    ctx = np.full(n, 1, dtype=np.int32)
    bt = np.arange(n, dtype=np.int32).reshape(n, 1)
    kc = np.zeros((n, 1, ps, D), dtype=np.uint8)
    vc = np.zeros_like(kc)
    mode = pa.PA_SCALE_PER_TOKEN_HEAD if per_token else pa.PA_SCALE_PER_TENSOR
    if per_token:
        sc = np.zeros((2, n, 1, ps), dtype=np.float32)
    dims = _dims(n, q_len, 1, D, ps, n, 1, True, mode)
    gk, gv, gs, st = _gpu_append(dims, nk, nv, bt, ctx, kc, vc, sc)
    wk, wv, ws, _ = cache.append(nk, nv, bt, ctx, q_len, ps, kc, vc, True, per_token, sc)
    assert st == 0
    bad = np.argwhere(gk != wk)
    assert np.array_equal(gk, wk), f"K bytes differ at {bad[:5].tolist()}"
    assert np.array_equal(gv, wv)
    if per_token:
        assert np.array_equal(gs.view(np.uint32), ws.view(np.uint32))


def test_tiny_rows_and_tiny_scales_encode_like_the_oracle():
    """Rows whose largest magnitude is tiny (per-token scales down to
    subnormal float32, where 1 / scale overflows) and tiny per-tensor scales:
    the quotient x / scale is still an ordinary number, and zeros keep their
    sign."""
    r = np.random.default_rng(21)
    D = 128
    mags = np.array([2.0 ** -133, 2.0 ** -126, 1e-38, 1e-37, 3e-36, 1e-30, 2.0 ** -61, 2.0 ** -59,
                     1e-12, 1.0])
    rows = []
    for m in mags:
        x = r.uniform(-1, 1, size=D) * m
        x[0] = m                                    # the row maximum
        x[1], x[2] = 0.0, -0.0
        rows.append(x)
    bits = _bf16_bits(np.array(rows))
    bits[:, 2] = 0x8000                             # an explicit -0
    say("[append] tiny per-token rows")
    _rows_case(bits, bits[::-1].copy(), per_token=True)
    for scale in (2.0 ** -149, 1e-40, 2.0 ** -70, 1e-30):
        say(f"[append] per-tensor scale {scale:g}")
        _rows_case(bits, bits[::-1].copy(), per_token=False,
                   sc=np.array([scale, scale * 0.75], dtype=np.float32))


def test_every_row_maximum_gives_the_oracle_scale_and_codes():
    """Per-token rows whose maximum magnitude is each positive finite bf16
    value in turn: the row scale max / 448 and every code match the oracle
    bit for bit (the other elements are the maximum times random fractions,
    rounded to bf16, with signs)."""
    r = np.random.default_rng(5)
    D = 128
    m_bits = np.arange(1, 0x7F80, dtype=np.uint32)          # +bf16 subnormals .. max finite
    m = (m_bits << np.uint32(16)).view(np.float32).astype(np.float64)
    x = r.uniform(-1, 1, size=(len(m), D)) * m[:, None]
    bits = _bf16_bits(x)
    bits[:, 0] = m_bits.astype(np.uint16)
    # bf16 rounding of the fractions may not exceed the maximum (|frac| < 1)
    say(f"[append] {len(m)} rows, every positive finite bf16 maximum")
    _rows_case(bits, np.roll(bits, 7, axis=0), per_token=True)
