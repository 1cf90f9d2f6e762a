"""Decode attention over a paged KV cache, in float64 (test infrastructure only).

What is computed. The pages name the operation — paged attention decode with
a block table, grouped query heads ("h16_kv1" in the shape keys of
hw-native-sys/simpler issue #998, table "Same-Shape Side-by-Side"), a
split-KV "split reducer" / "reduction kernel" (ROCm/FlyDSL PR #910, "Pull
request overview") and a paged KV cache read page by page (Ascend/RecSDK issue
#1281, section "背景与优化特性", background) — but never write the formula. The
plainest reading, used here, is scaled-dot-product softmax attention of each
query row over the gathered keys it may see:

  for sequence b with context length ctx (which counts the q_len appended
  tokens, already in the cache), query i in [0, q_len) and query head h:
    g      = h // (Hq / Hkv)                      (contiguous head groups)
    K[t]   = dequant(k_cache[block_table[b, t // ps], g, t % ps, :]), t < ctx
    V[t]   likewise
    seen   = { t : 0 <= t <= ctx - q_len + i }    (bottom-right causal mask)
    s_t    = scale * <q[b, i, h, :], K[t]>        for t in seen
    p      = exp(s - max s) / sum(exp(s - max s))
    out    = sum_t p_t V[t]

dequant is exact bf16 -> float, or e4m3fn(byte) * scale where the scale is
one number per tensor (K, V) or one per (page, kv head, slot).

The split form follows the same definition restricted to a token range
[t0, t1): it returns the normalised partial output and its log-sum-exp, and
partials merge by weights exp(lse_s - max lse). Both are exact identities of
the softmax, so the merged result equals the unsplit one up to rounding.
"""
from __future__ import annotations

import numpy as np

from .codecs import bf16_bits_to_f64, e4m3fn_to_f64, round_to_bf16

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3fn"
SCALE_NONE = "none"
SCALE_PER_TENSOR = "per_tensor"
SCALE_PER_TOKEN_HEAD = "per_token_head"


def _np(x):
    """torch tensor or array -> numpy (no copy for CPU tensors)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if str(x.dtype) == "torch.bfloat16":
            x = x.view(__import__("torch").int16)
        return x.numpy()
    return np.asarray(x)


def gather_rows(cache, block_table, b: int, g: int, ctx: int, page_size: int) -> np.ndarray:
    """Raw cache rows of (sequence b, kv head g) for tokens 0..ctx-1, in token order.

    Row t is cache[block_table[b, t // page_size], g, t % page_size, :]. The
    result keeps the cache's storage type (bf16 bits or e4m3fn bytes).
    """
    cache = _np(cache)
    bt = _np(block_table)
    t = np.arange(ctx)
    pages = bt[b, t // page_size].astype(np.int64)
    return cache[pages, g, t % page_size, :]


def _gather_scales(kv_scales, which: int, block_table, b, g, ctx, page_size):
    sc = _np(kv_scales)
    bt = _np(block_table)
    t = np.arange(ctx)
    return sc[which, bt[b, t // page_size].astype(np.int64), g, t % page_size].astype(np.float64)


def dequant_rows(raw, kv_dtype: str, scale_mode: str, kv_scales, which: int,
                 block_table=None, b=0, g=0, ctx=0, page_size=1) -> np.ndarray:
    """Gathered raw rows -> float64 values (which = 0 for K, 1 for V)."""
    if kv_dtype == KV_BF16:
        if scale_mode != SCALE_NONE:
            raise ValueError("bf16 KV takes no scales")
        return bf16_bits_to_f64(raw)
    if kv_dtype != KV_FP8:
        raise ValueError(kv_dtype)
    vals = e4m3fn_to_f64(raw)
    if scale_mode == SCALE_PER_TENSOR:
        return vals * float(_np(kv_scales)[which])
    if scale_mode == SCALE_PER_TOKEN_HEAD:
        s = _gather_scales(kv_scales, which, block_table, b, g, ctx, page_size)
        return vals * s[:, None]
    raise ValueError("fp8 KV needs a scale mode")


def _pair_inputs(q, k_cache, v_cache, block_table, context_lens, b, g, q_len, kv_dtype,
                 scale_mode, kv_scales, page_size):
    ctx = int(_np(context_lens)[b])
    qn = _np(q)
    Hq = qn.shape[2]
    Hkv = _np(k_cache).shape[1]
    group = Hq // Hkv
    K = dequant_rows(gather_rows(k_cache, block_table, b, g, ctx, page_size), kv_dtype,
                     scale_mode, kv_scales, 0, block_table, b, g, ctx, page_size)
    V = dequant_rows(gather_rows(v_cache, block_table, b, g, ctx, page_size), kv_dtype,
                     scale_mode, kv_scales, 1, block_table, b, g, ctx, page_size)
    # Query rows of this kv head, ordered r = i * group + local head.
    Q = bf16_bits_to_f64(qn[b, :, g * group:(g + 1) * group, :]).reshape(q_len * group, -1)
    return ctx, group, Q, K, V


def _visible(ctx: int, q_len: int, group: int, t0: int, t1: int) -> np.ndarray:
    """mask[r, t - t0] = key t visible to row r (query i = r // group)."""
    i = np.arange(q_len * group) // group
    t = np.arange(t0, t1)
    return t[None, :] <= (ctx - q_len + i)[:, None]


def decode(q, k_cache, v_cache, block_table, context_lens, q_len: int, scale: float,
           page_size: int, kv_dtype: str = KV_BF16, scale_mode: str = SCALE_NONE,
           kv_scales=None):
    """Decode attention output, float64 [B, q_len, Hq, D], and its bf16 rounding."""
    qn = _np(q)
    B, _, Hq, D = qn.shape
    Hkv = _np(k_cache).shape[1]
    out = np.zeros((B, q_len, Hq, D), dtype=np.float64)
    for b in range(B):
        for g in range(Hkv):
            ctx, group, Q, K, V = _pair_inputs(q, k_cache, v_cache, block_table, context_lens,
                                               b, g, q_len, kv_dtype, scale_mode, kv_scales,
                                               page_size)
            s = scale * (Q @ K.T)
            s = np.where(_visible(ctx, q_len, group, 0, ctx), s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            p = np.exp(s)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, g * group:(g + 1) * group, :] = (p @ V).reshape(q_len, group, D)
    return out, round_to_bf16(out)


def attend_range(q, k_cache, v_cache, block_table, context_lens, q_len: int, scale: float,
                 page_size: int, b: int, g: int, t0: int, t1: int, kv_dtype: str = KV_BF16,
                 scale_mode: str = SCALE_NONE, kv_scales=None):
    """Partial attention of the rows of pair (b, g) over keys [t0, t1).

    Returns (o [R, D], lse [R]) with R = q_len * group rows r = i * group + j:
      m = max of the visible scores, l = sum exp(s - m),
      o = sum exp(s - m) V / l,  lse = m + ln l.
    A row that sees no key of the range gets o = 0 and lse = -inf.
    """
    ctx, group, Q, K, V = _pair_inputs(q, k_cache, v_cache, block_table, context_lens, b, g,
                                       q_len, kv_dtype, scale_mode, kv_scales, page_size)
    R, D = Q.shape
    t1 = min(t1, ctx)
    o = np.zeros((R, D), dtype=np.float64)
    lse = np.full(R, -np.inf)
    if t1 <= t0:
        return o, lse
    s = scale * (Q @ K[t0:t1].T)
    vis = _visible(ctx, q_len, group, t0, t1)
    for r in range(R):
        sr = s[r][vis[r]]
        if sr.size == 0:
            continue
        m = sr.max()
        w = np.exp(sr - m)
        l = w.sum()
        o[r] = (w @ V[t0:t1][vis[r]]) / l
        lse[r] = m + np.log(l)
    return o, lse


def merge_partials(os_, lses):
    """Log-sum-exp merge: out = sum_s w_s o_s / sum_s w_s, w_s = exp(lse_s - max lse).

    os_ [S, R, D], lses [S, R]. A partial with lse = -inf has weight 0.
    """
    os_ = np.asarray(os_, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    M = lses.max(axis=0)
    w = np.where(np.isneginf(lses), 0.0, np.exp(lses - M[None, :]))
    return (w[:, :, None] * os_).sum(axis=0) / w.sum(axis=0)[:, None]


def decode_split(q, k_cache, v_cache, block_table, context_lens, q_len: int, scale: float,
                 page_size: int, partition: int, kv_dtype: str = KV_BF16,
                 scale_mode: str = SCALE_NONE, kv_scales=None):
    """Split-KV decode: partitions [k*P, min((k+1)*P, ctx)) counted from token 0,
    each attended alone, then merged by merge_partials. float64 [B, q_len, Hq, D]."""
    qn = _np(q)
    B, _, Hq, D = qn.shape
    Hkv = _np(k_cache).shape[1]
    group = Hq // Hkv
    ctxs = _np(context_lens)
    out = np.zeros((B, q_len, Hq, D), dtype=np.float64)
    for b in range(B):
        ctx = int(ctxs[b])
        for g in range(Hkv):
            parts = [attend_range(q, k_cache, v_cache, block_table, context_lens, q_len, scale,
                                  page_size, b, g, t0, t0 + partition, kv_dtype, scale_mode,
                                  kv_scales)
                     for t0 in range(0, ctx, partition)]
            o = merge_partials([p[0] for p in parts], [p[1] for p in parts])
            out[b, :, g * group:(g + 1) * group, :] = o.reshape(q_len, group, D)
    return out
