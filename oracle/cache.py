"""KV-cache append: the write side of the paged cache (test infrastructure only).

The pages read K and V page by page from a paged cache through a block table
(Ascend/RecSDK issue #1281, "背景与优化特性") and quantise the fp8 cache per
token and head or per tensor ("[Kernel][Perf] Optimize paged-attention
metadata decode", ROCm/FlyDSL PR #910, "Pull request overview"); how tokens
get into the cache is not written down. The plainest reading, which this
function follows:

  * sequence b's appended token i (of q_len) sits at position
    t = ctx_b - q_len + i, in physical page block_table[b, t // page_size],
    slot t % page_size, at kv head g;
  * a bf16 cache stores the token's K and V rows as they are;
  * an fp8 cache with per-token-head scales stores, for each of K and V,
    scale = max_d |x_d| / 448 (1 when the row is all zero) and the bytes
    e4m3fn(clamp(x_d / scale, -448, 448)), rounded to nearest even;
  * with a per-tensor scale the caller's scale is used the same way.

Every float decision that feeds an integer code (the maximum, the two
divisions, the clamp) is taken in float32, the precision the kernel works in;
the encoding itself is exact. A sequence whose context length lies outside
[max(1, q_len), max_pages_per_seq * page_size] is skipped and reported as bad
context (bit 1); a row whose page entry lies outside [0, num_pages) is
skipped and reported as a bad page (bit 2).
"""
from __future__ import annotations

import numpy as np

from .codecs import e4m3fn_encode

BAD_CONTEXT = 1
BAD_PAGE = 2
E4M3FN_MAX = np.float32(448.0)


def quantise_row(x_f32: np.ndarray, scale: np.float32) -> np.ndarray:
    """e4m3fn(clamp(x / scale, +-448)) with the division in float32 (a quotient
    past the float32 range is infinite, and the clamp takes it to +-448)."""
    with np.errstate(over="ignore"):
        y = (x_f32.astype(np.float32) / np.float32(scale)).astype(np.float32)
    y = np.clip(y, -E4M3FN_MAX, E4M3FN_MAX)
    return e4m3fn_encode(y)


def row_scale(x_f32: np.ndarray) -> np.float32:
    """max |x| / 448 in float32, or 1 for an all-zero row."""
    amax = np.float32(np.max(np.abs(x_f32.astype(np.float32))))
    return np.float32(1.0) if amax == 0 else np.float32(amax / E4M3FN_MAX)


def append(new_k_bits, new_v_bits, block_table, context_lens, q_len: int, page_size: int,
           k_cache, v_cache, fp8: bool, per_token: bool, kv_scales=None):
    """Returns (k_cache, v_cache, kv_scales, status) after the append; the
    inputs are not modified.

    new_k_bits, new_v_bits  [B, q_len, Hkv, D] bf16 bit patterns (uint16)
    k_cache, v_cache        [num_pages, Hkv, page_size, D] uint16 (bf16) or
                            uint8 (e4m3fn) arrays
    kv_scales               per token: [2, num_pages, Hkv, page_size] float32
                            (updated at the written slots); per tensor: [2]
                            float32 (read); None for bf16
    """
    nk = np.asarray(new_k_bits).astype(np.uint16)
    nv = np.asarray(new_v_bits).astype(np.uint16)
    kc = np.array(k_cache, copy=True)
    vc = np.array(v_cache, copy=True)
    sc = None if kv_scales is None else np.array(kv_scales, dtype=np.float32, copy=True)
    bt = np.asarray(block_table)
    ctxs = np.asarray(context_lens).astype(np.int64)
    B, QL, Hkv, D = nk.shape
    assert QL == q_len
    num_pages = kc.shape[0]
    cap = bt.shape[1] * page_size
    status = 0

    def to_f32(bits):
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)

    for b in range(B):
        ctx = int(ctxs[b])
        if ctx < max(1, q_len) or ctx > cap:
            status |= BAD_CONTEXT
            continue
        for i in range(q_len):
            t = ctx - q_len + i
            page = int(bt[b, t // page_size])
            if page < 0 or page >= num_pages:
                status |= BAD_PAGE
                continue
            slot = t % page_size
            for g in range(Hkv):
                for which, (src, dst) in enumerate(((nk, kc), (nv, vc))):
                    bits = src[b, i, g]
                    if not fp8:
                        dst[page, g, slot] = bits
                        continue
                    x = to_f32(bits)
                    if per_token:
                        s = row_scale(x)
                        sc[which, page, g, slot] = s
                    else:
                        s = np.float32(sc[which])
                    dst[page, g, slot] = quantise_row(x, s)
    return kc, vc, sc, status
