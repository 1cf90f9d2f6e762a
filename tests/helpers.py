"""Test helpers: contiguous <-> paged layout, brute-force attention, tolerances.

Nothing here is used by the library; the brute force is a second, independent
statement of decode attention (plain Python loops over rows, keys and dims on a
contiguous cache, no paging, no vectorisation) used to pin the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# Tolerances of |gpu - oracle| <= atol + rtol * |oracle|: the CPU FP32
# reference criterion rtol = atol = 8e-3 of Ascend/RecSDK issue #1281
# (section "其他相关讨论", correctness) for bf16 KV, and 2e-2 for fp8 KV.
TOL_BF16 = 8e-3
TOL_FP8 = 2e-2


def bf16_round(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def to_paged(kc: torch.Tensor, ctxs, page_size: int, pool: int, rng: np.random.Generator,
             fill=0):
    """Scatter contiguous rows kc [B, Hkv, T, D] into a page pool.

    Returns (cache [pool, Hkv, page_size, D], block_table [B, maxp] int32) with
    pages placed by a random permutation of the pool.
    """
    B, Hkv, T, D = kc.shape
    maxp = -(-T // page_size)
    need = sum(-(-int(c) // page_size) for c in ctxs)
    assert need <= pool
    perm = rng.permutation(pool)
    cache = torch.full((pool, Hkv, page_size, D), fill, dtype=kc.dtype)
    bt = torch.full((B, maxp), -1, dtype=torch.int32)
    off = 0
    for b in range(B):
        n = -(-int(ctxs[b]) // page_size)
        for j in range(n):
            pg = int(perm[off + j])
            bt[b, j] = pg
            t0, t1 = j * page_size, min((j + 1) * page_size, int(ctxs[b]))
            cache[pg, :, : t1 - t0] = kc[b, :, t0:t1]
        off += n
    return cache, bt


def brute_force(Q, K, V, ctxs, q_len: int, scale: float) -> np.ndarray:
    """Decode attention with explicit loops on contiguous float64 arrays.

    Q [B, q_len, Hq, D]; K, V [B, Hkv, T, D]. Query i of sequence b sees keys
    0..ctx_b - q_len + i; query head h reads kv head h // (Hq // Hkv).
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, _, Hq, D = Q.shape
    Hkv = K.shape[1]
    grp = Hq // Hkv
    out = np.zeros((B, q_len, Hq, D))
    for b in range(B):
        ctx = int(ctxs[b])
        for i in range(q_len):
            last = ctx - q_len + i
            for h in range(Hq):
                g = h // grp
                scores = []
                for t in range(last + 1):
                    acc = 0.0
                    for d in range(D):
                        acc += Q[b, i, h, d] * K[b, g, t, d]
                    scores.append(scale * acc)
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = sum(w)
                for d in range(D):
                    out[b, i, h, d] = sum(w[t] * V[b, g, t, d] for t in range(last + 1)) / z
    return out


def assert_close(got, want, tol, what=""):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - want)
    bound = tol + tol * np.abs(want)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[0]
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements out of tolerance {tol}; first at "
            f"{tuple(idx)}: got {got[tuple(idx)]!r} want {want[tuple(idx)]!r}; "
            f"max abs err {err.max():.3e}")
    return float(err.max())
