"""Seeded synthetic paged-KV decode workloads.

This module only draws inputs: context lengths, the physical page placement,
the block table, Q, the K/V page pool and (for fp8 KV) the quantised bytes and
their scales. It holds none of the attention arithmetic, so both the CPU oracle
and the GPU path can take their inputs from it without sharing any code.

Shapes follow the workloads the pages describe:
  * "Benchmark high-perf Paged Attention (#899) vs PA unroll on a2a3"
    (hw-native-sys/simpler issue #998), table "Same-Shape Side-by-Side": the
    b1_h16_kv1_s{128,512}_bs128_hd128_bf16 shapes (C1, C2 below).
  * Ascend/RecSDK issue #1281 (HSTU paged attention), section "测试方法"
    (test method): BF16, H=16, D=256, page size 32, small Q and large KV,
    seeds 2026/2029/2039 (C5 stands in for its 18-shape matrix).
  * "[Kernel][Perf] Optimize paged-attention metadata decode" (ROCm/FlyDSL
    PR #910), section "Performance (MI308X, gfx942, 80 CUs)": block size
    1024, 16 query heads, one KV head, head dim 128, several query lengths,
    per-token and per-tensor KV quantisation (C4 stands in for its shapes).
  * C3 is a batched grouped-query decode with small pages.

Recipe (every draw is a NumPy ``default_rng`` stream keyed by the seed and a
fixed stream id, so any part can be redrawn alone):
  stream [seed, 0]      context lengths, uniform integers in [ctx_lo, ctx_hi]
  stream [seed, 2]      a permutation of the physical page pool; sequence b
                        takes the next ceil(ctx_b / page_size) pages of it
  stream [seed, 1]      Q ~ N(0, 1) float32, rounded to bf16
  stream [seed, 100+T, i]  block i of the K (T=0) or V (T=1) pool, N(0, 1)
                        float32; blocks are runs of whole pages
fp8 KV: each float32 K/V value is quantised to OCP E4M3FN with torch's cast,
after division by a scale: per token and head, scale = max|x| over head_dim /
448 (1 when the row is all zero); per tensor, scale = max|x| over the whole
pool / 448. Values are clamped to +-448 before the cast (the cast does not
saturate). Unused pages and the slots of the last page past the context
length are poisoned with NaN (bf16 0x7FC0, e4m3fn 0x7F, NaN scales) so that a
kernel which reads them as live data is caught; unused block-table entries
are -1.

Decode loops (``decode_loop``) start the drawn workload ``steps * q_len``
tokens before its drawn lengths and draw each step's queries and new tokens'
K/V from streams [seed, 3], [seed, 4] and [seed, 5].
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional

import numpy as np
import torch

KV_BF16 = "bf16"
KV_FP8 = "fp8_e4m3fn"
SCALE_NONE = "none"
SCALE_PER_TENSOR = "per_tensor"
SCALE_PER_TOKEN_HEAD = "per_token_head"

E4M3FN_MAX = 448.0
_BF16_NAN = 0x7FC0
_E4M3FN_NAN = 0x7F


@dataclasses.dataclass(frozen=True)
class Spec:
    """Shape and distribution of one decode workload."""

    name: str
    batch: int
    q_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    ctx_lo: int
    ctx_hi: int                      # inclusive
    kv_dtype: str = KV_BF16
    kv_scale_mode: str = SCALE_NONE
    partition_size: int = 256
    pool_pages: int = 0              # > 0: fixed pool size; 0: see pool_slack
    pool_slack: float = 0.10         # pool = ceil((1 + slack) * pages needed)
    max_ctx: int = 0                 # block-table capacity in tokens (0: ctx_hi)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        """Query rows per (sequence, KV head) work unit: q_len * group."""
        return self.q_len * self.group

    @property
    def max_pages_per_seq(self) -> int:
        cap = self.max_ctx if self.max_ctx > 0 else self.ctx_hi
        return -(-cap // self.page_size)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


# The five workloads. C1/C2 are the Ascend issue's two same-shape cases; C3 a
# batched GQA decode; C4 the fp8 block-1024 persistent decode (four variants);
# C5 the HSTU-style small-Q / large-KV long-context case.
C1 = Spec("C1_tiny", 1, 1, 16, 1, 128, 128, 128, 128, pool_pages=8)
C2 = Spec("C2_single_seq", 1, 1, 16, 1, 128, 128, 512, 512, pool_pages=64)
C3 = Spec("C3_batched_gqa", 64, 1, 32, 8, 128, 16, 512, 8192)
C4_Q1_TOK = Spec("C4_fp8_q1_per_token", 32, 1, 16, 1, 128, 1024, 4096, 32768,
                 kv_dtype=KV_FP8, kv_scale_mode=SCALE_PER_TOKEN_HEAD)
C4_Q4_TOK = dataclasses.replace(C4_Q1_TOK, name="C4_fp8_q4_per_token", q_len=4)
C4_Q1_TEN = dataclasses.replace(C4_Q1_TOK, name="C4_fp8_q1_per_tensor",
                                kv_scale_mode=SCALE_PER_TENSOR)
C4_Q4_TEN = dataclasses.replace(C4_Q1_TEN, name="C4_fp8_q4_per_tensor", q_len=4)
C5 = Spec("C5_long_ctx_d256", 4, 8, 16, 16, 256, 32, 65536, 65536, pool_slack=0.0)

CONFIGS = {s.name: s for s in (C1, C2, C3, C4_Q1_TOK, C4_Q4_TOK, C4_Q1_TEN, C4_Q4_TEN, C5)}

# Chunked-prefill shapes (many query rows per kv head; not among the decode
# workloads above): the batched GQA heads and contexts with a 48-token chunk
# (192 rows per kv head), and the fp8 per-token heads and contexts with a
# 16-token chunk (256 rows).
P1 = dataclasses.replace(C3, name="P1_prefill_gqa_q48", q_len=48)
P2 = dataclasses.replace(C4_Q1_TOK, name="P2_prefill_fp8_q16", q_len=16)
PREFILL = {s.name: s for s in (P1, P2)}
SEEDS = (2026, 2029, 2039)


@dataclasses.dataclass
class Workload:
    """Host (CPU) tensors of one drawn workload, in the library's layouts.

    q            [B, q_len, Hq, D] bf16
    k_cache      [num_pages, Hkv, page_size, D] bf16, or uint8 e4m3fn bytes
    v_cache      same as k_cache
    block_table  [B, max_pages_per_seq] int32, -1 where unused
    context_lens [B] int32 (includes the q_len appended tokens)
    kv_scales    None; float32 [2] (per tensor: K, V); or float32
                 [2, num_pages, Hkv, page_size] (per token and head)
    """

    spec: Spec
    seed: int
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    context_lens: torch.Tensor
    kv_scales: Optional[torch.Tensor]
    num_pages: int

    def kv_bytes(self) -> int:
        """Algorithmic K+V payload bytes read by one decode (plus scales)."""
        s = self.spec
        elt = 1 if s.kv_dtype == KV_FP8 else 2
        toks = int(self.context_lens.to(torch.int64).sum())
        total = 2 * toks * s.num_kv_heads * s.head_dim * elt
        if s.kv_scale_mode == SCALE_PER_TOKEN_HEAD:
            total += 2 * toks * s.num_kv_heads * 4
        elif s.kv_scale_mode == SCALE_PER_TENSOR:
            total += 8
        return total


def _rng(*key: int) -> np.random.Generator:
    return np.random.default_rng(list(key))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _normal_pool(seed: int, stream: int, num_pages: int, page_elems: int) -> np.ndarray:
    """N(0,1) float32 pool of num_pages * page_elems values, drawn per block of pages."""
    pages_per_block = max(1, (1 << 22) // page_elems)
    nblk = -(-num_pages // pages_per_block)
    out = np.empty(num_pages * page_elems, dtype=np.float32)

    def fill(i: int) -> None:
        p0 = i * pages_per_block
        p1 = min(num_pages, p0 + pages_per_block)
        out[p0 * page_elems:p1 * page_elems] = _rng(seed, stream, i).standard_normal(
            (p1 - p0) * page_elems, dtype=np.float32)

    if nblk == 1:
        fill(0)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblk)))
    return out


def _to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(x).to(torch.bfloat16)


def quantise_e4m3fn(x: torch.Tensor, scale: torch.Tensor) -> torch.Tensor:
    """Bytes of e4m3fn(clamp(x / scale, +-448)), round to nearest even (torch cast)."""
    y = torch.clamp(x / scale, -E4M3FN_MAX, E4M3FN_MAX)
    return y.to(torch.float8_e4m3fn).view(torch.uint8)


def pool_size(spec: Spec, pages_needed: int) -> int:
    if spec.pool_pages > 0:
        if spec.pool_pages < pages_needed:
            raise ValueError(f"{spec.name}: pool of {spec.pool_pages} pages < {pages_needed} needed")
        return spec.pool_pages
    return int(math.ceil((1.0 + spec.pool_slack) * pages_needed - 1e-9))


def draw_context_lens(spec: Spec, seed: int) -> np.ndarray:
    """The context lengths of (spec, seed) alone (stream [seed, 0])."""
    if spec.ctx_lo == spec.ctx_hi:
        return np.full(spec.batch, spec.ctx_lo, dtype=np.int64)
    return _rng(seed, 0).integers(spec.ctx_lo, spec.ctx_hi + 1, size=spec.batch, dtype=np.int64)


def generate(spec: Spec, seed: int, poison: bool = True,
             context_lens: Optional[list] = None) -> Workload:
    """Draw one workload on the host. ``context_lens`` overrides the drawn lengths."""
    B, ps, D, Hkv = spec.batch, spec.page_size, spec.head_dim, spec.num_kv_heads
    if context_lens is None:
        ctx = draw_context_lens(spec, seed)
    else:
        ctx = np.asarray(context_lens, dtype=np.int64)
        assert ctx.shape == (B,)
    maxp = spec.max_pages_per_seq
    npages_b = -(-ctx // ps)
    if int(npages_b.max()) > maxp:
        raise ValueError("context longer than the block-table capacity")
    need = int(npages_b.sum())
    pool = pool_size(spec, need)
    perm = _rng(seed, 2).permutation(pool)
    bt = np.full((B, maxp), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        n = int(npages_b[b])
        bt[b, :n] = perm[off:off + n]
        off += n

    q = _to_bf16(_rng(seed, 1).standard_normal(B * spec.q_len * spec.num_q_heads * D, dtype=np.float32)
                 ).view(B, spec.q_len, spec.num_q_heads, D)
    page_elems = Hkv * ps * D
    shape = (pool, Hkv, ps, D)
    kf = _normal_pool(seed, 100, pool, page_elems)
    vf = _normal_pool(seed, 101, pool, page_elems)

    scales = None
    if spec.kv_dtype == KV_BF16:
        if spec.kv_scale_mode != SCALE_NONE:
            raise ValueError("bf16 KV takes no scales")
        k = _to_bf16(kf).view(shape)
        v = _to_bf16(vf).view(shape)
    elif spec.kv_dtype == KV_FP8:
        kt = torch.from_numpy(kf).view(shape)
        vt = torch.from_numpy(vf).view(shape)
        if spec.kv_scale_mode == SCALE_PER_TOKEN_HEAD:
            ks = kt.abs().amax(dim=-1) / E4M3FN_MAX
            vs = vt.abs().amax(dim=-1) / E4M3FN_MAX
            ks = torch.where(ks > 0, ks, torch.ones_like(ks))
            vs = torch.where(vs > 0, vs, torch.ones_like(vs))
            k = quantise_e4m3fn(kt, ks.unsqueeze(-1))
            v = quantise_e4m3fn(vt, vs.unsqueeze(-1))
            scales = torch.stack([ks, vs]).contiguous()
        elif spec.kv_scale_mode == SCALE_PER_TENSOR:
            ks = kt.abs().amax() / E4M3FN_MAX
            vs = vt.abs().amax() / E4M3FN_MAX
            ks = ks if ks > 0 else torch.tensor(1.0)
            vs = vs if vs > 0 else torch.tensor(1.0)
            k = quantise_e4m3fn(kt, ks)
            v = quantise_e4m3fn(vt, vs)
            scales = torch.stack([ks, vs]).to(torch.float32).contiguous()
        else:
            raise ValueError("fp8 KV needs a scale mode")
        del kt, vt
    else:
        raise ValueError(spec.kv_dtype)
    del kf, vf

    if poison:
        _poison(spec, k, v, scales, bt, ctx, perm[need:])

    return Workload(spec=spec, seed=seed, q=q.contiguous(), k_cache=k.contiguous(),
                    v_cache=v.contiguous(), block_table=torch.from_numpy(bt),
                    context_lens=torch.from_numpy(ctx.astype(np.int32)),
                    kv_scales=scales, num_pages=pool)


def _poison(spec: Spec, k, v, scales, bt, ctx, unused_pages) -> None:
    nan = _BF16_NAN if spec.kv_dtype == KV_BF16 else _E4M3FN_NAN
    kview = k.view(torch.int16) if spec.kv_dtype == KV_BF16 else k
    vview = v.view(torch.int16) if spec.kv_dtype == KV_BF16 else v
    fill = torch.tensor(nan, dtype=kview.dtype)
    per_tok = scales is not None and scales.dim() == 4
    if len(unused_pages):
        idx = torch.from_numpy(np.asarray(unused_pages, dtype=np.int64))
        kview[idx] = fill
        vview[idx] = fill
        if per_tok:
            scales[:, idx] = float("nan")
    ps = spec.page_size
    for b in range(spec.batch):
        c = int(ctx[b])
        n = -(-c // ps)
        tail = c - (n - 1) * ps
        if tail < ps:
            pg = int(bt[b, n - 1])
            kview[pg, :, tail:] = fill
            vview[pg, :, tail:] = fill
            if per_tok:
                scales[:, pg, :, tail:] = float("nan")


@dataclasses.dataclass
class DecodeLoop:
    """Inputs of ``steps`` consecutive decode steps of one workload.

    ``start`` is the state before the first step: its ``context_lens`` are the
    lengths before the step's tokens are appended; its block table already maps
    every page the steps will write; the slots the steps will fill are poisoned
    (so a decode that reads one before its append is caught). Step s appends
    ``new_k[s]`` / ``new_v[s]`` (bf16, [B, q_len, Hkv, D]) at positions
    [ctx + s q_len, ctx + (s+1) q_len) and decodes ``q[s]`` ([B, q_len, Hq, D])
    over the grown context. ``start.q`` is ``q[0]``.
    """

    start: Workload
    steps: int
    q: torch.Tensor
    new_k: torch.Tensor
    new_v: torch.Tensor

    def context_lens_at(self, step: int) -> torch.Tensor:
        """Context lengths seen by the decode of ``step`` (0-based)."""
        return self.start.context_lens + (step + 1) * self.start.spec.q_len


def decode_loop(spec: Spec, seed: int, steps: int,
                final_context_lens: Optional[list] = None) -> DecodeLoop:
    """Draw a decode loop: the workload of (spec, seed) at its final lengths
    (drawn, or ``final_context_lens``), started ``steps * q_len`` tokens
    earlier. Streams [seed, 3], [seed, 4] and [seed, 5] give the steps'
    queries, new K and new V, N(0, 1) rounded to bf16."""
    w = generate(spec, seed, context_lens=final_context_lens)
    B, ql, D, Hkv, ps = spec.batch, spec.q_len, spec.head_dim, spec.num_kv_heads, spec.page_size
    end = w.context_lens.numpy().astype(np.int64)
    start = end - steps * ql
    if int(start.min()) < ql:
        raise ValueError(f"{spec.name}: a context is shorter than q_len before the first step")
    nan = _BF16_NAN if spec.kv_dtype == KV_BF16 else _E4M3FN_NAN
    kview = w.k_cache.view(torch.int16) if spec.kv_dtype == KV_BF16 else w.k_cache
    vview = w.v_cache.view(torch.int16) if spec.kv_dtype == KV_BF16 else w.v_cache
    per_tok = w.kv_scales is not None and w.kv_scales.dim() == 4
    bt = w.block_table.numpy()
    for b in range(B):
        for t in range(int(start[b]), int(end[b])):
            pg, slot = int(bt[b, t // ps]), t % ps
            kview[pg, :, slot] = nan
            vview[pg, :, slot] = nan
            if per_tok:
                w.kv_scales[:, pg, :, slot] = float("nan")

    def draw(stream: int, heads: int) -> torch.Tensor:
        x = _rng(seed, stream).standard_normal(steps * B * ql * heads * D, dtype=np.float32)
        return _to_bf16(x).view(steps, B, ql, heads, D).contiguous()

    q = draw(3, spec.num_q_heads)
    nk, nv = draw(4, Hkv), draw(5, Hkv)
    w0 = Workload(spec=spec, seed=seed, q=q[0].contiguous(), k_cache=w.k_cache,
                  v_cache=w.v_cache, block_table=w.block_table,
                  context_lens=torch.from_numpy(start.astype(np.int32)), kv_scales=w.kv_scales,
                  num_pages=w.num_pages)
    return DecodeLoop(start=w0, steps=steps, q=q, new_k=nk, new_v=nv)


def scaled(spec: Spec, **changes) -> Spec:
    """A copy of ``spec`` with some fields changed (reduced-size test variants)."""
    return dataclasses.replace(spec, **changes)
