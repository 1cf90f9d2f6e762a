"""Helpers for the GPU tests: run a drawn workload through the C-ABI and
compare with the CPU oracle."""
from __future__ import annotations

import dataclasses
import sys

import numpy as np
import torch

import oracle
import paged_attention_decode_block_amd as pa
import workloads as W
from tests.helpers import TOL_BF16, TOL_FP8, assert_close

DEV = torch.device("cuda:0")

KV_CODE = {W.KV_BF16: pa.PA_KV_BF16, W.KV_FP8: pa.PA_KV_FP8_E4M3FN}
MODE_CODE = {W.SCALE_NONE: pa.PA_SCALE_NONE, W.SCALE_PER_TENSOR: pa.PA_SCALE_PER_TENSOR,
             W.SCALE_PER_TOKEN_HEAD: pa.PA_SCALE_PER_TOKEN_HEAD}


def say(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def tol(spec: W.Spec) -> float:
    return TOL_FP8 if spec.kv_dtype == W.KV_FP8 else TOL_BF16


def dims_for(w: W.Workload, partition: int | None = None, grid_multiplier: int = 0,
             flags: int = 0) -> pa.pa_dims:
    s = w.spec
    return pa.make_dims(batch=s.batch, q_len=s.q_len, num_q_heads=s.num_q_heads,
                        num_kv_heads=s.num_kv_heads, head_dim=s.head_dim, page_size=s.page_size,
                        num_pages=w.num_pages, max_pages_per_seq=s.max_pages_per_seq,
                        kv_dtype=KV_CODE[s.kv_dtype], kv_scale_mode=MODE_CODE[s.kv_scale_mode],
                        partition_size=partition or s.partition_size,
                        grid_multiplier=grid_multiplier, flags=flags)


@dataclasses.dataclass
class Dev:
    q: torch.Tensor
    k_cache: torch.Tensor
    v_cache: torch.Tensor
    block_table: torch.Tensor
    context_lens: torch.Tensor
    kv_scales: torch.Tensor | None


def upload(w: W.Workload) -> Dev:
    return Dev(w.q.to(DEV), w.k_cache.to(DEV), w.v_cache.to(DEV), w.block_table.to(DEV),
               w.context_lens.to(DEV), None if w.kv_scales is None else w.kv_scales.to(DEV))


def run(w: W.Workload, d: Dev | None = None, partition: int | None = None,
        grid_multiplier: int = 0, flags: int = 0, stream=None):
    """Plan + decode on the GPU. Returns (out bf16 on device, plan)."""
    d = d or upload(w)
    s = w.spec
    plan = pa.pa_plan(dims_for(w, partition, grid_multiplier, flags), d.context_lens, stream=stream)
    out = torch.empty_like(d.q)
    pa.pa_decode(plan, d.q, d.k_cache, d.v_cache, d.block_table, d.context_lens, s.q_len, s.scale,
                 MODE_CODE[s.kv_scale_mode], d.kv_scales, out, stream=stream)
    return out, plan


def oracle_out(w: W.Workload) -> np.ndarray:
    s = w.spec
    out, _ = oracle.decode(w.q, w.k_cache, w.v_cache, w.block_table, w.context_lens, s.q_len,
                           s.scale, s.page_size, s.kv_dtype, s.kv_scale_mode, w.kv_scales)
    return out


def to_f64(x: torch.Tensor) -> np.ndarray:
    return x.float().cpu().numpy().astype(np.float64)


def check(w: W.Workload, out: torch.Tensor, what: str = "") -> float:
    err = assert_close(to_f64(out), oracle_out(w), tol(w.spec), what or w.spec.name)
    return err


def plan_arrays(plan: pa.Plan, batch: int):
    """Device plan -> Python lists, in the oracle Plan's fields."""
    c = plan.c
    torch.cuda.synchronize()
    status = plan.region("status", 4).cpu().tolist()
    N, S = status[1], status[2]
    G, pairs = c.grid, c.num_pairs
    return dict(
        status=status[0], num_items=N, num_segs=S,
        wg_begin=plan.region("wg_begin", G + 1).cpu().tolist(),
        wg_seg_begin=plan.region("wg_seg_begin", G + 1).cpu().tolist(),
        items=[tuple(r) for r in plan.region("items", 4 * N).view(-1, 4).cpu().tolist()],
        segs=[tuple(r) for r in plan.region("segs", 4 * S).view(-1, 4).cpu().tolist()],
        nseg=plan.region("nseg", pairs).cpu().tolist(),
        seg_base=plan.region("seg_base", pairs + 1).cpu().tolist(),
        pseg_base=plan.region("pseg_base", pairs + 1).cpu().tolist(),
        batch_base=plan.region("batch_base", batch + 1).cpu().tolist(),
        seg_info=[tuple(r) for r in plan.region("seg_info", 8 * S).view(-1, 8).cpu().tolist()],
        wg_head=[tuple(r) for r in plan.region("wg_head", 16 * G).view(-1, 16).cpu().tolist()],
    )
