"""Paged-attention decode for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libpa.so`` (HIP kernels + C-ABI, declared in
``include/pa.h``). Every function here has the C name and only marshals
arguments: tensors become device pointers, the stream defaults to PyTorch's
current stream, and a negative status raises :class:`PaError`. All of the
work runs in the library's kernels; nothing here computes attention, and
there is no CPU fallback — if the library is missing, the calls raise.

Typical use::

    import paged_attention_decode_block_amd as pa
    dims = pa.make_dims(batch=B, q_len=1, num_q_heads=32, num_kv_heads=8,
                        head_dim=128, page_size=16, num_pages=P,
                        max_pages_per_seq=M)
    plan = pa.pa_plan(dims, context_lens)          # builds the work list
    pa.pa_decode(plan, q, k_cache, v_cache, block_table, context_lens,
                 q_len=1, scale=D ** -0.5, kv_scale_mode=pa.PA_SCALE_NONE,
                 kv_scales=None, out=out)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpa.so")

PA_OK = 0
PA_ERR_NULL = -1
PA_ERR_ALIGN = -2
PA_ERR_DIMS = -3
PA_ERR_UNSUPPORTED = -4
PA_ERR_WORKSPACE = -5
PA_ERR_PLAN_MISMATCH = -6
PA_ERR_SCALE_MODE = -7
PA_ERR_HIP = -8
PA_ERR_DEVICE = -9

PA_DEV_BAD_CONTEXT = 1
PA_DEV_BAD_PAGE = 2

PA_KV_BF16 = 0
PA_KV_FP8_E4M3FN = 1
PA_SCALE_NONE = 0
PA_SCALE_PER_TENSOR = 1
PA_SCALE_PER_TOKEN_HEAD = 2
PA_FLAG_DEBUG_BOUNDS = 1
PA_PLAN_MAGIC = 0x50414450


class PaError(RuntimeError):
    def __init__(self, code: int, text: str):
        super().__init__(f"{code}: {text}")
        self.code = code
        self.text = text


class pa_dims(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "batch", "q_len", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
        "max_pages_per_seq", "kv_dtype", "kv_scale_mode", "partition_size", "grid_multiplier",
        "flags")]


class pa_plan_t(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("device", ctypes.c_int32), ("dims", pa_dims),
        ("num_cus", ctypes.c_int32), ("grid", ctypes.c_int32), ("rows", ctypes.c_int32),
        ("num_pairs", ctypes.c_int32), ("max_items", ctypes.c_int32), ("max_segs", ctypes.c_int32),
        ("variant", ctypes.c_int32), ("q_block", ctypes.c_int32),
        ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_uint64),
        ("off_status", ctypes.c_uint64), ("off_wg_begin", ctypes.c_uint64),
        ("off_wg_seg_begin", ctypes.c_uint64), ("off_items", ctypes.c_uint64),
        ("off_segs", ctypes.c_uint64), ("off_nseg", ctypes.c_uint64),
        ("off_seg_base", ctypes.c_uint64), ("off_pseg_base", ctypes.c_uint64),
        ("off_batch_base", ctypes.c_uint64), ("off_partial_lse", ctypes.c_uint64),
        ("off_partial_o", ctypes.c_uint64), ("off_seg_info", ctypes.c_uint64),
        ("off_wg_head", ctypes.c_uint64), ("block_bytes", ctypes.c_uint64),
        ("reserved", ctypes.c_uint64),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libpa.so (in-tree). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -c 'import __graft_entry__ as g; g.build()')")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint64
        P = ctypes.POINTER
        sig = {
            "pa_query_device": (ctypes.c_int, [i32, P(i32)]),
            "pa_workspace_bytes": (ctypes.c_int, [P(pa_dims), i32, P(u64)]),
            "pa_plan": (ctypes.c_int, [P(pa_dims), vp, vp, u64, P(pa_plan_t), vp]),
            "pa_decode": (ctypes.c_int, [P(pa_plan_t), vp, vp, vp, vp, vp, i32, ctypes.c_float,
                                         i32, vp, vp, vp]),
            "pa_decode_partition": (ctypes.c_int, [P(pa_plan_t), vp, vp, vp, vp, vp, i32,
                                                   ctypes.c_float, i32, vp, vp, vp]),
            "pa_decode_reduce": (ctypes.c_int, [P(pa_plan_t), i32, i32, vp, vp]),
            "pa_plan_status": (ctypes.c_int, [P(pa_plan_t), P(i32), vp]),
            "pa_debug_gather": (ctypes.c_int, [P(pa_plan_t), vp, vp, vp, vp, vp, vp, vp]),
            "pa_cache_append": (ctypes.c_int, [P(pa_dims), vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "pa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "pa_last_error": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc: int) -> None:
    if rc != PA_OK:
        raise PaError(rc, lib().pa_last_error().decode() or lib().pa_status_string(rc).decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def make_dims(*, batch: int, q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
              page_size: int, num_pages: int, max_pages_per_seq: int, kv_dtype: int = PA_KV_BF16,
              kv_scale_mode: int = PA_SCALE_NONE, partition_size: int = 0,
              grid_multiplier: int = 0, flags: int = 0) -> pa_dims:
    return pa_dims(batch, q_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages,
                   max_pages_per_seq, kv_dtype, kv_scale_mode, partition_size, grid_multiplier,
                   flags)


class Plan:
    """A built plan (pa_plan_t) and the workspace tensor it points into."""

    def __init__(self, c: pa_plan_t, workspace: torch.Tensor):
        self.c = c
        self.workspace = workspace

    def region(self, name: str, count: int, dtype=torch.int32) -> torch.Tensor:
        """View of a workspace region (for tests and diagnostics)."""
        off = getattr(self.c, "off_" + name)
        esz = torch.empty(0, dtype=dtype).element_size()
        return self.workspace[off:off + count * esz].view(dtype)


def pa_query_device(device: int = 0) -> int:
    n = ctypes.c_int32(0)
    _check(lib().pa_query_device(device, ctypes.byref(n)))
    return n.value


def pa_workspace_bytes(dims: pa_dims, num_cus: int) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().pa_workspace_bytes(ctypes.byref(dims), num_cus, ctypes.byref(n)))
    return n.value


def pa_plan(dims: pa_dims, context_lens: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            stream=None) -> Plan:
    dev = context_lens.device
    if workspace is None:
        nbytes = pa_workspace_bytes(dims, pa_query_device(dev.index or 0))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    c = pa_plan_t()
    _check(lib().pa_plan(ctypes.byref(dims), _ptr(context_lens), _ptr(workspace),
                         workspace.numel(), ctypes.byref(c), _stream(stream)))
    return Plan(c, workspace)


def pa_decode(plan: Plan, q, k_cache, v_cache, block_table, context_lens, q_len: int,
              scale: float, kv_scale_mode: int, kv_scales, out, stream=None):
    _check(lib().pa_decode(ctypes.byref(plan.c), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                           _ptr(block_table), _ptr(context_lens), q_len, scale, kv_scale_mode,
                           _ptr(kv_scales), _ptr(out), _stream(stream)))
    return out


def pa_decode_partition(plan: Plan, q, k_cache, v_cache, block_table, context_lens, q_len: int,
                        scale: float, kv_scale_mode: int, kv_scales, out, stream=None):
    _check(lib().pa_decode_partition(ctypes.byref(plan.c), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                     _ptr(block_table), _ptr(context_lens), q_len, scale,
                                     kv_scale_mode, _ptr(kv_scales), _ptr(out), _stream(stream)))
    return out


def pa_decode_reduce(plan: Plan, q_len: int, kv_scale_mode: int, out, stream=None):
    _check(lib().pa_decode_reduce(ctypes.byref(plan.c), q_len, kv_scale_mode, _ptr(out),
                                  _stream(stream)))
    return out


def pa_plan_status(plan: Plan, stream=None) -> int:
    st = ctypes.c_int32(0)
    _check(lib().pa_plan_status(ctypes.byref(plan.c), ctypes.byref(st), _stream(stream)))
    return st.value


def pa_debug_gather(plan: Plan, k_cache, v_cache, block_table, context_lens, k_out, v_out,
                    stream=None):
    _check(lib().pa_debug_gather(ctypes.byref(plan.c), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(block_table), _ptr(context_lens), _ptr(k_out), _ptr(v_out),
                                 _stream(stream)))


def pa_cache_append(dims: pa_dims, new_k, new_v, block_table, context_lens, k_cache, v_cache,
                    kv_scales=None, device_status=None, stream=None):
    """Write the q_len new tokens' K/V rows of every sequence into the paged
    cache (include/pa.h, pa_cache_append)."""
    _check(lib().pa_cache_append(ctypes.byref(dims), _ptr(new_k), _ptr(new_v), _ptr(block_table),
                                 _ptr(context_lens), _ptr(k_cache), _ptr(v_cache), _ptr(kv_scales),
                                 _ptr(device_status), _stream(stream)))


def pa_status_string(code: int) -> str:
    return lib().pa_status_string(code).decode()


def pa_last_error() -> str:
    return lib().pa_last_error().decode()
