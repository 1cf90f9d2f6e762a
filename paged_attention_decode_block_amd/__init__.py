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

import numpy as np
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
PA_DEV_DEBUG_DEAD_ROW = 4

PA_KV_BF16 = 0
PA_KV_FP8_E4M3FN = 1
PA_SCALE_NONE = 0
PA_SCALE_PER_TENSOR = 1
PA_SCALE_PER_TOKEN_HEAD = 2
PA_FLAG_DEBUG_BOUNDS = 1
PA_FLAG_FUSED_REDUCE = 2
PA_FLAG_SEPARATE_REDUCE = 4
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
        ("off_counters", ctypes.c_uint64),
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
            "pa_plan_choice": (ctypes.c_int, [P(pa_dims), i32, P(pa_dims)]),
            "pa_plan": (ctypes.c_int, [P(pa_dims), vp, vp, u64, P(pa_plan_t), vp]),
            "pa_decode": (ctypes.c_int, [P(pa_plan_t), vp, vp, vp, vp, vp, i32, ctypes.c_float,
                                         i32, vp, vp, vp]),
            "pa_decode_partition": (ctypes.c_int, [P(pa_plan_t), vp, vp, vp, vp, vp, i32,
                                                   ctypes.c_float, i32, vp, vp, vp]),
            "pa_decode_reduce": (ctypes.c_int, [P(pa_plan_t), i32, i32, vp, vp]),
            "pa_plan_status": (ctypes.c_int, [P(pa_plan_t), P(i32), vp]),
            "pa_debug_gather": (ctypes.c_int, [P(pa_plan_t), vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp]),
            "pa_cache_append": (ctypes.c_int, [P(pa_dims), vp, vp, vp, vp, vp, vp, vp, vp, vp]),
            "pa_decode_static": (ctypes.c_int, [P(pa_dims), vp, vp, vp, vp, vp, i32,
                                                ctypes.c_float, i32, vp, vp, P(pa_plan_t), vp]),
            "pa_static_scratch_bytes": (u64, []),
            "pa_debug_read_probe": (ctypes.c_int, [vp, u64, vp, i32, i32, i32, i32, vp, vp]),
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


# Element types a buffer may carry (same width, any view of the bits).
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)
_FP8 = (torch.uint8, torch.int8, torch.float8_e4m3fn)
_I32 = (torch.int32,)
_F32 = (torch.float32,)


def _buf(t, name: str, dtypes, shape=None, optional: bool = False) -> Optional[int]:
    """Device pointer of a tensor argument after the checks that keep the
    kernels in bounds: an accepted element type, contiguous, and of the
    expected shape (or, for a shape given as an int, holding exactly that many
    elements). The device is checked by _on once every argument has passed
    these. Raises PaError."""
    if t is None:
        if optional:
            return None
        raise PaError(PA_ERR_NULL, f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise PaError(PA_ERR_DIMS, f"{name} must be a torch.Tensor, not {type(t).__name__}")
    if t.dtype not in dtypes:
        raise PaError(PA_ERR_DIMS, f"{name} has dtype {t.dtype}; expected one of "
                                   f"{', '.join(str(d) for d in dtypes)}")
    if not t.is_contiguous():
        raise PaError(PA_ERR_DIMS, f"{name} must be contiguous")
    if isinstance(shape, int):
        if t.numel() != shape:
            raise PaError(PA_ERR_DIMS, f"{name} holds {t.numel()} elements; expected {shape}")
    elif shape is not None and tuple(t.shape) != tuple(shape):
        raise PaError(PA_ERR_DIMS, f"{name} has shape {tuple(t.shape)}; expected {tuple(shape)}")
    return t.data_ptr()


def _on(dev: Optional[torch.device], **tensors) -> None:
    """Every given tensor is a GPU tensor on dev (on one common GPU when dev is
    None). Raises PaError."""
    for name, t in tensors.items():
        if t is None:
            continue
        if t.device.type != "cuda" or (dev is not None and t.device != dev):
            raise PaError(PA_ERR_DEVICE, f"{name} is on {t.device}; expected {dev or 'a GPU'}")
        dev = t.device


def _cache_args(d: pa_dims, k_cache, v_cache, kv_scales, mode: int):
    """Pointers of the caches and scales for dims d: caches [num_pages, Hkv,
    page_size, head_dim] (or flat with that many elements), scales [2] per
    tensor or [2, num_pages, Hkv, page_size] per token."""
    cdt = _FP8 if d.kv_dtype == PA_KV_FP8_E4M3FN else _BF16
    cshape = (d.num_pages, d.num_kv_heads, d.page_size, d.head_dim)
    shape_of = lambda t: cshape if t is not None and t.dim() == 4 else int(np.prod(cshape))  # noqa: E731
    k = _buf(k_cache, "k_cache", cdt, shape_of(k_cache))
    v = _buf(v_cache, "v_cache", cdt, shape_of(v_cache))
    if mode == PA_SCALE_NONE:
        if kv_scales is not None:
            raise PaError(PA_ERR_SCALE_MODE, "kv_scales must be None when kv_scale_mode is NONE")
        return k, v, None
    if mode == PA_SCALE_PER_TENSOR:
        return k, v, _buf(kv_scales, "kv_scales", _F32, 2)
    sshape = (2,) + cshape[:3]
    return k, v, _buf(kv_scales, "kv_scales", _F32,
                      sshape if kv_scales is not None and kv_scales.dim() == 4
                      else int(np.prod(sshape)))


def _plan_device(plan: "Plan") -> torch.device:
    return torch.device("cuda", plan.c.device)


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


def pa_plan_choice(dims: pa_dims, num_cus: int) -> pa_dims:
    """The dims pa_plan would use on a device of num_cus CUs: partition size,
    grid multiplier and reduce flag filled in from the tuning table or the
    defaults (include/pa.h, pa_plan_choice)."""
    out = pa_dims()
    _check(lib().pa_plan_choice(ctypes.byref(dims), num_cus, ctypes.byref(out)))
    return out


def pa_workspace_bytes(dims: pa_dims, num_cus: int) -> int:
    n = ctypes.c_uint64(0)
    _check(lib().pa_workspace_bytes(ctypes.byref(dims), num_cus, ctypes.byref(n)))
    return n.value


def pa_plan(dims: pa_dims, context_lens: torch.Tensor, workspace: Optional[torch.Tensor] = None,
            stream=None) -> Plan:
    _buf(context_lens, "context_lens", _I32, (dims.batch,))
    _on(None, context_lens=context_lens)
    dev = context_lens.device
    if workspace is None:
        nbytes = pa_workspace_bytes(dims, pa_query_device(dev.index or 0))
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _buf(workspace, "workspace", (torch.uint8,))
    _on(dev, workspace=workspace)
    c = pa_plan_t()
    _check(lib().pa_plan(ctypes.byref(dims), _ptr(context_lens), _ptr(workspace),
                         workspace.numel(), ctypes.byref(c), _stream(stream)))
    return Plan(c, workspace)


def _decode_ptrs(plan: Plan, q, k_cache, v_cache, block_table, context_lens, kv_scale_mode,
                 kv_scales, out):
    d = plan.c.dims
    qshape = (d.batch, d.q_len, d.num_q_heads, d.head_dim)
    k, v, sc = _cache_args(d, k_cache, v_cache, kv_scales, kv_scale_mode)
    ptrs = (_buf(q, "q", _BF16, qshape), k, v,
            _buf(block_table, "block_table", _I32, (d.batch, d.max_pages_per_seq)),
            _buf(context_lens, "context_lens", _I32, (d.batch,)), sc,
            _buf(out, "out", _BF16, qshape))
    _on(_plan_device(plan), q=q, k_cache=k_cache, v_cache=v_cache, block_table=block_table,
        context_lens=context_lens, kv_scales=kv_scales, out=out)
    return ptrs


def pa_decode(plan: Plan, q, k_cache, v_cache, block_table, context_lens, q_len: int,
              scale: float, kv_scale_mode: int, kv_scales, out, stream=None):
    pq, pk, pv, pbt, pctx, psc, pout = _decode_ptrs(plan, q, k_cache, v_cache, block_table,
                                                    context_lens, kv_scale_mode, kv_scales, out)
    _check(lib().pa_decode(ctypes.byref(plan.c), pq, pk, pv, pbt, pctx, q_len, scale,
                           kv_scale_mode, psc, pout, _stream(stream)))
    return out


def pa_decode_partition(plan: Plan, q, k_cache, v_cache, block_table, context_lens, q_len: int,
                        scale: float, kv_scale_mode: int, kv_scales, out, stream=None):
    pq, pk, pv, pbt, pctx, psc, pout = _decode_ptrs(plan, q, k_cache, v_cache, block_table,
                                                    context_lens, kv_scale_mode, kv_scales, out)
    _check(lib().pa_decode_partition(ctypes.byref(plan.c), pq, pk, pv, pbt, pctx, q_len, scale,
                                     kv_scale_mode, psc, pout, _stream(stream)))
    return out


def pa_decode_reduce(plan: Plan, q_len: int, kv_scale_mode: int, out, stream=None):
    d = plan.c.dims
    pout = _buf(out, "out", _BF16, (d.batch, d.q_len, d.num_q_heads, d.head_dim))
    _on(_plan_device(plan), out=out)
    _check(lib().pa_decode_reduce(ctypes.byref(plan.c), q_len, kv_scale_mode, pout,
                                  _stream(stream)))
    return out


def pa_decode_static(dims: pa_dims, q, k_cache, v_cache, block_table, context_lens, q_len: int,
                     scale: float, kv_scale_mode: int, kv_scales, out, stream=None) -> Plan:
    """pa_plan + pa_decode in the library's static scratch (include/pa.h,
    pa_decode_static): nothing is allocated. Returns the plan (its workspace
    is the scratch, valid until the next call on the device) for
    pa_plan_status."""
    qshape = (dims.batch, dims.q_len, dims.num_q_heads, dims.head_dim)
    k, v, sc = _cache_args(dims, k_cache, v_cache, kv_scales, kv_scale_mode)
    ptrs = (_buf(q, "q", _BF16, qshape), k, v,
            _buf(block_table, "block_table", _I32, (dims.batch, dims.max_pages_per_seq)),
            _buf(context_lens, "context_lens", _I32, (dims.batch,)))
    pout = _buf(out, "out", _BF16, qshape)
    _on(None, context_lens=context_lens, q=q, k_cache=k_cache, v_cache=v_cache,
        block_table=block_table, kv_scales=kv_scales, out=out)
    c = pa_plan_t()
    _check(lib().pa_decode_static(ctypes.byref(dims), *ptrs, q_len, scale, kv_scale_mode, sc,
                                  pout, ctypes.byref(c), _stream(stream)))
    return Plan(c, None)


def pa_static_scratch_bytes() -> int:
    return int(lib().pa_static_scratch_bytes())


def pa_plan_status(plan: Plan, stream=None) -> int:
    st = ctypes.c_int32(0)
    _check(lib().pa_plan_status(ctypes.byref(plan.c), ctypes.byref(st), _stream(stream)))
    return st.value


def pa_debug_gather(plan: Plan, k_cache, v_cache, block_table, context_lens, k_out, v_out,
                    kv_scales=None, scales_out=None, stream=None):
    """The decode's page loader alone (include/pa.h, pa_debug_gather): k_out /
    v_out [batch * Hkv, max_pages_per_seq * page_size, head_dim] in the cache's
    element type; scales_out [2, batch * Hkv, same rows] float32 in per-token
    mode."""
    d = plan.c.dims
    mode = d.kv_scale_mode
    k, v, sc = _cache_args(d, k_cache, v_cache, kv_scales, mode)
    rows = d.batch * d.num_kv_heads * d.max_pages_per_seq * d.page_size
    odt = _FP8 if d.kv_dtype == PA_KV_FP8_E4M3FN else _BF16
    n_out = rows * d.head_dim
    ptrs = (k, v, _buf(block_table, "block_table", _I32, (d.batch, d.max_pages_per_seq)),
            _buf(context_lens, "context_lens", _I32, (d.batch,)), sc,
            _buf(k_out, "k_out", odt, n_out), _buf(v_out, "v_out", odt, n_out),
            _buf(scales_out, "scales_out", _F32, 2 * rows,
                 optional=mode != PA_SCALE_PER_TOKEN_HEAD))
    _on(_plan_device(plan), k_cache=k_cache, v_cache=v_cache, block_table=block_table,
        context_lens=context_lens, kv_scales=kv_scales, k_out=k_out, v_out=v_out,
        scales_out=scales_out)
    _check(lib().pa_debug_gather(ctypes.byref(plan.c), *ptrs, _stream(stream)))


def pa_cache_append(dims: pa_dims, new_k, new_v, block_table, context_lens, k_cache, v_cache,
                    kv_scales=None, device_status=None, stream=None):
    """Write the q_len new tokens' K/V rows of every sequence into the paged
    cache (include/pa.h, pa_cache_append)."""
    nshape = (dims.batch, dims.q_len, dims.num_kv_heads, dims.head_dim)
    k, v, sc = _cache_args(dims, k_cache, v_cache, kv_scales, dims.kv_scale_mode)
    ptrs = (_buf(new_k, "new_k", _BF16, nshape), _buf(new_v, "new_v", _BF16, nshape),
            _buf(block_table, "block_table", _I32, (dims.batch, dims.max_pages_per_seq)),
            _buf(context_lens, "context_lens", _I32, (dims.batch,)), k, v, sc,
            _buf(device_status, "device_status", _I32, 1, optional=True))
    _on(None, context_lens=context_lens, new_k=new_k, new_v=new_v, block_table=block_table,
        k_cache=k_cache, v_cache=v_cache, kv_scales=kv_scales, device_status=device_status)
    _check(lib().pa_cache_append(ctypes.byref(dims), *ptrs, _stream(stream)))


def pa_debug_read_probe(buffer, blocks, row_bytes: int, linear: bool, waves: int, sink,
                        stream=None):
    """Read 16-row blocks of `buffer` in one K/V lane layout (include/pa.h,
    pa_debug_read_probe): measurement support for the load layout."""
    _buf(buffer, "buffer", (torch.uint8,))
    _buf(blocks, "blocks", _I32)
    _buf(sink, "sink", _F32)
    _on(None, buffer=buffer, blocks=blocks, sink=sink)
    if not 1 <= waves <= 16:
        raise PaError(PA_ERR_DIMS, f"waves {waves} outside [1, 16]")
    need = pa_query_device(sink.device.index) * waves * 64
    if sink.numel() < need:
        raise PaError(PA_ERR_DIMS, f"sink holds {sink.numel()} floats; one per lane of the grid, "
                                   f"{need}, is needed")
    _check(lib().pa_debug_read_probe(_ptr(buffer), buffer.numel(), _ptr(blocks), blocks.numel(),
                                     row_bytes, int(bool(linear)), waves, _ptr(sink),
                                     _stream(stream)))


def pa_status_string(code: int) -> str:
    return lib().pa_status_string(code).decode()


def pa_last_error() -> str:
    return lib().pa_last_error().decode()
