"""The C-ABI library without a GPU: it loads, exports every symbol include/pa.h
declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

import paged_attention_decode_block_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "pa.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = pa.lib()
    names = _declared()
    assert "pa_decode" in names and "pa_plan" in names
    for n in names:
        assert hasattr(L, n), n


def test_struct_sizes_match_header():
    # 13 int32 dims; the plan is 4-byte fields up to the pointers, then 8-byte ones
    assert ctypes.sizeof(pa.pa_dims) == 13 * 4
    assert ctypes.sizeof(pa.pa_plan_t) % 8 == 0
    assert pa.pa_plan_t.workspace.offset % 8 == 0


def _dims(**kw):
    base = dict(batch=2, q_len=1, num_q_heads=16, num_kv_heads=1, head_dim=128, page_size=16,
                num_pages=64, max_pages_per_seq=8)
    base.update(kw)
    return pa.make_dims(**base)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), pa.PA_ERR_DIMS),
    (dict(q_len=0), pa.PA_ERR_DIMS),
    (dict(num_q_heads=12, num_kv_heads=8), pa.PA_ERR_DIMS),
    (dict(num_pages=0), pa.PA_ERR_DIMS),
    (dict(grid_multiplier=17), pa.PA_ERR_DIMS),
    (dict(flags=8), pa.PA_ERR_DIMS),
    (dict(flags=pa.PA_FLAG_FUSED_REDUCE | pa.PA_FLAG_SEPARATE_REDUCE), pa.PA_ERR_DIMS),
    (dict(head_dim=64), pa.PA_ERR_UNSUPPORTED),
    (dict(head_dim=96), pa.PA_ERR_UNSUPPORTED),
    (dict(page_size=8), pa.PA_ERR_UNSUPPORTED),
    (dict(page_size=48), pa.PA_ERR_UNSUPPORTED),
    (dict(page_size=2048), pa.PA_ERR_UNSUPPORTED),
    (dict(partition_size=24), pa.PA_ERR_UNSUPPORTED),
    (dict(kv_dtype=2), pa.PA_ERR_UNSUPPORTED),
    (dict(kv_scale_mode=pa.PA_SCALE_PER_TENSOR), pa.PA_ERR_SCALE_MODE),
    (dict(kv_dtype=pa.PA_KV_FP8_E4M3FN), pa.PA_ERR_SCALE_MODE),
    # one query's rows past what a kernel holds (256 at head_dim 128, 64 at 256)
    (dict(q_len=1, num_q_heads=512, num_kv_heads=1), pa.PA_ERR_UNSUPPORTED),
    (dict(head_dim=256, q_len=2, num_q_heads=128, num_kv_heads=1), pa.PA_ERR_UNSUPPORTED),
])
def test_dims_rejected_on_host(kw, code):
    with pytest.raises(pa.PaError) as e:
        pa.pa_workspace_bytes(_dims(**kw), 256)
    assert e.value.code == code, e.value.text
    assert pa.pa_last_error()
    # pa_plan validates the same way before touching a device
    c = pa.pa_plan_t()
    rc = pa.lib().pa_plan(ctypes.byref(_dims(**kw)), 0x1000, 0x100000, 1 << 30, ctypes.byref(c), None)
    assert rc == code


def test_long_queries_take_one_workspace_block_per_query_block():
    # 16 rows per query: sixteen queries (256 rows) fit one kernel at head_dim
    # 128, so 17 and 32 queries take two blocks of sixteen, 33 take three; at
    # head_dim 256 (64 rows) blocks hold four queries
    one = pa.pa_workspace_bytes(_dims(q_len=16, num_q_heads=16, num_kv_heads=1), 256)
    assert one % 256 == 0
    for q_len, blocks in ((17, 2), (32, 2), (33, 3)):
        ws = pa.pa_workspace_bytes(_dims(q_len=q_len, num_q_heads=16, num_kv_heads=1), 256)
        assert ws == blocks * one, (q_len, ws, one)
    one256 = pa.pa_workspace_bytes(_dims(head_dim=256, q_len=4, num_q_heads=16, num_kv_heads=1), 256)
    assert pa.pa_workspace_bytes(_dims(head_dim=256, q_len=13, num_q_heads=16, num_kv_heads=1),
                                 256) == 4 * one256


def test_workspace_size_grows_with_work():
    small = pa.pa_workspace_bytes(_dims(), 256)
    big = pa.pa_workspace_bytes(_dims(batch=64, max_pages_per_seq=512), 256)
    assert 0 < small < big
    assert pa.pa_workspace_bytes(_dims(), 80) < small


def test_plan_argument_errors():
    L = pa.lib()
    c = pa.pa_plan_t()
    d = _dims()
    assert L.pa_plan(ctypes.byref(d), None, 0x100000, 1 << 30, ctypes.byref(c), None) == pa.PA_ERR_NULL
    assert L.pa_plan(ctypes.byref(d), 0x1000, None, 1 << 30, ctypes.byref(c), None) == pa.PA_ERR_WORKSPACE
    assert L.pa_plan(ctypes.byref(d), 0x1000, 0x100010, 1 << 30, ctypes.byref(c), None) == pa.PA_ERR_ALIGN
    assert L.pa_plan(ctypes.byref(d), 0x1002, 0x100000, 1 << 30, ctypes.byref(c), None) == pa.PA_ERR_ALIGN


def _fake_plan(**kw):
    c = pa.pa_plan_t()
    c.magic = pa.PA_PLAN_MAGIC
    c.dims = _dims(**kw)
    return c


def _decode(c, q=0x10000, k=0x20000, v=0x30000, bt=0x40000, ctx=0x50000, q_len=1,
            mode=pa.PA_SCALE_NONE, scales=None, out=0x60000):
    return pa.lib().pa_decode(ctypes.byref(c) if c is not None else None, q, k, v, bt, ctx, q_len,
                              0.1, mode, scales, out, None)


def test_decode_argument_errors_before_any_device_call():
    c = _fake_plan()
    assert _decode(None) == pa.PA_ERR_NULL
    assert _decode(c, q=None) == pa.PA_ERR_NULL
    assert _decode(c, out=None) == pa.PA_ERR_NULL
    unbuilt = pa.pa_plan_t()
    assert _decode(unbuilt) == pa.PA_ERR_PLAN_MISMATCH
    assert _decode(c, q=0x10008) == pa.PA_ERR_ALIGN
    assert _decode(c, k=0x20004) == pa.PA_ERR_ALIGN
    assert _decode(c, out=0x60002) == pa.PA_ERR_ALIGN
    assert _decode(c, bt=0x40002) == pa.PA_ERR_ALIGN
    assert _decode(c, q_len=2) == pa.PA_ERR_PLAN_MISMATCH
    assert _decode(c, mode=pa.PA_SCALE_PER_TENSOR, scales=0x70000) == pa.PA_ERR_PLAN_MISMATCH
    assert _decode(c, scales=0x70000) == pa.PA_ERR_SCALE_MODE
    f8 = _fake_plan(kv_dtype=pa.PA_KV_FP8_E4M3FN, kv_scale_mode=pa.PA_SCALE_PER_TOKEN_HEAD)
    assert _decode(f8, mode=pa.PA_SCALE_PER_TOKEN_HEAD) == pa.PA_ERR_SCALE_MODE
    assert _decode(f8, mode=pa.PA_SCALE_PER_TOKEN_HEAD, scales=0x70008) == pa.PA_ERR_ALIGN
    L = pa.lib()
    assert L.pa_decode_reduce(ctypes.byref(c), 2, 0, 0x60000, None) == pa.PA_ERR_PLAN_MISMATCH
    assert L.pa_decode_reduce(ctypes.byref(c), 1, 0, None, None) == pa.PA_ERR_NULL
    st = ctypes.c_int32()
    assert L.pa_plan_status(None, ctypes.byref(st), None) == pa.PA_ERR_NULL
    # pa_debug_gather(plan, k, v, block_table, ctx, kv_scales, k_out, v_out, scales_out, stream)
    assert L.pa_debug_gather(ctypes.byref(c), 0x20000, 0x30000, 0x40000, 0x50000, None, None,
                             0x80000, None, None) == pa.PA_ERR_NULL
    assert L.pa_debug_gather(ctypes.byref(c), 0x20000, 0x30000, 0x40000, 0x50000, 0x70000,
                             0x90000, 0x80000, None, None) == pa.PA_ERR_SCALE_MODE
    assert L.pa_debug_gather(ctypes.byref(f8), 0x20000, 0x30000, 0x40000, 0x50000, 0x70000,
                             0x90000, 0x80000, None, None) == pa.PA_ERR_NULL
    assert L.pa_debug_gather(ctypes.byref(c), 0x20000, 0x30000, 0x40000, 0x50000, None,
                             0x90008, 0x80000, None, None) == pa.PA_ERR_ALIGN


def test_status_strings():
    for code in range(-9, 1):
        s = pa.pa_status_string(code)
        assert s and s != "unknown status"
    assert pa.pa_status_string(-100) == "unknown status"


def _append(d, nk=0x10000, nv=0x18000, bt=0x40000, ctx=0x50000, k=0x20000, v=0x30000,
            scales=None, status=None):
    return pa.lib().pa_cache_append(ctypes.byref(d) if d is not None else None, nk, nv, bt, ctx,
                                    k, v, scales, status, None)


def test_cache_append_argument_errors_before_any_device_call():
    d = _dims()
    assert _append(None) == pa.PA_ERR_NULL
    assert _append(d, nk=None) == pa.PA_ERR_NULL
    assert _append(d, v=None) == pa.PA_ERR_NULL
    assert _append(_dims(head_dim=64)) == pa.PA_ERR_UNSUPPORTED
    assert _append(_dims(batch=0)) == pa.PA_ERR_DIMS
    assert _append(d, nk=0x10008) == pa.PA_ERR_ALIGN
    assert _append(d, k=0x20004) == pa.PA_ERR_ALIGN
    assert _append(d, ctx=0x50002) == pa.PA_ERR_ALIGN
    assert _append(d, status=0x90002) == pa.PA_ERR_ALIGN
    assert _append(d, scales=0x70000) == pa.PA_ERR_SCALE_MODE
    f8 = _dims(kv_dtype=pa.PA_KV_FP8_E4M3FN, kv_scale_mode=pa.PA_SCALE_PER_TOKEN_HEAD)
    assert _append(f8) == pa.PA_ERR_SCALE_MODE
    assert _append(f8, scales=0x70002) == pa.PA_ERR_ALIGN


# ---- the Python binding checks tensors before any call reaches the library


def _cpu_plan(**kw):
    """A plan record (never built) with a CPU workspace, for argument checks."""
    c = _fake_plan(**kw)
    c.device = 0
    return pa.Plan(c, torch.empty(0, dtype=torch.uint8))


def _decode_tensors(d, **over):
    t = dict(q=torch.zeros(d.batch, d.q_len, d.num_q_heads, d.head_dim, dtype=torch.bfloat16),
             k_cache=torch.zeros(d.num_pages, d.num_kv_heads, d.page_size, d.head_dim,
                                 dtype=torch.bfloat16),
             block_table=torch.zeros(d.batch, d.max_pages_per_seq, dtype=torch.int32),
             context_lens=torch.ones(d.batch, dtype=torch.int32),
             out=torch.zeros(d.batch, d.q_len, d.num_q_heads, d.head_dim, dtype=torch.bfloat16))
    t["v_cache"] = t["k_cache"].clone()
    t.update(over)
    return t


def _py_decode(plan, t, mode=pa.PA_SCALE_NONE, scales=None):
    d = plan.c.dims
    return pa.pa_decode(plan, t["q"], t["k_cache"], t["v_cache"], t["block_table"],
                        t["context_lens"], d.q_len, 0.1, mode, scales, t["out"])


@pytest.mark.parametrize("field,value,code", [
    ("q", None, pa.PA_ERR_NULL),
    ("q", "wrong dtype", pa.PA_ERR_DIMS),
    ("q", "wrong shape", pa.PA_ERR_DIMS),
    ("out", "transposed", pa.PA_ERR_DIMS),
    ("k_cache", "fewer pages", pa.PA_ERR_DIMS),
    ("k_cache", "flat, one row short", pa.PA_ERR_DIMS),
    ("block_table", "int64", pa.PA_ERR_DIMS),
    ("block_table", "short rows", pa.PA_ERR_DIMS),
    ("context_lens", "wrong batch", pa.PA_ERR_DIMS),
    ("q", "cpu", pa.PA_ERR_DEVICE),
])
def test_binding_rejects_bad_tensors(field, value, code):
    plan = _cpu_plan(batch=2, q_len=1, max_pages_per_seq=8)
    d = plan.c.dims
    good = _decode_tensors(d)
    bad = {
        None: None,
        "wrong dtype": good["q"].float(),
        "wrong shape": good["q"][:, :, :8],
        "transposed": good["out"].transpose(2, 3).contiguous().transpose(2, 3),
        "fewer pages": good["k_cache"][:-1],
        "flat, one row short": good["k_cache"].flatten()[:-d.head_dim],
        "int64": good["block_table"].long(),
        "short rows": good["block_table"][:, :-1].contiguous(),
        "wrong batch": good["context_lens"][:1],
        "cpu": good["q"],
    }[value]
    with pytest.raises(pa.PaError) as e:
        _py_decode(plan, dict(good, **{field: bad}))
    assert e.value.code == code, e.value.text


def test_binding_rejects_scales_that_disagree_with_the_mode():
    f8 = _cpu_plan(kv_dtype=pa.PA_KV_FP8_E4M3FN, kv_scale_mode=pa.PA_SCALE_PER_TOKEN_HEAD)
    d = f8.c.dims
    t = _decode_tensors(d, k_cache=torch.zeros(d.num_pages, 1, d.page_size, d.head_dim,
                                               dtype=torch.uint8))
    t["v_cache"] = t["k_cache"].clone()
    with pytest.raises(pa.PaError) as e:       # per-token scales of the wrong shape
        _py_decode(f8, t, pa.PA_SCALE_PER_TOKEN_HEAD, torch.zeros(2, dtype=torch.float32))
    assert e.value.code == pa.PA_ERR_DIMS
    with pytest.raises(pa.PaError) as e:       # bf16 caches for an fp8 plan
        _py_decode(f8, _decode_tensors(d), pa.PA_SCALE_PER_TOKEN_HEAD,
                   torch.zeros(2, d.num_pages, 1, d.page_size, dtype=torch.float32))
    assert e.value.code == pa.PA_ERR_DIMS
    bf = _cpu_plan()
    with pytest.raises(pa.PaError) as e:       # scales with a bf16 cache
        _py_decode(bf, _decode_tensors(bf.c.dims), pa.PA_SCALE_NONE,
                   torch.ones(2, dtype=torch.float32))
    assert e.value.code == pa.PA_ERR_SCALE_MODE


def test_binding_rejects_host_context_lens_before_planning():
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(_dims(), torch.ones(2, dtype=torch.int32))
    assert e.value.code == pa.PA_ERR_DEVICE
    with pytest.raises(pa.PaError) as e:
        pa.pa_plan(_dims(), torch.ones(3, dtype=torch.int32))
    assert e.value.code == pa.PA_ERR_DIMS


def test_host_calls_from_many_threads_keep_their_own_errors():
    """The host entry points run concurrently from several threads (ctypes
    releases the GIL for each call): every thread gets the same answers as a
    lone caller, and pa_last_error reports the calling thread's own last
    failure, not another thread's."""
    import threading

    good = [pa.make_dims(batch=b, q_len=q, num_q_heads=16, num_kv_heads=h, head_dim=d, page_size=ps,
                         num_pages=64, max_pages_per_seq=8)
            for b, q, h, d, ps in [(1, 1, 1, 128, 128), (64, 1, 8, 128, 16), (4, 8, 16, 256, 32),
                                   (32, 4, 1, 128, 1024), (7, 3, 2, 128, 64)]]
    want_bytes = [pa.pa_workspace_bytes(d_, 256) for d_ in good]
    want_choice = [tuple(getattr(pa.pa_plan_choice(d_, 256), f) for f, _ in pa.pa_dims._fields_)
                   for d_ in good]
    errors = []

    def worker(t):
        try:
            for it in range(200):
                i = (t + it) % len(good)
                assert pa.pa_workspace_bytes(good[i], 256) == want_bytes[i]
                got = pa.pa_plan_choice(good[i], 256)
                assert tuple(getattr(got, f) for f, _ in pa.pa_dims._fields_) == want_choice[i]
                # a failure whose message names this thread's own bad head_dim
                bad = pa.make_dims(batch=1, q_len=1, num_q_heads=1, num_kv_heads=1,
                                   head_dim=1000 + t, page_size=16, num_pages=1, max_pages_per_seq=1)
                with pytest.raises(pa.PaError) as e:
                    pa.pa_workspace_bytes(bad, 256)
                assert e.value.code == pa.PA_ERR_UNSUPPORTED
                assert f"head_dim {1000 + t} " in e.value.text, e.value.text
        except BaseException as ex:  # reported by the main thread
            errors.append((t, repr(ex)))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors
