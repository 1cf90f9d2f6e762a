"""The tuning table (tuning.csv) and the library's lookup of it, on the CPU.

The CSV utilities (read, write, lookup, upsert) round-trip and reject bad
rows; the library compiled from the committed table makes, for every row,
the choice the row records (pa_plan_choice, host-only), keeps fields the
caller set, and falls back to the defaults for shapes the table lacks."""
import os

import pytest

import paged_attention_decode_block_amd as pa
from paged_attention_decode_block_amd import tuning as T


def _entry(**kw):
    base = dict(num_cus=256, head_dim=128, kv_dtype=0, kv_scale_mode=0, row_tiles=1,
                page_size=16, pairs_log2=9, capacity_log2=13, grid_multiplier=1,
                partition_size=256, fused_reduce=0, decode_us=1.5, workload="w")
    base.update(kw)
    return T.Entry(**base)


def test_round_trip_and_upsert(tmp_path):
    path = os.path.join(tmp_path, "t.csv")
    assert T.read_table(path) == []
    a = _entry()
    b = _entry(page_size=32, grid_multiplier=2, fused_reduce=1, workload="x")
    table = T.upsert(T.upsert([], a), b)
    T.write_table(table, path)
    back = T.read_table(path)
    assert back == sorted([a, b], key=lambda e: e.key)
    # same key: replaced, not duplicated
    a2 = _entry(partition_size=128, decode_us=1.2)
    table = T.upsert(back, a2)
    assert len(table) == 2 and T.lookup(table, a.key) == a2
    assert T.lookup(table, _entry(page_size=64).key) is None


def test_bad_rows_are_rejected(tmp_path):
    for bad in (dict(grid_multiplier=0), dict(grid_multiplier=17), dict(partition_size=24),
                dict(fused_reduce=2), dict(head_dim=64)):
        with pytest.raises(ValueError):
            T.upsert([], _entry(**bad))
    path = os.path.join(tmp_path, "dup.csv")
    with open(path, "w") as f:
        f.write(",".join(T.COLUMNS) + "\n")
        row = ",".join(str(getattr(_entry(), c)) for c in T.COLUMNS)
        f.write(row + "\n" + row + "\n")
    with pytest.raises(ValueError):
        T.read_table(path)


def test_shape_key_matches_the_documented_classes():
    d = pa.make_dims(batch=64, q_len=1, num_q_heads=32, num_kv_heads=8, head_dim=128,
                     page_size=16, num_pages=100, max_pages_per_seq=512)
    assert T.shape_key(d, 256) == (256, 128, 0, 0, 1, 16, 9, 13)
    d = pa.make_dims(batch=32, q_len=4, num_q_heads=16, num_kv_heads=1, head_dim=128,
                     page_size=1024, num_pages=100, max_pages_per_seq=32,
                     kv_dtype=pa.PA_KV_FP8_E4M3FN, kv_scale_mode=pa.PA_SCALE_PER_TOKEN_HEAD)
    assert T.shape_key(d, 256) == (256, 128, 1, 2, 4, 1024, 5, 15)


def _dims_of(e: T.Entry, **kw):
    """pa_dims in entry e's shape class."""
    group = 16
    rows = 16 * e.row_tiles
    q_len = max(1, rows // group)
    cap = 1 << e.capacity_log2
    base = dict(batch=1 << e.pairs_log2, q_len=q_len, num_q_heads=group, num_kv_heads=1,
                head_dim=e.head_dim, page_size=e.page_size, num_pages=64,
                max_pages_per_seq=cap // e.page_size, kv_dtype=e.kv_dtype,
                kv_scale_mode=e.kv_scale_mode)
    base.update(kw)
    return pa.make_dims(**base)


def test_library_applies_the_committed_table():
    table = T.read_table()
    for e in table:
        d = _dims_of(e)
        assert T.shape_key(d, e.num_cus) == e.key
        c = pa.pa_plan_choice(d, e.num_cus)
        fused = bool(c.flags & pa.PA_FLAG_FUSED_REDUCE)
        assert (c.grid_multiplier, c.partition_size, int(fused)) == e.value, e
        assert bool(c.flags & pa.PA_FLAG_SEPARATE_REDUCE) != fused
        # fields the caller sets are kept
        c2 = pa.pa_plan_choice(_dims_of(e, partition_size=64, grid_multiplier=3,
                                        flags=pa.PA_FLAG_SEPARATE_REDUCE), e.num_cus)
        assert (c2.partition_size, c2.grid_multiplier) == (64, 3)
        assert c2.flags & pa.PA_FLAG_SEPARATE_REDUCE and not c2.flags & pa.PA_FLAG_FUSED_REDUCE
        # another CU count is another device class: defaults unless it has a row
        if T.lookup(table, (e.num_cus + 1,) + e.key[1:]) is None:
            c3 = pa.pa_plan_choice(d, e.num_cus + 1)
            assert (c3.grid_multiplier, c3.partition_size) == (1, 256)
            assert c3.flags & pa.PA_FLAG_SEPARATE_REDUCE


def test_defaults_without_an_entry():
    d = pa.make_dims(batch=3, q_len=1, num_q_heads=8, num_kv_heads=8, head_dim=128,
                     page_size=64, num_pages=64, max_pages_per_seq=5)
    assert T.lookup(T.read_table(), T.shape_key(d, 7)) is None
    c = pa.pa_plan_choice(d, 7)
    assert (c.grid_multiplier, c.partition_size) == (1, 256)
    assert c.flags == pa.PA_FLAG_SEPARATE_REDUCE
    c = pa.pa_plan_choice(pa.make_dims(batch=3, q_len=1, num_q_heads=8, num_kv_heads=8,
                                       head_dim=128, page_size=64, num_pages=64,
                                       max_pages_per_seq=5, flags=pa.PA_FLAG_FUSED_REDUCE), 7)
    assert c.flags == pa.PA_FLAG_FUSED_REDUCE
    # the workspace follows the choice: a fused plan needs the same bytes
    assert pa.pa_workspace_bytes(d, 7) > 0


def test_build_renders_every_row():
    table = T.read_table()
    text = T.render_rows(table)
    assert text.count("{") == len(table)
