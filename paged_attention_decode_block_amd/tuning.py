"""Tuned launch settings per shape class: the table the library compiles in.

"[Kernel][Perf] Optimize paged-attention metadata decode" (ROCm/FlyDSL PR
#910, "Pull request overview" and "Summary") keeps a tuned persistent-grid
choice per shape in a CSV file, read through lookup utilities, with one grid
per CU as the default where a shape has no entry. Here the table is
``tuning.csv`` beside this module. ``bench.py --tune`` writes it from HIP-graph
timings of the decode. The build turns it into C rows that ``pa_plan`` looks up
on the host (``pa_plan_choice`` in ``include/pa.h``). Only settings the caller
leaves unset take the table's value: partition_size and grid_multiplier at 0,
and neither reduce flag.

Key: (num_cus, head_dim, kv_dtype, kv_scale_mode, row_tiles, page_size,
pairs_log2, capacity_log2), where
row_tiles = ceil(q_len * num_q_heads / num_kv_heads / 16),
pairs_log2 = floor(log2(batch * num_kv_heads)) and
capacity_log2 = floor(log2(max_pages_per_seq * page_size)).
Value: (grid_multiplier, partition_size, fused_reduce). Two more columns are
informational: the decode time measured for the choice and the workload it
was tuned on.
"""
from __future__ import annotations

import csv
import dataclasses
import os
from typing import Iterable, List, Optional, Tuple

TABLE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tuning.csv")

KEY_COLUMNS = ("num_cus", "head_dim", "kv_dtype", "kv_scale_mode", "row_tiles", "page_size",
               "pairs_log2", "capacity_log2")
VALUE_COLUMNS = ("grid_multiplier", "partition_size", "fused_reduce")
INFO_COLUMNS = ("decode_us", "workload")
COLUMNS = KEY_COLUMNS + VALUE_COLUMNS + INFO_COLUMNS

Key = Tuple[int, int, int, int, int, int, int, int]


@dataclasses.dataclass(frozen=True)
class Entry:
    num_cus: int
    head_dim: int
    kv_dtype: int
    kv_scale_mode: int
    row_tiles: int
    page_size: int
    pairs_log2: int
    capacity_log2: int
    grid_multiplier: int
    partition_size: int
    fused_reduce: int
    decode_us: float = 0.0
    workload: str = ""

    @property
    def key(self) -> Key:
        return tuple(getattr(self, c) for c in KEY_COLUMNS)

    @property
    def value(self) -> Tuple[int, int, int]:
        return tuple(getattr(self, c) for c in VALUE_COLUMNS)


def _floor_log2(x: int) -> int:
    return int(x).bit_length() - 1


def shape_key(dims, num_cus: int) -> Key:
    """The shape class of a pa_dims (anything with its field names)."""
    rows = dims.q_len * (dims.num_q_heads // dims.num_kv_heads)
    return (int(num_cus), int(dims.head_dim), int(dims.kv_dtype), int(dims.kv_scale_mode),
            -(-rows // 16), int(dims.page_size), _floor_log2(dims.batch * dims.num_kv_heads),
            _floor_log2(dims.max_pages_per_seq * dims.page_size))


def validate(e: Entry) -> None:
    """Reject rows the library would refuse (it checks the same ranges)."""
    if not 1 <= e.grid_multiplier <= 16:
        raise ValueError(f"grid_multiplier {e.grid_multiplier} outside [1, 16]")
    if e.partition_size < 16 or e.partition_size % 16 or e.partition_size > 1 << 20:
        raise ValueError(f"partition_size {e.partition_size} is not a multiple of 16 in range")
    if e.fused_reduce not in (0, 1):
        raise ValueError(f"fused_reduce {e.fused_reduce} is not 0 or 1")
    if e.num_cus < 1 or e.head_dim not in (128, 256) or e.row_tiles < 1:
        raise ValueError(f"bad key {e.key}")


def read_table(path: str = TABLE) -> List[Entry]:
    if not os.path.exists(path):
        return []
    with open(path, newline="") as f:
        rows = [r for r in csv.reader(f) if r and not r[0].startswith("#")]
    if not rows:
        return []
    header = tuple(rows[0])
    if header != COLUMNS:
        raise ValueError(f"{path}: header {header} is not {COLUMNS}")
    out = []
    for r in rows[1:]:
        vals = dict(zip(COLUMNS, r))
        e = Entry(**{c: int(vals[c]) for c in KEY_COLUMNS + VALUE_COLUMNS},
                  decode_us=float(vals["decode_us"] or 0), workload=vals["workload"])
        validate(e)
        out.append(e)
    keys = [e.key for e in out]
    if len(set(keys)) != len(keys):
        raise ValueError(f"{path}: a shape class appears twice")
    return out


def write_table(entries: Iterable[Entry], path: str = TABLE) -> None:
    entries = sorted(entries, key=lambda e: e.key)
    tmp = path + ".tmp"
    with open(tmp, "w", newline="") as f:
        w = csv.writer(f, lineterminator="\n")
        w.writerow(COLUMNS)
        for e in entries:
            validate(e)
            w.writerow([getattr(e, c) for c in COLUMNS])
    os.replace(tmp, path)


def lookup(entries: Iterable[Entry], key: Key) -> Optional[Entry]:
    for e in entries:
        if e.key == tuple(key):
            return e
    return None


def upsert(entries: Iterable[Entry], entry: Entry) -> List[Entry]:
    """The table with `entry` replacing the row of its shape class, or added."""
    validate(entry)
    out = [e for e in entries if e.key != entry.key]
    out.append(entry)
    return sorted(out, key=lambda e: e.key)


def render_rows(entries: Iterable[Entry]) -> str:
    """The table as C initialisers for the library's build (one row each)."""
    lines = ["// generated from tuning.csv by the build; do not edit"]
    for e in sorted(entries, key=lambda e: e.key):
        vals = ", ".join(str(v) for v in e.key + e.value)
        lines.append(f"    {{{vals}}},  // {e.workload}")
    return "\n".join(lines) + "\n"
