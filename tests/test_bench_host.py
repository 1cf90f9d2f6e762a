"""Host-side parts of bench.py: the one-GPU guard and the committed counter
records it reports (HBM traffic and MFMA busy fraction of the partition
kernel), which count only while the kernel sources hash to the recorded
digest."""
import subprocess
import sys
from pathlib import Path

import bench
import workloads as W

ROOT = Path(__file__).resolve().parents[1]


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, str(ROOT / "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr and r.stdout == ""


def _records(path, tag):
    out = {}
    for ln in Path(path).read_text().splitlines():
        f = ln.split()
        if len(f) == 5 and f[0] == tag:
            out[f[1]] = f
    return out


def test_counter_records_cover_every_benched_workload():
    for path, tag in ((bench.TRAFFIC_FILE, "traffic"), (bench.MFMA_FILE, "mfma")):
        recs = _records(path, tag)
        assert set(recs) == set(W.CONFIGS), (path, sorted(recs))
        assert bench.HEADLINE in recs
        digests = {f[2] for f in recs.values()}
        assert len(digests) == 1 and len(digests.pop()) == 64


def test_records_are_dropped_when_the_sources_change(monkeypatch):
    recs = _records(bench.MFMA_FILE, "mfma")
    digest = recs[bench.HEADLINE][2]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: digest)
    m = bench.recorded_mfma(bench.HEADLINE)
    assert m is not None and 0 <= m["busy_frac"] <= 1 and m["flops_per_launch"] > 0
    t = bench.recorded_traffic(bench.HEADLINE)
    assert t is None or t["total_bytes"] == t["read_bytes"] + t["written_bytes"]
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.recorded_mfma(bench.HEADLINE) is None
    assert bench.recorded_traffic(bench.HEADLINE) is None
    assert bench.recorded_mfma("no_such_workload") is None


def _shared_tile_workloads():
    """Workloads whose partition kernel (as named in the committed kernel-trace
    record) shares K/V tiles between waves: its tenth template argument."""
    out = set()
    for ln in (ROOT / "profiles" / "pa_kernels_trace_all_workloads.md").read_text().splitlines():
        f = [x.strip() for x in ln.split("|")]
        if len(f) > 3 and f[2].startswith("`partition_kernel<"):
            args = f[2][len("`partition_kernel<"):-2].split(",")
            if args[9].strip() == "true":
                out.add(f[1])
    return out


def test_mfma_flops_match_the_padded_tile_count():
    """Executed bf16 MFMA flops per launch (counted on the GPU) = 4 x kv heads
    x head_dim x the query rows of a kv head rounded up to the 16-row MFMA tile
    x each sequence's tokens rounded up to the kernel's 32-token step (QK^T
    and PV, 2 flops per product each). A shared-tile kernel adds one 16-column
    PV tile of ones, its row sums: 2 x 16 more per token and row."""
    recs = _records(bench.MFMA_FILE, "mfma")
    shared = _shared_tile_workloads()
    assert shared == {"C4_fp8_q4_per_token", "C4_fp8_q4_per_tensor"}
    for name, f in recs.items():
        s = W.CONFIGS[name]
        t = int(((W.draw_context_lens(s, 2026) + 31) // 32 * 32).sum())
        rows = s.q_len * (s.num_q_heads // s.num_kv_heads)
        padded = -(-rows // 16) * 16
        cols = 2 * s.head_dim + (16 if name in shared else 0)
        assert int(f[4]) == 2 * t * s.num_kv_heads * padded * cols, name


def test_scale_sweep_shapes_are_valid():
    """Every scaled shape of the sweep keeps q_len <= ctx_lo <= ctx_hi and a
    block table wide enough for ctx_hi."""
    for name, factors in bench.SWEEP:
        base = W.CONFIGS[name]
        assert 1.0 in factors
        for f in factors:
            hi = int(base.ctx_hi * f)
            lo = max(int(base.ctx_lo * f), base.q_len)
            s = W.scaled(base, ctx_lo=lo, ctx_hi=hi, max_ctx=0)
            assert s.q_len <= s.ctx_lo <= s.ctx_hi
            assert s.max_pages_per_seq * s.page_size >= s.ctx_hi
            ctx = W.draw_context_lens(s, 2026)
            assert int(ctx.min()) >= lo and int(ctx.max()) <= hi


def test_plan_sweep_shapes_are_valid_dims():
    """Every batch of the plan sweep passes the library's host-side dims
    checks (no GPU call: the workspace size for 256 CUs)."""
    import paged_attention_decode_block_amd as pa
    for B, hkv in bench.PLAN_SWEEP:
        dims = pa.make_dims(batch=B, q_len=1, num_q_heads=4 * hkv, num_kv_heads=hkv, head_dim=128,
                            page_size=16, num_pages=B * 512, max_pages_per_seq=512,
                            kv_dtype=pa.PA_KV_BF16, kv_scale_mode=pa.PA_SCALE_NONE)
        assert pa.pa_workspace_bytes(dims, 256) > 0


def test_cpu_model_is_read_from_proc_cpuinfo():
    m = bench.cpu_model()
    assert m is None or (isinstance(m, str) and m)
