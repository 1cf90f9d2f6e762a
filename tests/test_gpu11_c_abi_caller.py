"""The C-ABI from a plain C caller.

Every other test reaches the library through the Python binding. Here
tests/c/pa_c_abi_decode.c, a C11 program built by build() against
include/pa.h and libpa.so alone, does what a C caller would: it allocates
device memory with hipMalloc, sizes the workspace with pa_workspace_bytes,
builds the plan and decodes on a stream of its own, and reads the device
status. It runs as a child process on inputs written to files. Its output
must equal the binding's on the same inputs bit for bit (same dims, so the
same plan and instantiation), and the oracle within the dtype's tolerance.
"""
import os
import subprocess

import numpy as np
import pytest
import torch

import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import KV_CODE, MODE_CODE, check, dims_for, run, say

pytestmark = pytest.mark.gpu

BIN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "c", "pa_c_abi_decode")

CASES = {
    "bf16 batched GQA": W.scaled(W.C3, batch=5, ctx_lo=100, ctx_hi=1200, max_ctx=1280),
    "bf16 single sequence (fused reduce by the table)": W.C2,
    "fp8 per-token q4 (shared tiles)": W.scaled(W.C4_Q4_TOK, batch=3, ctx_lo=300, ctx_hi=3000,
                                                max_ctx=3072),
    "fp8 per-tensor q1": W.scaled(W.C4_Q1_TEN, batch=3, ctx_lo=4, ctx_hi=3000, max_ctx=3072),
    "bf16 head_dim 256, q_len 8": W.scaled(W.C5, batch=2, ctx_lo=300, ctx_hi=1500,
                                           max_ctx=1536, pool_slack=0.2),
}


def _write(w: W.Workload, d: str) -> None:
    s = w.spec
    dims = dims_for(w)
    fields = [getattr(dims, f) for f, _ in pa.pa_dims._fields_]
    with open(os.path.join(d, "dims.txt"), "w") as f:
        f.write(" ".join(str(int(x)) for x in fields))
        f.write(f" {s.q_len} {s.scale!r} {MODE_CODE[s.kv_scale_mode]}\n")
    bits = lambda t: t.contiguous().view(torch.int16) if t.dtype == torch.bfloat16 else t.contiguous()
    bits(w.q).numpy().tofile(os.path.join(d, "q.bin"))
    bits(w.k_cache).numpy().tofile(os.path.join(d, "k.bin"))
    bits(w.v_cache).numpy().tofile(os.path.join(d, "v.bin"))
    w.block_table.to(torch.int32).contiguous().numpy().tofile(os.path.join(d, "bt.bin"))
    w.context_lens.to(torch.int32).contiguous().numpy().tofile(os.path.join(d, "ctx.bin"))
    if w.kv_scales is not None:
        w.kv_scales.to(torch.float32).contiguous().numpy().tofile(os.path.join(d, "scales.bin"))


@pytest.mark.parametrize("name", sorted(CASES))
def test_c_caller_matches_the_binding_and_the_oracle(name, tmp_path):
    assert os.path.exists(BIN), "tests/c/pa_c_abi_decode is built by __graft_entry__.build()"
    spec = CASES[name]
    w = W.generate(spec, 2026)
    assert KV_CODE[spec.kv_dtype] in (pa.PA_KV_BF16, pa.PA_KV_FP8_E4M3FN)
    _write(w, str(tmp_path))
    say(f"[c caller] {name}")
    res = subprocess.run([BIN, str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, f"C caller failed ({res.returncode}): {res.stdout}{res.stderr}"
    say(f"[c caller] {name}: {res.stdout.strip()}")
    got = np.fromfile(tmp_path / "out.bin", dtype=np.int16).reshape(tuple(w.q.shape))
    ref, plan = run(w)
    assert res.stdout.split()[:2] == ["status", "0"]
    assert int(res.stdout.split()[3]) == plan.c.grid and int(res.stdout.split()[5]) == plan.c.variant
    np.testing.assert_array_equal(got, ref.view(torch.int16).cpu().numpy())
    check(w, torch.from_numpy(got).view(torch.bfloat16), f"C caller, {name}")
