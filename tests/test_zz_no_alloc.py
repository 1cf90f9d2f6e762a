"""pa_decode_static: plan + decode in the library's static scratch, for
callers that cannot allocate. Its output must equal pa_plan + pa_decode's
(the same kernels over the same plan, so bitwise) on two calls in a row, the
second with a smaller problem, and both must match the oracle. A problem too
big for the scratch is rejected before any launch."""
import pytest
import torch

import paged_attention_decode_block_amd as pa
import workloads as W
from tests.gpu_util import DEV, MODE_CODE, check, dims_for, run, say, upload

pytestmark = pytest.mark.gpu


def _static(w: W.Workload, d):
    s = w.spec
    out = torch.full_like(d.q, float("nan"))
    plan = pa.pa_decode_static(dims_for(w), d.q, d.k_cache, d.v_cache, d.block_table,
                               d.context_lens, s.q_len, s.scale, MODE_CODE[s.kv_scale_mode],
                               d.kv_scales, out)
    return out, plan


@pytest.mark.parametrize("first,second", [
    (W.scaled(W.C3, batch=12, ctx_lo=300, ctx_hi=3000, max_ctx=4096),
     W.scaled(W.C3, batch=3, ctx_lo=20, ctx_hi=700, max_ctx=1024)),
    (W.scaled(W.C4_Q4_TOK, batch=6, ctx_lo=1000, ctx_hi=9000, max_ctx=10240),
     W.scaled(W.C4_Q4_TOK, batch=2, ctx_lo=5, ctx_hi=1500, max_ctx=2048)),
])
def test_static_scratch_matches_the_workspace_path(first, second):
    for i, spec in enumerate((first, second)):
        w = W.generate(spec, 2026 + i)
        say(f"[static] call {i}: {spec.name} batch {spec.batch} ctx {w.context_lens.tolist()}")
        d = upload(w)
        want, plan_ws = run(w, d)
        got, plan_st = _static(w, d)
        assert pa.pa_plan_status(plan_st) == 0 and pa.pa_plan_status(plan_ws) == 0
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), f"call {i}"
        check(w, got, f"static scratch, call {i}")


def test_static_scratch_rejects_problems_past_its_size():
    spec = W.scaled(W.C3, batch=64, max_ctx=1 << 20)      # a 2^20-token block table
    dims = dims_for(W.Workload(spec, 0, None, None, None, None, None, None, 16))
    need = pa.pa_workspace_bytes(dims, pa.pa_query_device(0))
    assert need > pa.pa_static_scratch_bytes()
    q = torch.zeros(spec.batch, 1, spec.num_q_heads, spec.head_dim, dtype=torch.bfloat16,
                    device=DEV)
    kc = torch.zeros(16, spec.num_kv_heads, spec.page_size, spec.head_dim, dtype=torch.bfloat16,
                     device=DEV)
    bt = torch.zeros(spec.batch, dims.max_pages_per_seq, dtype=torch.int32, device=DEV)
    ctx = torch.ones(spec.batch, dtype=torch.int32, device=DEV)
    out = torch.zeros_like(q)
    with pytest.raises(pa.PaError) as e:
        pa.pa_decode_static(dims, q, kc, kc, bt, ctx, 1, spec.scale, pa.PA_SCALE_NONE, None, out)
    assert e.value.code == pa.PA_ERR_WORKSPACE
    assert (out == 0).all()
