"""paged_attn_step_noalloc (the decode step for callers that cannot
allocate: its workspace is the library's static per-GPU scratch) against
paged_attn_step with a caller workspace, through the C ABI: bit-identical
outputs on two calls in a row, the second with a smaller batch, so the
second call runs on what the first left in the scratch."""
import pytest
import torch

import synth
from gpu_util import plan_for, run, pa_mod

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _noalloc(case_dev, plan):
    out = torch.full((case_dev.B, case_dev.Hq, case_dev.D), float("nan"), dtype=torch.float32,
                     device=DEV)
    pa_mod().paged_attn_step_noalloc(plan, case_dev.q, case_dev.k_pool, case_dev.v_pool, case_dev.table,
                                     case_dev.seq_len, out)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("pair", [("q4_0", "q4_0"), ("f16", "q8_0")])
def test_noalloc_step_equals_the_workspace_step(pair):
    big = synth.make_case([5000, 1200, 77, 0, 3000], k_fmt=pair[0], v_fmt=pair[1], seed=4101, junk="nan")
    small = synth.make_case([700, 31], k_fmt=pair[0], v_fmt=pair[1], seed=4102, junk="nan")
    for case, force in ((big, 0), (small, 3)):
        g = case.to(DEV)
        plan = plan_for(case, force_partitions=force)
        ref, ws = run(g, plan)
        assert pa_mod().paged_attn_status(ws) == 0
        got = _noalloc(g, plan)
        assert torch.equal(got, ref)


def test_noalloc_step_direct_mode():
    case = synth.workload("tiny_f16", seed=1000, junk="nan")
    g = case.to(DEV)
    plan = plan_for(case, force_partitions=1)
    ref, _ = run(g, plan)
    assert torch.equal(_noalloc(g, plan), ref)


def test_noalloc_step_refuses_plans_beyond_the_scratch():
    pa = pa_mod()
    shape = pa.shape_of(1024, 64, 4, 256, 16, 600000, 8192, "q4_0", "q4_0")
    plan = pa.paged_attn_plan(shape, 131072, num_cus=256, partition_tokens=256)
    assert plan.ws_bytes > 64 << 20
    x = torch.zeros(16, device=DEV)
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_step_noalloc(plan, x, x, x, x, x, x)
    assert e.value.code == pa.PA_ERR_INVALID and "static scratch" in str(e.value)
