"""The single-launch decode (plan.fused: the LDS-staged kernel also merges,
its workgroups claiming decode units and then merge slices from a counter in
the workspace; llama.cpp PR #13 HRX, Changes: the partials reduced by the
decode launch itself; lucebox PR #555, Roadmap item 4) against the
two-launch step (decode, then the merge kernel) on the same plan: the same
bits, always. Also: the workspace counters are zero after every call, a
counter left non-zero is detected (status bit, NaN columns) and cleared, and
repeated calls agree bit for bit."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_parity, plan_for, run, pa_mod

pytestmark = pytest.mark.gpu
DEV = "cuda"

CASES = {
    "ragged_q4_0": dict(lens=[3000, 1, 0, 700, 33, 1999], k_fmt="q4_0", v_fmt="q4_0"),
    "q8_0_f16": dict(lens=[5000, 4096, 17, 64], k_fmt="q8_0", v_fmt="f16", D=128, Hq=32, Hkv=8),
    "q4_0_q8_0_two_quads": dict(lens=[2500, 900, 0], k_fmt="q4_0", v_fmt="q8_0", Hq=24, Hkv=8),
    "f16_d128_r4": dict(lens=[4000, 129], k_fmt="f16", v_fmt="f16", D=128, Hq=32, Hkv=8),
    "q4_0_bs64": dict(lens=[3333, 640, 64], k_fmt="q4_0", v_fmt="q4_0", block_size=64),
}


def _counters_zero(ws, plan):
    raw = ws[:int(plan.part_offset)].cpu()
    return bool(torch.all(raw[4:12] == 0)) and bool(torch.all(raw[256:] == 0))


@pytest.mark.parametrize("name", sorted(CASES))
@pytest.mark.parametrize("force", [0, 3, 8])
def test_fused_equals_two_launches_bit_for_bit(name, force):
    kw = dict(CASES[name])
    lens = kw.pop("lens")
    case = synth.make_case(lens, seed=4200 + force, junk="nan", **kw)
    g = case.to(DEV)
    plan = plan_for(case, force_partitions=force)
    if plan.direct:
        pytest.skip("one partition: nothing to merge")
    assert plan.path == 2 and plan.fused == 0          # the planner's choice: two launches
    plan.fused = 1
    fused, ws = run(g, plan)
    assert pa_mod().paged_attn_status(ws) == 0
    assert _counters_zero(ws, plan)
    plan.fused = 0
    two, _ = run(g, plan)
    assert torch.equal(fused, two)
    check_parity(case, fused)


def test_fused_with_a_tiny_grid_and_repeats():
    """Two CUs' worth of workgroups: each claims many units and slices in turn;
    repeated calls on one workspace agree bit for bit and leave it clean."""
    case = synth.make_case([6000, 2000, 1, 0, 4097], k_fmt="q4_0", v_fmt="q4_0", seed=4301, junk="nan")
    g = case.to(DEV)
    plan = plan_for(case, num_cus=2, partition_tokens=256)
    plan.fused = 1
    assert plan.grid == 4
    ws = pa_mod().workspace(plan, DEV)
    outs = [run(g, plan, ws=ws)[0] for _ in range(3)]
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])
    assert _counters_zero(ws, plan)
    plan.fused = 0
    assert torch.equal(run(g, plan)[0], outs[0])
    check_parity(case, outs[0])


def test_counters_left_nonzero_are_flagged_and_cleared():
    """A workspace whose done counters were not zeroed (here: past any
    partition count) makes every merge slice give up at once: status bit
    PA_STATUS_MERGE_WAIT and NaN columns, no hang; the launch still zeroes
    the counters, so the next call is correct."""
    pa = pa_mod()
    case = synth.make_case([3000, 500], k_fmt="q4_0", v_fmt="q4_0", seed=4311, junk="nan")
    g = case.to(DEV)
    plan = plan_for(case)
    plan.fused = 1
    ws = pa.workspace(plan, DEV)
    n_done = case.B * (case.Hkv // 4)
    done = ws[256:int(plan.part_offset)].view(torch.int32)
    done[0:1040 * n_done:1040] = 0x7FFFFFF0           # one counter every 1040 words
    out, _ = run(g, plan, ws=ws)
    assert pa.paged_attn_status(ws) & pa.PA_STATUS_MERGE_WAIT
    assert bool(torch.isnan(out).all())
    assert _counters_zero(ws, plan)
    out, _ = run(g, plan, ws=ws)
    assert pa.paged_attn_status(ws) == 0
    check_parity(case, out)


@pytest.mark.parametrize("workload,L", [("uniform_q4_0", 32768), ("ragged_q4_0", 131072)])
def test_fused_equals_two_launches_at_full_size(workload, L):
    case = synth.workload(workload, B=8, L=L, seed=4400, device=DEV)
    plan = plan_for(case)
    plan.fused = 1
    fused, ws = run(case, plan)
    assert pa_mod().paged_attn_status(ws) == 0 and _counters_zero(ws, plan)
    plan.fused = 0
    two, _ = run(case, plan)
    assert torch.equal(fused, two)
    assert bool(torch.isfinite(fused).all())
