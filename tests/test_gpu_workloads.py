"""GPU parity at the pages' workload sizes, on every (sequence, kv-head) group
(the oracle computes them one by one from host copies of the blocks they
use), in the launch configuration bench.py times (automatic plan, all K/V
bytes resident on the device). The whole output must also be finite."""
import gc

import numpy as np
import pytest
import torch

import synth
from gpu_util import all_groups, plan_for, run, sampled_parity, pa_mod

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _free():
    gc.collect()
    torch.cuda.empty_cache()


def _run_auto(case):
    plan = plan_for(case)
    out, ws = run(case, plan)
    assert pa_mod().paged_attn_status(ws) == 0
    return out, plan


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_uniform_q8_0_4k(B):
    case = synth.workload("uniform_q8_0", B=B, L=4096, seed=1100 + B, device=DEV)
    out, _ = _run_auto(case)
    sampled_parity(case, out, all_groups(case))
    _free()


@pytest.mark.parametrize("B,L", [(B, L) for L in (32768, 131072) for B in (1, 2, 4, 8)])
def test_uniform_q4_0_long_context(B, L):
    case = synth.workload("uniform_q4_0", B=B, L=L, seed=1200 + B, device=DEV)
    out, plan = _run_auto(case)
    assert plan.p_max > 1
    sampled_parity(case, out, all_groups(case))
    _free()


def test_ragged_128k_plus_7x8k():
    case = synth.workload("ragged_q4_0", seed=1300, device=DEV)
    assert sum(case.seq_lens) == 188416
    out, _ = _run_auto(case)
    sampled_parity(case, out, all_groups(case))
    _free()


def test_ragged_small_4k_plus_7x256_all_heads():
    case = synth.workload("ragged_small_q4_0", seed=1301, device=DEV)
    out, _ = _run_auto(case)
    sampled_parity(case, out, all_groups(case))
    _free()


def test_slab_past_2pow32_elements_gather_and_decode():
    """F16 pool of 139,264 blocks of [32, 8, 128] (> 2^32 elements per side),
    B=8 x 65536 tokens with half of each sequence's blocks past element 2^32
    (mlxcel issue #2153: Problem, Acceptance Criteria)."""
    pa = pa_mod()
    case = synth.make_case([65536] * 8, Hq=32, Hkv=8, D=128, block_size=32, k_fmt="f16",
                           v_fmt="f16", nblocks=139264, table_mode="split", split_block=131072,
                           seed=1400, device=DEV, junk="random")
    assert case.k_pool.numel() // 2 > 2**32          # f16 elements per side
    high = case.table[:, :2048] >= 131072
    assert int(high.sum()) == 8 * 1024
    plan = plan_for(case)
    # bit-exact gather of a sequence whose rows straddle the 2^32 boundary
    rb = 256
    for which, pool in ((0, case.k_pool), (1, case.v_pool)):
        for b in (0, 5):
            n = 65536
            dst = torch.empty((n, 8, rb), dtype=torch.uint8, device=DEV)
            pa.paged_kv_gather(plan, pool, which, case.table, b, 0, n, dst)
            torch.cuda.synchronize()
            t = torch.arange(n, device=DEV)
            ids = case.table[b].to(DEV).long()[t // 32]
            ref = pool.view(-1, 32, 8, rb)[ids, t % 32]
            assert torch.equal(dst, ref)
            # a 32-bit wrap would read the row 2^32 elements lower instead
            hi = ids >= 131072
            wrapped = pool.view(-1, 32, 8, rb)[ids[hi] - 131072, (t % 32)[hi]]
            assert not torch.equal(dst[hi], wrapped)
            del dst, ref, wrapped
    out, _ = _run_auto(case)
    sampled_parity(case, out, all_groups(case))
    del case, out
    _free()


def test_uniform_f16_d256_32k_on_eight_slot_groups():
    """F16 K and V at D=256 (the lucebox page's head size): 16 slots of four
    heads' rows do not fit a ring slot, so the LDS-staged kernel streams
    8-slot groups; every (sequence, kv head) group is checked at 8 x 32K."""
    case = synth.workload("uniform_f16", B=8, L=32768, seed=1500, device=DEV)
    out, plan = _run_auto(case)
    assert plan.path == 2 and plan.p_max > 1
    sampled_parity(case, out, all_groups(case))
    _free()
