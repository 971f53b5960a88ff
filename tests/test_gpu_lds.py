"""GPU parity of the LDS-staged decode kernel (plan path 2) on the shapes
that exercise its own machinery: several kv-head quads per block (strided
4-row DMA runs), large blocks, the largest head group, segments of the block
table, and the fall-back to the register kernel for unaligned pools."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import check_parity, plan_for, run, pa_mod

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(lens, **kw):
    kw.setdefault("junk", "nan")
    return synth.make_case(lens, **kw)


@pytest.mark.parametrize("Hq,Hkv,D,pair", [
    (24, 8, 256, ("q4_0", "q4_0")),     # two quads, r = 3
    (48, 12, 128, ("q8_0", "f16")),     # three quads, r = 4
    (16, 16, 128, ("q4_0", "q8_0")),    # four quads, r = 1
])
def test_several_head_quads(Hq, Hkv, D, pair):
    case = _case([300, 33, 1, 129], Hq=Hq, Hkv=Hkv, D=D, k_fmt=pair[0], v_fmt=pair[1],
                 seed=101 + Hkv)
    g = case.to(DEV)
    for force in (0, 1, 3):
        out, _ = run(g, plan_for(case, path=2, force_partitions=force))
        check_parity(case, out)


@pytest.mark.parametrize("bs", [64, 256])
def test_large_blocks(bs):
    case = _case([bs * 3 + 17, bs - 1, 2 * bs], block_size=bs, k_fmt="q4_0", v_fmt="q4_0",
                 seed=200 + bs)
    g = case.to(DEV)
    for force in (0, 1, 4):
        out, _ = run(g, plan_for(case, path=2, force_partitions=force))
        check_parity(case, out)


def test_sixteen_query_heads_per_kv_head():
    case = _case([250, 70], Hq=64, Hkv=4, D=256, k_fmt="q4_0", v_fmt="q8_0", seed=211)
    g = case.to(DEV)
    for force in (0, 1, 2):
        out, _ = run(g, plan_for(case, path=2, force_partitions=force))
        check_parity(case, out)


def test_block_table_segments_in_one_partition():
    """A partition longer than the 512 block ids staged at a time (direct mode
    over 20000 tokens = 1250 blocks) walks three segments of the table."""
    case = _case([20000, 9000], k_fmt="q4_0", v_fmt="q4_0", seed=223, junk="zero")
    g = case.to(DEV)
    for force in (1, 0):
        out, _ = run(g, plan_for(case, path=2, force_partitions=force))
        check_parity(case, out)


def test_unaligned_pools_fall_back_to_the_register_kernel():
    """Pools that are not 16-byte aligned are decoded by the register kernel
    even under a path-2 plan: the result equals a path-1 run bit for bit."""
    case = _case([500, 77], k_fmt="q4_0", v_fmt="q4_0", seed=227)
    g = case.to(DEV)

    def shifted(pool):
        raw = torch.empty(pool.numel() + 4, dtype=torch.uint8, device=DEV)
        view = raw[4:].view(pool.shape)
        view.copy_(pool)
        assert view.data_ptr() % 16 == 4
        return view

    gu = case.to(DEV)
    gu.k_pool = shifted(g.k_pool)
    gu.v_pool = shifted(g.v_pool)
    plan2 = plan_for(case, path=2, force_partitions=3)
    plan1 = plan_for(case, path=1, force_partitions=3)
    out_u, _ = run(gu, plan2)
    out_1, _ = run(g, plan1)
    assert torch.equal(out_u, out_1)
    check_parity(case, out_u)


def test_unaligned_q_falls_back_to_the_register_kernel():
    """A q that is not 16-byte aligned (the LDS-staged kernel reads it with
    16-byte loads) is decoded by the register kernel even under a path-2
    plan: the result equals a path-1 run bit for bit."""
    case = _case([500, 77], k_fmt="q4_0", v_fmt="q8_0", seed=229)
    g = case.to(DEV)
    gu = case.to(DEV)
    raw = torch.empty(g.q.numel() + 1, dtype=torch.float32, device=DEV)
    gu.q = raw[1:].view(g.q.shape)
    gu.q.copy_(g.q)
    assert gu.q.data_ptr() % 16 == 4
    plan2 = plan_for(case, path=2, force_partitions=3)
    plan1 = plan_for(case, path=1, force_partitions=3)
    out_u, _ = run(gu, plan2)
    out_1, _ = run(g, plan1)
    assert torch.equal(out_u, out_1)
    check_parity(case, out_u)


def test_both_kernels_agree_within_tolerance():
    """Same inputs, same partitioning: the two kernels differ only in the
    order of fp32 accumulation."""
    case = _case([3000, 1234, 16], k_fmt="q8_0", v_fmt="q4_0", seed=229)
    g = case.to(DEV)
    plan1 = plan_for(case, path=1, force_partitions=3)
    plan2 = plan_for(case, path=2, force_partitions=3)
    o1, _ = run(g, plan1)
    o2, _ = run(g, plan2)
    d = (o1 - o2).abs().amax(dim=-1) / o1.abs().amax(dim=-1).clamp_min(1e-30)
    assert float(d.max()) < 2e-3
    check_parity(case, o2)
