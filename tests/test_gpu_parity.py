"""GPU parity of the HIP decode path against the fp64 oracle, through the C ABI.

Tolerance (on the per-row max-abs error relative to the row's max-abs
output): 2e-3 when K and V are F16, 5e-3 when either is quantised. Indexing
(the raw gather) is compared bit for bit; paged and contiguous layouts, and
repeated runs, must agree bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import check_parity, plan_for, run, shape_for, pa_mod, rel_err_rows, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = [(k, v) for k in synth.FORMATS for v in synth.FORMATS]
PATHS = [1, 2]      # decode kernel: register-streaming, LDS-staged


def _case(lens, **kw):
    kw.setdefault("junk", "nan")
    return synth.make_case(lens, **kw)


def test_tiny_f16_workload_all_partitionings():
    case = synth.workload("tiny_f16", seed=1000)
    g = case.to(DEV)
    for force in (0, 1, 2, 3, 7):
        plan = plan_for(case, force_partitions=force)
        out, ws = run(g, plan)
        check_parity(case, out)
        assert pa_mod().paged_attn_status(ws) == 0


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("D", [256, 128])
@pytest.mark.parametrize("pair", PAIRS, ids=[f"{k}-{v}" for k, v in PAIRS])
def test_nine_type_pairs(pair, D, path):
    k_fmt, v_fmt = pair
    Hq, Hkv = (24, 4) if D == 256 else (32, 8)
    lens = [200, 1, 16, 17, 33, 0, 95]
    case = _case(lens, Hq=Hq, Hkv=Hkv, D=D, block_size=16, k_fmt=k_fmt, v_fmt=v_fmt,
                 seed=7 + D + 3 * synth.FORMATS.index(k_fmt) + synth.FORMATS.index(v_fmt))
    g = case.to(DEV)
    for force in (1, 3):
        out, _ = run(g, plan_for(case, path=path, force_partitions=force))
        check_parity(case, out)
        assert np.all(out[5].cpu().numpy() == 0.0), "empty sequence must give a zero row"


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("L", [1, 15, 16, 17, 31, 32, 33, 64, 65, 200, 511, 1000])
@pytest.mark.parametrize("bs", [16, 32])
def test_block_boundaries(L, bs, path):
    case = _case([L, L + 1], block_size=bs, k_fmt="q4_0", v_fmt="q8_0", seed=L * 3 + bs)
    g = case.to(DEV)
    for force in (0, 1, 2):
        out, _ = run(g, plan_for(case, path=path, force_partitions=force))
        check_parity(case, out)


def test_gather_bit_exact_paged_and_contiguous():
    pa = pa_mod()
    for k_fmt, v_fmt in [("f16", "q4_0"), ("q8_0", "f16")]:
        case = _case([70, 33, 130], k_fmt=k_fmt, v_fmt=v_fmt, seed=5)
        g = case.to(DEV)
        plan = plan_for(case)
        for which, fmt, pool in ((0, k_fmt, case.k_pool), (1, v_fmt, case.v_pool)):
            rb = synth.row_bytes(fmt, case.D)
            flat = pool.reshape(-1, case.Hkv, rb)
            for b, L in enumerate(case.seq_lens):
                dst = torch.zeros((L, case.Hkv, rb), dtype=torch.uint8, device=DEV)
                pa.paged_kv_gather(plan, g.k_pool if which == 0 else g.v_pool, which, g.table, b, 0,
                                   L, dst)
                torch.cuda.synchronize()
                t = torch.arange(L)
                rows = case.table[b, t // case.block_size].long() * case.block_size + t % case.block_size
                assert torch.equal(dst.cpu(), flat[rows])
        # contiguous layout (null table)
        cc = synth.contiguous_copy(case)
        gc = cc.to(DEV)
        plan_c = plan_for(cc)
        rb = synth.row_bytes(k_fmt, case.D)
        for b, L in enumerate(case.seq_lens):
            dst = torch.zeros((L, case.Hkv, rb), dtype=torch.uint8, device=DEV)
            pa.paged_kv_gather(plan_c, gc.k_pool, 0, None, b, 0, L, dst)
            torch.cuda.synchronize()
            flat = cc.k_pool.reshape(-1, case.Hkv, rb)
            t = torch.arange(L)
            rows = (b * cc.max_blocks + t // case.block_size) * case.block_size + t % case.block_size
            assert torch.equal(dst.cpu(), flat[rows])


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pair", [("f16", "f16"), ("q4_0", "q4_0"), ("q8_0", "q4_0")])
def test_paged_equals_contiguous_bitwise_and_deterministic(pair, path):
    case = _case([700, 333, 1, 64], k_fmt=pair[0], v_fmt=pair[1], seed=11)
    cc = synth.contiguous_copy(case)
    g, gc = case.to(DEV), cc.to(DEV)
    for force in (0, 1, 3):
        plan = plan_for(case, path=path, force_partitions=force)
        out_p, _ = run(g, plan)
        out_p2, _ = run(g, plan)
        plan_c = plan_for(cc, path=path, force_partitions=force)
        assert plan_c.psize == plan.psize
        out_c, _ = run(gc, plan_c, table=None)
        assert torch.equal(out_p, out_p2), "repeated runs differ"
        assert torch.equal(out_p, out_c), "paged and contiguous runs differ"
        check_parity(case, out_p)


@pytest.mark.parametrize("pair", [("f16", "q4_0"), ("q4_0", "q8_0")])
def test_bad_block_id_sets_status_and_nans_only_that_sequence(pair):
    pa = pa_mod()
    case = _case([100, 64, 40], k_fmt=pair[0], v_fmt=pair[1], seed=13)
    g = case.to(DEV)
    for force in (1, 0, 3):
        plan = plan_for(case, force_partitions=force)
        for badid in (-1, case.nblocks, 2**31 - 1):
            tab = g.table.clone()
            tab[1, 2] = badid
            out, ws = run(g, plan, table=tab)
            assert pa.paged_attn_status(ws) & pa.PA_STATUS_BAD_BLOCK_ID
            o = out.cpu().numpy()
            assert np.isnan(o[1]).all(), "rows of the corrupt sequence must be NaN"
            ref = oracle.decode_case(case)
            for b in (0, 2):
                assert float(rel_err_rows(o[b], ref[b]).max()) <= tol_for(case)
            assert pa.paged_attn_status(ws) == 0, "status must clear after reading"


def test_seq_len_beyond_capacity_is_clamped_and_flagged():
    pa = pa_mod()
    case = _case([64, 40], k_fmt="q8_0", v_fmt="q8_0", seed=17, max_blocks=4)
    g = case.to(DEV)
    plan = plan_for(case, force_partitions=1)
    sl = g.seq_len.clone()
    sl[0] = 10_000          # beyond max_blocks*block_size = 64
    out, ws = pa_run_with_seq_len(g, plan, sl)
    assert pa.paged_attn_status(ws) & pa.PA_STATUS_BAD_SEQ_LEN
    check_parity(case, out)   # clamped to 64 = the case's own length


def pa_run_with_seq_len(g, plan, sl):
    pa = pa_mod()
    ws = pa.workspace(plan, DEV)
    out = torch.full((g.B, g.Hq, g.D), float("nan"), device=DEV)
    pa.paged_attn_step(plan, g.q, g.k_pool, g.v_pool, g.table, sl, ws, out)
    torch.cuda.synchronize()
    return out, ws


@pytest.mark.parametrize("pair", [("q4_0", "f16"), ("q8_0", "q4_0")])
@pytest.mark.parametrize("junk", ["nan", "big", "random"])
def test_junk_in_dead_slots_never_leaks(junk, pair):
    case = _case([33, 17, 1, 250], k_fmt=pair[0], v_fmt=pair[1], seed=19, junk=junk)
    g = case.to(DEV)
    for force in (0, 1, 2):
        out, _ = run(g, plan_for(case, force_partitions=force))
        check_parity(case, out)


def _oracle_partials(case, psize):
    kp, vp = case.k_pool.numpy().reshape(-1), case.v_pool.numpy().reshape(-1)
    return oracle.partials(case.q, kp, vp, case.table, case.seq_len, Hkv=case.Hkv, D=case.D,
                           block_size=case.block_size, k_fmt=case.k_fmt, v_fmt=case.v_fmt,
                           nblocks=case.nblocks, max_blocks=case.max_blocks, psize=psize,
                           scale=case.scale)


def _ws_partials(ws, plan, B, Hq, P, D):
    """(o [B,Hq,P,D] from binary16, ml [B,Hq,P,2] fp32) read from a workspace
    in the documented layout (partials from plan.part_offset)."""
    raw = ws.detach().cpu()
    n_o = B * Hq * P * D
    at = int(plan.part_offset)
    o = raw[at:at + 2 * n_o].view(torch.float16).reshape(B, Hq, P, D)
    ml = raw[at + 2 * n_o:at + 2 * n_o + 8 * B * Hq * P].view(torch.float32).reshape(B, Hq, P, 2)
    return o.double().numpy(), ml.double().numpy()


MERGE_CASES = {
    "p5": ([300, 0, 97, 31], 8, 2),
    "p10": ([600, 0, 97, 31], 8, 2),
    "p32": ([2000, 0, 97, 31], 8, 2),
    "p313": ([20000, 0, 97, 4100], 8, 2),       # the batched loads past the first 64
    # 44 sequences x 24 heads = 1056 rows of at most 5 partitions: the
    # row-per-thread merge layout
    "rows_p5": ([0, 1, 64, 65, 300, 17, 128, 129] * 5 + [0, 300, 33, 200], 24, 4),
    # ... and of at most 12 and 16 partitions (two lanes per row and 8 columns)
    "rows_p12": ([0, 1, 64, 65, 750, 17, 640, 129] * 5 + [0, 700, 33, 200], 24, 4),
    "rows_p16": ([0, 1, 64, 65, 1000, 17, 640, 129] * 5 + [0, 1000, 33, 200], 24, 4),
    # 27 x 24 = 648 rows of at most 24 and 32 partitions (four lanes; rows of
    # fewer partitions than lanes leave lanes with none)
    "rows_p24": ([0, 1, 64, 65, 1500, 17, 1280, 129] * 3 + [0, 1536, 33], 24, 4),
    "rows_p32": ([0, 1, 64, 65, 2000, 17, 1280, 129] * 3 + [0, 2048, 33], 24, 4),
}


@pytest.mark.parametrize("name", sorted(MERGE_CASES))
def test_merge_kernel_on_oracle_partials(name):
    """Write the oracle's own partials, o rounded to binary16, into the
    documented workspace layout and check the GPU merge against the oracle
    merge of the same values; and against the unrounded partials within what
    binary16 rounding of o can move the result (2^-11 of the largest |o_p|).
    Both merge layouts are covered: few rows (any partition count) and many
    rows of at most 6, 12, 16, 24 or 32 partitions (one, two or four lanes per
    row and 8 columns)."""
    pa = pa_mod()
    lens, Hq, Hkv = MERGE_CASES[name]
    case = _case(lens, k_fmt="f16", v_fmt="q8_0", seed=23, Hq=Hq, Hkv=Hkv)
    plan = plan_for(case, partition_tokens=64)
    plan.fused = 0                      # the separate merge kernel is what is tested here
    m, l, o, n = _oracle_partials(case, plan.psize)
    B, Hq, P, D = o.shape
    assert P == plan.p_max
    o16 = o.astype(np.float16)
    ml = np.stack([m, l], axis=-1).astype(np.float32)
    ws = pa.workspace(plan, "cpu")
    n_o = B * Hq * P * D
    at = int(plan.part_offset)
    ws[at:at + 2 * n_o] = torch.from_numpy(o16.reshape(-1)).view(torch.uint8)
    ws[at + 2 * n_o:at + 2 * n_o + 8 * B * Hq * P] = torch.from_numpy(ml.reshape(-1)).view(torch.uint8)
    wsd = ws.to(DEV)
    out = torch.full((B, Hq, D), float("nan"), device=DEV)
    pa.paged_attn_merge(plan, wsd, case.seq_len.to(DEV), out)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    ref16 = oracle.merge(m, l, o16.astype(np.float64), n)
    assert float(rel_err_rows(got, ref16).max()) <= 1e-5
    ref = oracle.merge(m, l, o, n)
    bound = 2.0 ** -11 * np.abs(o).max(axis=(2, 3)) + 1e-6 * np.abs(ref).max(axis=-1) + 1e-7
    assert np.all(np.abs(got - ref).max(axis=-1) <= bound)
    for b, L in enumerate(lens):
        if L == 0:
            assert np.all(got[b] == 0.0)


@pytest.mark.parametrize("name", ["p32", "rows_p5", "rows_p16", "rows_p32"])
def test_merge_nan_m_poisons_only_its_row(name):
    """A NaN m (what a partition that met a bad block id leaves) makes its
    whole row NaN on both merge layouts, whichever lane of a row's group
    holds that partition, and leaves every other row as it was."""
    pa = pa_mod()
    lens, Hq, Hkv = MERGE_CASES[name]
    case = _case(lens, k_fmt="f16", v_fmt="q8_0", seed=29, Hq=Hq, Hkv=Hkv)
    plan = plan_for(case, partition_tokens=64)
    plan.fused = 0
    m, l, o, n = _oracle_partials(case, plan.psize)
    B, Hq, P, D = o.shape
    b_long = int(np.argmax(n))
    bad = [(b_long, 1, int(n[b_long]) - 1), (b_long, Hq - 1, 1 % int(n[b_long]))]
    for b, h, p in bad:
        m[b, h, p] = np.nan
    ml = np.stack([m, l], axis=-1).astype(np.float32)
    ws = pa.workspace(plan, "cpu")
    n_o = B * Hq * P * D
    at = int(plan.part_offset)
    ws[at:at + 2 * n_o] = torch.from_numpy(o.astype(np.float16).reshape(-1)).view(torch.uint8)
    ws[at + 2 * n_o:at + 2 * n_o + 8 * B * Hq * P] = torch.from_numpy(ml.reshape(-1)).view(torch.uint8)
    out = torch.zeros((B, Hq, D), device=DEV)
    pa.paged_attn_merge(plan, ws.to(DEV), case.seq_len.to(DEV), out)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    poisoned = np.zeros((B, Hq), dtype=bool)
    for b, h, _ in bad:
        poisoned[b, h] = True
    assert np.all(np.isnan(got[poisoned]))
    assert np.all(np.isfinite(got[~poisoned]))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pair", [("q4_0", "q8_0"), ("f16", "q4_0")])
def test_decode_partials_match_the_oracle_split_form(pair, path):
    """The partials a decode kernel leaves in the workspace (binary16 o, fp32
    m and l, documented layout) against the oracle's split form with the same
    partition size: o to the format tolerance, m a reference value within 8
    (log2 units) below the partition's largest logit, and l * 2^m equal to the
    oracle's sum to the tolerance."""
    case = _case([300, 0, 97, 130], k_fmt=pair[0], v_fmt=pair[1], seed=31)
    plan = plan_for(case, path=path, partition_tokens=64)
    out, ws = run(case.to(DEV), plan)
    m_r, l_r, o_r, n = _oracle_partials(case, plan.psize)
    B, Hq, P, D = o_r.shape
    assert P == plan.p_max
    o, ml = _ws_partials(ws, plan, B, Hq, P, D)
    tol = tol_for(case)
    for b in range(B):
        for p in range(int(n[b])):
            assert float(rel_err_rows(o[b, :, p], o_r[b, :, p]).max()) <= tol
            m_g, l_g = ml[b, :, p, 0], ml[b, :, p, 1]
            assert np.all(m_g <= m_r[b, :, p] + 1e-2) and np.all(m_r[b, :, p] <= m_g + 8 + 1e-2)
            rel = np.abs(l_g * np.exp2(m_g - m_r[b, :, p]) / l_r[b, :, p] - 1.0)
            assert float(rel.max()) <= tol
    check_parity(case, out)


@pytest.mark.parametrize("path", PATHS)
def test_workspace_canary_untouched(path):
    case = _case([1000, 517, 3], k_fmt="q4_0", v_fmt="q4_0", seed=29)
    g = case.to(DEV)
    for force in (0, 1, 5):
        plan = plan_for(case, path=path, force_partitions=force)
        out, ws = run(g, plan, canary=4096)
        tail = ws[int(plan.ws_bytes):].cpu()
        assert torch.all(tail == 0xA5), "decode or merge wrote past plan.ws_bytes"
        check_parity(case, out)


def test_red_control_wrong_table_fails_parity():
    """A table whose first entry names a later block of the sequence must make
    the GPU result disagree with the oracle on the true table (TensorFold PR
    #1418, Kernel contract: the red control)."""
    case = _case([128], k_fmt="f16", v_fmt="f16", seed=31)
    g = case.to(DEV)
    tab = g.table.clone()
    tab[0, 0] = tab[0, 3]
    out, _ = run(g, plan_for(case, force_partitions=1), table=tab)
    ref = oracle.decode_case(case)
    assert float(rel_err_rows(out.cpu().double().numpy(), ref).max()) > 1e-2


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pair,std", [(("q4_0", "q4_0"), 400.0), (("q4_0", "f16"), 400.0),
                                      (("f16", "q4_0"), 400.0), (("q8_0", "q8_0"), 5000.0),
                                      (("q8_0", "q4_0"), 5000.0)])
def test_large_block_scales(pair, std, path):
    """Block scales far from O(1) (|d| in the hundreds to thousands, values up
    to ~1e4): the dequantisation must stay exact up to its one f16 rounding.
    q shrinks as K grows so the logits stay O(1), as in real attention (with
    f16 operands, logit error grows with |q|*|k|)."""
    case = _case([300, 77, 1000], k_fmt=pair[0], v_fmt=pair[1], seed=41, value_std=std,
                 q_std=min(1.0, 4.0 / std))
    g = case.to(DEV)
    for force in (0, 1, 3):
        out, _ = run(g, plan_for(case, path=path, force_partitions=force))
        check_parity(case, out)


def test_mixed_scales_within_one_sequence():
    """Large-scale rows only in part of the context, next to O(1) rows."""
    case = _case([2000, 500], k_fmt="q4_0", v_fmt="q4_0", seed=43)
    big = synth.make_case([2000, 500], k_fmt="q4_0", v_fmt="q4_0", seed=43, value_std=500.0,
                          nblocks=case.nblocks)
    case.q *= 0.002   # logits stay O(1) on the large rows (f16 operands: logit error ~ |q||k|)
    # splice the large-scale rows of blocks 10..20 of sequence 0 into the pool
    ids = case.table[0, 10:20].long()
    case.k_pool[ids] = big.k_pool[big.table[0, 10:20].long()]
    case.v_pool[ids] = big.v_pool[big.table[0, 10:20].long()]
    g = case.to(DEV)
    for force in (0, 1, 4):
        out, _ = run(g, plan_for(case, force_partitions=force))
        check_parity(case, out)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pair", [("q4_0", "q4_0"), ("q8_0", "f16")])
def test_more_units_than_workgroups(pair, path):
    """A plan for a 2-CU device: a handful of workgroups each take many
    (sequence, partition) units in turn, across sequences of different
    lengths (one empty), so every unit start after the first (block ids,
    q values, ring reuse) runs."""
    case = _case([3000, 77, 1000, 0, 513], k_fmt=pair[0], v_fmt=pair[1], seed=61)
    g = case.to(DEV)
    plan = plan_for(case, path=path, num_cus=2, partition_tokens=256)
    units = sum(-(-L // 256) for L in case.seq_lens) * (case.Hkv // 4 if plan.path == 2 else 1)
    assert plan.grid < units
    out, ws = run(g, plan)
    assert pa_mod().paged_attn_status(ws) == 0
    check_parity(case, out)


def test_register_kernel_sixteen_heads_per_group_f16_d256():
    """F16 K and V at D=256 with r = 16 (Hq = 64, Hkv = 4): a shape the LDS
    ring does not take, so the register kernel runs it, with more than the
    default 64 KiB of dynamic LDS for its cross-wave combine."""
    case = _case([300, 45, 0], Hq=64, Hkv=4, D=256, k_fmt="f16", v_fmt="f16", seed=331)
    g = case.to(DEV)
    for force in (0, 1, 3):
        plan = plan_for(case, path=1, force_partitions=force)
        out, ws = run(g, plan)
        check_parity(case, out)
        assert pa_mod().paged_attn_status(ws) == 0


def test_largest_batch_on_the_register_kernel():
    """B = 1024 short sequences (above the LDS kernel's 256): the batch prefix
    of live partitions alone is 8 KB of LDS."""
    rng = np.random.default_rng(337)
    lens = [int(x) for x in rng.integers(0, 40, size=1024)]
    case = _case(lens, k_fmt="q4_0", v_fmt="q8_0", seed=337)
    g = case.to(DEV)
    for force in (0, 2):
        plan = plan_for(case, force_partitions=force)
        assert plan.path == 1
        out, ws = run(g, plan)
        check_parity(case, out)
        assert pa_mod().paged_attn_status(ws) == 0
