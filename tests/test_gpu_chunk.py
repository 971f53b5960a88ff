"""GPU parity of the chunk path (multi-token queries with causal masking in
the chunk: lucebox PR #555, Roadmap item 3; TensorFold PR #1418, What:
paged equals contiguous bit for bit) against oracle.chunk, through the C ABI.

Tolerance as for decode (per-row max-abs error relative to the row's
max-abs output): 2e-3 when K and V are F16, 5e-3 when either is quantised.
Three kernels compute a chunk (plan path 1: tile conversion for any Tq;
path 2: the window kernel for few query rows per kv head; path 3: the
wide-tile kernel for many); the tests marked with a `path` parameter run
each on the same inputs."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_util import pa_mod, rel_err_rows, tol_for

pytestmark = pytest.mark.gpu

DEV = "cuda"
PAIRS = [(k, v) for k in synth.FORMATS for v in synth.FORMATS]


def _case(lens, Tq, seed, **kw):
    kw.setdefault("junk", "nan")
    c = synth.make_case(lens, seed=seed, **kw)
    g = torch.Generator().manual_seed(seed + 555)
    qc = torch.randn((c.B, Tq, c.Hq, c.D), generator=g)
    return c, qc


def window_ok(c, Tq):
    """Whether the window kernel (plan path 2) takes the chunk: quads of kv
    heads, one 16-slot group of K and V of four heads in a 36 KB ring slot
    (no F16 side at D=256), and at most 48 query rows (Tq*r) per kv head
    (three column groups of 16, over half of the head dimension per wave at
    D=256, where 33..48 rows take it for Q4_0 K and V only)."""
    rb = {"f16": 2 * c.D, "q8_0": 34 * c.D // 32, "q4_0": 18 * c.D // 32}
    per_group = sum(-(-16 * 4 * rb[f] // 1024) for f in (c.k_fmt, c.v_fmt)) * 1024
    rows = Tq * (c.Hq // c.Hkv)
    q4 = c.k_fmt == "q4_0" and c.v_fmt == "q4_0"
    return (c.Hkv % 4 == 0 and per_group <= 36864
            and (rows <= 32 or (rows <= 48 and (c.D == 128 or q4))))


def wide_paths(c, Tq):
    """The kernels the plan may pick besides the window kernel: the wide-tile
    kernel (plan path 3) takes more than 64 query rows per kv head, always in
    its paired form (every type pair at D=128; at D=256 all but F16 K and V
    together and F16 with Q8_0), in its four-wave form only if its units fill
    half the compute units, which the test does not mirror; the tile kernel
    (path 1) the rest."""
    rows = Tq * (c.Hq // c.Hkv)
    if rows <= 64:
        return {1}
    four_wave = c.D == 256 and ((c.k_fmt == "f16" and c.v_fmt != "q4_0") or
                                (c.v_fmt == "f16" and c.k_fmt != "q4_0"))
    return {1, 3} if four_wave else {3}


def _plan(c, Tq, path=None, **kw):
    """paged_attn_chunk_plan for the case; path=1/2/3 forces the kernel (a
    chunk the window kernel does not take is skipped for path 2; the tile and
    wide-tile kernels take any)."""
    pa = pa_mod()
    shape = pa.shape_of(c.B, c.Hq, c.Hkv, c.D, c.block_size, c.nblocks, c.max_blocks, c.k_fmt,
                        c.v_fmt)
    plan = pa.paged_attn_chunk_plan(shape, Tq, max(c.seq_lens), total_tokens=sum(c.seq_lens),
                                    scale=c.scale, **kw)
    assert plan.path in ({2} if window_ok(c, Tq) else wide_paths(c, Tq))
    if path is not None:
        if path == 2 and not window_ok(c, Tq):
            pytest.skip("the window kernel does not take this chunk")
        plan.path = path
    return plan


PATHS = [1, 2, 3]


def _run(c, qc, plan, table="case"):
    pa = pa_mod()
    g = c.to(DEV)
    ws = pa.workspace(plan, DEV)
    out = torch.full(tuple(qc.shape), float("nan"), dtype=torch.float32, device=DEV)
    tab = g.table if table == "case" else table
    pa.paged_attn_chunk(plan, qc.to(DEV), g.k_pool, g.v_pool, tab, g.seq_len, ws, out)
    torch.cuda.synchronize()
    return out, ws


def _ref(c, qc):
    kp, vp = c.k_pool.numpy().reshape(-1), c.v_pool.numpy().reshape(-1)
    return oracle.chunk(qc, kp, vp, c.table, c.seq_len, Hkv=c.Hkv, D=c.D, block_size=c.block_size,
                        k_fmt=c.k_fmt, v_fmt=c.v_fmt, nblocks=c.nblocks, max_blocks=c.max_blocks,
                        scale=c.scale)


def _check(c, qc, out):
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all(), "non-finite output"
    err = rel_err_rows(got, _ref(c, qc))
    worst = float(err.max())
    assert worst <= tol_for(c), f"max row error {worst:.3e}"
    return worst


@pytest.mark.parametrize("D", [256, 128])
@pytest.mark.parametrize("pair", PAIRS, ids=[f"{k}-{v}" for k, v in PAIRS])
def test_nine_type_pairs(pair, D):
    seed = 3 * synth.FORMATS.index(pair[0]) + synth.FORMATS.index(pair[1]) + D
    c, qc = _case([300, 77, 16], 9, seed=seed, k_fmt=pair[0], v_fmt=pair[1], D=D)
    for kw in ({}, {"force_partitions": 1}, {"partition_tokens": 64}):
        out, ws = _run(c, qc, _plan(c, 9, **kw))
        _check(c, qc, out)
        assert pa_mod().paged_attn_status(ws) == 0


@pytest.mark.parametrize("D", [256, 128])
@pytest.mark.parametrize("pair", PAIRS, ids=[f"{k}-{v}" for k, v in PAIRS])
def test_nine_type_pairs_wide(pair, D):
    """A 24-token chunk (144 query rows per kv head: a full and a partial
    128-row block) on the wide-tile kernel, with one and several
    partitions."""
    seed = 3 * synth.FORMATS.index(pair[0]) + synth.FORMATS.index(pair[1]) + D + 301
    c, qc = _case([300, 77, 40], 24, seed=seed, k_fmt=pair[0], v_fmt=pair[1], D=D)
    for kw in ({}, {"force_partitions": 1}, {"partition_tokens": 64}):
        plan = _plan(c, 24, path=3, **kw)
        out, ws = _run(c, qc, plan)
        _check(c, qc, out)
        assert pa_mod().paged_attn_status(ws) == 0


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("D", [256, 128])
@pytest.mark.parametrize("pair", PAIRS, ids=[f"{k}-{v}" for k, v in PAIRS])
def test_nine_type_pairs_short_window(pair, D, path):
    """A 5-token window (30 query rows per kv head) on both kernels."""
    seed = 3 * synth.FORMATS.index(pair[0]) + synth.FORMATS.index(pair[1]) + D + 77
    c, qc = _case([300, 77, 16], 5, seed=seed, k_fmt=pair[0], v_fmt=pair[1], D=D)
    for kw in ({}, {"force_partitions": 1}, {"partition_tokens": 64}):
        out, ws = _run(c, qc, _plan(c, 5, path=path, **kw))
        _check(c, qc, out)
        assert pa_mod().paged_attn_status(ws) == 0


@pytest.mark.parametrize("D", [256, 128])
@pytest.mark.parametrize("pair", PAIRS, ids=[f"{k}-{v}" for k, v in PAIRS])
def test_nine_type_pairs_two_token_window(pair, D):
    """A 2-token window (12 query rows per kv head): the window kernel at two
    workgroups per CU with the decode kernel's ring, for every type pair."""
    seed = 3 * synth.FORMATS.index(pair[0]) + synth.FORMATS.index(pair[1]) + D + 131
    c, qc = _case([300, 77, 16], 2, seed=seed, k_fmt=pair[0], v_fmt=pair[1], D=D)
    for kw in ({}, {"force_partitions": 1}, {"partition_tokens": 64}):
        out, ws = _run(c, qc, _plan(c, 2, path=2, **kw))
        _check(c, qc, out)
        assert pa_mod().paged_attn_status(ws) == 0


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("Tq", [1, 2, 16, 33, 130])
def test_chunk_lengths_and_partitions(Tq, path):
    """Query tiles from one to many, partitions that start past some rows'
    positions (those rows get empty partials), and a chunk as long as the
    sequence (its first token sees key 0 only)."""
    c, qc = _case([400, Tq, 1000], Tq, seed=Tq, k_fmt="q4_0", v_fmt="q8_0")
    for kw in ({}, {"force_partitions": 1}, {"partition_tokens": 96}, {"force_partitions": 5}):
        out, _ = _run(c, qc, _plan(c, Tq, path=path, **kw))
        _check(c, qc, out)


@pytest.mark.parametrize("path", PATHS)
def test_tq_one_is_a_decode_step(path):
    """A one-token chunk is a decode step: the same oracle, within tolerance of
    the decode kernels' output."""
    pa = pa_mod()
    c, qc = _case([700, 5, 129], 1, seed=41, k_fmt="q8_0", v_fmt="q4_0")
    out, _ = _run(c, qc, _plan(c, 1, path=path, partition_tokens=128))
    dc = dataclasses.replace(c, q=qc[:, 0].contiguous())
    ref = oracle.decode_case(dc)
    assert float(rel_err_rows(out[:, 0].cpu().double().numpy(), ref).max()) <= tol_for(c)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("pair", [("f16", "f16"), ("q4_0", "q4_0"), ("q8_0", "f16")])
def test_paged_equals_contiguous_bitwise_and_deterministic(pair, path):
    """TensorFold PR #1418, What: the paged chunk equals the contiguous one bit
    for bit (same tiles in the same order); repeated runs agree bit for bit."""
    Tq = {1: 12, 2: 4, 3: 24}[path]
    c, qc = _case([333, 64, 190], Tq, seed=7, k_fmt=pair[0], v_fmt=pair[1])
    cc = synth.contiguous_copy(c)
    for kw in ({}, {"partition_tokens": 64}):
        plan = _plan(c, Tq, path=path, **kw)
        plan_c = _plan(cc, Tq, path=path, **kw)  # the contiguous pool has its own nblocks
        assert (plan_c.psize, plan_c.grid) == (plan.psize, plan.grid)
        o1, _ = _run(c, qc, plan)
        o2, _ = _run(cc, qc, plan_c, table=None)
        o3, _ = _run(c, qc, plan)
        assert torch.equal(o1, o2) and torch.equal(o1, o3)
        _check(c, qc, o1)


@pytest.mark.parametrize("path", PATHS)
def test_empty_and_too_short_sequences(path):
    """L = 0 gives zero rows; 0 < L < Tq gives zero rows and the seq_len
    status bit; the other sequences are untouched."""
    pa = pa_mod()
    Tq = 6 if path == 1 else 5
    c, qc = _case([0, 3, 50], Tq, seed=13, k_fmt="q4_0", v_fmt="q8_0")
    for kw in ({}, {"force_partitions": 1}, {"partition_tokens": 32}):
        plan = _plan(c, Tq, path=path, **kw)
        g = c.to(DEV)
        ws = pa.workspace(plan, DEV)
        out = torch.full(tuple(qc.shape), float("nan"), device=DEV)
        pa.paged_attn_chunk(plan, qc.to(DEV), g.k_pool, g.v_pool, g.table, g.seq_len, ws, out)
        assert pa.paged_attn_status(ws) == pa.PA_STATUS_BAD_SEQ_LEN
        o = out.cpu()
        assert torch.all(o[0] == 0) and torch.all(o[1] == 0)
        ok = dataclasses.replace(c, B=1, seq_lens=[50], seq_len=c.seq_len[2:], q=c.q[2:],
                                 table=c.table[2:])
        err = rel_err_rows(o[2:].double().numpy(), _ref(ok, qc[2:]))
        assert float(err.max()) <= tol_for(c)


@pytest.mark.parametrize("path", PATHS)
def test_bad_block_id_sets_status_and_nans_only_that_sequence(path):
    pa = pa_mod()
    c, qc = _case([200, 150], 4, seed=17, k_fmt="q4_0", v_fmt="q4_0", junk="zero")
    bad_table = c.table.clone()
    bad_table[1, 3] = c.nblocks + 5
    plan = _plan(c, 4, path=path, partition_tokens=64)
    out, ws = _run(c, qc, plan, table=bad_table.to(DEV))
    assert pa.paged_attn_status(ws) & pa.PA_STATUS_BAD_BLOCK_ID
    o = out.cpu()
    assert torch.isnan(o[1]).all()
    good = dataclasses.replace(c, B=1, seq_lens=[200], seq_len=c.seq_len[:1], q=c.q[:1],
                               table=c.table[:1])
    assert float(rel_err_rows(o[:1].double().numpy(), _ref(good, qc[:1])).max()) <= tol_for(c)


@pytest.mark.parametrize("rows", [32, 48])
@pytest.mark.parametrize("heads", [(24, 4), (32, 8)], ids=["r6", "r4-two-quads"])
@pytest.mark.parametrize("pair", [("q4_0", "q4_0"), ("q8_0", "q4_0"), ("f16", "q8_0")])
@pytest.mark.parametrize("D", [256, 128])
def test_both_kernels_agree(pair, D, heads, rows):
    """The same chunk on both kernels with the same partitioning, to the
    format tolerance: besides the order of fp32 accumulation they round the
    quantised values differently (the window kernel folds the Q4_0 offset
    into correction MFMAs as the decode kernel does; the tile kernel converts
    (n - 8) * d directly). Hkv = 8 gives two kv-head quads per sequence."""
    Hq, Hkv = heads
    Tq = rows // (Hq // Hkv)
    c, qc = _case([2000, 700, 33], Tq, seed=101 + D + Hkv, k_fmt=pair[0], v_fmt=pair[1], D=D,
                  Hq=Hq, Hkv=Hkv)
    if not window_ok(c, Tq):
        pytest.skip("the window kernel does not take this chunk")
    for kw in ({}, {"partition_tokens": 256}):
        o1, _ = _run(c, qc, _plan(c, Tq, path=1, **kw))
        o2, _ = _run(c, qc, _plan(c, Tq, path=2, **kw))
        g1, g2 = o1.cpu().double().numpy(), o2.cpu().double().numpy()
        assert np.isfinite(g2).all()
        assert float(rel_err_rows(g2, g1).max()) <= tol_for(c)
        _check(c, qc, o2)


@pytest.mark.parametrize("rows", [72, 144, 384])
@pytest.mark.parametrize("pair", [("q4_0", "q4_0"), ("q8_0", "q4_0"), ("f16", "q8_0")])
@pytest.mark.parametrize("D", [256, 128])
def test_wide_and_tile_kernels_agree(pair, D, rows):
    """The same chunk on the tile and wide-tile kernels with the same
    partitioning, to the format tolerance (they convert the quantised values
    alike but accumulate in a different order)."""
    Tq = rows // 6
    c, qc = _case([2000, 700, 90], Tq, seed=131 + D + rows, k_fmt=pair[0], v_fmt=pair[1], D=D)
    for kw in ({}, {"partition_tokens": 256}):
        o1, _ = _run(c, qc, _plan(c, Tq, path=1, **kw))
        o3, _ = _run(c, qc, _plan(c, Tq, path=3, **kw))
        g1, g3 = o1.cpu().double().numpy(), o3.cpu().double().numpy()
        assert np.isfinite(g3).all()
        assert float(rel_err_rows(g3, g1).max()) <= tol_for(c)
        _check(c, qc, o3)


@pytest.mark.parametrize("bs", [32, 64])
@pytest.mark.parametrize("path,Tq,D,pair", [(1, 9, 256, ("q4_0", "q8_0")), (2, 4, 256, ("q4_0", "q4_0")),
                                            (3, 16, 256, ("q4_0", "q4_0")), (3, 16, 256, ("f16", "f16")),
                                            (3, 24, 128, ("q8_0", "q4_0"))])
def test_block_sizes_on_every_kernel(path, Tq, D, pair, bs):
    """Blocks of 32 and 64 tokens on each chunk kernel (the wide-tile kernel in
    both its forms), with sequence ends inside a block and inside a 16-key
    group: every kernel takes its 16-row groups from inside one block."""
    Hq, Hkv = (24, 4) if D == 256 else (32, 8)
    c, qc = _case([bs * 3 + 17, bs - 1 + Tq, 2 * bs + 5], Tq, seed=bs + 7 * path + D, k_fmt=pair[0],
                  v_fmt=pair[1], D=D, Hq=Hq, Hkv=Hkv, block_size=bs)
    o, _ = _run(c, qc, _plan(c, Tq, path=path, partition_tokens=64))
    _check(c, qc, o)


@pytest.mark.parametrize("path", [2, 3])
def test_unaligned_pools_run_the_tile_kernel(path):
    """Pools that are not 16-byte aligned run the tile-conversion kernel even
    under a window or wide-tile plan: the result equals a path-1 run bit for
    bit."""
    c, qc = _case([500, 77], 4, seed=231, k_fmt="q4_0", v_fmt="q8_0")
    g = c.to(DEV)

    def shifted(pool):
        raw = torch.empty(pool.numel() + 4, dtype=torch.uint8, device=DEV)
        view = raw[4:].view(pool.shape)
        view.copy_(pool)
        assert view.data_ptr() % 16 == 4
        return view

    plan2 = _plan(c, 4, path=path, partition_tokens=128)
    plan1 = _plan(c, 4, path=1, partition_tokens=128)
    pa = pa_mod()
    outs = []
    for plan, kp, vp in ((plan2, shifted(g.k_pool), shifted(g.v_pool)), (plan1, g.k_pool, g.v_pool)):
        ws = pa.workspace(plan, DEV)
        out = torch.full(tuple(qc.shape), float("nan"), dtype=torch.float32, device=DEV)
        pa.paged_attn_chunk(plan, qc.to(DEV), kp, vp, g.table, g.seq_len, ws, out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    _check(c, qc, outs[0])


@pytest.mark.parametrize("path", [2, 3])
def test_unaligned_q_runs_the_tile_kernel(path):
    """A q that is not 16-byte aligned runs the tile-conversion kernel even
    under a window or wide-tile plan (whose kernels read q with 16-byte
    loads): the result equals a path-1 run bit for bit."""
    c, qc = _case([500, 77], 4, seed=237, k_fmt="q4_0", v_fmt="q4_0")
    g = c.to(DEV)
    raw = torch.empty(qc.numel() + 1, dtype=torch.float32, device=DEV)
    qu = raw[1:].view(qc.shape)
    qu.copy_(qc.to(DEV))
    assert qu.data_ptr() % 16 == 4
    plan2 = _plan(c, 4, path=path, partition_tokens=128)
    plan1 = _plan(c, 4, path=1, partition_tokens=128)
    pa = pa_mod()
    outs = []
    for plan, q in ((plan2, qu), (plan1, qc.to(DEV))):
        ws = pa.workspace(plan, DEV)
        out = torch.full(tuple(qc.shape), float("nan"), dtype=torch.float32, device=DEV)
        pa.paged_attn_chunk(plan, q, g.k_pool, g.v_pool, g.table, g.seq_len, ws, out)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.equal(outs[0], outs[1])
    _check(c, qc, outs[0])


@pytest.mark.parametrize("Tq", [2, 4, 8])
def test_verify_windows_at_full_size(Tq):
    """Verify windows of 2, 4 and 8 tokens over Q4_0 K/V, B=8 x 32768 tokens
    (the chunk benchmark's workloads), on the automatic plan: the window
    kernel, a kv-head quad per workgroup for 12 query rows per kv head, a
    kv-head pair with the head dimension split over two waves for 24 and 48.
    Every output row (all sequences, tokens and query heads) is checked
    against the oracle."""
    pa = pa_mod()
    case = synth.workload("uniform_q4_0", B=8, L=32768, seed=1500 + Tq, device=DEV)
    qc = torch.randn((case.B, Tq, case.Hq, case.D), generator=torch.Generator().manual_seed(1600 + Tq))
    shape = pa.shape_of(case.B, case.Hq, case.Hkv, case.D, case.block_size, case.nblocks,
                        case.max_blocks, case.k_fmt, case.v_fmt)
    plan = pa.paged_attn_chunk_plan(shape, Tq, max(case.seq_lens), total_tokens=sum(case.seq_lens),
                                    scale=case.scale)
    assert plan.path == 2
    ws = pa.workspace(plan, DEV)
    out = torch.full(tuple(qc.shape), float("nan"), dtype=torch.float32, device=DEV)
    pa.paged_attn_chunk(plan, qc.to(DEV), case.k_pool, case.v_pool, case.table, case.seq_len, ws, out)
    torch.cuda.synchronize()
    assert pa.paged_attn_status(ws) == 0
    got = out.cpu().double().numpy()
    assert np.isfinite(got).all(), "non-finite output"
    kp, vp = case.k_pool.cpu().numpy().reshape(-1), case.v_pool.cpu().numpy().reshape(-1)
    ref = oracle.chunk(qc, kp, vp, case.table.cpu(), case.seq_len.cpu(), Hkv=case.Hkv, D=case.D,
                       block_size=case.block_size, k_fmt=case.k_fmt, v_fmt=case.v_fmt,
                       nblocks=case.nblocks, max_blocks=case.max_blocks, scale=case.scale)
    err = rel_err_rows(got, ref)                  # [B, Tq, Hq]
    worst = float(err.max())
    b, t, h = np.unravel_index(int(err.argmax()), err.shape)
    assert worst <= tol_for(case), f"max row error {worst:.3e} at sequence {b}, token {t}, head {h}"
    del case, ws, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pair", [("q4_0", "q4_0"), ("q8_0", "f16")])
def test_wide_partition_longer_than_a_segment(pair):
    """One partition of 9000 keys: the wide-tile kernel stages 512 block ids
    (8192 tokens at 16 per block) at a time and restarts its tile pipeline
    for the second segment."""
    c, qc = _case([9000, 300], 16, seed=88, k_fmt=pair[0], v_fmt=pair[1])
    plan = _plan(c, 16, path=3, force_partitions=1)
    assert plan.direct
    out, ws = _run(c, qc, plan)
    _check(c, qc, out)
    assert pa_mod().paged_attn_status(ws) == 0


def test_prefill_chunk_at_full_size():
    """The chunk benchmark's prefill chunk: 512 tokens over a Q4_0 sequence
    of 8192 (3072 query rows per kv head) on the plan's wide-tile kernel.
    Every output row is checked against the oracle; so are its first 6
    tokens once more as a 6-token chunk of the sequence cut after them (the
    keys each token sees are the same)."""
    pa = pa_mod()
    Tq, L = 512, 8192
    case = synth.workload("uniform_q4_0", B=1, L=L, seed=1700, device=DEV)
    qc = torch.randn((1, Tq, case.Hq, case.D), generator=torch.Generator().manual_seed(1701))
    shape = pa.shape_of(case.B, case.Hq, case.Hkv, case.D, case.block_size, case.nblocks,
                        case.max_blocks, case.k_fmt, case.v_fmt)
    plan = pa.paged_attn_chunk_plan(shape, Tq, L, total_tokens=L, scale=case.scale)
    assert plan.path == 3
    ws = pa.workspace(plan, DEV)
    out = torch.full(tuple(qc.shape), float("nan"), dtype=torch.float32, device=DEV)
    pa.paged_attn_chunk(plan, qc.to(DEV), case.k_pool, case.v_pool, case.table, case.seq_len, ws, out)
    torch.cuda.synchronize()
    assert pa.paged_attn_status(ws) == 0
    got = out.cpu()
    assert torch.isfinite(got).all()
    kp, vp = case.k_pool.cpu().numpy().reshape(-1), case.v_pool.cpu().numpy().reshape(-1)
    tab = case.table.cpu()
    for toks, n in ((slice(0, Tq), L), (slice(0, 6), L - Tq + 6)):
        ref = oracle.chunk(qc[:, toks], kp, vp, tab, torch.tensor([n], dtype=torch.int32), Hkv=case.Hkv,
                           D=case.D, block_size=case.block_size, k_fmt=case.k_fmt, v_fmt=case.v_fmt,
                           nblocks=case.nblocks, max_blocks=case.max_blocks, scale=case.scale)
        err = rel_err_rows(got[:, toks].double().numpy(), ref)
        worst = float(err.max())
        _, t, h = np.unravel_index(int(err.argmax()), err.shape)
        assert worst <= tol_for(case), f"tokens {toks}: max row error {worst:.3e} at token {t}, head {h}"
    del case, ws, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("Tq", [2, 5])
def test_more_units_than_workgroups(Tq, path):
    """A chunk plan for a 2-CU device: each workgroup takes many units in
    turn, across sequences of different lengths (one empty)."""
    c, qc = _case([3000, 77, 1000, 0, 513], Tq, seed=71 + Tq, k_fmt="q4_0", v_fmt="q4_0")
    plan = _plan(c, Tq, path=path, num_cus=2, partition_tokens=256)
    assert plan.grid < sum(-(-L // 256) for L in c.seq_lens)
    out, ws = _run(c, qc, plan)
    _check(c, qc, out)
    assert pa_mod().paged_attn_status(ws) == 0
