"""GPU checks of the paging-metadata entry points against oracle/metadata.py
(bit for bit), and an end-to-end decode over a shared prefix with
copy-on-write (lucebox PR #555, Summary: resident paging metadata updated
per fresh block; Roadmap item 6: prefix blocks shared under reference counts
and copied on write)."""
import numpy as np
import pytest
import torch

import oracle
import synth
from oracle.metadata import copy_blocks, table_update
from gpu_util import check_parity, pa_mod

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.mark.parametrize("n", [1, 37, 700])
def test_table_update_matches_the_oracle(n):
    """Random distinct (b, slot, value) entries, more than one launch's worth
    for n = 700; every other entry stays as it was."""
    pa = pa_mod()
    rng = np.random.default_rng(n)
    B, MB = 9, 300
    table = rng.integers(0, 5000, size=(B, MB), dtype=np.int32)
    seq = rng.integers(0, 4800, size=B, dtype=np.int32)
    keys = rng.choice(B * (MB + 1), size=n, replace=False)
    upd = [(int(k // (MB + 1)), int(k % (MB + 1)) - 1, int(rng.integers(-3, 1 << 20))) for k in keys]
    t_ref, s_ref = table_update(table, seq, upd)
    t_dev = torch.from_numpy(table).to(DEV)
    s_dev = torch.from_numpy(seq).to(DEV)
    pa.paged_table_update(t_dev, s_dev, upd)
    torch.cuda.synchronize()
    assert np.array_equal(t_dev.cpu().numpy(), t_ref)
    assert np.array_equal(s_dev.cpu().numpy(), s_ref)


@pytest.mark.parametrize("shape,npairs", [((200, 16, 4, 144), 100), ((9, 256, 8, 512), 3),
                                          ((40, 32, 2, 136), 17)])
def test_copy_blocks_matches_the_oracle(shape, npairs):
    """Whole-block copies (Q4_0 D=256 blocks; 1 MB F16 blocks; Q8_0 D=128
    blocks), more than one launch's worth of pairs for 100."""
    pa = pa_mod()
    rng = np.random.default_rng(npairs)
    pool = rng.integers(0, 256, size=shape, dtype=np.uint8)
    ids = rng.permutation(shape[0])
    src, dst = ids[:npairs].tolist(), ids[npairs:2 * npairs].tolist()
    ref = copy_blocks(pool, src, dst)
    dev = torch.from_numpy(pool).to(DEV)
    pa.paged_kv_copy_blocks(dev, src, dst)
    torch.cuda.synchronize()
    assert np.array_equal(dev.cpu().numpy(), ref)


@pytest.mark.parametrize("k_fmt,v_fmt", [("q4_0", "q4_0"), ("f16", "q8_0")])
def test_shared_prefix_with_copy_on_write_end_to_end(k_fmt, v_fmt):
    """Sequence A (87 tokens) is forked into B, which shares A's six blocks,
    including the partly filled sixth; B makes that block private (device
    copy) before appending tokens 87..126, then A appends tokens 87..100 in
    place. The device table and seq_len are only updated entry by entry. Both
    decodes match the oracle on the final pool, and B's first 87 rows are A's
    rows byte for byte."""
    pa = pa_mod()
    Hq, Hkv, D, bs, nblocks, MB = 24, 4, 256, 16, 24, 10
    rbk, rbv = synth.row_bytes(k_fmt, D), synth.row_bytes(v_fmt, D)
    gen = torch.Generator(device=DEV).manual_seed(77)
    kp = torch.empty((nblocks, bs, Hkv, rbk), dtype=torch.uint8, device=DEV)
    vp = torch.empty((nblocks, bs, Hkv, rbv), dtype=torch.uint8, device=DEV)
    synth.fill_junk(kp, k_fmt, D, "nan", gen)
    synth.fill_junk(vp, v_fmt, D, "nan", gen)

    def write_rows(ids, t0, t1):
        t = torch.arange(t0, t1, device=DEV)
        slot = torch.tensor(ids, device=DEV, dtype=torch.int64)[t // bs] * bs + t % bs
        for pool, fmt in ((kp, k_fmt), (vp, v_fmt)):
            vals = torch.randn((t1 - t0, Hkv, D), generator=gen, device=DEV)
            pool.view(nblocks * bs, Hkv, -1).index_copy_(0, slot, synth.encode(vals, fmt))

    alloc = pa.KvPool(nblocks)
    table = torch.zeros((2, MB), dtype=torch.int32, device=DEV)
    seq_len = torch.zeros(2, dtype=torch.int32, device=DEV)

    hA, idsA = alloc.alloc(6)
    write_rows(idsA, 0, 87)
    pa.paged_table_update(table, seq_len, [(0, i, b) for i, b in enumerate(idsA)] + [(0, -1, 87)])

    hB = alloc.fork(hA, 6)
    assert [alloc.refcount(i) for i in idsA] == [2] * 6
    new, old = alloc.cow(hB, 5)
    assert old == idsA[5] and new not in idsA
    pa.paged_kv_copy_blocks(kp, [old], [new])
    pa.paged_kv_copy_blocks(vp, [old], [new])
    _, more = alloc.alloc(2, hB)
    idsB = alloc.blocks(hB)
    assert idsB == idsA[:5] + [new] + more
    write_rows(idsB, 87, 127)
    pa.paged_table_update(table, seq_len, [(1, i, b) for i, b in enumerate(idsB)] + [(1, -1, 127)])

    assert alloc.cow(hA, 5) == (idsA[5], -1)          # private again: A writes in place
    _, moreA = alloc.alloc(1, hA)
    write_rows(idsA + moreA, 87, 101)
    pa.paged_table_update(table, seq_len, [(0, 6, moreA[0]), (0, -1, 101)])

    q = torch.randn((2, Hq, D), generator=gen, device=DEV)
    case = synth.Case(B=2, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, nblocks=nblocks, max_blocks=MB,
                      k_fmt=k_fmt, v_fmt=v_fmt, seq_lens=[101, 127], q=q, k_pool=kp, v_pool=vp,
                      table=table, seq_len=seq_len, scale=1.0 / 16, seed=77)
    shape = pa.shape_of(2, Hq, Hkv, D, bs, nblocks, MB, k_fmt, v_fmt)
    for force in (0, 1, 3):
        plan = pa.paged_attn_plan(shape, 127, total_tokens=228, force_partitions=force, scale=1.0 / 16)
        ws = pa.workspace(plan, DEV)
        out = torch.full((2, Hq, D), float("nan"), device=DEV)
        pa.paged_attn_step(plan, q, kp, vp, table, seq_len, ws, out)
        torch.cuda.synchronize()
        assert pa.paged_attn_status(ws) == 0
        check_parity(case.to("cpu"), out)

    # the shared prefix: B's rows 0..86 are A's rows, through both tables
    kf = kp.cpu().numpy().reshape(-1)
    tab = table.cpu().numpy()
    kw = dict(block_size=bs, Hkv=Hkv, nblocks=nblocks, max_blocks=MB, rbytes=rbk)
    for g in range(Hkv):
        ra = oracle.gather_rows(kf, oracle.row_offsets(tab, 0, g, 87, **kw), rbk)
        rb = oracle.gather_rows(kf, oracle.row_offsets(tab, 1, g, 87, **kw), rbk)
        assert np.array_equal(ra, rb)
    assert sorted(alloc.blocks(hA)[:5]) == sorted(idsB[:5])
