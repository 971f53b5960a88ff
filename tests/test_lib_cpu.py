"""CPU-side checks of the C-ABI library: it loads, exports every entry point
include/paged_attn.h declares, and its host logic (planner, argument
validation, error reporting, row sizes) behaves as documented. No kernel is
launched: every call here returns before touching a device."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "paged_attn.h")
LIB = os.environ.get("PAGED_ATTN_LIB") or os.path.join(ROOT, "paged_kv_gqa_attn_amd", "libpaged_attn.so")


def _ensure_built():
    """Build the library if nothing is built yet (without importing the
    package, whose import needs the library)."""
    if not os.path.exists(LIB):
        import importlib.util
        spec = importlib.util.spec_from_file_location(
            "_pa_build", os.path.join(ROOT, "paged_kv_gqa_attn_amd", "build.py"))
        mod = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(mod)
        mod.build()


_ensure_built()
import paged_kv_gqa_attn_amd as pa  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?([a-z_][a-z_0-9]*)\s*\(", text,
                                 flags=re.M)))


def test_header_declares_the_expected_entry_points():
    names = declared_functions()
    for must in ["paged_attn_plan", "paged_attn_decode", "paged_attn_merge", "paged_attn_step",
                 "paged_kv_gather", "paged_attn_status", "kv_pool_alloc", "kv_pool_release",
                 "kv_pool_create", "kv_pool_destroy", "kv_pool_reset", "pa_last_error",
                 "kv_pool_fork", "kv_pool_cow", "kv_pool_refcount", "paged_table_update",
                 "paged_kv_copy_blocks", "paged_attn_chunk_plan", "paged_attn_chunk",
                 "paged_attn_step_noalloc"]:
        assert must in names, must


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {l.split()[-1] for l in out.splitlines() if " T " in l}
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, f"declared but not exported: {missing}"
    L = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(L, n)


def test_binding_names_match_the_c_abi():
    for n in declared_functions():
        if n.startswith("kv_pool_"):
            continue                       # wrapped by the KvPool class
        assert hasattr(pa, n), n


def test_row_bytes():
    assert pa.pa_row_bytes(pa.PA_F16, 256) == 512
    assert pa.pa_row_bytes(pa.PA_Q8_0, 256) == 272
    assert pa.pa_row_bytes(pa.PA_Q4_0, 256) == 144
    assert pa.pa_row_bytes(pa.PA_Q4_0, 128) == 72
    with pytest.raises(pa.PaError) as e:
        pa.pa_row_bytes(pa.PA_Q4_0, 100)
    assert e.value.code == pa.PA_ERR_INVALID and "pa_row_bytes" in str(e.value)


def _shape(**kw):
    base = dict(B=8, Hq=24, Hkv=4, D=256, block_size=16, nblocks=100000, max_blocks=8192,
                k_type="q4_0", v_type="q4_0")
    base.update(kw)
    return pa.shape_of(**base)


def test_plan_automatic_partitions_for_long_context():
    p = pa.paged_attn_plan(_shape(), 131072, total_tokens=8 * 131072, num_cus=256)
    assert p.psize % 32 == 0 and p.psize >= 1024
    assert p.p_max == -(-131072 // p.psize)
    assert p.direct == 0
    # header, done[] counters of 8 sequences x 1 head quad (rounded to 256
    # bytes), then binary16 o rows and fp32 (m, l) pairs
    assert p.part_offset == 256 + 8 * 4160
    assert p.ws_bytes == p.part_offset + 8 * 24 * p.p_max * (2 * 256 + 8)
    assert 1 <= p.grid <= 256 * 8
    assert abs(p.scale - 1 / 16) < 1e-7


def test_plan_partial_traffic_floor_and_direct_mode():
    # a short batch: one partition covers it -> direct
    p = pa.paged_attn_plan(_shape(B=1), 200, num_cus=256)
    assert p.direct == 1 and p.p_max == 1 and p.ws_bytes == p.part_offset == 256 + 4352
    assert p.psize >= 200
    # register kernel (Hkv not a multiple of 4): the floor keeps partials
    # under ~4% of the K/V bytes of a partition
    p = pa.paged_attn_plan(_shape(Hq=12, Hkv=2), 32768, total_tokens=8 * 32768, num_cus=256)
    assert p.path == 1
    part = 12 * (2 * 256 + 8) * 2
    kv = p.psize * 2 * (144 + 144)
    assert part / kv <= 0.04 + 1e-9


def test_plan_lds_path_fills_two_workgroups_per_cu():
    for L in (32768, 131072):
        p = pa.paged_attn_plan(_shape(), L, total_tokens=8 * L, num_cus=256)
        assert p.path == 2 and p.grid == 512
        units = 8 * -(-L // p.psize)           # one unit per (sequence, partition) at Hkv = 4
        assert 480 <= units <= 512
    lens = [131072] + [8192] * 7
    p = pa.paged_attn_plan(_shape(), max(lens), total_tokens=sum(lens), num_cus=256)
    units = sum(-(-L // p.psize) for L in lens)
    assert p.path == 2 and units <= 512 and p.psize >= 64


@pytest.mark.parametrize("kw,path", [
    (dict(), 2),                                   # Q4_0/Q4_0, D=256, Hkv=4
    (dict(k_type="q8_0", v_type="q8_0"), 2),
    (dict(k_type="f16", v_type="f16"), 2),         # 8-slot groups: 16 slots of 4 F16 rows of D=256 are too big
    (dict(k_type="f16", v_type="q4_0"), 2),
    (dict(k_type="f16", v_type="f16", D=128, Hq=32, Hkv=8), 2),
    (dict(Hq=12, Hkv=2), 1),                       # no quad of kv heads
    (dict(Hq=24, Hkv=8), 2),
    (dict(B=300), 1),                              # batch prefix beyond the LDS budget
])
def test_plan_picks_the_decode_kernel(kw, path):
    p = pa.paged_attn_plan(_shape(**kw), 4096, num_cus=256)
    assert p.path == path


def test_plan_single_launch_merge_choice_and_checks():
    """fused (decode and merge in one launch) is the caller's choice (the
    planner leaves it 0: two launches measured faster on MI355X); it is
    accepted on the LDS kernel when partitions are merged with the wide
    layout, refused on the register kernel, in direct mode and where the
    merge takes the row-per-thread layout."""
    fake = 0x1000

    def decode(plan, out=fake):
        pa.paged_attn_decode(plan, fake, fake, fake, fake, fake, fake, out=out, stream=0,
                             ws_bytes=int(plan.ws_bytes))

    p = pa.paged_attn_plan(_shape(), 32768, total_tokens=8 * 32768, num_cus=256)
    assert p.path == 2 and p.fused == 0 and p.direct == 0 and p.grid == 512
    d = pa.paged_attn_plan(_shape(B=1), 200, num_cus=256)
    assert d.direct == 1 and d.fused == 0
    d.fused = 1
    with pytest.raises(pa.PaError) as e:
        decode(d)
    assert e.value.code == pa.PA_ERR_INVALID and "fused" in str(e.value)
    # 64 sequences x 24 heads = 1536 rows of 16 partitions: row-per-thread merge
    w = pa.paged_attn_plan(_shape(B=64, nblocks=200000), 4096, num_cus=256, force_partitions=16)
    assert w.path == 2 and w.p_max <= 16 and w.fused == 0
    w.fused = 1
    with pytest.raises(pa.PaError) as e:
        decode(w)
    assert e.value.code == pa.PA_ERR_INVALID and "fused" in str(e.value)
    p.fused = 1
    p.path = 1
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_decode(p, fake, fake, fake, fake, fake, fake, out=fake, stream=0,
                             ws_bytes=int(p.ws_bytes))
    assert e.value.code == pa.PA_ERR_INVALID and "fused" in str(e.value)
    p.path, p.fused = 2, 1
    with pytest.raises(pa.PaError) as e:          # a fused decode writes out
        pa.paged_attn_decode(p, fake, fake, fake, fake, fake, fake, out=None, stream=0,
                             ws_bytes=int(p.ws_bytes))
    assert e.value.code == pa.PA_ERR_INVALID
    pa.paged_attn_merge(p, fake, fake, fake, stream=0, ws_bytes=int(p.ws_bytes))   # no-op
    p.part_offset = 256
    with pytest.raises(pa.PaError):
        pa.paged_attn_merge(p, fake, fake, fake, stream=0, ws_bytes=int(p.ws_bytes))


def test_plan_path_two_refused_where_the_shape_does_not_fit():
    p = pa.paged_attn_plan(_shape(Hq=12, Hkv=2), 4096, num_cus=256)
    p.path = 2
    fake = 0x1000
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_decode(p, fake, fake, fake, fake, fake, fake, out=fake, stream=0,
                             ws_bytes=int(p.ws_bytes))
    assert e.value.code == pa.PA_ERR_UNSUPPORTED and "path 2" in str(e.value)
    p.path = 3
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_merge(p, fake, fake, fake, stream=0, ws_bytes=int(p.ws_bytes))
    assert e.value.code == pa.PA_ERR_INVALID


def test_plan_forced_partitions_and_tokens():
    p = pa.paged_attn_plan(_shape(), 1000, num_cus=256, force_partitions=1)
    assert p.direct == 1 and p.psize >= 1000
    p = pa.paged_attn_plan(_shape(), 1000, num_cus=256, force_partitions=7)
    assert p.p_max <= 7 and p.psize % 32 == 0 and p.p_max == -(-1000 // p.psize)
    p = pa.paged_attn_plan(_shape(), 1000, num_cus=256, partition_tokens=100)
    assert p.psize == 128 and p.p_max == 8
    p = pa.paged_attn_plan(_shape(), 0, num_cus=256)
    assert p.direct == 1


def test_plan_ragged_grid_follows_total_tokens():
    lens = [131072] + [8192] * 7
    p1 = pa.paged_attn_plan(_shape(), max(lens), total_tokens=sum(lens), num_cus=256)
    p2 = pa.paged_attn_plan(_shape(), max(lens), total_tokens=0, num_cus=256)
    assert p1.grid <= p2.grid


@pytest.mark.parametrize("kw,code,word", [
    (dict(Hq=25), pa.PA_ERR_INVALID, "multiple of Hkv"),
    (dict(D=64), pa.PA_ERR_UNSUPPORTED, "D=64"),
    (dict(block_size=24), pa.PA_ERR_INVALID, "power of two"),
    (dict(block_size=8), pa.PA_ERR_UNSUPPORTED, "block_size"),
    (dict(Hq=68, Hkv=4), pa.PA_ERR_UNSUPPORTED, "query heads per K/V head"),
    (dict(B=0), pa.PA_ERR_INVALID, ">= 1"),
    (dict(B=2000), pa.PA_ERR_UNSUPPORTED, "B=2000"),
    (dict(k_type=7), pa.PA_ERR_INVALID, "type"),
])
def test_plan_refusals_name_the_entry_point(kw, code, word):
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_plan(_shape(**kw), 100, num_cus=256)
    assert e.value.code == code
    assert "paged_attn_plan" in str(e.value) and word in str(e.value)


def test_plan_rejects_seq_len_beyond_table():
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_plan(_shape(max_blocks=10), 161, num_cus=256)
    assert e.value.code == pa.PA_ERR_INVALID


def test_decode_argument_checks_before_any_launch():
    plan = pa.paged_attn_plan(_shape(), 4096, num_cus=256)
    fake = 0x1000            # never dereferenced: every call below is refused first
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_decode(plan, fake, fake, fake, fake, fake, fake, out=fake, stream=0,
                             ws_bytes=int(plan.ws_bytes) - 1)
    assert e.value.code == pa.PA_ERR_INVALID and "workspace" in str(e.value)
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_decode(plan, None, fake, fake, fake, fake, fake, out=fake, stream=0,
                             ws_bytes=int(plan.ws_bytes))
    assert "paged_attn_decode" in str(e.value)
    bad = pa.PaPlan()
    bad.shape = _shape()
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_merge(bad, fake, fake, fake, stream=0, ws_bytes=1 << 20)
    assert "not produced by paged_attn_plan" in str(e.value)
    with pytest.raises(pa.PaError):
        pa.paged_kv_gather(plan, fake, 2, fake, 0, 0, 1, fake, stream=0)
    with pytest.raises(pa.PaError):
        pa.paged_kv_gather(plan, fake, 0, fake, 8, 0, 1, fake, stream=0)
    with pytest.raises(pa.PaError):
        pa.paged_kv_gather(plan, fake, 0, fake, 0, 8192 * 16, 1, fake, stream=0)


def test_noalloc_step_refuses_plans_beyond_its_scratch_before_any_launch():
    """paged_attn_step_noalloc checks the plan's workspace against its 64 MiB
    static scratch before it touches the device."""
    plan = pa.paged_attn_plan(_shape(B=1024, Hq=64, nblocks=600000), 131072, num_cus=256,
                              partition_tokens=256)
    assert plan.ws_bytes > 64 << 20
    fake = 0x1000
    rc = pa.lib.paged_attn_step_noalloc(ctypes.byref(plan), fake, fake, fake, fake, fake, fake, 0)
    assert rc == pa.PA_ERR_INVALID
    assert "paged_attn_step_noalloc" in pa.pa_last_error() and "static scratch" in pa.pa_last_error()


def test_noalloc_step_refuses_fused_plans_before_any_launch():
    """A fused plan's counters must start at zero, which the shared static
    scratch does not keep: paged_attn_step_noalloc refuses it before it
    touches the device."""
    plan = pa.paged_attn_plan(_shape(B=8), 32768, num_cus=256)
    assert plan.path == 2 and plan.direct == 0
    plan.fused = 1
    fake = 0x1000
    rc = pa.lib.paged_attn_step_noalloc(ctypes.byref(plan), fake, fake, fake, fake, fake, fake, 0)
    assert rc == pa.PA_ERR_INVALID
    assert "paged_attn_step_noalloc" in pa.pa_last_error() and "start at zero" in pa.pa_last_error()


def test_direct_plan_merge_is_a_no_op():
    plan = pa.paged_attn_plan(_shape(B=1), 100, num_cus=256)
    assert plan.direct == 1
    pa.paged_attn_merge(plan, 0x1000, 0x1000, 0x1000, stream=0, ws_bytes=256)


def _i32(vals):
    arr = (ctypes.c_int32 * max(len(vals), 1))(*vals)
    return arr


def test_table_update_refusals_before_any_launch():
    """paged_table_update validates every triple on the host and launches
    nothing when one is out of range or two name the same entry (lucebox PR
    #555, Summary: the resident table is updated entry by entry)."""
    fake = 0x1000
    cases = [
        ([2, 0, 7], "outside"),             # b = 2 >= B
        ([0, 4, 7], "outside"),             # slot = max_blocks
        ([0, -2, 7], "outside"),            # slot < -1
        ([0, 1, 7, 0, 1, 8], "same entry"),
        ([1, -1, 3, 1, -1, 4], "same entry"),
    ]
    for flat, word in cases:
        rc = pa.lib.paged_table_update(fake, fake, 2, 4, _i32(flat), len(flat) // 3, 0)
        assert rc == pa.PA_ERR_INVALID and word in pa.pa_last_error()
        assert "paged_table_update" in pa.pa_last_error()
    assert pa.lib.paged_table_update(fake, fake, 2, 4, None, 0, 0) == pa.PA_OK      # nothing to do
    assert pa.lib.paged_table_update(None, fake, 2, 4, _i32([0, 0, 1]), 1, 0) == pa.PA_ERR_INVALID


def test_copy_blocks_refusals_before_any_launch():
    fake = 0x1000
    cases = [
        ([0], [4], 4, 64, "outside"),         # dst >= nblocks
        ([-1], [2], 4, 64, "outside"),
        ([0, 1], [2, 2], 4, 64, "named twice"),
        ([0, 2], [2, 3], 4, 64, "both a source and a destination"),
        ([0], [1], 4, 40, "multiple of 16"),
    ]
    for src, dst, nb, bb, word in cases:
        rc = pa.lib.paged_kv_copy_blocks(fake, bb, nb, _i32(src), _i32(dst), len(src), 0)
        assert rc == pa.PA_ERR_INVALID and word in pa.pa_last_error(), (src, dst, pa.pa_last_error())
        assert "paged_kv_copy_blocks" in pa.pa_last_error()
    rc = pa.lib.paged_kv_copy_blocks(fake + 8, 64, 4, _i32([0]), _i32([1]), 1, 0)
    assert rc == pa.PA_ERR_INVALID and "aligned" in pa.pa_last_error()
    assert pa.lib.paged_kv_copy_blocks(fake, 64, 4, None, None, 0, 0) == pa.PA_OK


def test_chunk_plan_partitions_and_workspace():
    """paged_attn_chunk_plan: a four-wave workgroup per (sequence, partition,
    kv head, 64 query rows at D=256), two per compute unit, or per 128 query
    rows on the wide-tile kernel, one per compute unit; partials of 2D+8
    bytes per query row and partition."""
    p = pa.paged_attn_chunk_plan(_shape(), 9, 32768, total_tokens=8 * 32768, num_cus=256)
    assert p.tq == 9 and p.psize % 32 == 0 and p.direct == 0 and p.path == 1
    assert p.p_max == -(-32768 // p.psize)
    units = 8 * p.p_max * 4 * 1                      # 9*6 = 54 rows per kv head: one block
    assert p.grid == min(units, 256 * 2)
    big = pa.paged_attn_chunk_plan(_shape(B=1), 512, 8192, num_cus=256)
    assert big.path == 3 and big.grid == min(1 * big.p_max * 4 * 24, 256)   # 3072 rows: 24 blocks of 128
    assert p.part_offset == 256 + 8 * 4160
    assert p.ws_bytes == -(-(p.part_offset + 8 * 9 * 24 * p.p_max * (2 * 256 + 8)) // 256) * 256
    d = pa.paged_attn_chunk_plan(_shape(B=1), 16, 200, num_cus=256)
    assert d.direct == 1 and d.p_max == 1 and d.ws_bytes == 256 + 4352
    f = pa.paged_attn_chunk_plan(_shape(), 4, 1000, num_cus=256, partition_tokens=64)
    assert f.psize == 64 and f.p_max == 16


def test_chunk_plan_kernel_choice():
    """The window kernel (path 2) for at most 48 query rows per kv head: a
    workgroup per (sequence, partition, kv-head quad), except 17..48 rows at
    D=256, where the head dimension is split over two waves and a workgroup
    takes a kv-head pair, two per compute unit; the wide-tile kernel (path 3)
    for more than 64 rows, a workgroup per (sequence, partition, kv head, 128
    rows), one per compute unit (in its four-wave form, for F16 K and V at
    D=256 and F16 with Q8_0, only where its units fill at least half the
    CUs); the tile-conversion
    kernel (path 1) otherwise. A plan forced to path 2 where it does not apply, or to a path
    that does not exist, is refused before launch."""
    p = pa.paged_attn_chunk_plan(_shape(), 9, 32768, total_tokens=8 * 32768, num_cus=256)
    assert p.path == 1                                   # 54 rows
    w8 = pa.paged_attn_chunk_plan(_shape(), 8, 32768, total_tokens=8 * 32768, num_cus=256)
    assert w8.path == 2 and w8.grid == min(8 * w8.p_max * 2, 512)  # 48 rows: kv-head pairs
    q8 = pa.paged_attn_chunk_plan(_shape(k_type="q8_0"), 8, 32768, total_tokens=8 * 32768, num_cus=256)
    assert q8.path == 1                                  # 48 rows at D=256 with a Q8_0 side
    w = pa.paged_attn_chunk_plan(_shape(), 4, 32768, total_tokens=8 * 32768, num_cus=256)
    assert w.path == 2 and w.grid == min(8 * w.p_max * 2, 512)     # 24 rows: kv-head pairs
    w2 = pa.paged_attn_chunk_plan(_shape(), 2, 32768, total_tokens=8 * 32768, num_cus=256)
    assert w2.path == 2 and w2.grid == min(8 * w2.p_max * 1, 512)  # 12 rows
    w128 = pa.paged_attn_chunk_plan(_shape(D=128), 8, 32768, total_tokens=8 * 32768, num_cus=256)
    assert w128.path == 2                                # 48 rows at D=128
    assert pa.paged_attn_chunk_plan(_shape(D=128), 9, 32768, num_cus=256).path == 1
    for D in (256, 128):
        wide = pa.paged_attn_chunk_plan(_shape(D=D), 12, 32768, total_tokens=8 * 32768, num_cus=256)
        assert wide.path == 3 and wide.grid == min(8 * wide.p_max * 4 * 1, 256)    # 72 rows
        pre = pa.paged_attn_chunk_plan(_shape(D=D, B=1), 512, 8192, total_tokens=8192, num_cus=256)
        assert pre.path == 3 and pre.grid == min(pre.p_max * 4 * 24, 256)         # 3072 rows
    # the paired form takes every chunk of more than 64 rows: 192 rows, and a
    # 64-token chunk over 8K (72 units)
    assert pa.paged_attn_chunk_plan(_shape(), 32, 32768, total_tokens=8 * 32768, num_cus=256).path == 3
    assert pa.paged_attn_chunk_plan(_shape(B=1), 64, 8192, total_tokens=8192, num_cus=256).path == 3
    # the four-wave form (F16 K and V at D=256) needs units for half the CUs:
    # 72 at a 64-token chunk over 8K are too few, 144 at 128 tokens enough
    f16 = dict(k_type="f16", v_type="f16")
    assert pa.paged_attn_chunk_plan(_shape(B=1, **f16), 64, 8192, total_tokens=8192, num_cus=256).path == 1
    t128 = pa.paged_attn_chunk_plan(_shape(B=1, **f16), 128, 8192, total_tokens=8192, num_cus=256)
    assert t128.path == 3 and t128.grid == 144
    assert pa.paged_attn_chunk_plan(_shape(**f16), 32, 32768, total_tokens=8 * 32768, num_cus=256).path == 3
    assert pa.paged_attn_chunk_plan(_shape(D=128), 32, 32768, total_tokens=8 * 32768, num_cus=256).path == 3
    p.path = 2
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_chunk(p, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                            stream=0, ws_bytes=int(p.ws_bytes))
    assert e.value.code == pa.PA_ERR_UNSUPPORTED and "window" in str(e.value)
    w.path = 4
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_chunk(w, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                            stream=0, ws_bytes=int(w.ws_bytes))
    assert e.value.code == pa.PA_ERR_INVALID


def test_chunk_refusals_before_any_launch():
    for tq in (0, 4097):
        with pytest.raises(pa.PaError) as e:
            pa.paged_attn_chunk_plan(_shape(), tq, 100, num_cus=256)
        assert e.value.code == pa.PA_ERR_INVALID and "paged_attn_chunk_plan" in str(e.value)
    bogus = pa.PaChunkPlan()
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_chunk(bogus, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                            stream=0, ws_bytes=1 << 20)
    assert e.value.code == pa.PA_ERR_INVALID and "paged_attn_chunk" in str(e.value)
    p = pa.paged_attn_chunk_plan(_shape(), 4, 4096, num_cus=256)
    with pytest.raises(pa.PaError) as e:
        pa.paged_attn_chunk(p, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000, 0x1000,
                            stream=0, ws_bytes=int(p.ws_bytes) - 1)
    assert e.value.code == pa.PA_ERR_INVALID and "workspace" in str(e.value)


def test_smoke_cases_take_the_kernels_smoke_expects():
    """__graft_entry__.smoke() checks that each of its decode and chunk cases
    is planned on a given kernel; the planner (host code) must agree, for
    every partitioning smoke runs."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("_graft_entry", os.path.join(ROOT, "__graft_entry__.py"))
    ge = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(ge)
    for label, case, _, path in ge.smoke_cases():
        shape = pa.shape_of(case.B, case.Hq, case.Hkv, case.D, case.block_size, case.nblocks,
                            case.max_blocks, case.k_fmt, case.v_fmt)
        for force in (0, 1, 3):
            plan = pa.paged_attn_plan(shape, max(case.seq_lens), num_cus=256, force_partitions=force)
            assert plan.path == path, (label, force, plan.path)
    for label, case, Tq, path in ge.smoke_chunk_cases():
        shape = pa.shape_of(case.B, case.Hq, case.Hkv, case.D, case.block_size, case.nblocks,
                            case.max_blocks, case.k_fmt, case.v_fmt)
        plan = pa.paged_attn_chunk_plan(shape, Tq, max(case.seq_lens), total_tokens=sum(case.seq_lens),
                                        num_cus=256, partition_tokens=256, scale=case.scale)
        assert plan.path == path, (label, plan.path)


@pytest.mark.parametrize("Hq,Hkv,D,Tq,kt,vt,per_cu,heads", [
    (24, 4, 256, 2, "q4_0", "q4_0", 2, 4),    # 12 rows: one column group
    (24, 4, 256, 4, "q4_0", "q4_0", 2, 2),    # 24 rows at D=256: the head dimension split over kv-head pairs
    (24, 4, 256, 8, "q4_0", "q4_0", 2, 2),    # 48 rows at D=256: the same
    (32, 8, 128, 8, "q4_0", "q4_0", 2, 4),    # 32 rows at D=128, quantised: registers fit twice
    (32, 8, 128, 8, "f16", "f16", 1, 4),      # F16/F16 keeps the larger ring
    (32, 8, 128, 12, "q8_0", "q4_0", 2, 4),   # 48 rows at D=128: two per CU where measured faster
    (32, 8, 128, 12, "q4_0", "q8_0", 1, 4),   # ... but not Q4_0 K with Q8_0 V
])
def test_window_kernel_occupancy(Hq, Hkv, D, Tq, kt, vt, per_cu, heads):
    """The window chunk kernel's workgroups per CU and kv heads per workgroup
    for each shape class: the plan's grid is min(units, per_cu * num_cus) with
    units = B * p_max * Hkv / heads."""
    s = _shape(Hq=Hq, Hkv=Hkv, D=D, k_type=kt, v_type=vt, max_blocks=4096)
    p = pa.paged_attn_chunk_plan(s, Tq, 32768, total_tokens=8 * 32768, num_cus=256)
    assert p.path == 2
    assert p.grid == min(8 * p.p_max * Hkv // heads, per_cu * 256), (p.grid, p.p_max)
