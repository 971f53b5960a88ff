"""Calls that pass every host check and reach a kernel launcher, run only
against the host-only sanitizer build (whose launchers refuse with
PA_ERR_HIP): the full host path of each entry point - plan checks, workspace
carving, argument packing, chunking of long update and copy lists - executes
under AddressSanitizer and UndefinedBehaviorSanitizer. The device pointers
passed here are never dereferenced. Not collected by the default test run;
tests/test_host_sanitized.py runs this file in its sanitized child process."""
import ctypes

import pytest

import paged_kv_gqa_attn_amd as pa

if not hasattr(pa.lib, "pa_host_only_build"):
    pytest.skip("needs the host-only sanitizer build (its launchers refuse)", allow_module_level=True)

FAKE = 0x10000


def _shape(**kw):
    base = dict(B=8, Hq=24, Hkv=4, D=256, block_size=16, nblocks=100000, max_blocks=8192,
                k_type="q4_0", v_type="q4_0")
    base.update(kw)
    return pa.shape_of(**base)


def _refused_at_launch(fn):
    with pytest.raises(pa.PaError) as e:
        fn()
    assert e.value.code == pa.PA_ERR_HIP, str(e.value)
    assert "launch failed" in str(e.value)


@pytest.mark.parametrize("kw", [dict(), dict(k_type="f16", v_type="f16"), dict(Hkv=8, Hq=32, D=128),
                                dict(B=1024, nblocks=2000, max_blocks=64)])
@pytest.mark.parametrize("force", [0, 1, 5])
def test_decode_merge_step_reach_the_launcher(kw, force):
    shape = _shape(**kw)
    plan = pa.paged_attn_plan(shape, min(4096, shape.max_blocks * shape.block_size), num_cus=256,
                              force_partitions=force)
    ws = int(plan.ws_bytes)
    _refused_at_launch(lambda: pa.paged_attn_decode(plan, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, out=FAKE,
                                                    stream=0, ws_bytes=ws))
    _refused_at_launch(lambda: pa.paged_attn_decode(plan, FAKE, FAKE, FAKE, None, FAKE, FAKE, out=FAKE,
                                                    stream=0, ws_bytes=ws))
    if plan.direct or plan.fused:                  # merged by the decode (or nothing to merge)
        pa.paged_attn_merge(plan, FAKE, FAKE, FAKE, stream=0, ws_bytes=ws)
    else:
        _refused_at_launch(lambda: pa.paged_attn_merge(plan, FAKE, FAKE, FAKE, stream=0, ws_bytes=ws))
    if plan.fused:                                 # two launches: both reach a launcher
        plan.fused = 0
        _refused_at_launch(lambda: pa.paged_attn_merge(plan, FAKE, FAKE, FAKE, stream=0, ws_bytes=ws))
        plan.fused = 1
    _refused_at_launch(lambda: pa.paged_attn_step(plan, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0,
                                                  ws_bytes=ws))
    _refused_at_launch(lambda: pa.paged_kv_gather(plan, FAKE, 1, FAKE, 0, 16, 100, FAKE, stream=0))


@pytest.mark.parametrize("tq", [1, 2, 8, 512])
def test_chunk_reaches_the_launcher(tq):
    plan = pa.paged_attn_chunk_plan(_shape(), tq, 8192, num_cus=256)
    _refused_at_launch(lambda: pa.paged_attn_chunk(plan, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, stream=0,
                                                   ws_bytes=int(plan.ws_bytes)))


def test_long_update_and_copy_lists_reach_the_launcher():
    n = 1000                                  # several launches' worth of triples and pairs
    flat = []
    for i in range(n):
        flat += [i % 8, i // 8, i]
    upd = (ctypes.c_int32 * len(flat))(*flat)
    assert pa.lib.paged_table_update(FAKE, FAKE, 8, 512, upd, n, 0) == pa.PA_ERR_HIP
    src = (ctypes.c_int32 * n)(*range(n))
    dst = (ctypes.c_int32 * n)(*range(n, 2 * n))
    assert pa.lib.paged_kv_copy_blocks(FAKE, 4096, 2 * n, src, dst, n, 0) == pa.PA_ERR_HIP
