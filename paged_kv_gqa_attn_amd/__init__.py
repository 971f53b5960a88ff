"""Python binding of libpaged_attn (paged GQA decode attention on MI355X).

Argument marshalling only: every function forwards to the C-ABI entry point of
the same name in libpaged_attn.so (declared in include/paged_attn.h); all
computation happens in the library's HIP kernels. Torch tensors are accepted
for device buffers (their data_ptr() is passed) and the current torch stream
is used when no stream is given. Importing this package fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# PAGED_ATTN_LIB names another build of the same C ABI (the tests' host-only
# sanitizer build, whose kernel launchers all refuse); by default the in-tree
# HIP library.
LIB_PATH = os.environ.get("PAGED_ATTN_LIB") or os.path.join(_HERE, "libpaged_attn.so")

PA_F16, PA_Q8_0, PA_Q4_0 = 0, 1, 2
PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_CAPACITY, PA_ERR_STALE_HANDLE, PA_ERR_HIP = (
    0, -1, -2, -3, -4, -5)
PA_STATUS_BAD_BLOCK_ID, PA_STATUS_BAD_SEQ_LEN, PA_STATUS_MERGE_WAIT = 1, 2, 4
TYPES = {"f16": PA_F16, "q8_0": PA_Q8_0, "q4_0": PA_Q4_0}

__all__ = ["PaShape", "PaPlan", "PaError", "lib", "pa_row_bytes", "pa_last_error",
           "paged_attn_plan", "paged_attn_decode", "paged_attn_merge", "paged_attn_step",
           "paged_attn_step_noalloc", "paged_kv_gather", "paged_attn_status", "KvPool", "workspace", "shape_of"]


class PaShape(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Hq", ctypes.c_int32), ("Hkv", ctypes.c_int32),
                ("D", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("nblocks", ctypes.c_int32), ("max_blocks", ctypes.c_int32),
                ("k_type", ctypes.c_int32), ("v_type", ctypes.c_int32)]


class PaPlan(ctypes.Structure):
    _fields_ = [("shape", PaShape), ("scale", ctypes.c_float), ("psize", ctypes.c_int32),
                ("p_max", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("num_cus", ctypes.c_int32),
                ("direct", ctypes.c_int32), ("path", ctypes.c_int32),
                ("fused", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("ws_bytes", ctypes.c_uint64), ("part_offset", ctypes.c_uint64)]

    def __repr__(self):
        s = self.shape
        return (f"PaPlan(B={s.B}, Hq={s.Hq}, Hkv={s.Hkv}, D={s.D}, bs={s.block_size}, "
                f"psize={self.psize}, p_max={self.p_max}, grid={self.grid}, "
                f"direct={self.direct}, path={self.path}, fused={self.fused}, "
                f"ws_bytes={self.ws_bytes}, part_offset={self.part_offset})")


class PaChunkPlan(ctypes.Structure):
    _fields_ = [("shape", PaShape), ("tq", ctypes.c_int32), ("scale", ctypes.c_float),
                ("psize", ctypes.c_int32), ("p_max", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("num_cus", ctypes.c_int32), ("direct", ctypes.c_int32),
                ("path", ctypes.c_int32), ("ws_bytes", ctypes.c_uint64),
                ("part_offset", ctypes.c_uint64)]

    def __repr__(self):
        s = self.shape
        return (f"PaChunkPlan(B={s.B}, Tq={self.tq}, Hq={s.Hq}, Hkv={s.Hkv}, D={s.D}, "
                f"psize={self.psize}, p_max={self.p_max}, grid={self.grid}, direct={self.direct}, "
                f"path={self.path}, ws_bytes={self.ws_bytes})")


class PaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


def _load():
    # torch ships its own HIP runtime under the same soname (libamdhip64.so.7);
    # importing torch first makes this library bind to that copy, so device
    # memory and streams handed over from torch live in the same runtime.
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()' "
            "or python paged_kv_gqa_attn_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    i32, u32, u64, i64, vp = ctypes.c_int32, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
    P = ctypes.POINTER
    sig = {
        "pa_row_bytes": (i32, [i32, i32]),
        "pa_last_error": (ctypes.c_char_p, []),
        "paged_attn_plan": (i32, [P(PaShape), i32, i64, i32, i32, i32, ctypes.c_float, P(PaPlan)]),
        "paged_attn_decode": (i32, [P(PaPlan), vp, vp, vp, vp, vp, vp, u64, vp, vp]),
        "paged_attn_merge": (i32, [P(PaPlan), vp, u64, vp, vp, vp]),
        "paged_attn_step": (i32, [P(PaPlan), vp, vp, vp, vp, vp, vp, u64, vp, vp]),
        "paged_attn_step_noalloc": (i32, [P(PaPlan), vp, vp, vp, vp, vp, vp, vp]),
        "paged_kv_gather": (i32, [P(PaPlan), vp, i32, vp, i32, i32, i32, vp, vp, vp]),
        "paged_attn_status": (i32, [vp, vp, P(u32)]),
        "kv_pool_create": (i32, [i32, P(vp)]),
        "kv_pool_destroy": (i32, [vp]),
        "kv_pool_alloc": (i32, [vp, i32, P(i32), P(u64)]),
        "kv_pool_release": (i32, [vp, u64]),
        "kv_pool_reset": (i32, [vp]),
        "kv_pool_free_count": (i32, [vp]),
        "kv_pool_count": (i32, [vp, u64]),
        "kv_pool_blocks": (i32, [vp, u64, P(i32), i32]),
        "kv_pool_fork": (i32, [vp, u64, i32, P(u64)]),
        "kv_pool_cow": (i32, [vp, u64, i32, P(i32), P(i32)]),
        "kv_pool_refcount": (i32, [vp, i32]),
        "paged_table_update": (i32, [vp, vp, i32, i32, P(i32), i32, vp]),
        "paged_attn_chunk_plan": (i32, [P(PaShape), i32, i32, i64, i32, i32, i32, ctypes.c_float,
                                        P(PaChunkPlan)]),
        "paged_attn_chunk": (i32, [P(PaChunkPlan), vp, vp, vp, vp, vp, vp, u64, vp, vp]),
        "paged_kv_copy_blocks": (i32, [vp, u64, i32, P(i32), P(i32), i32, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    return L


lib = _load()


def pa_last_error() -> str:
    return lib.pa_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise PaError(rc, pa_last_error())
    return rc


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def pa_row_bytes(type_: int, D: int) -> int:
    return _check(lib.pa_row_bytes(type_, D))


def shape_of(B, Hq, Hkv, D, block_size, nblocks, max_blocks, k_type, v_type) -> PaShape:
    kt = TYPES.get(k_type, k_type)
    vt = TYPES.get(v_type, v_type)
    return PaShape(B, Hq, Hkv, D, block_size, nblocks, max_blocks, kt, vt)


def paged_attn_plan(shape: PaShape, max_seq_len: int, total_tokens: int = 0, num_cus: int = 0,
                    force_partitions: int = 0, partition_tokens: int = 0,
                    scale: float = 0.0) -> PaPlan:
    plan = PaPlan()
    _check(lib.paged_attn_plan(ctypes.byref(shape), max_seq_len, total_tokens, num_cus,
                               force_partitions, partition_tokens, scale, ctypes.byref(plan)))
    return plan


def paged_attn_decode(plan: PaPlan, q, k_pool, v_pool, block_table, seq_len, ws, out=None,
                      stream=None, ws_bytes: Optional[int] = None) -> None:
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(lib.paged_attn_decode(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                 _ptr(block_table), _ptr(seq_len), _ptr(ws), nb, _ptr(out),
                                 _stream(stream)))


def paged_attn_merge(plan: PaPlan, ws, seq_len, out, stream=None,
                     ws_bytes: Optional[int] = None) -> None:
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(lib.paged_attn_merge(ctypes.byref(plan), _ptr(ws), nb, _ptr(seq_len), _ptr(out),
                                _stream(stream)))


def paged_attn_step(plan: PaPlan, q, k_pool, v_pool, block_table, seq_len, ws, out,
                    stream=None, ws_bytes: Optional[int] = None) -> None:
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(lib.paged_attn_step(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                               _ptr(block_table), _ptr(seq_len), _ptr(ws), nb, _ptr(out),
                               _stream(stream)))


def paged_attn_step_noalloc(plan: PaPlan, q, k_pool, v_pool, block_table, seq_len, out,
                            stream=None) -> None:
    """paged_attn_step with the library's static per-GPU scratch as workspace
    (no allocation; calls overlapping on one GPU race)."""
    _check(lib.paged_attn_step_noalloc(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                       _ptr(block_table), _ptr(seq_len), _ptr(out), _stream(stream)))


def paged_kv_gather(plan: PaPlan, pool, which: int, block_table, b: int, t0: int, n: int, dst,
                    ws=None, stream=None) -> None:
    _check(lib.paged_kv_gather(ctypes.byref(plan), _ptr(pool), which, _ptr(block_table), b, t0,
                               n, _ptr(dst), _ptr(ws), _stream(stream)))


def paged_attn_status(ws, stream=None) -> int:
    flags = ctypes.c_uint32(0)
    _check(lib.paged_attn_status(_ptr(ws), _stream(stream), ctypes.byref(flags)))
    return flags.value


def paged_attn_chunk_plan(shape: PaShape, tq: int, max_seq_len: int, total_tokens: int = 0,
                          num_cus: int = 0, force_partitions: int = 0, partition_tokens: int = 0,
                          scale: float = 0.0) -> PaChunkPlan:
    plan = PaChunkPlan()
    _check(lib.paged_attn_chunk_plan(ctypes.byref(shape), tq, max_seq_len, total_tokens, num_cus,
                                     force_partitions, partition_tokens, scale, ctypes.byref(plan)))
    return plan


def paged_attn_chunk(plan: PaChunkPlan, q, k_pool, v_pool, block_table, seq_len, ws, out,
                     stream=None, ws_bytes: Optional[int] = None) -> None:
    """Chunk attention (q, out: fp32 [B, Tq, Hq, D]), merge included."""
    nb = ws_bytes if ws_bytes is not None else ws.numel() * ws.element_size()
    _check(lib.paged_attn_chunk(ctypes.byref(plan), _ptr(q), _ptr(k_pool), _ptr(v_pool),
                                _ptr(block_table), _ptr(seq_len), _ptr(ws), nb, _ptr(out),
                                _stream(stream)))


def _i32_array(values):
    flat = [int(v) for v in values]
    return (ctypes.c_int32 * max(len(flat), 1))(*flat), len(flat)


def paged_table_update(table, seq_len, updates, stream=None) -> None:
    """Write (b, slot, value) triples into the device table [B, max_blocks]
    (slot >= 0) or seq_len [B] (slot == -1); the triples are host values."""
    B, max_blocks = table.shape
    flat, n3 = _i32_array(v for t in updates for v in t)
    _check(lib.paged_table_update(_ptr(table), _ptr(seq_len), B, max_blocks, flat, n3 // 3,
                                  _stream(stream)))


def paged_kv_copy_blocks(pool, src_ids, dst_ids, stream=None) -> None:
    """Copy whole blocks src_ids[i] -> dst_ids[i] inside a device pool
    [nblocks, block_size, Hkv, row_bytes] (host id lists)."""
    nblocks = pool.shape[0]
    block_bytes = pool[0].numel() * pool.element_size() if nblocks else 0
    src, n = _i32_array(src_ids)
    dst, m = _i32_array(dst_ids)
    if n != m:
        raise ValueError("src_ids and dst_ids differ in length")
    _check(lib.paged_kv_copy_blocks(_ptr(pool), block_bytes, nblocks, src, dst, n, _stream(stream)))


def workspace(plan: PaPlan, device="cuda", extra: int = 0):
    """A zero-filled uint8 workspace tensor of plan.ws_bytes (+ extra) bytes."""
    import torch
    return torch.zeros(int(plan.ws_bytes) + extra, dtype=torch.uint8, device=device)


class KvPool:
    """Handle-based fixed-block allocator (kv_pool_* entry points)."""

    def __init__(self, nblocks: int):
        h = ctypes.c_void_p()
        _check(lib.kv_pool_create(nblocks, ctypes.byref(h)))
        self._h = h

    def close(self):
        if self._h:
            _check(lib.kv_pool_destroy(self._h))
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int, handle: int = 0):
        ids = (ctypes.c_int32 * max(n, 1))()
        h = ctypes.c_uint64(handle)
        _check(lib.kv_pool_alloc(self._h, n, ids, ctypes.byref(h)))
        return h.value, list(ids[:n])

    def release(self, handle: int) -> None:
        _check(lib.kv_pool_release(self._h, handle))

    def reset(self) -> None:
        _check(lib.kv_pool_reset(self._h))

    def free_count(self) -> int:
        return _check(lib.kv_pool_free_count(self._h))

    def count(self, handle: int) -> int:
        return _check(lib.kv_pool_count(self._h, handle))

    def fork(self, src: int, n_shared: int) -> int:
        """A new allocation holding the first n_shared blocks of src."""
        h = ctypes.c_uint64(0)
        _check(lib.kv_pool_fork(self._h, src, n_shared, ctypes.byref(h)))
        return h.value

    def cow(self, handle: int, index: int):
        """Make block `index` private: returns (id, copy_from), copy_from = -1
        when no copy is needed."""
        i, c = ctypes.c_int32(0), ctypes.c_int32(0)
        _check(lib.kv_pool_cow(self._h, handle, index, ctypes.byref(i), ctypes.byref(c)))
        return i.value, c.value

    def refcount(self, block_id: int) -> int:
        return _check(lib.kv_pool_refcount(self._h, block_id))

    def blocks(self, handle: int):
        n = _check(lib.kv_pool_blocks(self._h, handle, None, 0))
        ids = (ctypes.c_int32 * max(n, 1))()
        _check(lib.kv_pool_blocks(self._h, handle, ids, n))
        return list(ids[:n])
