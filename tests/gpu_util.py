"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare with the fp64 oracle on the same seeded bytes."""
import numpy as np
import torch

import oracle
import synth

TOL = {"f16": 2e-3, "q8_0": 5e-3, "q4_0": 5e-3}


def tol_for(case):
    return max(TOL[case.k_fmt], TOL[case.v_fmt])


def pa_mod():
    import paged_kv_gqa_attn_amd as pa
    return pa


def shape_for(case):
    pa = pa_mod()
    return pa.shape_of(case.B, case.Hq, case.Hkv, case.D, case.block_size, case.nblocks,
                       case.max_blocks, case.k_fmt, case.v_fmt)


def lds_path_ok(case):
    """Whether the LDS-staged decode kernel (plan path 2) takes the case's shape:
    quads of kv heads, B <= 256, and one group of 16 (else 8) token slots of K
    and V of four heads in a 36 KB ring slot."""
    rb = {"f16": 2 * case.D, "q8_0": 34 * case.D // 32, "q4_0": 18 * case.D // 32}
    fits = any(sum(-(-gs * 4 * rb[f] // 1024) for f in (case.k_fmt, case.v_fmt)) * 1024 <= 36864
               for gs in (16, 8))
    return case.Hkv % 4 == 0 and case.B <= 256 and fits


def plan_for(case, path=None, **kw):
    """paged_attn_plan for the case; path=1/2 forces the decode kernel (a case
    the LDS-staged kernel does not take is skipped for path 2)."""
    import pytest
    pa = pa_mod()
    kw.setdefault("total_tokens", sum(case.seq_lens))
    plan = pa.paged_attn_plan(shape_for(case), max(max(case.seq_lens), 0), **kw)
    assert plan.path == (2 if lds_path_ok(case) else 1)
    if path is not None:
        if path == 2 and not lds_path_ok(case):
            pytest.skip("the LDS-staged kernel does not take this shape")
        plan.path = path
        if path == 1:
            plan.fused = 0               # the single-launch merge is the LDS kernel's
    return plan


def run(case_dev, plan, table="case", ws=None, canary=0):
    """One decode step (decode + merge) on the GPU. Returns (out, ws)."""
    pa = pa_mod()
    dev = case_dev.q.device
    if ws is None:
        ws = pa.workspace(plan, dev, extra=canary)
        if canary:
            ws[int(plan.ws_bytes):] = 0xA5
    out = torch.full((case_dev.B, case_dev.Hq, case_dev.D), float("nan"), dtype=torch.float32,
                     device=dev)
    tab = case_dev.table if table == "case" else table
    pa.paged_attn_step(plan, case_dev.q, case_dev.k_pool, case_dev.v_pool, tab, case_dev.seq_len,
                       ws, out)
    torch.cuda.synchronize()
    return out, ws


def rel_err_rows(got, ref):
    """Per-row max_d |got-ref| / max_d |ref| (zero rows compared absolutely)."""
    got = np.asarray(got, dtype=np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return num / den


def check_parity(case, out, heads=None):
    """Compare out [B,Hq,D] with the oracle (all rows, or selected (b,g) groups)."""
    got = out.detach().cpu().double().numpy()
    tol = tol_for(case)
    if heads is None:
        ref = oracle.decode_case(case)
        err = rel_err_rows(got, ref)
        assert np.isfinite(got).all(), "non-finite output"
        worst = float(err.max())
        assert worst <= tol, f"max row error {worst:.3e} > {tol}"
        return worst
    res = oracle.decode_case(case, heads=heads)
    r = case.Hq // case.Hkv
    worst = 0.0
    for (b, g), ref in res.items():
        gg = got[b, g * r:(g + 1) * r]
        assert np.isfinite(gg).all(), f"non-finite output at b={b} g={g}"
        e = float(rel_err_rows(gg, ref).max())
        worst = max(worst, e)
        assert e <= tol, f"b={b} g={g}: max row error {e:.3e} > {tol}"
    return worst


class BlockSubset:
    """Host copy of selected blocks of a device pool, serving the oracle's row
    reads by byte offset (the oracle computes the offsets itself). Reading a
    row of a block that was not copied raises."""

    def __init__(self, pool_dev, block_ids):
        self.shape = tuple(pool_dev.shape)          # [nblocks, bs, Hkv, rb]
        self.ids = np.unique(np.asarray(list(block_ids), dtype=np.int64))
        sel = torch.from_numpy(self.ids).to(pool_dev.device)
        self.data = pool_dev.index_select(0, sel).cpu().numpy()

    def read_rows(self, offsets, rbytes):
        nb, bs, hkv, rb = self.shape
        assert rb == rbytes
        offsets = np.asarray(offsets, dtype=np.int64)
        if offsets.size and (offsets % rb).any():
            raise ValueError("unaligned row offset")
        row = offsets // rb
        blk = row // (bs * hkv)
        within = row % (bs * hkv)
        k = np.searchsorted(self.ids, blk)
        if blk.size and (k.max() >= self.ids.size or (self.ids[np.minimum(k, self.ids.size - 1)] != blk).any()):
            raise KeyError("row of a block that was not copied")
        flat = self.data.reshape(self.ids.size, bs * hkv, rb)
        return flat[k, within]


def all_groups(case):
    """Every (sequence, kv head) group of a case."""
    return [(b, g) for b in range(case.B) for g in range(case.Hkv)]


def sampled_parity(case_dev, out, items):
    """Oracle check of selected (b, g) groups of a device-resident case; the
    pool bytes the oracle reads are host copies of just those sequences'
    blocks. The whole output must be finite, sampled or not."""
    import types
    assert bool(torch.isfinite(out).all()), "non-finite values in the output"
    tab = case_dev.table.cpu()
    blocks = set()
    for b, _ in items:
        n = -(-case_dev.seq_lens[b] // case_dev.block_size)
        blocks |= set(tab[b, :n].tolist())
    host = types.SimpleNamespace(**{k: getattr(case_dev, k) for k in (
        "B", "Hq", "Hkv", "D", "block_size", "nblocks", "max_blocks", "k_fmt", "v_fmt",
        "seq_lens", "scale", "seed")})
    host.q = case_dev.q.cpu()
    host.table = tab
    host.seq_len = case_dev.seq_len.cpu()
    host.k_pool = BlockSubset(case_dev.k_pool, blocks)
    host.v_pool = BlockSubset(case_dev.v_pool, blocks)
    return check_parity(host, out, heads=items)
