"""Pins for the fp64 oracle, independent of the oracle's own code.

Each test checks the oracle against something the pages or the mathematics fix:
byte counts the pages print (golden fixtures), exhaustive closed forms for the
byte decoders, a separate pure-Python brute force on tiny shapes, closed-form
attention results, paging invariance under shuffled tables with junk blocks,
a red control, and the merge invariant of the split form. The mutation test at
the end plants plausible mistakes in the oracle and checks that these pins
catch every one.
"""
import math
import struct

import numpy as np
import pytest
import torch

import oracle
import synth
from conftest import read_golden


# ----------------------------------------------------------------------------
# independent helpers (struct-based binary16 decoding, pure-Python loops)
# ----------------------------------------------------------------------------

def f16_from_bytes(lo: int, hi: int) -> float:
    return struct.unpack("<e", bytes([lo, hi]))[0]


def brute_row(raw: bytes, fmt: str, D: int):
    """Decode one row with plain Python and struct."""
    if fmt == "f16":
        return [struct.unpack_from("<e", raw, 2 * i)[0] for i in range(D)]
    out = []
    if fmt == "q8_0":
        for blk in range(D // 32):
            base = 34 * blk
            d = struct.unpack_from("<e", raw, base)[0]
            for j in range(32):
                q = struct.unpack_from("<b", raw, base + 2 + j)[0]
                out.append(d * q)
        return out
    if fmt == "q4_0":
        for blk in range(D // 32):
            base = 18 * blk
            d = struct.unpack_from("<e", raw, base)[0]
            vals = [0.0] * 32
            for j in range(16):
                byte = raw[base + 2 + j]
                vals[j] = d * ((byte & 0xF) - 8)
                vals[j + 16] = d * ((byte >> 4) - 8)
            out.extend(vals)
        return out
    raise ValueError(fmt)


def brute_decode(case):
    """Pure-Python decode step: loops over tokens, struct decoding, math.exp."""
    q = case.q.double().tolist()
    kp = bytes(case.k_pool.reshape(-1).tolist())
    vp = bytes(case.v_pool.reshape(-1).tolist())
    table = case.table.tolist()
    kb, vb = synth.row_bytes(case.k_fmt, case.D), synth.row_bytes(case.v_fmt, case.D)
    r = case.Hq // case.Hkv
    out = np.zeros((case.B, case.Hq, case.D))
    for b, L in enumerate(case.seq_lens):
        for h in range(case.Hq):
            g = h // r
            Ks, Vs = [], []
            for t in range(L):
                p = table[b][t // case.block_size]
                s = t % case.block_size
                row = (p * case.block_size + s) * case.Hkv + g
                Ks.append(brute_row(kp[row * kb:(row + 1) * kb], case.k_fmt, case.D))
                Vs.append(brute_row(vp[row * vb:(row + 1) * vb], case.v_fmt, case.D))
            if L == 0:
                continue
            z = [case.scale * sum(q[b][h][d] * k[d] for d in range(case.D)) for k in Ks]
            zmax = max(z)
            w = [math.exp(zi - zmax) for zi in z]
            sw = sum(w)
            for d in range(case.D):
                out[b, h, d] = sum(w[t] * Vs[t][d] for t in range(L)) / sw
    return out


def rel_err(a, b):
    """max over rows of max_d |a-b| / max_d |b| (rows of exactly zero compare absolutely)."""
    num = np.abs(a - b).max(axis=-1)
    den = np.abs(b).max(axis=-1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if num.size else 0.0


# ----------------------------------------------------------------------------
# byte accounting printed by the pages
# ----------------------------------------------------------------------------

def test_capacity_numbers_from_lucebox_page():
    g = read_golden("capacity_lucebox.txt")
    D, Hkv, bs = int(g["D"]), int(g["Hkv"]), int(g["block_size"])
    lens = [int(x) for x in g["seq_lens"].split(",")]
    live = sum(-(-L // bs) * bs for L in lens)
    assert live == int(g["live_tokens"])
    assert len(lens) * max(lens) == int(g["padded_slots"])
    per_token = Hkv * (oracle.row_bytes("q4_0", D) * 2)       # K and V
    MiB, GiB = 2**20, 2**30
    assert per_token * int(g["padded_slots"]) == int(g["one_layer_padded_MiB"]) * MiB
    assert round(per_token * live / MiB) == int(g["one_layer_paged_MiB"])
    layers = int(g["layers"])
    assert f"{per_token * int(g['padded_slots']) * layers / GiB:.3f}" == g["all_layers_padded_GiB"]
    assert f"{per_token * live * layers / GiB:.3f}" == g["all_layers_paged_GiB"]
    assert f"{int(g['padded_slots']) / live:.2f}" == g["ratio_x"]
    assert f"{100 * (1 - live / int(g['padded_slots'])):.2f}" == g["saving_percent"]


def test_wrap_point_from_mlxcel_page():
    g = read_golden("wrap_mlxcel.txt")
    Hkv, D, bs = int(g["Hkv"]), int(g["D"]), int(g["block_size"])
    slots = int(g["wrap_token_slots"])
    assert slots * Hkv * D == 2**32
    assert int(g["wrap_blocks"]) * bs == slots
    assert slots * Hkv * oracle.row_bytes("f16", D) == int(g["bytes_per_side_GiB_f16"]) * 2**30
    nblocks = int(g["test_pool_blocks"])
    rb = oracle.row_bytes("f16", D)
    # last element of a pool of exactly 2^32 elements is addressable
    table = np.array([[int(g["wrap_blocks"]) - 1]], dtype=np.int32)
    off = oracle.row_offsets(table, 0, Hkv - 1, bs, block_size=bs, Hkv=Hkv, rbytes=rb,
                             nblocks=nblocks, max_blocks=1)
    last_row = int(off[-1])
    assert last_row // 2 + D - 1 == 2**32 - 1                # element index (2-byte f16)
    # first row past 2^32 elements: the block named by the page's 131,073-block pool
    table = np.array([[int(g["wrap_blocks"])]], dtype=np.int32)
    off = oracle.row_offsets(table, 0, 0, 1, block_size=bs, Hkv=Hkv, rbytes=rb,
                             nblocks=nblocks, max_blocks=1)
    assert int(off[0]) == 2**32 * 2
    # same offsets as unbounded Python integers for random rows
    rng = np.random.default_rng(5)
    ids = rng.integers(0, nblocks, size=(1, 64)).astype(np.int32)
    for gg in range(Hkv):
        off = oracle.row_offsets(ids, 0, gg, 64 * bs, block_size=bs, Hkv=Hkv, rbytes=rb,
                                 nblocks=nblocks, max_blocks=64)
        for t in range(0, 64 * bs, 37):
            p = int(ids[0, t // bs])
            assert int(off[t]) == ((p * bs + t % bs) * Hkv + gg) * rb


# ----------------------------------------------------------------------------
# byte decoders: exhaustive closed forms
# ----------------------------------------------------------------------------

SCALES = [0.0, 1.0, -2.5, 0.1, 2.0**-24, 65504.0, -65504.0, 1.0 / 3.0, 6.1e-5]


def f16_bytes(x):
    return list(struct.pack("<e", x))


def test_f16_decode_matches_struct_including_specials():
    allbits = np.arange(65536, dtype=np.uint16)
    raw = allbits.view(np.uint8).reshape(1, -1)
    got = oracle.dequant_rows(raw, "f16", 65536)[0]
    for bits in list(range(0, 65536, 97)) + [0x0001, 0x03FF, 0x0400, 0x7BFF, 0x7C00, 0xFC00,
                                             0x8001, 0x7E00, 0x3C00, 0xBC00]:
        ref = f16_from_bytes(bits & 0xFF, bits >> 8)
        if math.isnan(ref):
            assert math.isnan(got[bits])
        else:
            assert got[bits] == ref


def test_q8_0_decode_exhaustive():
    for d in SCALES:
        raw = np.zeros((8, 34), dtype=np.uint8)  # 8 blocks x 32 = all 256 byte values
        for blk in range(8):
            raw[blk, 0:2] = f16_bytes(d)
            raw[blk, 2:34] = np.arange(32 * blk, 32 * blk + 32)
        got = oracle.dequant_rows(raw.reshape(1, -1), "q8_0", 256)[0]
        dd = f16_from_bytes(*f16_bytes(d))
        for v in range(256):
            signed = v - 256 if v >= 128 else v
            assert got[v] == dd * signed


def test_q4_0_decode_exhaustive():
    for d in SCALES:
        raw = np.zeros((16, 18), dtype=np.uint8)   # 16 blocks x 16 bytes = all 256 values
        for blk in range(16):
            raw[blk, 0:2] = f16_bytes(d)
            raw[blk, 2:18] = np.arange(16 * blk, 16 * blk + 16)
        got = oracle.dequant_rows(raw.reshape(1, -1), "q4_0", 512)[0]
        dd = f16_from_bytes(*f16_bytes(d))
        for blk in range(16):
            for j in range(16):
                byte = 16 * blk + j
                assert got[32 * blk + j] == dd * ((byte & 15) - 8)
                assert got[32 * blk + j + 16] == dd * ((byte >> 4) - 8)


def test_decoders_roundtrip_synth_encoders():
    """Values encoded by the generator decode back within the format's step
    (Q4_0: a value at the opposite extreme of the max-|x| one clamps at 15,
    so its error reaches one full step amax/8)."""
    x = torch.randn(64, 256, generator=torch.Generator().manual_seed(3))
    for fmt, tol in [("f16", 2**-11), ("q8_0", 0.5 / 127 + 2**-10), ("q4_0", 1 / 8 + 2**-9)]:
        raw = synth.encode(x, fmt).numpy()
        back = oracle.dequant_rows(raw, fmt, 256)
        amax = np.abs(x.numpy().reshape(64, 8, 32)).max(-1, keepdims=True)
        err = np.abs(back.reshape(64, 8, 32) - x.numpy().reshape(64, 8, 32)) / amax
        assert err.max() <= tol * 1.01, fmt


# ----------------------------------------------------------------------------
# brute force on tiny shapes, all nine K/V format pairs
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("k_fmt", synth.FORMATS)
@pytest.mark.parametrize("v_fmt", synth.FORMATS)
def test_brute_force_all_pairs(k_fmt, v_fmt):
    case = synth.make_case([37, 5, 64], Hq=6, Hkv=2, D=32, block_size=4, k_fmt=k_fmt,
                           v_fmt=v_fmt, seed=3 * synth.FORMATS.index(k_fmt) + synth.FORMATS.index(v_fmt),
                           junk="nan")
    got = oracle.decode_case(case)
    ref = brute_decode(case)
    assert rel_err(got, ref) <= 1e-13


@pytest.mark.parametrize("L", [0, 1, 15, 16, 17, 31, 32, 33, 70])
def test_brute_force_block_boundaries(L):
    case = synth.make_case([L, 3], Hq=4, Hkv=1, D=64, block_size=16, k_fmt="q4_0",
                           v_fmt="f16", seed=L, junk="nan")
    got = oracle.decode_case(case)
    ref = brute_decode(case)
    assert rel_err(got, ref) <= 1e-13
    if L == 0:
        assert np.all(got[0] == 0.0)


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def _case_from_values(K, V, q, *, bs=4, scale=None, Hkv=1):
    """A one-sequence case whose pool rows are given F16 values [L, Hkv, D]."""
    K = torch.as_tensor(K, dtype=torch.float32)
    V = torch.as_tensor(V, dtype=torch.float32)
    L, _, D = K.shape
    c = synth.make_case([L], Hq=q.shape[0], Hkv=Hkv, D=D, block_size=bs, k_fmt="f16",
                        v_fmt="f16", seed=L + 17, junk="nan", scale=scale)
    kflat = c.k_pool.view(-1, Hkv, 2 * D)
    vflat = c.v_pool.view(-1, Hkv, 2 * D)
    for t in range(L):
        slot = int(c.table[0, t // bs]) * bs + t % bs
        kflat[slot] = synth.encode(K[t], "f16")
        vflat[slot] = synth.encode(V[t], "f16")
    c.q = torch.as_tensor(q, dtype=torch.float32).reshape(1, q.shape[0], D)
    return c


def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(1)
    K, V = rng.standard_normal((1, 1, 32)), rng.standard_normal((1, 1, 32))
    c = _case_from_values(K, V, rng.standard_normal((2, 32)))
    out = oracle.decode_case(c)
    vv = np.float64(np.float16(V[0, 0]))
    assert np.array_equal(out[0, 0], vv) and np.array_equal(out[0, 1], vv)


def test_constant_value_rows_and_zero_query_mean():
    rng = np.random.default_rng(2)
    L, D = 23, 32
    K = rng.standard_normal((L, 1, D))
    row = rng.standard_normal(D)
    V = np.tile(row, (L, 1, 1))
    c = _case_from_values(K, V, rng.standard_normal((3, D)))
    out = oracle.decode_case(c)
    assert np.allclose(out[0], np.float16(row).astype(np.float64), rtol=0, atol=1e-14)
    V2 = rng.standard_normal((L, 1, D))
    c2 = _case_from_values(K, V2, np.zeros((1, D)))
    out2 = oracle.decode_case(c2)
    mean = np.float16(V2[:, 0]).astype(np.float64).mean(axis=0)
    assert np.allclose(out2[0, 0], mean, rtol=0, atol=1e-14)


def test_two_tokens_sigmoid_and_scale():
    D = 64
    q = np.zeros((1, D)); q[0, 0] = 2.0
    K = np.zeros((2, 1, D)); K[0, 0, 0] = 3.0; K[1, 0, 0] = -1.0   # q.k = 6, -2
    V = np.zeros((2, 1, D)); V[0, 0, :] = 1.0; V[1, 0, :] = -1.0
    c = _case_from_values(K, V, q)
    out = oracle.decode_case(c)
    a = 1.0 / (1.0 + math.exp(-(6.0 - (-2.0)) / math.sqrt(D)))   # softmax weight of token 0
    assert abs(out[0, 0, 0] - (a * 1.0 + (1 - a) * -1.0)) < 1e-15
    # an explicit scale overrides 1/sqrt(D)
    c.scale = 0.5
    out = oracle.decode_case(c)
    a = 1.0 / (1.0 + math.exp(-0.5 * 8.0))
    assert abs(out[0, 0, 5] - (2 * a - 1)) < 1e-15


def test_dominant_logit_selects_its_row():
    rng = np.random.default_rng(4)
    L, D = 40, 32
    q = np.zeros((1, D)); q[0, 3] = 1.0
    K = rng.standard_normal((L, 1, D)) * 0.01
    K[17, 0, 3] = 40.0 * math.sqrt(D)        # logit 40 above the rest (|others| < 0.1)
    V = rng.standard_normal((L, 1, D))
    c = _case_from_values(K, V, q)
    out = oracle.decode_case(c)
    vt = np.float16(V[17, 0]).astype(np.float64)
    vmax = np.abs(np.float16(V).astype(np.float64)).max()
    assert np.abs(out[0, 0] - vt).max() <= (L - 1) * math.exp(-39.8) * 2 * vmax


def test_gqa_head_to_kv_group_mapping():
    """Query head h reads kv head floor(h / (Hq/Hkv)): with V constant per kv
    head (+1 for head 0, -1 for head 1), rows 0..2 are +1 and rows 3..5 -1."""
    rng = np.random.default_rng(6)
    L, D, Hkv = 19, 32, 2
    K = rng.standard_normal((L, Hkv, D))
    V = np.zeros((L, Hkv, D)); V[:, 0] = 1.0; V[:, 1] = -1.0
    c = _case_from_values(K, V, rng.standard_normal((6, D)), Hkv=Hkv)
    out = oracle.decode_case(c)
    assert np.allclose(out[0, :3], 1.0, atol=1e-15)
    assert np.allclose(out[0, 3:], -1.0, atol=1e-15)


def test_identical_query_heads_give_identical_rows():
    c = synth.make_case([50], Hq=4, Hkv=1, D=64, k_fmt="q8_0", v_fmt="q4_0", seed=9)
    c.q[0, 1:] = c.q[0, 0]
    out = oracle.decode_case(c)
    for h in range(1, 4):
        assert np.array_equal(out[0, h], out[0, 0])


# ----------------------------------------------------------------------------
# paging invariance, junk, red control, corrupt tables
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("fmts", [("f16", "f16"), ("q4_0", "q8_0"), ("q8_0", "q4_0")])
def test_paged_equals_contiguous_bitwise_with_nan_junk(fmts):
    c = synth.make_case([45, 0, 16, 100], Hq=6, Hkv=2, D=64, block_size=16,
                        k_fmt=fmts[0], v_fmt=fmts[1], seed=21, junk="nan")
    cc = synth.contiguous_copy(c)
    a = oracle.decode_case(c)
    b = oracle.decode_case(cc, table=None)
    assert np.array_equal(a, b)
    assert np.isfinite(a).all()
    # same result with 'big' junk in the unused blocks and dead slots
    c2 = synth.make_case([45, 0, 16, 100], Hq=6, Hkv=2, D=64, block_size=16,
                         k_fmt=fmts[0], v_fmt=fmts[1], seed=21, junk="big")
    assert np.array_equal(oracle.decode_case(c2), a)


def test_red_control_corrupted_table_differs():
    """A table whose first entry names a later block of the same sequence must
    change the result (TensorFold PR #1418, Kernel contract, red control)."""
    c = synth.make_case([64], Hq=4, Hkv=1, D=64, block_size=16, seed=31)
    a = oracle.decode_case(c)
    bad = c.table.clone()
    bad[0, 0] = bad[0, 2]
    b = oracle.decode_case(c, table=bad)
    assert rel_err(b, a) > 1e-3


def test_out_of_range_block_id_raises():
    c = synth.make_case([40], Hq=4, Hkv=1, D=32, block_size=16, seed=32)
    for badid in (-1, c.nblocks):
        bad = c.table.clone()
        bad[0, 1] = badid
        with pytest.raises(ValueError):
            oracle.decode_case(c, table=bad)


# ----------------------------------------------------------------------------
# merge invariant of the split form
# ----------------------------------------------------------------------------

@pytest.mark.parametrize("psize", [1, 3, 16, 32, 50, 1000])
def test_merge_of_partials_equals_direct(psize):
    c = synth.make_case([97, 0, 1, 33], Hq=6, Hkv=3, D=64, block_size=16, k_fmt="q4_0",
                        v_fmt="q8_0", seed=40 + psize)
    kw = dict(Hkv=c.Hkv, D=c.D, block_size=c.block_size, k_fmt=c.k_fmt, v_fmt=c.v_fmt,
              nblocks=c.nblocks, max_blocks=c.max_blocks, scale=c.scale)
    kp, vp = c.k_pool.numpy().reshape(-1), c.v_pool.numpy().reshape(-1)
    m, l, o, n = oracle.partials(c.q, kp, vp, c.table, c.seq_len, psize=psize, **kw)
    assert list(n) == [-(-L // psize) for L in c.seq_lens]
    merged = oracle.merge(m, l, o, n)
    direct = oracle.decode_case(c)
    assert rel_err(merged, direct) <= 1e-12
    assert np.all(merged[1] == 0.0)


def test_merge_closed_form_two_partitions():
    """Two partitions with m=(0, 1), l=(1, 1): weights 2^-1 and 1."""
    m = np.array([[[0.0, 1.0]]]); l = np.array([[[1.0, 1.0]]])
    o = np.zeros((1, 1, 2, 4)); o[0, 0, 0] = 3.0; o[0, 0, 1] = 0.0
    out = oracle.merge(m, l, o, np.array([2]))
    assert np.allclose(out[0, 0], 3.0 * 0.5 / 1.5, atol=1e-15)


# ----------------------------------------------------------------------------
# mutation check: plausible mistakes in the oracle are caught by the pins
# ----------------------------------------------------------------------------

def _mutants():
    orig_deq = oracle.dequant_rows
    orig_off = oracle.row_offsets
    orig_att = oracle.attend

    def nibble_swap(raw, fmt, D):
        if fmt != "q4_0":
            return orig_deq(raw, fmt, D)
        raw = np.array(raw, dtype=np.uint8).reshape(raw.shape[0], D // 32, 18)
        raw[:, :, 2:] = ((raw[:, :, 2:] & 0x0F) << 4) | (raw[:, :, 2:] >> 4)
        return orig_deq(raw.reshape(raw.shape[0], -1), fmt, D)

    def unsigned_q8(raw, fmt, D):
        if fmt != "q8_0":
            return orig_deq(raw, fmt, D)
        n = raw.shape[0]
        blk = np.ascontiguousarray(raw).reshape(n, D // 32, 34)
        d = blk[:, :, 0:2].copy().view("<f2").astype(np.float64)
        return (d * blk[:, :, 2:].astype(np.float64)).reshape(n, D)

    def head_major(table, b, g, L, **kw):
        # reads the pool as [nblocks, Hkv, block_size, row] instead of
        # [nblocks, block_size, Hkv, row]
        bs, Hkv, rb = kw["block_size"], kw["Hkv"], kw["rbytes"]
        t = np.arange(L, dtype=np.int64)
        p = np.asarray(table, dtype=np.int64)[b][t // bs]
        return ((p * Hkv + g) * bs + t % bs) * rb

    def slot_off_by_one(table, b, g, L, **kw):
        bs, Hkv, rb = kw["block_size"], kw["Hkv"], kw["rbytes"]
        t = np.arange(L, dtype=np.int64)
        p = np.asarray(table, dtype=np.int64)[b][t // bs]
        return ((p * bs + (t + 1) % bs) * Hkv + g) * rb

    def wrong_group(table, b, g, L, **kw):
        return orig_off(table, b, (g + 1) % kw["Hkv"], L, **kw)

    def no_scale(q, K, V, scale):
        return orig_att(q, K, V, 1.0)

    def no_max_shift_sign(q, K, V, scale):
        if K.shape[0] == 0:
            return orig_att(q, K, V, scale)
        z = scale * (q @ K.T)
        w = np.exp(-(z - z.max(axis=1, keepdims=True)))
        return (w @ V) / w.sum(axis=1, keepdims=True)

    return {
        "q4_0 nibble order": ("dequant_rows", nibble_swap),
        "q8_0 read unsigned": ("dequant_rows", unsigned_q8),
        "head-major layout": ("row_offsets", head_major),
        "slot off by one": ("row_offsets", slot_off_by_one),
        "kv group": ("row_offsets", wrong_group),
        "dropped scale": ("attend", no_scale),
        "softmax sign": ("attend", no_max_shift_sign),
    }


@pytest.mark.parametrize("name", list(_mutants()))
def test_pins_catch_planted_oracle_mistakes(name, monkeypatch):
    attr, fn = _mutants()[name]
    monkeypatch.setattr(oracle, attr, fn)
    caught = False
    c = synth.make_case([21, 9], Hq=4, Hkv=2, D=32, block_size=4, k_fmt="q4_0",
                        v_fmt="q8_0", seed=77)
    try:
        caught |= not rel_err(oracle.decode_case(c), brute_decode(c)) <= 1e-9
    except Exception:
        caught = True
    c2 = synth.make_case([21, 9], Hq=4, Hkv=2, D=32, block_size=4, k_fmt="f16",
                         v_fmt="q4_0", seed=78)
    try:
        caught |= not rel_err(oracle.decode_case(c2), brute_decode(c2)) <= 1e-9
    except Exception:
        caught = True
    assert caught, f"mutant '{name}' survived the brute-force pin"
