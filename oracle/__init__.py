"""fp64 CPU oracle for paged GQA decode attention.

TEST INFRASTRUCTURE ONLY. Only the tests, the package smoke check and the
benchmark's CPU-baseline leg may import this module; the product path (the
C-ABI library and its Python binding) never does, and shares no code with it.

What it computes is the plain definition of one decode step, written out in
float64 with no blocking, fusion or reordering:

  for every sequence b, query head h, with kv head g = floor(h / (Hq/Hkv)) and
  L = seq_len[b]:
    1. for t < L, look up physical block  p = table[b][t // block_size],
       slot s = t % block_size, and read the encoded row at byte offset
       ((p*block_size + s)*Hkv + g) * row_bytes      (exact integer math);
    2. decode each row to float64 exactly (F16 widening; Q8_0 d*q;
       Q4_0 (nibble-8)*d);
    3. z_t = scale * sum_d q[b,h,d] * k_t[d];  w_t = exp(z_t - max z);
       out[b,h,:] = sum_t w_t v_t / sum_t w_t;
    4. L = 0 gives a zero row.

Sources (page titles and sections):
  * lucebox PR #555 "paged-attention monolithic decode-only AR foundation",
    Summary: single-query paged attention over a pool of fixed-size blocks,
    D=256 with grouped query heads, K/V stored as F16, Q4_0 or Q8_0, one pass
    over a K/V row serving every query head that shares it, partitions
    recombined by a max-shifted merge; Validation: checked against a float64
    reference with and without partitions, on zero-length sequences, block
    edges, permuted block order and tables with out-of-range entries.
  * mlxcel issue #2153 "use 64-bit pool offsets in the fused decode kernels",
    Current Behavior and Proposed Solution: a row's pool offset (block id
    times block size plus slot, times the token stride, plus the head's
    offset) must be formed in 64-bit arithmetic before any product; Scope: the gather path (gather through the table, then dense
    attention) is the reference the fused kernels are checked against.
  * TensorFold PR #1418, Kernel contract: a float64 attention reference and
    shuffled pages with spare junk pages.

`partials` / `merge` give the split form: per context partition the running
max m (base-2 logits), the sum l and the normalised output o, then the stable
max-rescaling merge (lucebox PR #555, Summary: the partitions are recombined
by a numerically stable merge of the split softmax; llama.cpp PR #13 HRX,
Changes: the multi-pass KV-block reduction). In exact
arithmetic merge(partials(...)) equals decode(...).
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

LOG2E = 1.0 / math.log(2.0)

__all__ = ["row_bytes", "dequant_rows", "row_offsets", "gather_rows", "attend",
           "decode", "decode_heads", "partials", "merge", "chunk", "LOG2E"]


def row_bytes(fmt: str, D: int) -> int:
    """Bytes of one encoded row: F16 2 bytes per value; Q8_0 34 bytes and
    Q4_0 18 bytes per block of 32 values (f16 scale + 32 int8 / 16 nibble
    bytes)."""
    if fmt == "f16":
        return 2 * D
    if D % 32 != 0:
        raise ValueError("quantised rows need D % 32 == 0")
    return {"q8_0": 34, "q4_0": 18}[fmt] * (D // 32)


def _f16(raw: np.ndarray) -> np.ndarray:
    """Little-endian IEEE binary16 bytes [..., 2k] -> float64 [..., k] (exact)."""
    return np.ascontiguousarray(raw).view("<f2").astype(np.float64)


def dequant_rows(raw: np.ndarray, fmt: str, D: int) -> np.ndarray:
    """Decode uint8 rows [n, row_bytes] to float64 [n, D] exactly."""
    raw = np.ascontiguousarray(raw, dtype=np.uint8)
    n = raw.shape[0]
    if fmt == "f16":
        return _f16(raw).reshape(n, D)
    nb = D // 32
    if fmt == "q8_0":
        blk = raw.reshape(n, nb, 34)
        d = _f16(blk[:, :, 0:2]).reshape(n, nb, 1)
        q = blk[:, :, 2:34].view(np.int8).astype(np.float64)
        return (d * q).reshape(n, D)
    if fmt == "q4_0":
        blk = raw.reshape(n, nb, 18)
        d = _f16(blk[:, :, 0:2]).reshape(n, nb, 1)
        b = blk[:, :, 2:18].astype(np.int64)
        lo = (b & 0x0F) - 8          # element j of the block, j < 16
        hi = (b >> 4) - 8            # element j + 16
        x = np.concatenate([lo, hi], axis=2).astype(np.float64)
        return (d * x).reshape(n, D)
    raise ValueError(fmt)


def row_offsets(table: Optional[np.ndarray], b: int, g: int, L: int, *, block_size: int,
                Hkv: int, rbytes: int, nblocks: int, max_blocks: int) -> np.ndarray:
    """Byte offsets (int64) of the rows of tokens 0..L-1 of sequence b, kv head g.

    table None means the contiguous layout: sequence b's logical block j is
    physical block b*max_blocks + j. A block id outside [0, nblocks) raises.
    """
    t = np.arange(L, dtype=np.int64)
    j = t // block_size
    if table is None:
        p = b * max_blocks + j
    else:
        p = np.asarray(table, dtype=np.int64)[b][j]
    if L and (p.min() < 0 or p.max() >= nblocks):
        raise ValueError(f"block table of sequence {b} names a block outside the pool")
    slot = t % block_size
    # widened to 64 bits before any multiply (mlxcel #2153, Implementation Notes)
    return ((p * block_size + slot) * Hkv + g) * rbytes


def gather_rows(pool, offsets: np.ndarray, rbytes: int) -> np.ndarray:
    """Read rows of rbytes bytes at the given byte offsets.

    `pool` is a flat uint8 array of the whole pool, or any object with a
    `read_rows(offsets, rbytes)` method serving the same bytes.
    """
    if hasattr(pool, "read_rows"):
        return pool.read_rows(offsets, rbytes)
    flat = np.asarray(pool).reshape(-1)
    if offsets.size and (offsets % rbytes).any():
        raise ValueError("row offsets must be multiples of the row size")
    rows = flat.view(np.uint8)[: (flat.size // rbytes) * rbytes].reshape(-1, rbytes)
    return rows[offsets // rbytes]


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float) -> np.ndarray:
    """softmax(scale * q K^T) V for q [r, D], K, V [L, D] (float64)."""
    r, D = q.shape
    if K.shape[0] == 0:
        return np.zeros((r, V.shape[1]), dtype=np.float64)
    z = scale * (q @ K.T)                       # [r, L]
    m = z.max(axis=1, keepdims=True)
    w = np.exp(z - m)
    return (w @ V) / w.sum(axis=1, keepdims=True)


def _np(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.asarray(x)


def decode_heads(q, k_pool, v_pool, table, seq_len, *, Hkv: int, D: int, block_size: int,
                 k_fmt: str, v_fmt: str, nblocks: int, max_blocks: int,
                 scale: Optional[float] = None, items: Optional[Sequence[tuple]] = None):
    """Oracle output for selected (b, g) kv-head groups.

    Returns {(b, g): float64 [r, D]} for the query heads g*r .. g*r+r-1.
    """
    q = _np(q).astype(np.float64)
    B, Hq, _ = q.shape
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    r = Hq // Hkv
    seq_len = _np(seq_len).astype(np.int64)
    tab = None if table is None else _np(table)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kb, vb = row_bytes(k_fmt, D), row_bytes(v_fmt, D)
    if items is None:
        items = [(b, g) for b in range(B) for g in range(Hkv)]
    out = {}
    for b, g in items:
        L = int(seq_len[b])
        if L < 0 or L > max_blocks * block_size:
            raise ValueError(f"seq_len[{b}]={L} outside [0, max_blocks*block_size]")
        kw = dict(block_size=block_size, Hkv=Hkv, nblocks=nblocks, max_blocks=max_blocks)
        ko = row_offsets(tab, b, g, L, rbytes=kb, **kw)
        vo = row_offsets(tab, b, g, L, rbytes=vb, **kw)
        K = dequant_rows(gather_rows(k_pool, ko, kb), k_fmt, D)
        V = dequant_rows(gather_rows(v_pool, vo, vb), v_fmt, D)
        out[(b, g)] = attend(q[b, g * r:(g + 1) * r], K, V, scale)
    return out


def decode(q, k_pool, v_pool, table, seq_len, *, Hkv: int, D: int, block_size: int,
           k_fmt: str, v_fmt: str, nblocks: int, max_blocks: int,
           scale: Optional[float] = None) -> np.ndarray:
    """Full oracle output float64 [B, Hq, D]."""
    qn = _np(q)
    B, Hq, _ = qn.shape
    r = Hq // Hkv
    res = decode_heads(qn, k_pool, v_pool, table, seq_len, Hkv=Hkv, D=D,
                       block_size=block_size, k_fmt=k_fmt, v_fmt=v_fmt, nblocks=nblocks,
                       max_blocks=max_blocks, scale=scale)
    out = np.zeros((B, Hq, D), dtype=np.float64)
    for (b, g), o in res.items():
        out[b, g * r:(g + 1) * r] = o
    return out


def decode_case(case, heads: Optional[Sequence[tuple]] = None, table="case"):
    """Convenience: run the oracle on a synthetic case object (host copies of
    its tensors). `heads` selects (b, g) groups; table=None forces the
    contiguous layout."""
    tab = case.table if table == "case" else table
    kw = dict(Hkv=case.Hkv, D=case.D, block_size=case.block_size, k_fmt=case.k_fmt,
              v_fmt=case.v_fmt, nblocks=case.nblocks, max_blocks=case.max_blocks,
              scale=case.scale)
    kp = _np(case.k_pool).reshape(-1) if not hasattr(case.k_pool, "read_rows") else case.k_pool
    vp = _np(case.v_pool).reshape(-1) if not hasattr(case.v_pool, "read_rows") else case.v_pool
    if heads is None:
        return decode(case.q, kp, vp, tab, case.seq_len, **kw)
    return decode_heads(case.q, kp, vp, tab, case.seq_len, items=heads, **kw)


def chunk(q, k_pool, v_pool, table, seq_len, *, Hkv: int, D: int, block_size: int,
          k_fmt: str, v_fmt: str, nblocks: int, max_blocks: int,
          scale: Optional[float] = None) -> np.ndarray:
    """Multi-token query over the paged pool with causal masking inside the
    chunk (lucebox PR #555, Roadmap item 3: several query tokens per sequence
    attend over the K/V already in the pool, causally inside the chunk;
    TensorFold PR #1418, What: paged prompt-chunk attention equal to the
    contiguous one).

    q is [B, Tq, Hq, D]; seq_len[b] = L counts the chunk's own tokens, which
    are the last Tq of the sequence, so chunk token t sits at position
    L - Tq + t and attends to the keys at positions 0 .. L - Tq + t. A
    sequence with L = 0 gives zero rows; 0 < L < Tq raises. Returns float64
    [B, Tq, Hq, D].
    """
    qn = _np(q).astype(np.float64)
    B, Tq, Hq, _ = qn.shape
    r = Hq // Hkv
    seq_len = _np(seq_len).astype(np.int64)
    tab = None if table is None else _np(table)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kb, vb = row_bytes(k_fmt, D), row_bytes(v_fmt, D)
    kw = dict(block_size=block_size, Hkv=Hkv, nblocks=nblocks, max_blocks=max_blocks)
    out = np.zeros((B, Tq, Hq, D), dtype=np.float64)
    for b in range(B):
        L = int(seq_len[b])
        if L == 0:
            continue
        if L < Tq or L > max_blocks * block_size:
            raise ValueError(f"seq_len[{b}]={L} outside [Tq, max_blocks*block_size]")
        for g in range(Hkv):
            K = dequant_rows(gather_rows(k_pool, row_offsets(tab, b, g, L, rbytes=kb, **kw), kb),
                             k_fmt, D)
            V = dequant_rows(gather_rows(v_pool, row_offsets(tab, b, g, L, rbytes=vb, **kw), vb),
                             v_fmt, D)
            for t in range(Tq):
                n = L - Tq + t + 1                 # keys 0 .. L - Tq + t
                out[b, t, g * r:(g + 1) * r] = attend(qn[b, t, g * r:(g + 1) * r], K[:n], V[:n],
                                                      scale)
    return out


def partials(q, k_pool, v_pool, table, seq_len, *, Hkv: int, D: int, block_size: int,
             k_fmt: str, v_fmt: str, nblocks: int, max_blocks: int, psize: int,
             scale: Optional[float] = None):
    """Split form over context partitions of psize tokens.

    For partition p of sequence b (tokens p*psize .. min(L, (p+1)*psize)-1) and
    head h, with base-2 logits y_t = log2(e) * scale * q.k_t:
        m = max_t y_t,  l = sum_t 2^(y_t - m),  o = sum_t 2^(y_t - m) v_t / l.
    Returns (m [B,Hq,P], l [B,Hq,P], o [B,Hq,P,D], nparts [B]) with
    P = max_b ceil(L_b/psize); unused partition slots hold m=-inf, l=0, o=0.
    """
    q = _np(q).astype(np.float64)
    B, Hq, _ = q.shape
    r = Hq // Hkv
    seq_len = _np(seq_len).astype(np.int64)
    tab = None if table is None else _np(table)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    kb, vb = row_bytes(k_fmt, D), row_bytes(v_fmt, D)
    nparts = np.array([(int(L) + psize - 1) // psize for L in seq_len], dtype=np.int64)
    P = max(int(nparts.max()) if B else 0, 1)
    m = np.full((B, Hq, P), -np.inf)
    l = np.zeros((B, Hq, P))
    o = np.zeros((B, Hq, P, D))
    kw = dict(block_size=block_size, Hkv=Hkv, nblocks=nblocks, max_blocks=max_blocks)
    for b in range(B):
        L = int(seq_len[b])
        for g in range(Hkv):
            K = dequant_rows(gather_rows(k_pool, row_offsets(tab, b, g, L, rbytes=kb, **kw), kb),
                             k_fmt, D)
            V = dequant_rows(gather_rows(v_pool, row_offsets(tab, b, g, L, rbytes=vb, **kw), vb),
                             v_fmt, D)
            y = LOG2E * scale * (q[b, g * r:(g + 1) * r] @ K.T)     # [r, L]
            for p in range(int(nparts[b])):
                t0, t1 = p * psize, min(L, (p + 1) * psize)
                yp = y[:, t0:t1]
                mp = yp.max(axis=1)
                w = np.exp2(yp - mp[:, None])
                lp = w.sum(axis=1)
                m[b, g * r:(g + 1) * r, p] = mp
                l[b, g * r:(g + 1) * r, p] = lp
                o[b, g * r:(g + 1) * r, p] = (w @ V[t0:t1]) / lp[:, None]
    return m, l, o, nparts


def merge(m: np.ndarray, l: np.ndarray, o: np.ndarray, nparts: np.ndarray) -> np.ndarray:
    """Numerically stable merge of the partitions' split-softmax partials.

    For each (b, h) over its live partitions p < nparts[b]:
        M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p.
    A sequence with no live partition gives a zero row.
    """
    B, Hq, P, D = o.shape
    out = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(nparts[b])
        if n == 0:
            continue
        mb, lb, ob = m[b, :, :n], l[b, :, :n], o[b, :, :n]
        M = mb.max(axis=1, keepdims=True)
        w = np.exp2(mb - M) * lb                   # [Hq, n]
        out[b] = np.einsum("hp,hpd->hd", w, ob) / w.sum(axis=1)[:, None]
    return out
