"""Pins of oracle.chunk (multi-token queries with causal masking inside the
chunk: lucebox PR #555, Roadmap item 3; TensorFold PR #1418, What)
against things other than its own formula: the pure-Python brute-force
decode of test_oracle.py run on the sequence cut at each chunk token's
position, the reduction to a decode step at Tq = 1, and planted mistakes
in the causal limit that these pins catch."""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import synth
from test_oracle import brute_decode, rel_err


def _chunk_case(lens, Tq, **kw):
    """A decode case plus a chunk query q [B, Tq, Hq, D] (seeded)."""
    c = synth.make_case(lens, **kw)
    g = torch.Generator().manual_seed(kw.get("seed", 0) + 99)
    qc = torch.randn((c.B, Tq, c.Hq, c.D), generator=g)
    return c, qc


def _oracle_chunk(c, qc):
    kp, vp = c.k_pool.numpy().reshape(-1), c.v_pool.numpy().reshape(-1)
    return oracle.chunk(qc, kp, vp, c.table, c.seq_len, Hkv=c.Hkv, D=c.D, block_size=c.block_size,
                        k_fmt=c.k_fmt, v_fmt=c.v_fmt, nblocks=c.nblocks, max_blocks=c.max_blocks,
                        scale=c.scale)


def _brute_chunk(c, qc):
    """Row t of sequence b: the brute-force decode of the same pool with
    seq_len cut to L - Tq + t + 1 and query qc[b, t]."""
    B, Tq = qc.shape[:2]
    out = np.zeros(tuple(qc.shape), dtype=np.float64)
    for t in range(Tq):
        lens = [L - Tq + t + 1 if L else 0 for L in c.seq_lens]
        cut = dataclasses.replace(c, seq_lens=lens, seq_len=torch.tensor(lens, dtype=torch.int32),
                                  q=qc[:, t].contiguous())
        out[:, t] = brute_decode(cut)
    return out


@pytest.mark.parametrize("k_fmt,v_fmt", [("q4_0", "f16"), ("f16", "q8_0"), ("q8_0", "q4_0")])
def test_chunk_matches_brute_force_cut_sequences(k_fmt, v_fmt):
    c, qc = _chunk_case([11, 0, 6], 5, Hq=4, Hkv=2, D=32, block_size=4, k_fmt=k_fmt, v_fmt=v_fmt,
                        seed=5, junk="nan")
    got = _oracle_chunk(c, qc)
    ref = _brute_chunk(c, qc)
    assert rel_err(got, ref) <= 1e-13
    assert np.all(got[1] == 0.0)


def test_chunk_of_one_token_is_a_decode_step():
    c, qc = _chunk_case([37, 5, 64], 1, Hq=6, Hkv=2, D=32, block_size=4, k_fmt="q4_0",
                        v_fmt="q8_0", seed=9, junk="nan")
    got = _oracle_chunk(c, qc)[:, 0]
    ref = oracle.decode_case(dataclasses.replace(c, q=qc[:, 0].contiguous()))
    assert rel_err(got, ref) <= 1e-13


def test_first_chunk_token_sees_only_the_earlier_keys_and_itself():
    """Tq = L: token 0 attends to key 0 alone, so it returns V row 0 exactly."""
    c, qc = _chunk_case([6], 6, Hq=2, Hkv=1, D=32, block_size=4, k_fmt="f16", v_fmt="f16", seed=3,
                        junk="nan")
    got = _oracle_chunk(c, qc)
    v0 = oracle.dequant_rows(c.v_pool.numpy().reshape(-1, 64)[int(c.table[0, 0]) * 4][None], "f16", 32)[0]
    assert np.array_equal(got[0, 0, 0], v0) and np.array_equal(got[0, 0, 1], v0)


def test_chunk_longer_than_the_sequence_raises():
    c, qc = _chunk_case([3], 4, Hq=2, Hkv=1, D=32, block_size=4, seed=1)
    with pytest.raises(ValueError):
        _oracle_chunk(c, qc)


@pytest.mark.parametrize("shift", [-1, 1, "none"])
def test_pins_catch_a_wrong_causal_limit(shift):
    """Planted mistakes: the limit one key early or late, or no causal mask."""
    c, qc = _chunk_case([9, 7], 3, Hq=2, Hkv=1, D=32, block_size=4, k_fmt="q8_0", v_fmt="f16",
                        seed=21, junk="zero")
    ref = _brute_chunk(c, qc)

    def chunk_mut(q, k_pool, v_pool, table, seq_len, **kw):
        qn = np.asarray(q, dtype=np.float64)
        B, Tq, Hq, D = qn.shape
        out = np.zeros(qn.shape)
        for b in range(B):
            L = int(seq_len[b])
            for t in range(Tq):
                n = L if shift == "none" else min(L, max(1, L - Tq + t + 1 + shift))
                lens = torch.tensor([n if bb == b else 0 for bb in range(B)], dtype=torch.int32)
                q1 = torch.zeros((B, Hq, D), dtype=torch.float64)
                q1[b] = torch.as_tensor(qn[b, t])
                out[b, t] = oracle.decode(q1, k_pool, v_pool, table, lens, **kw)[b]
        return out

    kp, vp = c.k_pool.numpy().reshape(-1), c.v_pool.numpy().reshape(-1)
    got = chunk_mut(qc.numpy(), kp, vp, c.table, c.seq_len, Hkv=c.Hkv, D=c.D,
                    block_size=c.block_size, k_fmt=c.k_fmt, v_fmt=c.v_fmt, nblocks=c.nblocks,
                    max_blocks=c.max_blocks, scale=c.scale)
    assert rel_err(got, ref) > 1e-3
