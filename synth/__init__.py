"""Seeded synthetic inputs for paged GQA decode attention.

This module only *makes* inputs: query vectors, K/V values, their F16 / Q8_0 /
Q4_0 byte encodings laid into a paged pool, block tables and sequence lengths.
It holds none of the decode arithmetic (no dequantisation, no dot products, no
softmax), so both the fp64 oracle and the HIP path can consume what it makes.

Everything is torch, so the same code runs on the CPU (for tests without a GPU)
and on a GPU (to build the multi-GB pools of the long-context workloads in
seconds). Randomness comes from explicitly seeded torch.Generator objects.

Workload facts used here (all from the lucebox PR #555 page, "Benchmark
results" and "K/V capacity" sections, and the mlxcel issue #2153 page,
"Problem / Background"):
  * the pages' model attention shape: D=256, Hq=24, Hkv=4, blocks of 16 tokens;
  * K/V in F16, Q8_0 or Q4_0, K and V types independent;
  * ragged batches 128K + 7x8K with the blocks of all sequences interleaved
    randomly in one pool;
  * a Llama-style slab (Hkv=8, D=128, blocks of 32) that passes 2^32 elements.

Byte formats (the reading this project takes of "ggml Q8_0 / Q4_0"):
  * F16: IEEE binary16, little endian, D values per row.
  * Q8_0: D/32 blocks of 34 bytes: f16 scale d, then 32 signed int8 q;
    value = d * q.
  * Q4_0: D/32 blocks of 18 bytes: f16 scale d, then 16 bytes; byte j holds
    element j in its low nibble and element j+16 in its high nibble;
    value = (nibble - 8) * d.
A pool is uint8 [nblocks, block_size, Hkv, row_bytes]; one row is the D values
of one (token slot, kv head).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import torch

FORMATS = ("f16", "q8_0", "q4_0")
INT32_MAX = 2**31 - 1


def row_bytes(fmt: str, D: int) -> int:
    """Bytes of one encoded row of D values."""
    if fmt == "f16":
        return 2 * D
    if D % 32:
        raise ValueError(f"{fmt} needs D % 32 == 0, got D={D}")
    if fmt == "q8_0":
        return 34 * (D // 32)
    if fmt == "q4_0":
        return 18 * (D // 32)
    raise ValueError(f"unknown format {fmt!r}")


# ----------------------------------------------------------------------------
# encoders (values -> bytes). Quantisation shapes the inputs only: the oracle
# and the kernels both read back exactly the bytes written here.
# ----------------------------------------------------------------------------

def _round_half_away(x: torch.Tensor) -> torch.Tensor:
    return torch.sign(x) * torch.floor(torch.abs(x) + 0.5)


def encode(x: torch.Tensor, fmt: str) -> torch.Tensor:
    """Encode float32 values [..., D] into uint8 rows [..., row_bytes]."""
    x = x.float()
    D = x.shape[-1]
    lead = x.shape[:-1]
    if fmt == "f16":
        return x.half().contiguous().view(torch.uint8).reshape(*lead, 2 * D)
    nb = D // 32
    blk = x.reshape(*lead, nb, 32)
    if fmt == "q8_0":
        amax = blk.abs().amax(-1)
        d32 = amax / 127.0
        inv = torch.where(d32 > 0, 1.0 / torch.where(d32 > 0, d32, 1.0), 0.0)
        q = _round_half_away(blk * inv.unsqueeze(-1)).clamp(-127, 127).to(torch.int8)
        d16 = d32.half().contiguous().view(torch.uint8).reshape(*lead, nb, 2)
        out = torch.cat([d16, q.view(torch.uint8)], dim=-1)
        return out.reshape(*lead, 34 * nb)
    if fmt == "q4_0":
        idx = blk.abs().argmax(-1, keepdim=True)
        m = torch.gather(blk, -1, idx).squeeze(-1)  # signed value of max |x|
        d32 = m / -8.0
        inv = torch.where(d32 != 0, 1.0 / torch.where(d32 != 0, d32, 1.0), 0.0)
        q = (_round_half_away(blk * inv.unsqueeze(-1)) + 8).clamp(0, 15).to(torch.uint8)
        packed = q[..., :16] | (q[..., 16:] << 4)
        d16 = d32.half().contiguous().view(torch.uint8).reshape(*lead, nb, 2)
        out = torch.cat([d16, packed], dim=-1)
        return out.reshape(*lead, 18 * nb)
    raise ValueError(f"unknown format {fmt!r}")


# ----------------------------------------------------------------------------
# junk for dead slots and unused blocks
# ----------------------------------------------------------------------------

_F16_NAN = 0x7E00


def fill_junk(pool: torch.Tensor, fmt: str, D: int, mode: str, gen: Optional[torch.Generator]):
    """Overwrite every byte of `pool` ([..., row_bytes] uint8) with junk.

    mode 'nan'  : F16 rows all NaN; quantised rows get a NaN scale and random
                  quants.
    mode 'big'  : F16 rows +-30000; quantised rows get scale 30000 and random
                  quants (large but finite).
    mode 'zero' : all zero bytes (cheap, for timing runs).
    mode 'random': uniformly random bytes (may hold NaN/Inf patterns).
    """
    rb = pool.shape[-1]
    flat = pool.view(-1, rb)
    if mode == "zero":
        flat.zero_()
        return
    if mode == "random":
        flat.copy_(torch.randint(0, 256, flat.shape, generator=gen, dtype=torch.uint8,
                                 device=flat.device))
        return
    if mode not in ("nan", "big"):
        raise ValueError(mode)
    if fmt == "f16":
        if mode == "nan":
            val = torch.full((flat.shape[0], D), _F16_NAN, dtype=torch.int16, device=flat.device)
            flat.copy_(val.view(torch.uint8))
        else:
            sign = torch.randint(0, 2, (flat.shape[0], D), generator=gen, device=flat.device) * 2 - 1
            flat.copy_((sign.float() * 30000.0).half().view(torch.uint8))
        return
    nb = D // 32
    bsz = rb // nb
    blocks = flat.view(-1, nb, bsz)
    blocks.copy_(torch.randint(0, 256, blocks.shape, generator=gen, dtype=torch.uint8,
                               device=flat.device))
    scale = torch.full(blocks.shape[:2], float("nan") if mode == "nan" else 30000.0,
                       dtype=torch.float16, device=flat.device)
    blocks[..., 0:2].copy_(scale.contiguous().view(torch.uint8).view(*blocks.shape[:2], 2))


# ----------------------------------------------------------------------------
# block tables
# ----------------------------------------------------------------------------

def blocks_needed(L: int, bs: int) -> int:
    return (L + bs - 1) // bs


def make_table(seq_lens: Sequence[int], bs: int, nblocks: int, max_blocks: int,
               mode: str, gen: torch.Generator, split_block: int = 0) -> torch.Tensor:
    """Block table int32 [B, max_blocks]; entries past a sequence's live blocks
    hold INT32_MAX.

    mode 'shuffled'   : a seeded random permutation of all pool blocks; the
                        first sum(ceil(L_b/bs)) go to the sequences interleaved
                        (logical block j of every sequence before block j+1),
                        the rest stay unused junk.
    mode 'contiguous' : sequence b's block j is physical block b*max_blocks + j
                        (the layout the kernels assume when no table is given).
    mode 'split'      : half of every sequence's blocks are drawn from ids
                        >= split_block and half from below, in random order
                        (used to put half of each sequence past a 2^32-element
                        offset).
    """
    B = len(seq_lens)
    need = [blocks_needed(L, bs) for L in seq_lens]
    if max(need, default=0) > max_blocks:
        raise ValueError("sequence longer than max_blocks*bs")
    table = torch.full((B, max_blocks), INT32_MAX, dtype=torch.int32)
    if mode == "contiguous":
        if B * max_blocks > nblocks:
            raise ValueError("contiguous layout needs nblocks >= B*max_blocks")
        for b in range(B):
            table[b, : need[b]] = torch.arange(need[b], dtype=torch.int32) + b * max_blocks
        return table
    if mode == "shuffled":
        total = sum(need)
        if total > nblocks:
            raise ValueError("pool too small")
        perm = torch.randperm(nblocks, generator=gen)[:total].to(torch.int32)
        # interleaved order: all sequences' logical block j before block j+1
        bb = torch.cat([torch.full((n,), b, dtype=torch.int64) for b, n in enumerate(need)]
                       or [torch.zeros(0, dtype=torch.int64)])
        jj = torch.cat([torch.arange(n, dtype=torch.int64) for n in need]
                       or [torch.zeros(0, dtype=torch.int64)])
        order = torch.argsort(jj * B + bb)
        table[bb[order], jj[order]] = perm
        return table
    if mode == "split":
        hi_pool = torch.randperm(nblocks - split_block, generator=gen).to(torch.int32) + split_block
        lo_pool = torch.randperm(split_block, generator=gen).to(torch.int32)
        hk = lk = 0
        for b in range(B):
            n = need[b]
            nh = n // 2
            ids = torch.cat([hi_pool[hk:hk + nh], lo_pool[lk:lk + n - nh]])
            if ids.numel() != n:
                raise ValueError("pool too small for split table")
            hk += nh
            lk += n - nh
            ids = ids[torch.randperm(n, generator=gen)]
            table[b, :n] = ids
        return table
    raise ValueError(mode)


# ----------------------------------------------------------------------------
# one decode-step case
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class Case:
    B: int
    Hq: int
    Hkv: int
    D: int
    block_size: int
    nblocks: int
    max_blocks: int
    k_fmt: str
    v_fmt: str
    seq_lens: List[int]
    q: torch.Tensor            # float32 [B, Hq, D]
    k_pool: torch.Tensor       # uint8 [nblocks, bs, Hkv, row_bytes(k_fmt)]
    v_pool: torch.Tensor       # uint8 [nblocks, bs, Hkv, row_bytes(v_fmt)]
    table: torch.Tensor        # int32 [B, max_blocks]
    seq_len: torch.Tensor      # int32 [B]
    scale: float
    seed: int

    @property
    def live_tokens(self) -> int:
        return sum(self.seq_lens)

    def to(self, device) -> "Case":
        return dataclasses.replace(
            self, q=self.q.to(device), k_pool=self.k_pool.to(device),
            v_pool=self.v_pool.to(device), table=self.table.to(device),
            seq_len=self.seq_len.to(device))


def make_case(seq_lens: Sequence[int], *, Hq: int = 24, Hkv: int = 4, D: int = 256,
              block_size: int = 16, k_fmt: str = "f16", v_fmt: str = "f16",
              nblocks: Optional[int] = None, max_blocks: Optional[int] = None,
              table_mode: str = "shuffled", junk: str = "nan", seed: int = 0,
              device="cpu", split_block: int = 0, scale: Optional[float] = None,
              value_std: float = 1.0, q_std: float = 1.0, chunk_tokens: int = 1 << 16) -> Case:
    """Build one seeded decode-step case.

    q ~ N(0, q_std^2) fp32; live K and V values ~ N(0, value_std^2) then
    encoded in k_fmt / v_fmt. The pool defaults to 1.25x the used blocks (rounded up);
    every unused block and every dead slot of a partly filled block holds junk.
    """
    seq_lens = [int(L) for L in seq_lens]
    B = len(seq_lens)
    bs = block_size
    need = [blocks_needed(L, bs) for L in seq_lens]
    if max_blocks is None:
        max_blocks = max(max(need, default=1), 1)
    if nblocks is None:
        if table_mode == "contiguous":
            nblocks = B * max_blocks
        else:
            nblocks = max(int(math.ceil(sum(need) * 1.25)), 1)
    gen_cpu = torch.Generator().manual_seed(seed)
    dev = torch.device(device)
    gen_dev = torch.Generator(device=dev).manual_seed(seed + 1)
    table = make_table(seq_lens, bs, nblocks, max_blocks, table_mode, gen_cpu, split_block)
    q = torch.randn((B, Hq, D), generator=gen_dev, device=dev, dtype=torch.float32) * q_std

    def build_pool(fmt: str, salt: int) -> torch.Tensor:
        rb = row_bytes(fmt, D)
        pool = torch.empty((nblocks, bs, Hkv, rb), dtype=torch.uint8, device=dev)
        gj = torch.Generator(device=dev).manual_seed(seed * 7 + salt)
        fill_junk(pool, fmt, D, junk, gj)
        flat = pool.view(nblocks * bs, Hkv, rb)
        gv = torch.Generator(device=dev).manual_seed(seed * 131 + salt)
        for b, L in enumerate(seq_lens):
            if L == 0:
                continue
            ids = table[b, : need[b]].to(torch.int64).to(dev)
            for t0 in range(0, L, chunk_tokens):
                t1 = min(L, t0 + chunk_tokens)
                t = torch.arange(t0, t1, device=dev, dtype=torch.int64)
                slot = ids[t // bs] * bs + (t % bs)
                vals = torch.randn((t1 - t0, Hkv, D), generator=gv, device=dev) * value_std
                flat.index_copy_(0, slot, encode(vals, fmt))
        return pool

    k_pool = build_pool(k_fmt, 11)
    v_pool = build_pool(v_fmt, 23)
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    return Case(B=B, Hq=Hq, Hkv=Hkv, D=D, block_size=bs, nblocks=nblocks,
                max_blocks=max_blocks, k_fmt=k_fmt, v_fmt=v_fmt, seq_lens=seq_lens,
                q=q, k_pool=k_pool, v_pool=v_pool, table=table.to(dev),
                seq_len=torch.tensor(seq_lens, dtype=torch.int32, device=dev),
                scale=scale, seed=seed)


def contiguous_copy(case: Case) -> Case:
    """The same live rows re-laid so sequence b's block j is physical block
    b*max_blocks + j (the layout used when the kernels get no block table)."""
    bs, B, mb = case.block_size, case.B, case.max_blocks
    dev = case.k_pool.device

    def relay(pool: torch.Tensor) -> torch.Tensor:
        out = torch.zeros((B * mb,) + tuple(pool.shape[1:]), dtype=torch.uint8, device=dev)
        for b, L in enumerate(case.seq_lens):
            n = blocks_needed(L, bs)
            if n:
                ids = case.table[b, :n].to(torch.int64).to(dev)
                out[b * mb: b * mb + n] = pool[ids]
        return out

    table = make_table(case.seq_lens, bs, B * mb, mb, "contiguous", torch.Generator())
    return dataclasses.replace(case, k_pool=relay(case.k_pool), v_pool=relay(case.v_pool),
                               nblocks=B * mb, table=table.to(case.table.device))


# ----------------------------------------------------------------------------
# named workloads (sizes from the pages' benchmarks)
# ----------------------------------------------------------------------------

def workload(name: str, *, B: int = 8, L: int = 4096, seed: int = 1000, device="cpu",
             junk: str = "nan") -> Case:
    """Named decode-step workloads.

    tiny_f16     : B=1, L=200 (last block partly filled), 32-block pool, F16.
    uniform_q8_0 : B sequences of L tokens, Q8_0 K/V (L=4096 in the pages' 4K row).
    uniform_q4_0 : B sequences of L tokens, Q4_0 K/V (L in {32768, 131072}).
    uniform_f16  : B sequences of L tokens, F16 K/V (D=256, Hq=24, Hkv=4).
    ragged_q4_0  : 131072 + 7 x 8192 tokens, blocks interleaved in one pool.
    ragged_small_q4_0 : 4096 + 7 x 256 tokens.
    uniform_q4_0_d128 : B sequences of L tokens, Q4_0 K/V in the D=128 shape
                   of slab_f16 (Hq=32, Hkv=8, blocks of 32).
    slab_f16     : D=128, Hq=32, Hkv=8, blocks of 32, 139,264-block pool
                   (more than 2^32 elements per side), B=8 x 65536 tokens with
                   half of each sequence's blocks past element 2^32.
    """
    if name == "tiny_f16":
        return make_case([200], k_fmt="f16", v_fmt="f16", nblocks=32, seed=seed,
                         device=device, junk=junk)
    if name == "uniform_q8_0":
        return make_case([L] * B, k_fmt="q8_0", v_fmt="q8_0", seed=seed, device=device, junk=junk)
    if name == "uniform_q4_0":
        return make_case([L] * B, k_fmt="q4_0", v_fmt="q4_0", seed=seed, device=device, junk=junk)
    if name == "uniform_q4_0_d128":
        return make_case([L] * B, Hq=32, Hkv=8, D=128, block_size=32, k_fmt="q4_0", v_fmt="q4_0",
                         seed=seed, device=device, junk=junk)
    if name == "uniform_f16":
        return make_case([L] * B, k_fmt="f16", v_fmt="f16", seed=seed, device=device, junk=junk)
    if name == "ragged_q4_0":
        return make_case([131072] + [8192] * 7, k_fmt="q4_0", v_fmt="q4_0", seed=seed,
                         device=device, junk=junk)
    if name == "ragged_small_q4_0":
        return make_case([4096] + [256] * 7, k_fmt="q4_0", v_fmt="q4_0", seed=seed,
                         device=device, junk=junk)
    if name == "slab_f16":
        return make_case([65536] * 8, Hq=32, Hkv=8, D=128, block_size=32, k_fmt="f16",
                         v_fmt="f16", nblocks=139264, table_mode="split", split_block=131072,
                         seed=seed, device=device, junk=junk)
    raise ValueError(name)
