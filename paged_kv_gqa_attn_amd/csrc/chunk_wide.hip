// Multi-token queries with many query rows per kv head (prefill chunks): the
// wide-tile kernel.
//
// What it computes is what chunk.hip computes (lucebox PR #555, Roadmap item
// 3: several query tokens per sequence attend over the K/V already in the
// pool, causally inside the chunk; TensorFold PR #1418, What: paged
// prompt-chunk attention): chunk token t of sequence b (length L) sits at
// position L - Tq + t and attends to the keys at positions 0 .. L - Tq + t of
// kv head g = h / r, with the Tq*r query rows of a kv head (row n = t*r +
// h - g*r) sharing every converted K/V tile.
//
// How it maps onto gfx950 (a prefill chunk is MFMA-bound: 4*D flops per
// visible query row and key):
//   * 32x32x16 f16 MFMAs. Scores come as S^T = K Q^T, 32 keys by 32 query
//     rows per MFMA, with the rows' Q^T held in registers as the B operand;
//     the S^T accumulators are, lane for lane, the B operand P^T of
//     O^T += V^T P^T once converted to f16 (the V^T operand lists its keys
//     in the accumulators' order), so P never moves between lanes. Each lane
//     holds one query row (lanes l and l+32 split its keys), so the row max
//     is 15 in-lane max operations and one lane swap. Every operand the
//     MFMAs read from LDS serves 32 rows: 1 KB per 32x32x16 MFMA, twice the
//     rows per operand byte of the 16x16 tiles of chunk.hip.
//   * A workgroup takes a unit (sequence b, key partition p, kv head g, 128
//     query rows). The raw K/V rows of each 32-key tile arrive by DMA in an
//     LDS ring, the 16 rows of a group of kv head g back to back, through
//     the block table (64-bit row addresses, mlxcel issue #2153); a group
//     that crosses the end of the keys gets a buffer resource over its live
//     rows, so junk slots land as zeros. Every tile is converted to f16 once
//     per workgroup into LDS in MFMA operand order, one barrier per tile.
//   * Paired form (chunk_pair_kernel; every type pair at D = 128, all but
//     F16/F16, F16/Q8_0 and Q8_0/F16 at D = 256): eight waves, two per SIMD.
//     Score wave w holds the Q^T of rows 32w .. 32w+31 and per tile kt runs
//     the softmax of kt, the scores of kt+1 and the PV of the first half of
//     the d-tiles, leaving its P^T operands and rescale flags in LDS; the
//     conversion wave on its SIMD DMAs and converts one side (K or V) of one
//     16-key group of every tile, from registers loaded a tile ahead, and
//     runs the PV of the second half of the d-tiles for kt-1. No AGPRs (the
//     compiler would split the 256 registers of two waves per SIMD evenly
//     between VGPRs and AGPRs); one instantiation of the body per role.
//   * Four-wave form (chunk_wide_kernel; F16/F16, F16/Q8_0 and Q8_0/F16 at
//     D = 256, whose raw tiles leave no LDS for the paired form's ring): wave
//     w owns rows 32w .. 32w+31, holds its Q^T (D/4 registers) and O^T
//     (D/2) in AGPRs at one workgroup per CU with 512 registers per lane, and
//     converts a quarter of each tile; the score MFMAs of kt+1 alternate with
//     the PV MFMAs of kt, operand reads streaming ahead of them.
//   * Causal limit per row; tiles past the workgroup's last row are not
//     read and only tiles that cross some row's limit are masked. Partials
//     (normalised binary16 o, fp32 m and l) use the decode layout with Tq*Hq
//     rows per sequence and go through the same merge.
#include <type_traits>

#include "decode_common.h"
#include "lds_ring.h"
#include "wide_plan.h"

namespace pa {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kWThreads = 256;
constexpr int kWRows = 128;     // query rows per workgroup (32 per wave)
constexpr int kWNid = 512;      // block ids staged per segment of a partition
constexpr int kWTile = 32;      // keys per tile

// 32x32x16 f16 -> f32: A lane l (row l%32, k 8*(l/32)+i), B lane l (col l%32,
// k 8*(l/32)+i), C lane l register r (row 8*(r/4) + 4*(l/32) + r%4, col l%32).
__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// Wait states after the last MFMAs of a loop, before a block after it reads
// their results (see mfma_settle), kept in place by a scheduling barrier.
// Inside the loop every MFMA result is read an iteration after the MFMA.
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// s_waitcnt vmcnt(n) lgkmcnt(0), then the workgroup barrier: the wave's DMA
// but the last n instructions has landed and its LDS writes are done, so
// every wave reads them after the barrier (n wave-uniform; above 15 it waits
// for more than needed, which is safe).
__device__ __forceinline__ void wait_all_then_barrier(int n) {
#define PA_WAIT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ") lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  switch (n < 15 ? n : 15) {
    PA_WAIT_CASE(0) PA_WAIT_CASE(1) PA_WAIT_CASE(2) PA_WAIT_CASE(3) PA_WAIT_CASE(4)
    PA_WAIT_CASE(5) PA_WAIT_CASE(6) PA_WAIT_CASE(7) PA_WAIT_CASE(8) PA_WAIT_CASE(9)
    PA_WAIT_CASE(10) PA_WAIT_CASE(11) PA_WAIT_CASE(12) PA_WAIT_CASE(13) PA_WAIT_CASE(14)
    default: asm volatile("s_waitcnt vmcnt(15) lgkmcnt(0)\n\ts_barrier" ::: "memory"); break;
  }
#undef PA_WAIT_CASE
}

// s_waitcnt vmcnt(n): the wave's own vector memory operations but the last n
// have completed (n wave-uniform; above 15 it waits for more than needed).
__device__ __forceinline__ void wait_vm(int n) {
#define PA_WAIT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")" ::: "memory"); break;
  switch (n < 15 ? n : 15) {
    PA_WAIT_CASE(0) PA_WAIT_CASE(1) PA_WAIT_CASE(2) PA_WAIT_CASE(3) PA_WAIT_CASE(4)
    PA_WAIT_CASE(5) PA_WAIT_CASE(6) PA_WAIT_CASE(7) PA_WAIT_CASE(8) PA_WAIT_CASE(9)
    PA_WAIT_CASE(10) PA_WAIT_CASE(11) PA_WAIT_CASE(12) PA_WAIT_CASE(13) PA_WAIT_CASE(14)
    default: asm volatile("s_waitcnt vmcnt(15)" ::: "memory"); break;
  }
#undef PA_WAIT_CASE
}
// The wave's LDS operations have completed.
__device__ __forceinline__ void lds_drain() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Key of register r of an S^T accumulator, within its 32-key tile, for lane half h.
__host__ __device__ constexpr int skey(int r, int h) { return 8 * (r / 4) + 4 * h + r % 4; }
// Key of slot e of a P^T (and V^T) operand half of k-step t: the accumulator
// registers 8t .. 8t+7 in order.
__host__ __device__ constexpr int pkey(int t, int h, int e) { return skey(8 * t + e, h); }

// Byte-pair conversion order (bytes 0, 2 then 1, 3 of each dword).
__host__ __device__ constexpr int word_order(int s) { return (s & 4) + ((s & 1) << 1) + ((s >> 1) & 1); }

// v_perm_b32 selector for bytes [s, s+4) of {hi:lo}, s in 0..4.
__device__ __forceinline__ uint32_t shift_sel(uint32_t s) { return 0x03020100u + s * 0x01010101u; }

// ===========================================================================
// K formats: the A operand of S^T = K Q^T. Lane l holds key l%32 of the tile
// and, for step c (0 .. D/16-1), head positions kd(c, l/32, 0..7). Every wave
// converts a quarter of a tile's K: 8 keys, its lane kk + 8q the operand
// slots of key kk for half h = q & 1 and the CQ = D/64 steps of quarter
// cq = q >> 1 (c = cq*CQ + cc). `load` reads the lane's bytes of its staged
// row into kWords dwords, `op` converts step cc.
// ===========================================================================
template <int KT, int D> struct WK;

// Every format also converts a run of NS steps c0 .. c0+NS-1 for one lane
// (`loadn`, `opn`; c0 and NS even), the unit of the paired form's K waves.
template <int D> struct WK<kF16, D> {
  static constexpr int CQ = D / 64;
  template <int NS> static constexpr int words() { return 4 * NS; }
  static constexpr int kWords = words<CQ>();
  __host__ __device__ static constexpr int kd(int c, int h, int s) { return 16 * c + 8 * h + s; }
  template <int NS>
  __device__ static void loadn(uint32_t* w, const unsigned char* row, int h, int c0) {
#pragma unroll
    for (int cc = 0; cc < NS; ++cc) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(row + 32 * (c0 + cc) + 16 * h);
#pragma unroll
      for (int k = 0; k < 4; ++k) w[4 * cc + k] = a[k];
    }
  }
  template <int NS>
  __device__ static f16x8 opn(const uint32_t* w, int cc, int, uint32_t) {
    return bitcast<f16x8>(u32x4{w[4 * cc], w[4 * cc + 1], w[4 * cc + 2], w[4 * cc + 3]});
  }
  __device__ static void load(uint32_t* w, const unsigned char* row, int h, int cq) { loadn<CQ>(w, row, h, cq * CQ); }
  __device__ static f16x8 op(const uint32_t* w, int cc, int cq, uint32_t mg) { return opn<CQ>(w, cc, cq * CQ, mg); }
};

// Quantised K: step c = 2*bk + x covers ggml block bk, quant bytes [16x + 8h,
// +8) for Q8_0, nibble x of quant bytes [8h, +8) for Q4_0, in word_order.
// The 8 bytes start 2 bytes into a dword for even bk: three dwords from the
// 4-aligned base below them are read and realigned (v_alignbyte).
template <int D> struct WK<kQ4_0, D> {
  static constexpr int CQ = D / 64;
  template <int NS> static constexpr int words() { return 4 * (NS / 2); }   // block j: w[3j..3j+2], scale w[3NB + j]
  static constexpr int kWords = words<CQ>();
  __host__ __device__ static constexpr int kd(int c, int h, int s) {
    return 32 * (c / 2) + 16 * (c % 2) + 8 * h + word_order(s);
  }
  template <int NS>
  __device__ static void loadn(uint32_t* w, const unsigned char* row, int h, int c0) {
    constexpr int NB = NS / 2;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int bk = c0 / 2 + j;
      const uint32_t* q = reinterpret_cast<const uint32_t*>(row + ((18 * bk + 2 + 8 * h) & ~3));
      w[3 * j] = q[0];
      w[3 * j + 1] = q[1];
      w[3 * j + 2] = q[2];
      w[3 * NB + j] = *reinterpret_cast<const uint16_t*>(row + 18 * bk);
    }
  }
  template <int NS>
  __device__ static f16x8 opn(const uint32_t* w, int cc, int c0, uint32_t mg) {
    constexpr int NB = NS / 2;
    const int j = cc / 2, x = cc % 2;
    const uint32_t sh = ((c0 / 2 + j) & 1) ? 0u : 2u;
    uint32_t w0 = align_bytes(w[3 * j + 1], w[3 * j], sh);
    uint32_t w1 = align_bytes(w[3 * j + 2], w[3 * j + 1], sh);
    if (x) { w0 >>= 4; w1 >>= 4; }
    const f16x2 d2 = splat2(bitcast<f16>(uint16_t(w[3 * NB + j])));
    return pack8(nib_pair_to_f16(w0, d2, mg), nib_pair_to_f16(w0 >> 8, d2, mg),
                 nib_pair_to_f16(w1, d2, mg), nib_pair_to_f16(w1 >> 8, d2, mg));
  }
  __device__ static void load(uint32_t* w, const unsigned char* row, int h, int cq) { loadn<CQ>(w, row, h, cq * CQ); }
  __device__ static f16x8 op(const uint32_t* w, int cc, int cq, uint32_t mg) { return opn<CQ>(w, cc, cq * CQ, mg); }
};

template <int D> struct WK<kQ8_0, D> {
  static constexpr int CQ = D / 64;
  template <int NS> static constexpr int words() { return 7 * (NS / 2); }   // chunk x of block j: w[6j + 3x ..], scale w[6NB + j]
  static constexpr int kWords = words<CQ>();
  __host__ __device__ static constexpr int kd(int c, int h, int s) {
    return 32 * (c / 2) + 16 * (c % 2) + 8 * h + word_order(s);
  }
  template <int NS>
  __device__ static void loadn(uint32_t* w, const unsigned char* row, int h, int c0) {
    constexpr int NB = NS / 2;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int bk = c0 / 2 + j;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const uint32_t* q = reinterpret_cast<const uint32_t*>(row + ((34 * bk + 2 + 16 * x + 8 * h) & ~3));
        w[6 * j + 3 * x] = q[0];
        w[6 * j + 3 * x + 1] = q[1];
        w[6 * j + 3 * x + 2] = q[2];
      }
      w[6 * NB + j] = *reinterpret_cast<const uint16_t*>(row + 34 * bk);
    }
  }
  template <int NS>
  __device__ static f16x8 opn(const uint32_t* w, int cc, int c0, uint32_t mg) {
    constexpr int NB = NS / 2;
    const int j = cc / 2, o = 6 * j + 3 * (cc % 2);
    const uint32_t sh = ((c0 / 2 + j) & 1) ? 0u : 2u;
    const uint32_t u0 = align_bytes(w[o + 1], w[o], sh);
    const uint32_t u1 = align_bytes(w[o + 2], w[o + 1], sh);
    const f16x2 d2 = splat2(bitcast<f16>(uint16_t(w[6 * NB + j])));
    const uint32_t a = u0 ^ 0x80808080u, b = u1 ^ 0x80808080u;
    return pack8(i8pair_to_f16(a, d2, mg), i8pair_to_f16(a >> 8, d2, mg), i8pair_to_f16(b, d2, mg),
                 i8pair_to_f16(b >> 8, d2, mg));
  }
  __device__ static void load(uint32_t* w, const unsigned char* row, int h, int cq) { loadn<CQ>(w, row, h, cq * CQ); }
  __device__ static f16x8 op(const uint32_t* w, int cc, int cq, uint32_t mg) { return opn<CQ>(w, cc, cq * CQ, mg); }
};

// ===========================================================================
// V formats: the A operand of O^T += V^T P^T. Lane l = i + 32h holds, for
// k-step t (16-key group t of the tile) and d-tile dt (0 .. D/32-1), head
// position vd(dt, i) of keys pkey(t, h, 0..7). Every wave converts a quarter
// of a tile's V: of one 16-key group, the keys pkey(t, h, 4k .. 4k+3) of
// every operand lane (k = 0 or 1), written as the f16x4 half k of the lane's
// f16x8. `load` reads those 4 keys' bytes from the staged rows (r0: the row
// of the first, pkey(t, h, 4k); the others pkey(0, 0, e) rows on) into
// kWords dwords, `prep` realigns them in place, `op` converts d-tile dt.
// dnext(dt) is the d-tile holding position vd(dt, i) + 1 (for every i), or
// -1: the pairs of adjacent positions the binary16 partial rows are stored by.
// ===========================================================================
template <int VT, int D> struct WV;

template <int D> struct WV<kF16, D> {
  static constexpr int NDT = D / 32;
  static constexpr int NW = NDT / 2;          // dwords of a key the lane reads
  static constexpr int kWords = 4 * NW;
  struct Lane { uint32_t voff; };
  __host__ __device__ static constexpr int vd(int dt, int i) { return NDT * i + dt; }
  __host__ __device__ static constexpr int dnext(int dt) { return dt % 2 ? -1 : dt + 1; }
  __device__ static Lane lane(int i) { return Lane{2u * NDT * i}; }
  __device__ static void load(uint32_t* w, const unsigned char* r0, const Lane& L) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned char* p = r0 + pkey(0, 0, e) * (2 * D) + L.voff;
      if constexpr (NW == 4) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int k = 0; k < 4; ++k) w[4 * e + k] = a[k];
      } else {
        const u32x2 a = *reinterpret_cast<const u32x2*>(p);
        w[2 * e] = a[0];
        w[2 * e + 1] = a[1];
      }
    }
  }
  __device__ static void prep(uint32_t*, const Lane&) {}
  __device__ static f16x4 op(const uint32_t* w, const Lane&, int dt, uint32_t) {
    const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;
    u32x2 o;
#pragma unroll
    for (int q = 0; q < 2; ++q) o[q] = perm_bytes(w[NW * (2 * q + 1) + dt / 2], w[NW * (2 * q) + dt / 2], sel);
    return bitcast<f16x4>(o);
  }
};

// Q4_0 V. D = 256: lane row i = 4bk + c (block bk, quant dword c), d-tile
// dt = 2b + x (byte b of the dword, nibble x): position 32bk + 16x + 4c + b.
// D = 128: i = 16x + 4bk + c, dt = b, the same position. Key e: window
// w[2e], w[2e+1], scale w[8 + e].
template <int D> struct WV<kQ4_0, D> {
  static constexpr int NDT = D / 32;
  static constexpr int RB = 18 * (D / 32);
  static constexpr int kWords = 12;
  struct Lane { uint32_t voff, sel, doff, xs; };
  __host__ __device__ static constexpr int vbk(int i) { return D == 256 ? i / 4 : (i / 4) % 4; }
  __host__ __device__ static constexpr int vx(int dt, int i) { return D == 256 ? dt % 2 : i / 16; }
  __host__ __device__ static constexpr int vb(int dt) { return D == 256 ? dt / 2 : dt; }
  __host__ __device__ static constexpr int vd(int dt, int i) {
    return 32 * vbk(i) + 16 * vx(dt, i) + 4 * (i % 4) + vb(dt);
  }
  __host__ __device__ static constexpr int dnext(int dt) {
    return D == 256 ? ((dt / 2) % 2 ? -1 : dt + 2) : (dt % 2 ? -1 : dt + 1);
  }
  // quant dword c of block bk at o = 18bk + 2 + 4c; two dwords are read from
  // the 4-aligned base at or below o (kept inside the row) and the dword
  // picked out with a byte permute
  __device__ static Lane lane(int i) {
    const uint32_t o = 18u * vbk(i) + 2u + 4u * (i % 4);
    const uint32_t base = min(o & ~3u, uint32_t(RB - 8));
    return Lane{base, shift_sel(o - base), 18u * vbk(i), D == 256 ? 0u : 4u * uint32_t(i / 16)};
  }
  __device__ static void load(uint32_t* w, const unsigned char* r0, const Lane& L) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned char* row = r0 + pkey(0, 0, e) * RB;
      const uint32_t* q = reinterpret_cast<const uint32_t*>(row + L.voff);
      w[2 * e] = q[0];
      w[2 * e + 1] = q[1];
      w[8 + e] = *reinterpret_cast<const uint16_t*>(row + L.doff);
    }
  }
  // the quant dword of key e into w[2e]; scale pairs of keys (2k, 2k+1) into w[8 + 2k]
  __device__ static void prep(uint32_t* w, const Lane& L) {
#pragma unroll
    for (int e = 0; e < 4; ++e) w[2 * e] = perm_bytes(w[2 * e + 1], w[2 * e], L.sel);
#pragma unroll
    for (int k = 0; k < 2; ++k) w[8 + 2 * k] = (w[8 + 2 * k] & 0xFFFFu) | (w[9 + 2 * k] << 16);
  }
  __device__ static f16x4 op(const uint32_t* w, const Lane& L, int dt, uint32_t mg) {
    const uint32_t b = uint32_t(vb(dt));
    const uint32_t sel = b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);
    f16x2 o[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      uint32_t y = perm_bytes(w[4 * k + 2], w[4 * k], sel);
      if constexpr (D == 256) {
        if (dt % 2) y >>= 4;
      } else {
        y >>= L.xs;
      }
      o[k] = nib_pair_to_f16(y, bitcast<f16x2>(w[8 + 2 * k]), mg);
    }
    return f16x4{o[0][0], o[0][1], o[1][0], o[1][1]};
  }
};

// Q8_0 V. D = 256: lane row i = 4bk + c, quant bytes [8c, +8) of block bk,
// d-tile dt = byte: position 32bk + 8c + dt. D = 128: i = 8bk + c, bytes
// [4c, +4), position 32bk + 4c + dt. Key e: window w[NWIN*e ..], scale
// w[4*NWIN + e].
template <int D> struct WV<kQ8_0, D> {
  static constexpr int NDT = D / 32;
  static constexpr int RB = 34 * (D / 32);
  static constexpr int QB = NDT;                // quant bytes per key and lane
  static constexpr int NWIN = QB / 4 + 1;       // window dwords
  static constexpr int SC = 4 * NWIN;           // first scale word
  static constexpr int kWords = 4 * NWIN + 4;
  struct Lane { uint32_t voff, sel, doff; };
  __host__ __device__ static constexpr int vbk(int i) { return D == 256 ? i / 4 : i / 8; }
  __host__ __device__ static constexpr int vc(int i) { return D == 256 ? i % 4 : i % 8; }
  __host__ __device__ static constexpr int vd(int dt, int i) { return 32 * vbk(i) + QB * vc(i) + dt; }
  __host__ __device__ static constexpr int dnext(int dt) { return dt % 2 ? -1 : dt + 1; }
  __device__ static Lane lane(int i) {
    const uint32_t o = 34u * vbk(i) + 2u + uint32_t(QB) * vc(i);
    const uint32_t base = min(o & ~3u, uint32_t(RB - 4 * NWIN));
    return Lane{base, shift_sel(o - base), 34u * vbk(i)};
  }
  __device__ static void load(uint32_t* w, const unsigned char* r0, const Lane& L) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const unsigned char* row = r0 + pkey(0, 0, e) * RB;
      const uint32_t* q = reinterpret_cast<const uint32_t*>(row + L.voff);
#pragma unroll
      for (int k = 0; k < NWIN; ++k) w[NWIN * e + k] = q[k];
      w[SC + e] = *reinterpret_cast<const uint16_t*>(row + L.doff);
    }
  }
  // quant dwords of key e into w[NWIN*e + k], k < QB/4; scale pairs into w[SC + 2k]
  __device__ static void prep(uint32_t* w, const Lane& L) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int k = 0; k < QB / 4; ++k) w[NWIN * e + k] = perm_bytes(w[NWIN * e + k + 1], w[NWIN * e + k], L.sel);
#pragma unroll
    for (int k = 0; k < 2; ++k) w[SC + 2 * k] = (w[SC + 2 * k] & 0xFFFFu) | (w[SC + 2 * k + 1] << 16);
  }
  __device__ static f16x4 op(const uint32_t* w, const Lane&, int dt, uint32_t) {
    const uint32_t b = uint32_t(dt % 4);
    const uint32_t sel = b | (0x0Cu << 8) | ((4u + b) << 16) | (0x0Cu << 24);
    f16x2 o[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const uint32_t y =
          perm_bytes(w[NWIN * (2 * k + 1) + dt / 4], w[NWIN * (2 * k) + dt / 4], sel) ^ 0x64806480u;
      o[k] = (bitcast<f16x2>(y) - f16x2{1152.0f16, 1152.0f16}) * bitcast<f16x2>(w[SC + 2 * k]);
    }
    return f16x4{o[0][0], o[0][1], o[1][0], o[1][1]};
  }
};

template <typename VF>
__host__ __device__ constexpr bool pairs_ok() {
  for (int dt = 0; dt < VF::NDT; ++dt) {
    const int n = VF::dnext(dt);
    for (int i = 0; i < 32; ++i) {
      if (n >= 0 && (VF::vd(n, i) != VF::vd(dt, i) + 1 || VF::vd(dt, i) % 2)) return false;
    }
  }
  int seen = 0;
  for (int dt = 0; dt < VF::NDT; ++dt) seen += VF::dnext(dt) >= 0 ? 2 : 0;
  return seen == VF::NDT;
}

// Staging of raw K/V rows: a side (K or V) of one 16-key group is DMA'd as
// NI instructions of 64 chunks of CB bytes (16, or 4 where a row is not a
// whole number of 16-byte chunks), the 16 rows of kv head g back to back.
template <int T, int D> struct Stage {
  static constexpr int RB = row_bytes_of(T, D);
  static constexpr int CB = RB % 16 == 0 ? 16 : 4;
  static constexpr int CPR = RB / CB;                 // chunks per row
  static constexpr int NI = (16 * CPR + 63) / 64;     // instructions per group
  static constexpr int GB = NI * 64 * CB;             // LDS bytes per group
  // pool offset (from the group's first row) of chunk 64*j + lane, or past
  // any resource (reads as 0) for the instruction's unused lanes
  __device__ static uint32_t off(int j, int lane, uint32_t stride) {
    const int c = 64 * j + lane;
    const int row = c / CPR;
    return c < 16 * CPR ? uint32_t(row) * stride + uint32_t(c - row * CPR) * CB : 0x80000000u;
  }
};

template <int KT, int VT, int D> struct WideLds {
  using SK = Stage<KT, D>;
  using SV = Stage<VT, D>;
  static constexpr int KBUF = (D / 16) * 64 * 16;          // K operands of a tile
  static constexpr int VBUF = 2 * (D / 32) * 64 * 16;      // V operands of a tile
  static constexpr int SLOT = 2 * (SK::GB + SV::GB);       // raw rows of a tile
  static constexpr int IDS = 4 * (kWNid + 4);              // block ids of a segment
  static constexpr int OPS = 2 * KBUF + 3 * VBUF;
  // raw tiles in the ring: up to four (RR-1 in flight while one is
  // converted), as many as fit the 160 KB of a CU
  static constexpr int RR = OPS + 4 * SLOT + IDS <= 160 * 1024   ? 4
                            : OPS + 3 * SLOT + IDS <= 160 * 1024 ? 3
                                                                 : 2;
  static constexpr int RAW = OPS;
  static constexpr int ID0 = RAW + RR * SLOT;
  static constexpr int BYTES = ID0 + IDS;
  static constexpr int NT = 2 * (SK::NI + SV::NI);          // DMA instructions per tile
  static_assert(BYTES <= 160 * 1024, "LDS of one CU");
};

// One DMA instruction: lane l's CB bytes at pool offset voff land at LDS
// byte dst + CB*l (cached loads: the tiles are read again by the other
// query-row blocks of the kv head).
template <int CB>
__device__ __forceinline__ void dma_lds(rsrc_t R, uint32_t dst, uint32_t voff) {
  if constexpr (CB == 16)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R, (lds_ptr_t)(g_lds + dst), 16, voff, 0, 0, 0);
  else
    __builtin_amdgcn_raw_ptr_buffer_load_lds(R, (lds_ptr_t)(g_lds + dst), 4, voff, 0, 0, 0);
}

template <int KT, int VT, int D>
__global__ void __launch_bounds__(kWThreads, 1) chunk_wide_kernel(const ChunkArgs a) {
  using KF = WK<KT, D>;
  using VF = WV<VT, D>;
  using LY = WideLds<KT, VT, D>;
  using SK = typename LY::SK;
  using SV = typename LY::SV;
  static_assert(pairs_ok<VF>(), "d-tile pairs cover adjacent even/odd positions");
  constexpr int C = D / 16;                       // score MFMA steps
  constexpr int CQ = D / 64;                      // steps per converting lane
  constexpr int NDT = D / 32;                     // PV d-tiles
  constexpr int KBUF = LY::KBUF, VBUF = LY::VBUF, RR = LY::RR;
  constexpr int KRB = SK::RB, VRB = SV::RB;

  unsigned char* const kbuf = g_lds;
  unsigned char* const vbuf = g_lds + 2 * KBUF;
  int32_t* const ids = reinterpret_cast<int32_t*>(g_lds + LY::ID0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int li = lane & 31;             // query row of the lane (column of its MFMAs)
  const int h = lane >> 5;              // key half of its accumulators
  // conversion: every wave converts a quarter of each tile, K of keys
  // 8*wave .. 8*wave+7 (lane kk + 8q: half k_h = q & 1, step quarter
  // k_cq = q >> 1) and V of 16-key group v_grp, keys pkey(v_grp, h,
  // 4*v_half .. 4*v_half+3) of every operand lane
  const int kk = lane & 7, k_h = (lane >> 3) & 1, k_cq = lane >> 4;
  const int kslot = 8 * wave + kk + 32 * k_h;     // the operand lane it fills
  const int v_grp = wave >> 1, v_half = wave & 1;
  const int R = a.Tq * a.r;
  const int QG = (R + kWRows - 1) / kWRows;
  const int n_units = a.B * a.p_max * a.Hkv * QG;
  const int Gd = gridDim.x;
  const int logical = xcd_logical(blockIdx.x, Gd);

  const uint32_t kstride = uint32_t(a.Hkv) * KRB;
  const uint32_t vstride = uint32_t(a.Hkv) * VRB;
  // where the lane's conversion job reads inside a staged raw tile
  // where the lane's conversion reads inside a staged raw tile
  const uint32_t k_row = uint32_t(((8 * wave + kk) >> 4) * SK::GB + ((8 * wave + kk) & 15) * KRB);
  const auto vl = VF::lane(li);
  const uint32_t v_row0 = uint32_t(2 * SK::GB + v_grp * SV::GB + pkey(0, h, 4 * v_half) * VRB);
  const uint32_t mg = opaque_vgpr(kMagic);
  const int seg_tokens = kWNid << a.bs_shift;
  // the DMA of a tile: wave w issues every instruction of one side (K for
  // even w, V for odd) of 16-key group w >> 1, at lane offsets that do not
  // change from tile to tile
  const int d_grp = wave >> 1;
  const bool d_v = (wave & 1) != 0;
  const int n_dma = d_v ? SV::NI : SK::NI;
  constexpr int NIM = SK::NI > SV::NI ? SK::NI : SV::NI;
  uint32_t d_off[NIM];
#pragma unroll
  for (int j = 0; j < NIM; ++j)
    d_off[j] = d_v ? (j < SV::NI ? SV::off(j, lane, vstride) : 0u) : (j < SK::NI ? SK::off(j, lane, kstride) : 0u);

  for (int u = logical; u < n_units; u += Gd) {
    // ---- locate the unit: ((b*Hkv + g)*QG + qg)*p_max + p ------------------
    // (the partition varies fastest, so the units that read one Q run side by
    // side on one XCD, whose L2 then serves that Q once for all of them)
    const int p = u % a.p_max;
    const int qg = (u / a.p_max) % QG;
    const int g = (u / (a.p_max * QG)) % a.Hkv;
    const int b = u / (a.p_max * QG * a.Hkv);
    int L = a.seq_len[b];
    if (L < 0 || L > a.cap_tokens) {
      if (tid == 0 && p == 0 && g == 0 && qg == 0) atomicOr(a.status, 2u);
      L = L < 0 ? 0 : a.cap_tokens;
    }
    if (L > 0 && L < a.Tq) {             // the chunk is longer than the sequence
      if (tid == 0 && p == 0 && g == 0 && qg == 0) atomicOr(a.status, 2u);
      L = 0;
    }
    L = __builtin_amdgcn_readfirstlane(L);
    const int P = L > 0 ? (L + a.psize - 1) / a.psize : 0;
    const int t_begin = p * a.psize;
    const int t_end = min(L, t_begin + a.psize);
    // this lane's query row
    const int row = qg * kWRows + 32 * wave + li;
    const bool valid = row < R;
    const int tq = valid ? row / a.r : 0;
    const int hq = g * a.r + (valid ? row - tq * a.r : 0);
    const int64_t orow = (int64_t(b) * a.Tq + tq) * a.Hq + hq;   // row of out / partials
    const int lim = valid ? min(L - a.Tq + tq, t_end - 1) : t_begin - 1;
    if (L == 0) {
      // an empty (or refused) sequence: zero rows in direct mode; the merge
      // writes its zero rows otherwise
      if (a.direct && valid && h == 0)
        for (int d = 0; d < D; ++d) a.out[orow * D + d] = 0.0f;
      continue;
    }
    if (p >= P) continue;                 // no such partition: nothing to write
    int lim_min = valid ? lim : INT32_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);
    // last key any row of the workgroup reads: that of its last valid row
    const int row_hi = min(R - 1, qg * kWRows + kWRows - 1);
    const int t_stop = min(t_end, L - a.Tq + row_hi / a.r + 1);

    // ---- Q^T operands: slot s of step c holds q[row][kd(c, h, s)] ----------
    f16x8 qop[C];
    {
      const float* qr = a.q + orow * D;
      const float keep = valid ? a.qscale : 0.0f;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        // kd(c, h, 0..7) is 8 consecutive positions in word_order
        const float* q8 = qr + (KF::kd(c, h, 0) & ~7);
        const float4 A = valid ? *reinterpret_cast<const float4*>(q8) : float4{0, 0, 0, 0};
        const float4 B = valid ? *reinterpret_cast<const float4*>(q8 + 4) : float4{0, 0, 0, 0};
        const float v[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
#pragma unroll
        for (int s = 0; s < 8; ++s) qop[c][s] = f16(v[KF::kd(0, 0, s)] * keep);
        // Q^T stays in AGPRs (the MFMAs read their B operand from there),
        // leaving the VGPRs to the operand reads, softmax and conversion
        asm volatile("" : "+a"(qop[c]));
      }
    }

    // reference max: +inf for rows past R (their p are exactly 0); -inf until
    // the row has seen a key
    float m_run = valid ? -INFINITY : INFINITY;
    float l_lane = 0.0f;
    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[dt] = f32x16{};
    int bad = 0;

    // ---- one tile's steps (scores, softmax, PV) and the conversion job, in
    // two regions per tile with no branch inside, so the scheduler can put
    // VALU work between the MFMAs (a wave issues in order, and at one wave
    // per SIMD nothing else fills the gaps) -------------------------------------
    // the causal and end-of-partition mask of the scores of the tile at t0
    // (a branch, taken only where some row's limit falls inside the tile)
    auto mask = [&](f32x16& s, int t0) __attribute__((always_inline)) {
      if (t0 + kWTile - 1 > lim_min) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + skey(r, h) > lim) s[r] = -INFINITY;
      }
    };
    // S^T = K Q^T over the D/16 steps, read by the softmax an iteration later
    auto scores = [&](const unsigned char* kops, f32x16& sc) __attribute__((always_inline)) {
      f16x8 kop[C];
#pragma unroll
      for (int c = 0; c < C; ++c) kop[c] = *reinterpret_cast<const f16x8*>(kops + (c * 64 + lane) * 16);
      sc = f32x16{};
#pragma unroll
      for (int c = 0; c < C; ++c) sc = mfma32(kop[c], qop[c], sc);
    };
    auto row_max = [&](const f32x16& s) __attribute__((always_inline)) {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    // lazy rescale (lucebox PR #555, Summary: skip the rescale when the max is
    // unchanged): the reference moves only when a row's max exceeds it by more
    // than kSlack; rows with no key yet (m = -inf) and rows past R (m = +inf)
    // keep their sums as they are
    auto rescale = [&](float mx) __attribute__((always_inline)) {
      // a scalar branch around the rare rescale: taken by the whole wave or
      // skipped (the asm keeps the compiler from running it on every tile
      // with a factor of 1)
      if (__builtin_amdgcn_readfirstlane(__any(mx > m_run + kSlack) ? 1 : 0)) {
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_lane *= alpha;
        // element by element through a VGPR: the accumulators stay in AGPRs
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float x;
            asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(x) : "a"(acc[dt][r]));
            x *= alpha;
            asm volatile("v_accvgpr_write_b32 %0, %1" : "=a"(acc[dt][r]) : "v"(x));
          }
        m_run = m_new;
      }
    };
    // exp2 of the scores against the reference, their sum, P^T operands
    auto probs = [&](const f32x16& s, f16x8 (&pop)[2]) __attribute__((always_inline)) {
      const float m_use = m_run == -INFINITY ? 0.0f : m_run;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r += 4) ls += (pr[r] + pr[r + 1]) + (pr[r + 2] + pr[r + 3]);
      l_lane += ls;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[t][e] = f16(pr[8 * t + e]);
    };

    for (int seg_t0 = t_begin; seg_t0 < t_stop; seg_t0 += seg_tokens) {
      const int seg_t1 = min(t_stop, seg_t0 + seg_tokens);
      const int jb0 = seg_t0 >> a.bs_shift;
      const int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
      __syncthreads();                       // ids[] and every LDS buffer are free
      int badl = 0;
      for (int i = tid; i < nb; i += kWThreads) {
        int32_t id = block_of(a.table, b, a.max_blocks, jb0 + i);
        if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
        ids[i] = id;
      }
      bad |= __syncthreads_or(badl);
      const int ntiles = (seg_t1 - seg_t0 + kWTile - 1) / kWTile;

      // ---- DMA of tile t's raw rows into ring slot t % RR --------------------
      // (a group at or past seg_t1 gets a zero-size resource and reads
      // nothing, one that crosses it a resource over its live rows; the
      // instruction count per wave stays the same)
      auto issue = [&](int t) __attribute__((always_inline)) {
        const uint32_t slot = uint32_t(LY::RAW + (t % RR) * LY::SLOT);
        const int tg = seg_t0 + t * kWTile + 16 * d_grp;
        const bool live = tg < seg_t1;
        const int32_t id = live ? __builtin_amdgcn_readfirstlane(ids[(tg >> a.bs_shift) - jb0]) : 0;
        const int slot0 = live ? (tg & ((1 << a.bs_shift) - 1)) : 0;
        // rows past seg_t1 (junk slots, maybe NaN) lie outside the resource
        // and land as zeros: their p is 0, and 0 * NaN would not be
        const uint32_t nlive = live ? uint32_t(min(16, seg_t1 - tg)) : 0u;
        if (!d_v) {
          const rsrc_t kr = make_rsrc(a.k_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, SK::RB),
                                      nlive * kstride);
#pragma unroll
          for (int j = 0; j < SK::NI; ++j) dma_lds<SK::CB>(kr, slot + d_grp * SK::GB + j * 64 * SK::CB, d_off[j]);
        } else {
          const rsrc_t vr = make_rsrc(a.v_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, SV::RB),
                                      nlive * vstride);
#pragma unroll
          for (int j = 0; j < SV::NI; ++j)
            dma_lds<SV::CB>(vr, slot + 2 * SK::GB + d_grp * SV::GB + j * 64 * SV::CB, d_off[j]);
        }
      };
      // ---- this wave's quarter of the conversion of tile kt: staged raw rows
      // into f16 operands in LDS (a tile past the segment converts whatever
      // the ring holds into buffers nothing reads) -----------------------------
      struct ConvRaw { uint32_t kw[KF::kWords], vw[VF::kWords]; };
      auto conv_load = [&](int kt, ConvRaw& cr) __attribute__((always_inline)) {
        const unsigned char* raw = g_lds + LY::RAW + (kt % RR) * LY::SLOT;
        KF::load(cr.kw, raw + k_row, k_h, k_cq);
        VF::load(cr.vw, raw + v_row0, vl);
      };
      auto conv_store = [&](int kt, ConvRaw& cr) __attribute__((always_inline)) {
        VF::prep(cr.vw, vl);
        unsigned char* kops = kbuf + (kt & 1) * KBUF;
#pragma unroll
        for (int cc = 0; cc < CQ; ++cc)
          *reinterpret_cast<f16x8*>(kops + ((k_cq * CQ + cc) * 64 + kslot) * 16) = KF::op(cr.kw, cc, k_cq, mg);
        unsigned char* vops = vbuf + (kt % 3) * VBUF;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          *reinterpret_cast<f16x4*>(vops + ((v_grp * NDT + dt) * 64 + lane) * 16 + 8 * v_half) =
              VF::op(cr.vw, vl, dt, mg);
      };
      auto convert = [&](int kt) __attribute__((always_inline)) {
        ConvRaw cr;
        conv_load(kt, cr);
        conv_store(kt, cr);
      };

      // ---- the pipeline: one barrier per tile. Iteration kt issues the DMA
      // of tile kt+RR+1, computes the scores of kt+1, converts kt+2 and runs
      // the softmax and PV of kt; before its barrier the DMA of kt+3 has
      // landed (RR-2 tiles of DMA stay in flight). ---------------------------
      f32x16 s0, s1;
#pragma unroll
      for (int t = 0; t < RR; ++t) issue(t);
      wait_dma_then_barrier((RR - 1) * n_dma);
      convert(0);
      wait_all_then_barrier((RR - 2) * n_dma);
      issue(RR);
      scores(kbuf, s0);
      convert(1);
      wait_all_then_barrier((RR - 2) * n_dma);
      auto step = [&](int kt, f32x16& s_cur, f32x16& s_next) __attribute__((always_inline)) {
        issue(kt + RR + 1);
        mask(s_cur, seg_t0 + kt * kWTile);
        // the staged rows of tile kt+2 first (LDS returns in order), the row
        // max and the rare rescale
        ConvRaw cr;
        conv_load(kt + 2, cr);
        const float mx = row_max(s_cur);
        rescale(mx);
        // then the score MFMAs of kt+1 alternate with the PV MFMAs of kt, the
        // operand reads streaming kLead reads ahead of them (the LDS counter
        // holds at most 15) and the probabilities and the conversion of kt+2
        // between them
        f16x8 kop[C];
        f16x8 vop[2][NDT];
        {
          const unsigned char* kops = kbuf + ((kt + 1) & 1) * KBUF;
          const unsigned char* vops = vbuf + (kt % 3) * VBUF;
#pragma unroll
          for (int i = 0; i < C; ++i) {
            kop[i] = *reinterpret_cast<const f16x8*>(kops + (i * 64 + lane) * 16);
            vop[i / NDT][i % NDT] = *reinterpret_cast<const f16x8*>(vops + (i * 64 + lane) * 16);
          }
        }
        f16x8 pop[2];
        probs(s_cur, pop);
        s_next = f32x16{};
#pragma unroll
        for (int i = 0; i < C; ++i) {
          s_next = mfma32(kop[i], qop[i], s_next);
          acc[i % NDT] = mfma32(vop[i / NDT][i % NDT], pop[i / NDT], acc[i % NDT]);
        }
        conv_store(kt + 2, cr);
        constexpr int kLead = 12;
        __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 24, 0);
#pragma unroll
        for (int i = 0; i < 2 * C; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);
          if (i + kLead < 2 * C) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x200, 16, 0);
        // the accumulators are carried from tile to tile in AGPRs (without
        // this the compiler moves all of them to VGPRs and back every tile)
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) asm volatile("" : "+a"(acc[dt]));
        wait_all_then_barrier((RR - 2) * n_dma);
      };
      for (int kt = 0; kt < ntiles; kt += 2) {
        step(kt, s0, s1);
        if (kt + 1 >= ntiles) break;
        step(kt + 1, s1, s0);
      }
      // the DMA of tiles past the segment (zeros) lands before the ring is reused
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }

    // ---- partial (or final) rows -------------------------------------------
    mfma_drain();                          // the last tile's PV MFMAs wrote acc
    if (bad && tid == 0) atomicOr(a.status, 1u);
    float l_run;
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
      l_run = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
    if (!valid) continue;
    const float inv = bad ? __builtin_nanf("") : (l_run > 0.0f ? 1.0f / l_run : 0.0f);
    if (a.direct) {
      float* dst = a.out + orow * D;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) dst[VF::vd(dt, skey(r, h))] = acc[dt][r] * inv;
    } else {
      const int64_t prow = orow * a.p_max + p;
      f16* dst = reinterpret_cast<f16*>(a.part_o) + prow * D;
      if (h == 0) {
        a.part_ml[2 * prow] = bad ? __builtin_nanf("") : (l_run > 0.0f ? m_run : -INFINITY);
        a.part_ml[2 * prow + 1] = l_run;
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int dn = VF::dnext(dt);
        if (dn < 0) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          store_f16_pair(dst, VF::vd(dt, skey(r, h)), acc[dt][r] * inv, acc[dn][r] * inv);
      }
    }
  }
}

// ===========================================================================
// The paired form: eight waves, two per SIMD. Waves w and w + 4 (on one SIMD)
// share query rows 32w .. 32w+31: the score wave (w < 4) holds their Q^T,
// computes the scores of tile kt+1, the softmax of tile kt and the PV of the
// first half of the d-tiles; the conversion wave (w >= 4) issues the DMA,
// converts tile kt+2 (a quarter of it, as in the four-wave form) and runs the
// PV of the second half of the d-tiles for tile kt-1, with the P^T operands
// and the rescale factors its partner left in LDS one tile earlier. Each
// SIMD keeps the four-wave form's MFMA and vector work, but two waves issue
// it, so one wave's LDS waits are filled with the other's instructions.
// ===========================================================================
constexpr int kPThreads = 512;

// Whether every stored pair of d-tiles (dt, dnext(dt)) lies inside one half
// of the d-tiles, with the same pattern in both halves.
template <typename VF>
__host__ __device__ constexpr bool halves_ok() {
  constexpr int NH = VF::NDT / 2;
  for (int j = 0; j < NH; ++j) {
    const int a = VF::dnext(j), b = VF::dnext(NH + j);
    if ((a < 0) != (b < 0)) return false;
    if (a >= 0 && (a >= NH || b != NH + a)) return false;
  }
  return true;
}
constexpr int kPNid = 256;      // block ids staged per segment
// LDS row stride of the staged Q rows and partial rows (binary16): 16 bytes
// of padding spread a wave's rows over the banks
constexpr int stage_row(int D) { return 2 * D + 16; }

template <int KT, int VT, int D> struct PairLds {
  using SK = Stage<KT, D>;
  using SV = Stage<VT, D>;
  static constexpr int KBUF = (D / 16) * 64 * 16;          // K operands of a tile
  static constexpr int VBUF = 2 * (D / 32) * 64 * 16;      // V operands of a tile
  static constexpr int PBUF = 4 * 2 * 64 * 16;             // P^T operands of the four score waves
  static constexpr int XBUF = 4 * 256;                     // per score wave: flag, 32 row factors
  static constexpr int SLOT = 2 * (SK::GB + SV::GB);       // raw rows of a tile
  static constexpr int IDS = 4 * (kPNid + 4);
  static constexpr int K0 = 0;
  static constexpr int V0 = K0 + 2 * KBUF;                 // four V buffers (tiles kt-1 .. kt+2)
  static constexpr int P0 = V0 + 4 * VBUF;                 // two tiles of P^T
  static constexpr int X0 = P0 + 2 * PBUF;                 // two tiles of flags and factors
  static constexpr int L0 = X0 + 2 * XBUF;                 // row sums for the epilogue
  static constexpr int OPS = L0 + 4 * 32 * 4;
  static constexpr int RR = OPS + 3 * SLOT + IDS <= 160 * 1024 ? 3 : 2;
  static constexpr int RAW = OPS;
  static constexpr int ID0 = RAW + RR * SLOT;
  static constexpr int BYTES = ID0 + IDS;
  static constexpr bool kFits = BYTES <= 160 * 1024;
};

// Roles of the paired form's waves.
constexpr int kRoleScore = 0, kRoleConvK = 1, kRoleConvV = 2;

// The whole body of one role, instantiated once per role so that no role's
// registers stay live across another's code; every role runs the same
// sequence of barriers. Score wave pw (waves 0-3) holds query rows 32pw ..
// 32pw+31; conversion wave 4 + pw shares its SIMD and rows and, by pw,
// handles one side (K for even pw, V for odd) of 16-key group pw >> 1 of
// every tile: it DMAs those rows, waits for its own DMA only, loads the raw
// rows of tile kt+3 into registers during tile kt, and converts tile kt+2
// from the registers loaded during tile kt-1, so no LDS latency stands
// between a tile's start and its conversion.
template <int KT, int VT, int D, int ROLE>
__device__ __forceinline__ void pair_role(const ChunkArgs& a) {
  using KF = WK<KT, D>;
  using VF = WV<VT, D>;
  using LY = PairLds<KT, VT, D>;
  using SK = typename LY::SK;
  using SV = typename LY::SV;
  static_assert(pairs_ok<VF>(), "d-tile pairs cover adjacent even/odd positions");
  static_assert(LY::kFits, "LDS of one CU");
  constexpr int C = D / 16;                       // score MFMA steps
  constexpr int NDT = D / 32;                     // PV d-tiles
  constexpr int NH = NDT / 2;                     // d-tiles per wave of a pair
  constexpr int KBUF = LY::KBUF, VBUF = LY::VBUF, RR = LY::RR;
  constexpr int KRB = SK::RB, VRB = SV::RB;
  constexpr bool sw = ROLE == kRoleScore;
  constexpr bool cv = ROLE == kRoleConvV;
  static_assert(2 * NH == NDT && halves_ok<VF>(), "the d-tile pairs stay inside a half");
  constexpr int kStageRow = stage_row(D);
  static_assert(kWRows * kStageRow <= LY::P0, "staged rows fit the operand buffers");

  unsigned char* const kbuf = g_lds + LY::K0;
  unsigned char* const vbuf = g_lds + LY::V0;
  int32_t* const ids = reinterpret_cast<int32_t*>(g_lds + LY::ID0);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pw = wave & 3;                        // the pair: query rows 32pw .. 32pw+31
  const int li = lane & 31;                       // query row of the lane (column of its MFMAs)
  const int h = lane >> 5;                        // key half of its accumulators
  const int R = a.Tq * a.r;
  const int QG = (R + kWRows - 1) / kWRows;
  const int n_units = a.B * a.p_max * a.Hkv * QG;
  const int Gd = gridDim.x;
  const int logical = xcd_logical(blockIdx.x, Gd);

  const uint32_t kstride = uint32_t(a.Hkv) * KRB;
  const uint32_t vstride = uint32_t(a.Hkv) * VRB;
  const uint32_t mg = opaque_vgpr(kMagic);
  const int seg_tokens = kPNid << a.bs_shift;
  // conversion waves: the 16-key group and its DMA (NI instructions of the
  // side, lane offsets fixed for the kernel)
  const int grp = pw >> 1;
  constexpr int NI = cv ? SV::NI : SK::NI;
  const int n_dma = sw ? 0 : NI;
  uint32_t d_off[NI];
#pragma unroll
  for (int j = 0; j < NI; ++j) d_off[j] = cv ? SV::off(j, lane, vstride) : SK::off(j, lane, kstride);
  // K conversion: lane = kk + 16 (k_h + 2 k_c2) converts the operand slots of
  // key 16 grp + kk for half k_h and the C/2 steps k_c2*C/2 ..
  constexpr int KS = C / 2;
  const int kk = lane & 15, k_h = (lane >> 4) & 1, k_c2 = lane >> 5;
  const int kslot = 16 * grp + kk + 32 * k_h;
  // V conversion: every operand lane of group grp, both halves of its keys
  const auto vl = VF::lane(li);
  // P^T operands, flags and row factors of the pair, by tile parity
  auto pslot = [&](int kt) __attribute__((always_inline)) {
    return g_lds + LY::P0 + (kt & 1) * LY::PBUF + pw * 2048;
  };
  auto xslot = [&](int kt) __attribute__((always_inline)) {
    return g_lds + LY::X0 + (kt & 1) * LY::XBUF + pw * 256;
  };
  float* const lsum = reinterpret_cast<float*>(g_lds + LY::L0) + 32 * pw;

  for (int u = logical; u < n_units; u += Gd) {
    // ---- locate the unit: ((b*Hkv + g)*QG + qg)*p_max + p ------------------
    // (the partition varies fastest, so the units that read one Q run side by
    // side on one XCD, whose L2 then serves that Q once for all of them)
    const int p = u % a.p_max;
    const int qg = (u / a.p_max) % QG;
    const int g = (u / (a.p_max * QG)) % a.Hkv;
    const int b = u / (a.p_max * QG * a.Hkv);
    int L = a.seq_len[b];
    if (L < 0 || L > a.cap_tokens) {
      if (tid == 0 && p == 0 && g == 0 && qg == 0) atomicOr(a.status, 2u);
      L = L < 0 ? 0 : a.cap_tokens;
    }
    if (L > 0 && L < a.Tq) {             // the chunk is longer than the sequence
      if (tid == 0 && p == 0 && g == 0 && qg == 0) atomicOr(a.status, 2u);
      L = 0;
    }
    L = __builtin_amdgcn_readfirstlane(L);
    const int P = L > 0 ? (L + a.psize - 1) / a.psize : 0;
    const int t_begin = p * a.psize;
    const int t_end = min(L, t_begin + a.psize);
    // this lane's query row
    const int row = qg * kWRows + 32 * pw + li;
    const bool valid = row < R;
    const int tq = valid ? row / a.r : 0;
    const int hq = g * a.r + (valid ? row - tq * a.r : 0);
    const int64_t orow = (int64_t(b) * a.Tq + tq) * a.Hq + hq;   // row of out / partials
    const int lim = valid ? min(L - a.Tq + tq, t_end - 1) : t_begin - 1;
    if (L == 0) {
      // an empty (or refused) sequence: zero rows in direct mode; the merge
      // writes its zero rows otherwise
      if (a.direct && sw && valid && h == 0)
        for (int d = 0; d < D; ++d) a.out[orow * D + d] = 0.0f;
      continue;
    }
    if (p >= P) continue;                 // no such partition: nothing to write
    int lim_min = valid ? lim : INT32_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);
    // last key any row of the workgroup reads: that of its last valid row
    const int row_hi = min(R - 1, qg * kWRows + kWRows - 1);
    const int t_stop = min(t_end, L - a.Tq + row_hi / a.r + 1);

    // ---- Q^T operands (score waves): slot s of step c holds q[row][kd(c, h, s)].
    // The workgroup's 128 rows are read whole by all its threads (16-byte
    // loads, every row contiguous, all in flight at once), scaled, rounded to
    // f16 into LDS and read back by the score waves in operand order; rows
    // past R are zeros.
    __syncthreads();                      // the LDS staging of the last unit is read
    {
      constexpr int CPR4 = D / 4;                       // 16-byte chunks of a row
      constexpr int NQ = kWRows * CPR4 / kPThreads;     // per thread
      float4 v[NQ];
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        const int c = tid + k * kPThreads;
        const int grow = qg * kWRows + c / CPR4;
        v[k] = float4{0.0f, 0.0f, 0.0f, 0.0f};
        if (grow < R) {
          const int tq2 = grow / a.r;
          const int64_t orow2 = (int64_t(b) * a.Tq + tq2) * a.Hq + g * a.r + (grow - tq2 * a.r);
          v[k] = *reinterpret_cast<const float4*>(a.q + orow2 * D + 4 * (c % CPR4));
        }
      }
#pragma unroll
      for (int k = 0; k < NQ; ++k) {
        const int c = tid + k * kPThreads;
        *reinterpret_cast<f16x4*>(g_lds + (c / CPR4) * kStageRow + 8 * (c % CPR4)) =
            f16x4{f16(v[k].x * a.qscale), f16(v[k].y * a.qscale), f16(v[k].z * a.qscale), f16(v[k].w * a.qscale)};
      }
    }
    __syncthreads();
    f16x8 qop[C];
    if (sw) {
      const unsigned char* qs = g_lds + (32 * pw + li) * kStageRow;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const f16x8 q8 = *reinterpret_cast<const f16x8*>(qs + 2 * (KF::kd(c, h, 0) & ~7));
#pragma unroll
        for (int s = 0; s < 8; ++s) qop[c][s] = q8[KF::kd(0, 0, s)];
      }
    }

    // reference max: +inf for rows past R (their p are exactly 0); -inf until
    // the row has seen a key (score waves)
    float m_run = valid ? -INFINITY : INFINITY;
    float l_lane = 0.0f;
    f32x16 acc[NH];
#pragma unroll
    for (int dt = 0; dt < NH; ++dt) acc[dt] = f32x16{};
    int bad = 0;

    auto mask = [&](f32x16& s, int t0) __attribute__((always_inline)) {
      if (t0 + kWTile - 1 > lim_min) {
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (t0 + skey(r, h) > lim) s[r] = -INFINITY;
      }
    };
    auto scores = [&](const unsigned char* kops, f32x16& sc) __attribute__((always_inline)) {
      f16x8 kop[C];
#pragma unroll
      for (int c = 0; c < C; ++c) kop[c] = *reinterpret_cast<const f16x8*>(kops + (c * 64 + lane) * 16);
      sc = f32x16{};
#pragma unroll
      for (int c = 0; c < C; ++c) sc = mfma32(kop[c], qop[c], sc);
    };
    auto row_max = [&](const f32x16& s) __attribute__((always_inline)) {
      float mx = s[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      return fmaxf(__uint_as_float(sw2[0]), __uint_as_float(sw2[1]));
    };
    auto scale_acc = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < NH; ++dt) acc[dt] *= alpha;
    };
    // lazy rescale (lucebox PR #555, Summary: skip the rescale when the max is
    // unchanged), as in the four-wave form; the score wave also leaves the
    // flag of tile kt (and, when set, each row's factor) for its partner
    auto rescale = [&](float mx, int kt) __attribute__((always_inline)) {
      unsigned char* xs = xslot(kt);
      const int take = __builtin_amdgcn_readfirstlane(__any(mx > m_run + kSlack) ? 1 : 0);
      if (lane == 0) *reinterpret_cast<uint32_t*>(xs) = uint32_t(take);
      if (take) {
        asm volatile("" ::: "memory");
        const float m_new = fmaxf(m_run, mx);
        const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
        l_lane *= alpha;
        scale_acc(alpha);
        reinterpret_cast<float*>(xs + 4)[li] = alpha;
        m_run = m_new;
      }
    };
    auto probs = [&](const f32x16& s, f16x8 (&pop)[2]) __attribute__((always_inline)) {
      const float m_use = m_run == -INFINITY ? 0.0f : m_run;
      float pr[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) pr[r] = __builtin_amdgcn_exp2f(s[r] - m_use);
      float ls = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; r += 4) ls += (pr[r] + pr[r + 1]) + (pr[r + 2] + pr[r + 3]);
      l_lane += ls;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 8; ++e) pop[t][e] = f16(pr[8 * t + e]);
    };

    for (int seg_t0 = t_begin; seg_t0 < t_stop; seg_t0 += seg_tokens) {
      const int seg_t1 = min(t_stop, seg_t0 + seg_tokens);
      const int jb0 = seg_t0 >> a.bs_shift;
      const int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
      __syncthreads();                       // ids[] and every LDS buffer are free
      int badl = 0;
      for (int i = tid; i < nb; i += kPThreads) {
        int32_t id = block_of(a.table, b, a.max_blocks, jb0 + i);
        if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
        ids[i] = id;
      }
      bad |= __syncthreads_or(badl);
      const int ntiles = (seg_t1 - seg_t0 + kWTile - 1) / kWTile;

      // ---- DMA of the wave's side of group grp of tile t into ring slot
      // t % RR (a group at or past seg_t1 gets a zero-size resource and reads
      // nothing, one that crosses it a resource over its live rows: rows past
      // seg_t1, junk slots maybe holding NaN, land as zeros, so their p of 0
      // meets no NaN) -----------------------------------------------------------
      // the block id of the group of tile t, read from LDS (0 past seg_t1);
      // issue_id takes it read a tile earlier, so the DMA issue does not
      // wait for LDS
      auto id_load = [&](int t) __attribute__((always_inline)) {
        const int tg = seg_t0 + t * kWTile + 16 * grp;
        return tg < seg_t1 ? ids[(tg >> a.bs_shift) - jb0] : 0;
      };
      auto issue_id = [&](int t, int32_t idv) __attribute__((always_inline)) {
        const uint32_t slot = uint32_t(LY::RAW + (t % RR) * LY::SLOT);
        const int tg = seg_t0 + t * kWTile + 16 * grp;
        const bool live = tg < seg_t1;
        const int32_t id = __builtin_amdgcn_readfirstlane(idv);
        const int slot0 = live ? (tg & ((1 << a.bs_shift) - 1)) : 0;
        const uint32_t nlive = live ? uint32_t(min(16, seg_t1 - tg)) : 0u;
        if (!cv) {
          const rsrc_t kr = make_rsrc(a.k_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, SK::RB),
                                      nlive * kstride);
#pragma unroll
          for (int j = 0; j < SK::NI; ++j) dma_lds<SK::CB>(kr, slot + grp * SK::GB + j * 64 * SK::CB, d_off[j]);
        } else {
          const rsrc_t vr = make_rsrc(a.v_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, SV::RB),
                                      nlive * vstride);
#pragma unroll
          for (int j = 0; j < SV::NI; ++j)
            dma_lds<SV::CB>(vr, slot + 2 * SK::GB + grp * SV::GB + j * 64 * SV::CB, d_off[j]);
        }
      };
      auto issue = [&](int t) __attribute__((always_inline)) { issue_id(t, id_load(t)); };
      // ---- the raw rows of tile t in registers, and their conversion into
      // f16 operands in LDS (a tile past the segment converts the zeros of
      // its zero-size DMA into buffers nothing reads) ---------------------------
      struct Raw {
        uint32_t w[cv ? 2 * VF::kWords : KF::template words<KS>()];
      };
      auto raw_load = [&](int t, Raw& r) __attribute__((always_inline)) {
        const unsigned char* raw = g_lds + LY::RAW + (t % RR) * LY::SLOT;
        if constexpr (cv) {
#pragma unroll
          for (int k = 0; k < 2; ++k)
            VF::load(r.w + k * VF::kWords, raw + 2 * SK::GB + grp * SV::GB + pkey(0, h, 4 * k) * VRB, vl);
        } else {
          KF::template loadn<KS>(r.w, raw + grp * SK::GB + kk * KRB, k_h, k_c2 * KS);
        }
      };
      // (in two halves: steps or d-tiles [lo, hi) of the lane's job; the
      // first half also realigns the raw V words)
      auto raw_store = [&](int t, Raw& r, int lo, int hi) __attribute__((always_inline)) {
        if constexpr (cv) {
          if (lo == 0) {
#pragma unroll
            for (int k = 0; k < 2; ++k) VF::prep(r.w + k * VF::kWords, vl);
          }
          unsigned char* vops = vbuf + (t & 3) * VBUF;
#pragma unroll
          for (int dt = lo; dt < hi; ++dt) {
            const f16x4 lo = VF::op(r.w, vl, dt, mg), hi = VF::op(r.w + VF::kWords, vl, dt, mg);
            *reinterpret_cast<f16x8*>(vops + ((grp * NDT + dt) * 64 + lane) * 16) =
                f16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
          }
        } else {
          unsigned char* kops = kbuf + (t & 1) * KBUF;
#pragma unroll
          for (int cc = lo * KS / NDT; cc < hi * KS / NDT; ++cc)
            *reinterpret_cast<f16x8*>(kops + ((k_c2 * KS + cc) * 64 + kslot) * 16) =
                KF::template opn<KS>(r.w, cc, k_c2 * KS, mg);
        }
      };
      // ---- PV of tile kt on the conversion wave's d-tiles: the partner's
      // flag, P^T operands and (when it rescaled) row factors of tile kt ------
      auto pair_pv_load = [&](int kt, f16x8 (&pop)[2], f16x8 (&vop)[2][NH]) __attribute__((always_inline)) {
        const unsigned char* ps = pslot(kt);
#pragma unroll
        for (int t = 0; t < 2; ++t) pop[t] = *reinterpret_cast<const f16x8*>(ps + (t * 64 + lane) * 16);
        const unsigned char* vops = vbuf + (kt & 3) * VBUF;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int dt = 0; dt < NH; ++dt)
            vop[t][dt] = *reinterpret_cast<const f16x8*>(vops + ((t * NDT + NH + dt) * 64 + lane) * 16);
      };
      auto pair_pv_mfma = [&](int kt, const f16x8 (&pop)[2], const f16x8 (&vop)[2][NH]) __attribute__((always_inline)) {
        const unsigned char* xs = xslot(kt);
        if (__builtin_amdgcn_readfirstlane(*reinterpret_cast<const uint32_t*>(xs))) {
          asm volatile("" ::: "memory");
          scale_acc(reinterpret_cast<const float*>(xs + 4)[li]);
        }
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int dt = 0; dt < NH; ++dt) acc[dt] = mfma32(vop[t][dt], pop[t], acc[dt]);
      };

      // ---- the pipeline: one barrier per tile. Iteration kt: the score waves
      // run the softmax of kt (leaving its P^T and rescale flag), the scores
      // of kt+1 and their half of the PV of kt; the conversion waves issue
      // their DMA of tile kt+RR+2, load tile kt+3's raw rows into registers
      // (their own DMA of it has landed), convert kt+2 from the registers
      // loaded during kt-1 and run their half of the PV of kt-1. -------------
      f32x16 s0, s1;
      if constexpr (sw) {
        wait_all_then_barrier(0);
        scores(kbuf, s0);
        wait_all_then_barrier(0);
        auto s_step = [&](int kt, f32x16& s_cur, f32x16& s_next) __attribute__((always_inline)) {
          mask(s_cur, seg_t0 + kt * kWTile);
          const float mx = row_max(s_cur);
          rescale(mx, kt);
          // the score MFMAs of kt+1 alternate with the PV MFMAs of kt, the
          // operand reads streaming ahead of them
          f16x8 kop[C];
          f16x8 vop[2][NH];
          {
            const unsigned char* kops = kbuf + ((kt + 1) & 1) * KBUF;
            const unsigned char* vops = vbuf + (kt & 3) * VBUF;
#pragma unroll
            for (int i = 0; i < C; ++i) {
              kop[i] = *reinterpret_cast<const f16x8*>(kops + (i * 64 + lane) * 16);
              if (i < 2 * NH)
                vop[i / NH][i % NH] =
                    *reinterpret_cast<const f16x8*>(vops + (((i / NH) * NDT + i % NH) * 64 + lane) * 16);
            }
          }
          f16x8 pop[2];
          probs(s_cur, pop);
          unsigned char* ps = pslot(kt);
#pragma unroll
          for (int t = 0; t < 2; ++t) *reinterpret_cast<f16x8*>(ps + (t * 64 + lane) * 16) = pop[t];
          s_next = f32x16{};
#pragma unroll
          for (int i = 0; i < C; ++i) {
            s_next = mfma32(kop[i], qop[i], s_next);
            if (i < 2 * NH) acc[i % NH] = mfma32(vop[i / NH][i % NH], pop[i / NH], acc[i % NH]);
          }
          constexpr int kLead = 8, kReads = C + 2 * NH, kMfma = C + 2 * NH;
          __builtin_amdgcn_sched_group_barrier(0x100, kLead, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
          __builtin_amdgcn_sched_group_barrier(0x200, 2, 0);
#pragma unroll
          for (int i = 0; i < kMfma; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
            if (i + kLead < kReads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
        };
        for (int kt = 0; kt < ntiles; kt += 2) {
          s_step(kt, s0, s1);
          wait_all_then_barrier(0);
          if (kt + 1 >= ntiles) break;
          s_step(kt + 1, s1, s0);
          wait_all_then_barrier(0);
        }
      } else {
        // the conversion waves set the pace of a tile: their instructions
        // issue before the score waves' when both are ready
        __builtin_amdgcn_s_setprio(2);
        // prologue: the first RR tiles in flight; tiles 0 and 1 converted (0
        // before the first barrier, which the score waves wait for to compute
        // the scores of tile 0), tile 2 loaded
        const int vm_keep = (RR - 1) * n_dma;
#pragma unroll
        for (int t = 0; t < RR; ++t) issue(t);
        Raw cur, nxt;
        wait_vm(vm_keep);
        raw_load(0, cur);
        raw_store(0, cur, 0, NDT);
        lds_drain();                          // the rows of tile 0 are read before its slot is refilled
        issue(RR);
        lds_barrier();
        wait_vm(vm_keep);
        raw_load(1, cur);
        raw_store(1, cur, 0, NDT);
        lds_drain();
        issue(RR + 1);
        wait_vm(vm_keep);
        raw_load(2, cur);
        lds_barrier();
        // (tile 0: no PV of the tile before it; every later tile's PV sits
        // after the conversion, which needs no LDS wait)
        int32_t idn = id_load(RR + 2);
        auto c_step = [&](int kt, bool pv) __attribute__((always_inline)) {
          issue_id(kt + RR + 2, idn);
          idn = id_load(kt + RR + 3);
          wait_vm(vm_keep);                   // own DMA of tile kt+3 has landed
          raw_load(kt + 3, nxt);
          f16x8 pop[2];
          f16x8 vop[2][NH];
          if (pv) pair_pv_load(kt - 1, pop, vop);
          raw_store(kt + 2, cur, 0, NDT / 2);
          if (pv) pair_pv_mfma(kt - 1, pop, vop);
          raw_store(kt + 2, cur, NDT / 2, NDT);
          if (pv) {
#pragma unroll
            for (int i = 0; i < 2 * NH; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
              __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
            }
          }
          cur = nxt;
        };
        c_step(0, false);
        lds_barrier();
        for (int kt = 1; kt < ntiles; ++kt) {
          c_step(kt, true);
          lds_barrier();
        }
        // the last tile's half of the PV; the DMA of tiles past the segment
        // (zeros) lands before the ring is reused
        {
          f16x8 pop[2];
          f16x8 vop[2][NH];
          pair_pv_load(ntiles - 1, pop, vop);
          pair_pv_mfma(ntiles - 1, pop, vop);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_setprio(0);
      }
    }

    // ---- partial (or final) rows: each wave of a pair writes its d-tiles ---
    mfma_drain();                          // the last PV MFMAs wrote acc
    if (bad && tid == 0) atomicOr(a.status, 1u);
    float l_run = 0.0f;
    if (sw) {
      const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_lane), __float_as_uint(l_lane), false, false);
      l_run = __uint_as_float(sw2[0]) + __uint_as_float(sw2[1]);
      lsum[li] = l_run;
    }
    __syncthreads();                       // also: every LDS buffer is free
    if (!sw) l_run = lsum[li];
    const float inv = bad ? __builtin_nanf("") : (l_run > 0.0f ? 1.0f / l_run : 0.0f);
    constexpr int H0 = sw ? 0 : NH;        // the wave's first d-tile
    if (a.direct) {
      if (valid) {
        float* dst = a.out + orow * D;
#pragma unroll
        for (int j = 0; j < NH; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[VF::vd(H0 + j, skey(r, h))] = acc[j][r] * inv;
      }
    } else {
      // binary16 rows staged in LDS (row stride kStageRow), then copied out
      // 16 bytes a thread, each row's D values contiguous
      f16* st = reinterpret_cast<f16*>(g_lds + (32 * pw + li) * kStageRow);
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int dn = VF::dnext(H0 + j);
        if (dn < 0) continue;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          store_f16_pair(st, VF::vd(H0 + j, skey(r, h)), acc[j][r] * inv, acc[dn - H0][r] * inv);
      }
      if (sw && h == 0 && valid) {
        const int64_t prow = orow * a.p_max + p;
        a.part_ml[2 * prow] = bad ? __builtin_nanf("") : (l_run > 0.0f ? m_run : -INFINITY);
        a.part_ml[2 * prow + 1] = l_run;
      }
      __syncthreads();
      constexpr int CPR16 = D / 8;         // 16-byte chunks per row
      for (int c = tid; c < kWRows * CPR16; c += kPThreads) {
        const int rr = c / CPR16, col = c - rr * CPR16;
        const int grow = qg * kWRows + rr;
        if (grow < R) {
          const int tq2 = grow / a.r;
          const int64_t prow2 = ((int64_t(b) * a.Tq + tq2) * a.Hq + g * a.r + (grow - tq2 * a.r)) * a.p_max + p;
          *reinterpret_cast<u32x4*>(reinterpret_cast<f16*>(a.part_o) + prow2 * D + col * 8) =
              *reinterpret_cast<const u32x4*>(g_lds + rr * kStageRow + col * 16);
        }
      }
    }
  }
}

template <int KT, int VT, int D>
__global__ void __launch_bounds__(kPThreads, 1) chunk_pair_kernel(const ChunkArgs a) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (w < 4) pair_role<KT, VT, D, kRoleScore>(a);
  else if ((w & 1) == 0) pair_role<KT, VT, D, kRoleConvK>(a);
  else pair_role<KT, VT, D, kRoleConvV>(a);
}

template <int KT, int VT, int D>
hipError_t launch_pair(const ChunkArgs& a, hipStream_t stream) {
  constexpr size_t lds = PairLds<KT, VT, D>::BYTES;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chunk_pair_kernel<KT, VT, D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((chunk_pair_kernel<KT, VT, D>), dim3(a.grid), dim3(kPThreads), lds, stream, a);
  return hipGetLastError();
}

template <int KT, int VT, int D>
hipError_t launch_wide(const ChunkArgs& a, hipStream_t stream) {
  static_assert(kF16 == PA_F16 && kQ8_0 == PA_Q8_0 && kQ4_0 == PA_Q4_0, "type codes");
  static_assert(PairLds<KT, VT, D>::kFits == chunk_wide_paired(KT, VT, D), "the planner's form matches the LDS layout");
  if constexpr (chunk_wide_paired(KT, VT, D)) return launch_pair<KT, VT, D>(a, stream);
  constexpr size_t lds = WideLds<KT, VT, D>::BYTES;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chunk_wide_kernel<KT, VT, D>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((chunk_wide_kernel<KT, VT, D>), dim3(a.grid), dim3(kWThreads), lds, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_wide_d(const ChunkArgs& a, hipStream_t stream) {
  switch (a.k_type * 3 + a.v_type) {
    case 0: return launch_wide<kF16, kF16, D>(a, stream);
    case 1: return launch_wide<kF16, kQ8_0, D>(a, stream);
    case 2: return launch_wide<kF16, kQ4_0, D>(a, stream);
    case 3: return launch_wide<kQ8_0, kF16, D>(a, stream);
    case 4: return launch_wide<kQ8_0, kQ8_0, D>(a, stream);
    case 5: return launch_wide<kQ8_0, kQ4_0, D>(a, stream);
    case 6: return launch_wide<kQ4_0, kF16, D>(a, stream);
    case 7: return launch_wide<kQ4_0, kQ8_0, D>(a, stream);
    case 8: return launch_wide<kQ4_0, kQ4_0, D>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_wide(const ChunkArgs& a, hipStream_t stream) {
  if (a.D == 256) return launch_wide_d<256>(a, stream);
  if (a.D == 128) return launch_wide_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
