// Paged GQA decode attention: the partition kernel.
//
// What it computes (lucebox PR #555, Summary): for each live (sequence b,
// K/V head g, context partition p) the r = Hq/Hkv query heads of the group
// attend over the partition's tokens; the kernel writes each head's running
// max m (base-2 logits), sum l and normalised output o, or the final output
// when a single partition covers the sequence ("direct" mode).
//
// How it maps onto gfx950 (the lucebox design - one warp per K/V group, q8_1
// pre-quantised Q, 32-token score tiles, exp2 softmax - is prior art; this
// is a CDNA4 design around the fact that decode attention is HBM-bound):
//   * Workgroup = 4 wave64s working on one (b, g, p) unit. Wave w takes the
//     32-token tiles w, w+4, w+8, ... of the partition and the four partial
//     softmax states are combined through LDS at the end, so a unit gets four
//     tiles in flight without more partial-result traffic.
//   * The r query heads of the group form the N side of 16x16x32 f16 MFMAs
//     (padded to 16 columns). Scores: S^T[t,h] = K[t,:] . Q[h,:]. PV:
//     O^T[d,h] += V^T[d,t] P^T[t,h]; the score MFMA's output layout (lane
//     holds head lane%16, tokens 4*(lane/16)+i) is exactly the B operand of
//     the PV MFMA, and both MFMAs keep head = lane%16, so the online softmax
//     never moves data between lanes except for two xor-shuffle reductions.
//   * K/V rows stream from HBM straight into registers in MFMA operand
//     order, double-buffered per wave: the next tile's loads are in flight
//     while the current tile is computed. The contraction index of the score
//     MFMA (the head dimension) is permuted per format so every lane reads
//     whole 16-byte chunks (F16) or whole ggml blocks (Q8_0/Q4_0); Q is laid
//     out with the same permutation. V is transposed in registers (v_perm).
//   * The block table is read once per 16-row group (block_size >= 16) with a
//     scalar load; the row address is 64-bit (mlxcel issue #2153).
//   * Dead slots (t >= seq_len in the last block, or a clamped group past the
//     end) are never used: their scores are selected to -inf and their V
//     values zeroed before the PV MFMA, so NaN/Inf junk cannot leak.
//   * Units are spread over the grid with an XCD-aware swizzle so the Hkv
//     units of one (b, p) - which share cache lines of the pool for the
//     quantised formats - run on the same XCD and L2.
#include <type_traits>

#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr uint32_t kMagic = 0x64006400u;   // f16 1024.0 in both halves
constexpr float kSlack = 8.0f;             // lazy-rescale slack (log2 units)

__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f16x2 splat2(f16 x) { return f16x2{x, x}; }

// Reductions over the four lanes that hold the same head (lane, lane^16,
// lane^32, lane^48). v_permlane16_swap / v_permlane32_swap with both operands
// set to x leave {own value, partner value} in the two results, so each
// butterfly step is one VALU swap and one max/add (no LDS round trip), and
// every lane of a head ends with the bitwise-same result.
__device__ __forceinline__ float max_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float sum_over_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// ---------------------------------------------------------------------------
// Integer -> f16 conversion. A byte or nibble placed under the f16 exponent of
// 1024 (0x64xx) reads as 1024 + x exactly. `mg` is 0x64006400 held in a VGPR
// (see and_or). Two forms, the same values up to the single rounding:
//   exact form: (1024 + x - off) * d  - the subtraction is exact, one rounding;
//   fma form:   (1024 + x) * d - 1024 * d in one v_pk_fma_f16 - the product
//               and the subtraction are exact inside the FMA, one rounding,
//               and the constant offset of the format (-8 for Q4_0, -128 for
//               Q8_0 after the sign flip) is added back once per block by a
//               correction MFMA instead of per value. -1024*d must be a
//               finite f16, so this form needs |d| < 64 (see fast_ok).
// High Q4_0 nibbles are taken in place with the mask 0x00F000F0, which reads
// 1024 + 16n: they live in a "x16" frame (K: the matching q is pre-divided by
// 16; V: those output columns are scaled by 1/16 at the end).
// ---------------------------------------------------------------------------
__device__ __forceinline__ f16x2 cvt_exact(uint32_t w, uint32_t mask, f16 off, f16x2 d2, uint32_t mg) {
  const uint32_t v = and_or(w, mask, mg);
  return (bitcast<f16x2>(v) - f16x2{off, off}) * d2;
}
__device__ __forceinline__ f16x2 cvt_fma(uint32_t w, uint32_t mask, f16x2 d2, f16x2 c2, uint32_t mg) {
  const uint32_t v = and_or(w, mask, mg);
  return __builtin_elementwise_fma(bitcast<f16x2>(v), d2, c2);
}
constexpr uint32_t kLoNib = 0x000F000Fu, kHiNib = 0x00F000F0u, kByte = 0x00FF00FFu;

// |d| < 64 (and finite) for both halves / one f16, from the bit pattern.
__device__ __forceinline__ bool scale_ok2(uint32_t x) {
  return ((x & 0x7FFFu) < 0x5400u) && (((x >> 16) & 0x7FFFu) < 0x5400u);
}
__device__ __forceinline__ bool scale_ok(f16 d) { return (bitcast<uint16_t>(d) & 0x7FFFu) < 0x5400u; }

__device__ __forceinline__ f16x8 pack8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// ===========================================================================
// K formats: the A operand of the score MFMA. Lane (m = lane%16, j = lane/16)
// holds token row m of a 16-row group and, for MFMA step s, 8 head-dimension
// values at positions dslot(j, s, 0..7). Loads go through a buffer resource
// whose base is the group's first row; `voff` is the lane's fixed offset.
// ===========================================================================
template <int KT, int D> struct KFmt;

template <int D> struct KFmt<kF16, D> {
  static constexpr int RB = 2 * D;
  static constexpr int S = D / 32;
  struct Raw { u32x4 c[S]; };
  // chunk s of lane j = bytes [64s + 16j, +16): 64 contiguous bytes per row
  // per instruction across the 4 lanes of a row.
  __device__ static uint32_t lane_off(int j) { return 16u * j; }
  __device__ static void load(Raw& r, rsrc_t R, uint32_t voff) {
#pragma unroll
    for (int s = 0; s < S; ++s) r.c[s] = buf_u32x4(R, voff + 64 * s, 0);
  }
  static constexpr bool kQuant = false;
  static constexpr int NBL = 0;            // no block scales
  static constexpr float kOffset = 0.0f;
  __device__ static f16 dscale(const Raw&, int, uint32_t) { return f16(0); }
  template <bool FAST>
  __device__ static f16x8 op(const Raw& r, int s, uint32_t, uint32_t) { return bitcast<f16x8>(r.c[s]); }
  __host__ __device__ static int dslot(int j, int s, int i) { return 32 * s + 8 * j + i; }
  __host__ __device__ static bool hi_slot(int) { return false; }
  __device__ static uint32_t shift(int) { return 0; }
};

// Quantised K: lane j owns the contiguous bytes [j*LB, (j+1)*LB) of the row,
// i.e. whole ggml blocks (2 blocks at D=256, 1 at D=128).
template <int KT, int D> struct KQuantBase {
  static constexpr int RB = row_bytes_of(KT, D);
  static constexpr int S = D / 32;
  static constexpr int LB = RB / 4;
  static constexpr bool kAligned = (LB % 4) == 0;        // every lane window 4-aligned
  static constexpr int NW = kAligned ? LB / 4 : (LB + 2 + 3) / 4;
  struct Raw { uint32_t w[NW]; };
  __device__ static uint32_t shift(int j) { return uint32_t(j * LB) & 3u; }
  __device__ static uint32_t lane_off(int j) { return uint32_t(j * LB) & ~3u; }
  __device__ static void load(Raw& r, rsrc_t R, uint32_t voff) {
    int i = 0;
#pragma unroll
    for (; i + 4 <= NW; i += 4) {
      const u32x4 v = buf_u32x4(R, voff + 4 * i, 0);
      r.w[i] = v[0]; r.w[i + 1] = v[1]; r.w[i + 2] = v[2]; r.w[i + 3] = v[3];
    }
#pragma unroll
    for (; i < NW; ++i) r.w[i] = buf_u32(R, voff + 4 * i, 0);
  }
  // dword at lane byte c (c even, compile-time after unrolling), given the
  // lane window's misalignment sh in {0, 2}.
  __device__ static uint32_t dw(const Raw& r, int c, uint32_t sh) {
    if (c % 4 == 0) {
      const uint32_t a0 = r.w[c / 4];
      if (kAligned) return a0;
      return sh ? align_bytes(r.w[c / 4 + 1], r.w[c / 4], 2) : a0;
    }
    const uint32_t a0 = align_bytes(r.w[c / 4 + 1], r.w[c / 4], 2);
    if (kAligned) return a0;
    return sh ? r.w[c / 4 + 1] : a0;
  }
  // f16 at lane byte c (c even).
  __device__ static f16 half_at(const Raw& r, int c, uint32_t sh) {
    uint32_t w;
    if (c % 4 == 0) {
      w = (kAligned || !sh) ? r.w[c / 4] : (r.w[c / 4] >> 16);
    } else {
      w = (kAligned || !sh) ? (r.w[c / 4] >> 16) : r.w[c / 4 + 1];
    }
    return bitcast<f16>(uint16_t(w & 0xFFFFu));
  }
};

template <int D> struct KFmt<kQ8_0, D> : KQuantBase<kQ8_0, D> {
  using B = KQuantBase<kQ8_0, D>;
  using typename B::Raw;
  static constexpr bool kQuant = true;
  static constexpr int NBL = D / 128;   // ggml blocks per lane
  static constexpr float kOffset = -128.0f;   // fma form holds (q + 128) * d
  __device__ static f16 dscale(const Raw& r, int blk, uint32_t sh) { return B::half_at(r, 34 * blk, sh); }
  // step s: block s/4 of the lane, quants 8*(s%4) .. +7, emitted in the order
  // (0,2),(1,3),(4,6),(5,7) by the byte-pair conversion.
  template <bool FAST>
  __device__ static f16x8 op(const Raw& r, int s, uint32_t sh, uint32_t mg) {
    const int blk = s / 4, base = 8 * (s % 4);
    const f16x2 d2 = splat2(dscale(r, blk, sh));
    const uint32_t u0 = B::dw(r, 34 * blk + 2 + base, sh) ^ 0x80808080u;
    const uint32_t u1 = B::dw(r, 34 * blk + 2 + base + 4, sh) ^ 0x80808080u;
    if constexpr (FAST) {
      const f16x2 c2 = d2 * f16x2{-1024.0f16, -1024.0f16};
      return pack8(cvt_fma(u0, kByte, d2, c2, mg), cvt_fma(u0 >> 8, kByte, d2, c2, mg),
                   cvt_fma(u1, kByte, d2, c2, mg), cvt_fma(u1 >> 8, kByte, d2, c2, mg));
    } else {
      const f16 o = 1152.0f16;
      return pack8(cvt_exact(u0, kByte, o, d2, mg), cvt_exact(u0 >> 8, kByte, o, d2, mg),
                   cvt_exact(u1, kByte, o, d2, mg), cvt_exact(u1 >> 8, kByte, o, d2, mg));
    }
  }
  __host__ __device__ static int dslot(int j, int s, int i) {
    const int order[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    return 32 * (j * NBL + s / 4) + 8 * (s % 4) + order[i];
  }
  __host__ __device__ static bool hi_slot(int) { return false; }
};

template <int D> struct KFmt<kQ4_0, D> : KQuantBase<kQ4_0, D> {
  using B = KQuantBase<kQ4_0, D>;
  using typename B::Raw;
  static constexpr bool kQuant = true;
  static constexpr int NBL = D / 128;
  static constexpr float kOffset = -8.0f;     // fma form holds n * d
  __device__ static f16 dscale(const Raw& r, int blk, uint32_t sh) { return B::half_at(r, 18 * blk, sh); }
  // step s: block s/4, nibble bytes 4c..4c+3 (c = s%4) -> elements
  // 4c, 4c+2, 16+4c, 18+4c, 4c+1, 4c+3, 17+4c, 19+4c; in the fma form the
  // high nibbles (slots 2, 3, 6, 7) are in the x16 frame.
  template <bool FAST>
  __device__ static f16x8 op(const Raw& r, int s, uint32_t sh, uint32_t mg) {
    const int blk = s / 4, c = s % 4;
    const f16x2 d2 = splat2(dscale(r, blk, sh));
    const uint32_t w = B::dw(r, 18 * blk + 2 + 4 * c, sh);
    const uint32_t w8 = w >> 8;
    if constexpr (FAST) {
      const f16x2 c2 = d2 * f16x2{-1024.0f16, -1024.0f16};
      return pack8(cvt_fma(w, kLoNib, d2, c2, mg), cvt_fma(w, kHiNib, d2, c2, mg),
                   cvt_fma(w8, kLoNib, d2, c2, mg), cvt_fma(w8, kHiNib, d2, c2, mg));
    } else {
      // exact form in true values (no x16 frame: it would overflow f16 once
      // |d| > 512); the caller multiplies the q of slots 2, 3, 6, 7 back by 16
      const f16 o = 1032.0f16;
      return pack8(cvt_exact(w, kLoNib, o, d2, mg), cvt_exact(w >> 4, kLoNib, o, d2, mg),
                   cvt_exact(w8, kLoNib, o, d2, mg), cvt_exact(w >> 12, kLoNib, o, d2, mg));
    }
  }
  __host__ __device__ static int dslot(int j, int s, int i) {
    const int c = s % 4;
    const int order[8] = {0, 2, 16, 18, 1, 3, 17, 19};
    return 32 * (j * NBL + s / 4) + 4 * c + order[i];
  }
  __host__ __device__ static bool hi_slot(int i) { return (i & 2) != 0; }
};

// ===========================================================================
// V formats: the A operand of the PV MFMA is V^T. Lane (m, j) holds, for
// d-tile e, head-dimension position dv(m, e) of the lane's 8 token rows
// (rows 4j..4j+3 of group 0 and 16+4j..16+4j+3 of group 1). A load names the
// lane's first row by `voff`; row i of the group is reached with the scalar
// offset i*stride.
// ===========================================================================
template <int VT, int D> struct VFmt;

template <int D> struct VFmt<kF16, D> {
  static constexpr int RB = 2 * D;
  static constexpr int E = D / 16;       // d-tiles
  static constexpr int NCH = D / 128;    // 16-byte chunks per row per lane
  static constexpr bool kQuant = false;
  __host__ __device__ static bool hi_col(int) { return false; }
  struct Lane { uint32_t voff, sh; };
  struct Raw { u32x4 c[NCH]; };
  // 16 lanes m read 256 contiguous bytes of a row per instruction.
  __device__ static Lane lane(int m, uint32_t row0) { return Lane{row0 + 16u * m, 0}; }
  __device__ static void load(Raw& r, rsrc_t R, const Lane& L, uint32_t soff) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) r.c[c] = buf_u32x4(R, L.voff + 256 * c, soff);
  }
  __device__ static void kill(Raw& r) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) r.c[c] = u32x4{0, 0, 0, 0};
  }
  __host__ __device__ static int dv(int m, int e) { return 8 * (m + 16 * (e / 8)) + e % 8; }
  // Pack half k of chunk e/8 of rows (2p, 2p+1) into dword p.
  __device__ static f16x8 op(const Raw* R, int e) {
    const int c = e / 8, k = e % 8;
    const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p) o[p] = perm_bytes(R[2 * p + 1].c[c][k / 2], R[2 * p].c[c][k / 2], sel);
    return bitcast<f16x8>(o);
  }
};

// Quantised V: lane m covers EPL = D/16 head positions, all inside one ggml
// block; the quant bytes are fetched through a dword window and realigned.
template <int VT, int D> struct VQuantBase {
  static constexpr int RB = row_bytes_of(VT, D);
  static constexpr int E = D / 16;
  static constexpr int EPL = D / 16;           // positions per lane
  static constexpr bool kQuant = true;
  static constexpr int BB = (VT == kQ8_0) ? 34 : 18;       // ggml block bytes
  static constexpr int QB = (VT == kQ8_0) ? EPL : EPL / 2; // quant bytes per lane
  static constexpr int ND = QB / 4;            // realigned quant dwords
  static constexpr int NW = ND + 1;            // window dwords (covers a 2-byte skew)
  struct Lane { uint32_t voff, last, doff, sh; };
  struct Raw { uint32_t w[NW]; f16 d; };
  __device__ static Lane lane(int m, uint32_t row0) {
    // quant bytes of lane m start at byte qoff of the row
    const int per_blk = (VT == kQ8_0) ? 32 : 16;           // quant bytes per block
    const int qidx = m * QB;
    const int blk = qidx / per_blk, st = qidx % per_blk;
    const uint32_t qoff = uint32_t(BB * blk + 2 + st);
    const uint32_t woff = qoff & ~3u;
    // the last window dword is only needed when the window is skewed; keep
    // its address inside the row so the last row of a pool is never over-read
    const uint32_t lastoff = woff + 4u * (NW - 1);
    Lane L;
    L.voff = row0 + woff;
    L.last = row0 + (lastoff + 4u <= uint32_t(RB) ? lastoff : uint32_t(RB) - 4u);
    L.doff = row0 + uint32_t(BB * blk);
    L.sh = qoff & 3u;
    return L;
  }
  __device__ static void load(Raw& r, rsrc_t R, const Lane& L, uint32_t soff) {
    if constexpr (NW - 1 == 4) {
      const u32x4 v = buf_u32x4(R, L.voff, soff);
      r.w[0] = v[0]; r.w[1] = v[1]; r.w[2] = v[2]; r.w[3] = v[3];
    } else if constexpr (NW - 1 == 2) {
      const u32x2 v = buf_u32x2(R, L.voff, soff);
      r.w[0] = v[0]; r.w[1] = v[1];
    } else {
#pragma unroll
      for (int i = 0; i < NW - 1; ++i) r.w[i] = buf_u32(R, L.voff + 4 * i, soff);
    }
    r.w[NW - 1] = buf_u32(R, L.last, soff);
    r.d = bitcast<f16>(buf_u16(R, L.doff, soff));
  }
  __device__ static void kill(Raw& r) { r.d = f16(0); }
  __device__ static void realign(const Raw& r, uint32_t sh, uint32_t* q) {
#pragma unroll
    for (int i = 0; i < ND; ++i) q[i] = align_bytes(r.w[i + 1], r.w[i], sh);
  }
};

template <int D> struct VFmt<kQ8_0, D> : VQuantBase<kQ8_0, D> {
  using B = VQuantBase<kQ8_0, D>;
  static constexpr float kOffset = -128.0f;   // fma form holds (q + 128) * d
  __host__ __device__ static int dv(int m, int e) { return m * B::EPL + e; }
  __host__ __device__ static bool hi_col(int) { return false; }
  // q: realigned quant dwords of the 8 rows [row][ND]; dd[p] = (d_2p, d_2p+1),
  // cc[p] = -1024 * dd[p]. perm gives (q_A, 0, q_B, 0); XOR 0x64806480 flips
  // the sign bits and plants the exponent bytes in one instruction.
  template <bool FAST>
  __device__ static f16x8 op_q(const uint32_t (*q)[B::ND], const f16x2* dd, const f16x2* cc, int e,
                               uint32_t) {
    const int k = e % 4, i = e / 4;
    const uint32_t sel = uint32_t(k) | (0x0Cu << 8) | (uint32_t(4 + k) << 16) | (0x0Cu << 24);
    f16x2 o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const f16x2 x = bitcast<f16x2>(perm_bytes(q[2 * p + 1][i], q[2 * p][i], sel) ^ 0x64806480u);
      if constexpr (FAST) o[p] = __builtin_elementwise_fma(x, dd[p], cc[p]);
      else o[p] = (x - f16x2{1152.0f16, 1152.0f16}) * dd[p];
    }
    return pack8(o[0], o[1], o[2], o[3]);
  }
};

template <int D> struct VFmt<kQ4_0, D> : VQuantBase<kQ4_0, D> {
  using B = VQuantBase<kQ4_0, D>;
  static constexpr float kOffset = -8.0f;     // fma form holds n * d
  // e < QB: low nibble of quant byte e; e >= QB: high nibble of byte e-QB
  // (in the x16 frame).
  __host__ __device__ static int dv(int m, int e) {
    const int qidx = m * B::QB;
    const int blk = qidx / 16, st = qidx % 16;
    return 32 * blk + (e < B::QB ? st + e : 16 + st + (e - B::QB));
  }
  __host__ __device__ static bool hi_col(int e) { return e >= B::QB; }
  template <bool FAST>
  __device__ static f16x8 op_q(const uint32_t (*q)[B::ND], const f16x2* dd, const f16x2* cc, int e,
                               uint32_t mg) {
    const bool hi = e >= B::QB;
    const int byte = hi ? e - B::QB : e;
    const int k = byte % 4, i = byte / 4;
    const uint32_t sel = uint32_t(k) | (0x0Cu << 8) | (uint32_t(4 + k) << 16) | (0x0Cu << 24);
    const uint32_t mask = hi ? kHiNib : kLoNib;
    f16x2 o[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t x = perm_bytes(q[2 * p + 1][i], q[2 * p][i], sel);
      if constexpr (FAST) o[p] = cvt_fma(x, mask, dd[p], cc[p], mg);
      else o[p] = cvt_exact(hi ? (x >> 4) : x, kLoNib, 1032.0f16, dd[p], mg);   // true values
    }
    return pack8(o[0], o[1], o[2], o[3]);
  }
};

// ===========================================================================
// The kernel
// ===========================================================================
// 16-row groups per tile: 4 (64 tokens) when both formats are Q4_0, whose
template <int KT, int VT>
struct TileGroups {
  static constexpr int value = 2;
};

template <int KT, int VT, int D>
struct Tile {
  using KF = KFmt<KT, D>;
  using VF = VFmt<VT, D>;
  static constexpr int NG = TileGroups<KT, VT>::value;
  typename KF::Raw k[NG];
  typename VF::Raw v[NG / 2][8];   // per group pair: the lane's 8 token rows
};

struct Unit {
  int b, g, p, t_begin, t_end;
};


// LDS layout of a workgroup (in 4-byte words):
//   unit_start[B+1] | lens[B] | pad | ids[kNid+1] | qop[D/32][64][4] | qs[r*D]
//   | comb[3*(r*D+32)]
// qop is the Q operand of the score MFMA in lane order (one 16-byte operand
// per lane and step, shared by the four waves); comb doubles as the scratch
// of the start-up prefix scan (needs kThreads words).
constexpr int kNid = 2048;     // block ids staged per segment of a partition

__host__ __device__ inline int lds_words(int B, int r, int D) {
  const int pre = ((2 * B + 1) + 3) & ~3;
  const int ids = (kNid + 1 + 3) & ~3;
  const int qop = (D / 32) * 64 * 4;
  const int comb = 3 * (r * D + 32) > kThreads ? 3 * (r * D + 32) : kThreads;
  return pre + ids + qop + r * D + comb;
}

// Workgroups per CU the register allocation is held to: two (256 VGPRs per
// wave, two waves per SIMD) where the kernel fits without spilling - small
// rows (Q4_0 K and V) or D=128 - else one.
template <int KT, int VT, int D>
struct MinBlocks {
  static constexpr int value = (D == 128 || (KT == kQ4_0 && VT == kQ4_0)) ? 2 : 1;
};

template <int KT, int VT, int D>
__global__ void __launch_bounds__(kThreads, (MinBlocks<KT, VT, D>::value))
decode_kernel(const DecodeArgs a) {
  using KF = KFmt<KT, D>;
  using VF = VFmt<VT, D>;
  using T = Tile<KT, VT, D>;
  constexpr int S = D / 32;      // score MFMA steps
  constexpr int E = D / 16;      // PV d-tiles
  constexpr int NG = T::NG;      // 16-row groups per tile
  constexpr int kTile = 16 * NG; // tokens per tile

  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* unit_start = reinterpret_cast<int32_t*>(smem);
  int32_t* lens = unit_start + (a.B + 1);
  int32_t* ids = reinterpret_cast<int32_t*>(smem) + (((2 * a.B + 1) + 3) & ~3);
  f16x8* qop_lds = reinterpret_cast<f16x8*>(ids + ((kNid + 1 + 3) & ~3));
  float* qs = reinterpret_cast<float*>(qop_lds + S * 64);
  float* comb = qs + a.r * D;
  const int comb_stride = a.r * D + 32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int m = lane & 15;
  const int j = lane >> 4;

  // ---- per-workgroup prefix of live partitions per sequence -------------
  {
    const int per = (a.B + kThreads - 1) / kThreads;
    const int b0 = tid * per;
    const int cap = a.cap_tokens;
    int local = 0;
    uint32_t st = 0;
    for (int b = b0; b < b0 + per && b < a.B; ++b) {
      int L = a.seq_len[b];
      if (L < 0 || L > cap) { st |= 2u; L = L < 0 ? 0 : cap; }
      lens[b] = L;
      local += (L + a.psize - 1) / a.psize;
    }
    if (st && blockIdx.x == 0) atomicOr(a.status, st);
    // block-wide inclusive scan of `local` (Hillis-Steele over LDS)
    int* scan = reinterpret_cast<int*>(comb);
    scan[tid] = local;
    __syncthreads();
    for (int off = 1; off < kThreads; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    int run = scan[tid] - local;
    for (int b = b0; b < b0 + per && b < a.B; ++b) {
      unit_start[b] = run;
      run += (lens[b] + a.psize - 1) / a.psize;
    }
    if (tid == kThreads - 1) unit_start[a.B] = scan[tid];
    __syncthreads();
  }
  const int n_bp = __builtin_amdgcn_readfirstlane(unit_start[a.B]);
  const int n_units = n_bp * a.Hkv;
  const int G = gridDim.x;

  // In direct mode no merge follows: an empty sequence's rows are zeroed here.
  if (a.direct) {
    for (int b = blockIdx.x; b < a.B; b += G) {
      if (lens[b] != 0) continue;
      float* o = a.out + int64_t(b) * a.Hq * D;
      for (int i = tid; i < a.Hq * D; i += kThreads) o[i] = 0.0f;
    }
  }

  // ---- XCD-aware order: consecutive logical units land on one XCD -------
  const int xcd = blockIdx.x % 8, kk = blockIdx.x / 8;
  const int cb = G / 8, rem = G % 8;
  const int logical = xcd * cb + (xcd < rem ? xcd : rem) + kk;

  const uint32_t kstride = uint32_t(a.Hkv) * KF::RB;   // bytes between token rows
  const uint32_t vstride = uint32_t(a.Hkv) * VF::RB;
  const uint32_t ksh = KF::shift(j);
  const uint32_t kvoff = m * kstride + KF::lane_off(j);
  const auto vl = VF::lane(m, 4u * j * vstride);
  const uint32_t mg = opaque_vgpr(kMagic);
  const int bs_mask = (1 << a.bs_shift) - 1;
  const int seg_tokens = kNid << a.bs_shift;

  for (int u = logical; u < n_units; u += G) {
    // ---- locate the unit ---------------------------------------------------
    const int bp = u / a.Hkv;
    Unit U;
    U.g = u - bp * a.Hkv;
    {
      int lo = 0, hi = a.B - 1;            // largest b with unit_start[b] <= bp
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (unit_start[mid] <= bp) lo = mid; else hi = mid - 1;
      }
      U.b = __builtin_amdgcn_readfirstlane(lo);
    }
    U.p = bp - __builtin_amdgcn_readfirstlane(unit_start[U.b]);
    U.t_begin = U.p * a.psize;
    U.t_end = min(__builtin_amdgcn_readfirstlane(lens[U.b]), U.t_begin + a.psize);

    // ---- stage the group's r query rows (scaled by scale*log2 e) ----------
    {
      const float* qg = a.q + (int64_t(U.b) * a.Hq + U.g * a.r) * D;
      for (int i = tid; i < a.r * D / 4; i += kThreads) {
        float4 v = reinterpret_cast<const float4*>(qg)[i];
        v.x *= a.qscale; v.y *= a.qscale; v.z *= a.qscale; v.w *= a.qscale;
        reinterpret_cast<float4*>(qs)[i] = v;
      }
    }

    f16x8 kcorr;           // B operand of the K offset correction (fma form)
    bool q_fast = true;    // the correction operand is representable in f16
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[E];
    f32x4 vcorr = f32x4{0.f, 0.f, 0.f, 0.f};   // sum_t d_t * p_t (V offset correction)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    int bad = 0;
    bool redo = false;     // a tile needed the exact conversion

    // ---- tile loader: one block id per 16-row group ------------------------
    // A tile index past the range still issues its loads, through a
    // zero-size buffer resource: they return 0 without touching memory, so
    // every path through the loop has the same loads in flight and the
    // compiler's wait counts stay exact.
    auto load_tile = [&](T& t, int base_t, int nt, int kt, auto get_id) __attribute__((always_inline)) {
      const bool valid = kt < nt;
      const int t0 = base_t + (valid ? kt : nt - 1) * kTile;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        const int tg = t0 + 16 * gi;
        const bool live = tg < U.t_end;
        const int tq = live ? tg : U.t_end - 1;
        const int32_t id = get_id(tq >> a.bs_shift);
        const int slot0 = live ? (tg & bs_mask) : 0;
        const rsrc_t kr = make_rsrc(a.k_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, U.g, KF::RB),
                                    valid ? 16u * kstride : 0u);
        const rsrc_t vr = make_rsrc(a.v_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, U.g, VF::RB),
                                    valid ? 16u * vstride : 0u);
        KF::load(t.k[gi], kr, kvoff);
#pragma unroll
        for (int i = 0; i < 4; ++i) VF::load(t.v[gi / 2][4 * (gi % 2) + i], vr, vl, i * vstride);
      }
    };

    // ---- tile compute: scores, online softmax (exp2), PV ----------------
    auto compute_tile = [&](T& t, int t0, auto fast_c) __attribute__((always_inline)) {
      constexpr bool FAST = decltype(fast_c)::value;
      const bool full = t0 + kTile <= U.t_end;
      if (!full) {
        // zero V rows past the end so 0 * junk never reaches the PV MFMA
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + 16 * gi + 4 * j + i >= U.t_end) VF::kill(t.v[gi / 2][4 * (gi % 2) + i]);
      }
      // The fma-form conversions need every live block scale below 64 in
      // magnitude (dead V rows have a zeroed scale; dead K rows are ignored).
      if constexpr (FAST && (KF::kQuant || VF::kQuant)) {
        bool ok = q_fast;
        if constexpr (KF::kQuant) {
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            const bool live_row = t0 + 16 * gi + m < U.t_end;
#pragma unroll
            for (int bl = 0; bl < KF::NBL; ++bl)
              ok = ok && (!live_row || scale_ok(KF::dscale(t.k[gi], bl, ksh)));
          }
        }
        if constexpr (VF::kQuant) {
#pragma unroll
          for (int pp = 0; pp < NG / 2; ++pp)
#pragma unroll
            for (int i = 0; i < 8; ++i) ok = ok && scale_ok(t.v[pp][i].d);
        }
        redo |= !__all(ok);
      }

      f32x4 sc[NG];
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) sc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
      {
        constexpr bool F = FAST;
#pragma unroll
        for (int s = 0; s < S; ++s) {
          f16x8 qv = qop_lds[s * 64 + lane];
          if constexpr (!F) {
#pragma unroll
            for (int i = 0; i < 8; ++i)
              if (KF::hi_slot(i)) qv[i] *= 16.0f16;   // the exact form holds true values
          }
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) sc[gi] = mfma(KF::template op<F>(t.k[gi], s, ksh, mg), qv, sc[gi]);
        }
        if constexpr (F && KF::kQuant) {
          // sum over the lane's blocks of d * offset * sum(q): one MFMA per group
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) {
            f16x8 ca = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
            for (int bl = 0; bl < KF::NBL; ++bl) {
              const f16 d = KF::dscale(t.k[gi], bl, ksh);
              ca[2 * bl] = d;
              ca[2 * bl + 1] = d;
            }
            sc[gi] = mfma(ca, kcorr, sc[gi]);
          }
        }
      }
      if (!full) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + 16 * gi + 4 * j + i >= U.t_end) sc[gi][i] = -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        mx = fmaxf(mx, fmaxf(fmaxf(sc[gi][0], sc[gi][1]), fmaxf(sc[gi][2], sc[gi][3])));
      mx = max_over_rows(mx);
      // Lazy rescale: the softmax is invariant to the reference m, so m_run
      // only moves when some head's max exceeds it by more than kSlack
      // (then p <= 2^kSlack, safe in f16) - the accumulators are rescaled
      // a handful of times per partition instead of at most tiles (the
      // lucebox page skips the rescale when the max is unchanged).
      if (__any(mx > m_run + kSlack)) {
        const float m_new = fmaxf(m_run, mx);
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
        l_run *= alpha;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] *= alpha;
        vcorr *= alpha;
        m_run = m_new;
      }
      float ps = 0.0f;
#pragma unroll
      for (int pp = 0; pp < NG / 2; ++pp) {
        float p[8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[4 * h2 + i] = __builtin_amdgcn_exp2f(sc[2 * pp + h2][i] - m_run);
        ps += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
        f16x8 pop;
#pragma unroll
        for (int i = 0; i < 8; ++i) pop[i] = f16(p[i]);
        if constexpr (VF::kQuant) {
          uint32_t q[8][VF::ND];
          f16x2 dd[4];
#pragma unroll
          for (int i = 0; i < 8; ++i) VF::realign(t.v[pp][i], vl.sh, q[i]);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dd[qq] = f16x2{t.v[pp][2 * qq].d, t.v[pp][2 * qq + 1].d};
          if constexpr (FAST) {
            f16x2 cc[4];
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) cc[qq] = dd[qq] * f16x2{-1024.0f16, -1024.0f16};
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = mfma(VF::template op_q<true>(q, dd, cc, e, mg), pop, acc[e]);
            // sum_t d_t p_t per (row block, head): the offset correction
            vcorr = mfma(pack8(dd[0], dd[1], dd[2], dd[3]), pop, vcorr);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = mfma(VF::template op_q<false>(q, dd, dd, e, mg), pop, acc[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = mfma(VF::op(t.v[pp], e), pop, acc[e]);
        }
      }
      l_run += sum_over_rows(ps);
    };

    for (int seg_t0 = U.t_begin; seg_t0 < U.t_end; seg_t0 += seg_tokens) {
      const int seg_t1 = min(U.t_end, seg_t0 + seg_tokens);
      const int jb0 = seg_t0 >> a.bs_shift;
      const int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
      __syncthreads();                       // earlier readers of ids[] are done
      int badl = 0;
      for (int i = tid; i < nb; i += kThreads) {
        int32_t id = block_of(a.table, U.b, a.max_blocks, jb0 + i);
        if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
        ids[i] = id;
      }
      bad |= __syncthreads_or(badl);         // also publishes ids[] and qs[]

      if (seg_t0 == U.t_begin) {
        // Q operand: column n = lane%16 holds head g*r+n (zero when n >= r);
        // slots that meet x16-frame K values hold q/16. Every wave builds it
        // (it needs its own correction operand), wave 0 publishes it to LDS.
        f16x8 qop[S];
        const int n = m < a.r ? m : a.r - 1;
        const float keep = m < a.r ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i)
            qop[s][i] = f16(qs[n * D + KF::dslot(j, s, i)] * (KF::hi_slot(i) ? keep * 0.0625f : keep));
        if (wave == 0) {
#pragma unroll
          for (int s = 0; s < S; ++s) qop_lds[s * 64 + lane] = qop[s];
        }
        if constexpr (KF::kQuant) {
          // Correction operand of the fma form: for each of the lane's ggml
          // blocks, offset * (sum of the q values this lane's slots carry for
          // that block), split into an f16 high and low part so the product
          // with the block scale is carried to ~22 bits.
          constexpr int NBL = KF::NBL;
          float qsum[NBL];
#pragma unroll
          for (int bl = 0; bl < NBL; ++bl) {
            float acc_q = 0.0f;
#pragma unroll
            for (int s = 4 * bl; s < 4 * bl + 4; ++s)
#pragma unroll
              for (int i = 0; i < 8; ++i) acc_q += float(qop[s][i]) * (KF::hi_slot(i) ? 16.0f : 1.0f);
            qsum[bl] = acc_q * KF::kOffset;
          }
          kcorr = f16x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
          for (int bl = 0; bl < NBL; ++bl) {
            q_fast = q_fast && fabsf(qsum[bl]) < 32768.0f;
            const f16 hi = f16(qsum[bl]);
            kcorr[2 * bl] = hi;
            kcorr[2 * bl + 1] = f16(qsum[bl] - float(hi));
          }
        }
        __syncthreads();                     // qop_lds published
      }

      const int ntiles = (seg_t1 - seg_t0 + kTile - 1) / kTile;
      // ---- wave w streams tiles w, w+4, ... with one tile prefetched ------
      // (block ids come from the LDS copy of this segment)
      auto seg_id = [&](int jb) __attribute__((always_inline)) {
        return __builtin_amdgcn_readfirstlane(ids[jb - jb0]);
      };
      int k = wave;
      if (k < ntiles) {
        T A, Bt;
        load_tile(A, seg_t0, ntiles, k, seg_id);
        while (true) {
          load_tile(Bt, seg_t0, ntiles, k + kWaves, seg_id);
          compute_tile(A, seg_t0 + k * kTile, std::true_type{});
          k += kWaves;
          if (k >= ntiles) break;
          load_tile(A, seg_t0, ntiles, k + kWaves, seg_id);
          compute_tile(Bt, seg_t0 + k * kTile, std::true_type{});
          k += kWaves;
          if (k >= ntiles) break;
        }
      }
    }

    // ---- rare path: a tile had a block scale the fma form cannot take -----
    // The wave drops what it accumulated and recomputes all its tiles of the
    // unit with the exact conversion (block ids read from the table).
    if constexpr (KF::kQuant || VF::kQuant) {
      if (redo) {
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
        vcorr = f32x4{0.f, 0.f, 0.f, 0.f};
        auto table_id = [&](int jb) __attribute__((always_inline)) {
          int32_t id = block_of(a.table, U.b, a.max_blocks, jb);
          return uint32_t(id) < uint32_t(a.nblocks) ? id : 0;   // bad ids already flagged
        };
        const int nt_all = (U.t_end - U.t_begin + kTile - 1) / kTile;
        for (int kr = wave; kr < nt_all; kr += kWaves) {
          T A;
          load_tile(A, U.t_begin, nt_all, kr, table_id);
          compute_tile(A, U.t_begin + kr * kTile, std::false_type{});
        }
      }
    }

    // ---- undo the x16 frame and add the V offset correction ---------------
    // (a wave that recomputed with the exact form holds true values already)
    if constexpr (VF::kQuant) {
      if (!redo) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float sc = VF::hi_col(e) ? 0.0625f : 1.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[e][i] = acc[e][i] * sc + VF::kOffset * vcorr[i];
      }
      }
    }

    // ---- combine the four waves through LDS -------------------------------
    const int n = m;
    if (wave > 0) {
      float* cw = comb + (wave - 1) * comb_stride;
      if (n < a.r) {
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) cw[n * D + VF::dv(4 * j + i, e)] = acc[e][i];
        if (j == 0) {
          cw[a.r * D + n] = m_run;
          cw[a.r * D + 16 + n] = l_run;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      float M = m_run;
      float mw[3], lw[3];
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        const float* cw = comb + w * comb_stride;
        mw[w] = n < a.r ? cw[a.r * D + n] : -INFINITY;
        lw[w] = n < a.r ? cw[a.r * D + 16 + n] : 0.0f;
        M = fmaxf(M, mw[w]);
      }
      const float c0 = __builtin_amdgcn_exp2f(m_run - M);
      float cwt[3];
      float l = l_run * c0;
#pragma unroll
      for (int w = 0; w < 3; ++w) {
        cwt[w] = __builtin_amdgcn_exp2f(mw[w] - M);
        l += lw[w] * cwt[w];
      }
      const float inv = 1.0f / l;
      const int h = U.g * a.r + n;
      if (bad && lane == 0) atomicOr(a.status, 1u);
      if (n < a.r) {
        float* dst;
        if (a.direct) {
          dst = a.out + (int64_t(U.b) * a.Hq + h) * D;
        } else {
          const int64_t row = (int64_t(U.b) * a.Hq + h) * a.p_max + U.p;
          dst = a.part_o + row * D;
          if (j == 0) {
            a.part_ml[2 * row] = bad ? __builtin_nanf("") : M;
            a.part_ml[2 * row + 1] = l;
          }
        }
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d = VF::dv(4 * j + i, e);
            float v = acc[e][i] * c0;
#pragma unroll
            for (int w = 0; w < 3; ++w) v += comb[w * comb_stride + n * D + d] * cwt[w];
            dst[d] = bad ? __builtin_nanf("") : v * inv;
          }
      }
    }
    __syncthreads();
  }
}

template <int KT, int VT, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = size_t(lds_words(a.B, a.r, D)) * 4;
  hipLaunchKernelGGL((decode_kernel<KT, VT, D>), dim3(a.grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.k_type * 3 + a.v_type) {
    case 0: return launch_typed<kF16, kF16, D>(a, s);
    case 1: return launch_typed<kF16, kQ8_0, D>(a, s);
    case 2: return launch_typed<kF16, kQ4_0, D>(a, s);
    case 3: return launch_typed<kQ8_0, kF16, D>(a, s);
    case 4: return launch_typed<kQ8_0, kQ8_0, D>(a, s);
    case 5: return launch_typed<kQ8_0, kQ4_0, D>(a, s);
    case 6: return launch_typed<kQ4_0, kF16, D>(a, s);
    case 7: return launch_typed<kQ4_0, kQ8_0, D>(a, s);
    case 8: return launch_typed<kQ4_0, kQ4_0, D>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 256) return launch_d<256>(a, stream);
  if (a.D == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
