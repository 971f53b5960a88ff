// Device code shared by the two decode kernels (register-streaming and
// LDS-staged): MFMA wrappers, the per-head reductions, the integer -> f16
// conversions and the K/V row formats in MFMA operand order, plus the
// per-workgroup prefix of live partitions that both kernels schedule from.
#pragma once
#include "pa_device.h"
#include "pa_host.h"

namespace pa {

constexpr uint32_t kMagic = 0x64006400u;   // f16 1024.0 in both halves
constexpr float kSlack = 8.0f;             // lazy-rescale slack (log2 units)

// 16x16x32 f16 -> f32: A lane (row l%16, k 8*(l/16)+i), B lane (col l%16,
// k 8*(l/16)+i), C lane (rows 4*(l/16)+i, col l%16).
__device__ __forceinline__ f32x4 mfma(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// 16x16x16 f16 -> f32: the same layout with k 4*(l/16)+i.
__device__ __forceinline__ f32x4 mfma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
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
// Integer -> f16 conversion: a byte or nibble placed under the f16 exponent
// of 1024 (0x64xx) reads as 1024 + x exactly; subtracting the offset is exact,
// so the only rounding is the multiplication by the block scale d.
// `mg` is 0x64006400 held in a VGPR (see and_or).
// ---------------------------------------------------------------------------
// Signed int8 bytes 0 and 2 of `u` (already XORed with 0x80) -> d * q.
__device__ __forceinline__ f16x2 i8pair_to_f16(uint32_t u_shifted, f16x2 d2, uint32_t mg) {
  const uint32_t v = and_or(u_shifted, 0x00FF00FFu, mg);
  return (bitcast<f16x2>(v) - f16x2{1152.0f16, 1152.0f16}) * d2;
}
// Nibbles at bits 0-3 and 16-19 -> (n - 8) * d.
__device__ __forceinline__ f16x2 nib_pair_to_f16(uint32_t w_shifted, f16x2 d2, uint32_t mg) {
  const uint32_t v = and_or(w_shifted, 0x000F000Fu, mg);
  return (bitcast<f16x2>(v) - f16x2{1032.0f16, 1032.0f16}) * d2;
}

// Nibble value times scale, offset left out: n*d from x = 1024 + n (the
// magic-number f16). Two forms of the same single rounding of n*d:
//   fma form:   fma(x, d, -1024*d) - the product and the subtraction are exact
//               inside the FMA; needs -1024*d finite, i.e. |d| < 64;
//   exact form: (x - 1024) * d - the subtraction is exact.
// The format offset (-8 for Q4_0) is added back once per block by a
// correction term, so both forms give bit-identical results.
template <bool FMA>
__device__ __forceinline__ f16x2 nd_pair(uint32_t w_shifted, f16x2 d2, f16x2 c2, uint32_t mg) {
  const f16x2 x = bitcast<f16x2>(and_or(w_shifted, 0x000F000Fu, mg));
  if constexpr (FMA) return __builtin_elementwise_fma(x, d2, c2);
  else return (x - f16x2{1024.0f16, 1024.0f16}) * d2;
}
// The same in place for both nibbles of bytes 0 and 2 of w (no shift): the low
// nibble gives n*d, the high nibble, taken under the mask 0x00F000F0, reads as
// 1024 + 16n and gives 16*n*d - the "x16 frame", undone by the consumer (q/16
// for K, 1/16 on the output columns for V). fma form only: |d| < 64 keeps
// -1024*d finite and 16*15*|d| inside the f16 range.
__device__ __forceinline__ f16x2 nd_lo(uint32_t w, f16x2 d2, f16x2 c2, uint32_t mg) {
  return __builtin_elementwise_fma(bitcast<f16x2>(and_or(w, 0x000F000Fu, mg)), d2, c2);
}
__device__ __forceinline__ f16x2 nd_hi16(uint32_t w, f16x2 d2, f16x2 c2, uint32_t mg) {
  return __builtin_elementwise_fma(bitcast<f16x2>(and_or(w, 0x00F000F0u, mg)), d2, c2);
}
// Power-of-two shift k >= 0 that brings |d| below 64 (d * 2^-k keeps -1024*d
// finite for the fma form), from the f16 exponent field: 64 has field 21.
__device__ __forceinline__ int scale_shift(f16 d) {
  const int e = int((bitcast<uint16_t>(d) & 0x7FFFu) >> 10);
  return e > 20 ? e - 20 : 0;
}
// 2^-k as an f16 pair (0 <= k <= 11; exact).
__device__ __forceinline__ f16x2 pow2_neg_f16x2(int k) {
  const uint32_t h = uint32_t(15 - k) << 10;
  return bitcast<f16x2>(h | (h << 16));
}
// Largest k of the wave, given each lane's k (usually all zero; the loop over
// thresholds only runs when some lane needs a shift).
__device__ __forceinline__ int wave_max_shift(int k) {
  if (!__any(k > 0)) return 0;
  for (int t = 11; t > 1; --t)
    if (__any(k >= t)) return t;
  return 1;
}

__device__ __forceinline__ f16x8 pack8(f16x2 a, f16x2 b, f16x2 c, f16x2 d) {
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// NP f16 pairs -> the A operand of a 16x16x(8*NP) MFMA.
template <int NP> struct OpVec;
template <> struct OpVec<4> {
  typedef f16x8 type;
  __device__ static f16x8 pack(const f16x2* o) { return pack8(o[0], o[1], o[2], o[3]); }
  __device__ static f16x8 from(const u32x4& w) { return bitcast<f16x8>(w); }
};
template <> struct OpVec<2> {
  typedef f16x4 type;
  __device__ static f16x4 pack(const f16x2* o) { return f16x4{o[0][0], o[0][1], o[1][0], o[1][1]}; }
  __device__ static f16x4 from(const u32x4& w) { return bitcast<f16x4>(u32x2{w[0], w[1]}); }
};

// ===========================================================================
// K formats: the A operand of the score MFMA. Lane (m = lane%16, j = lane/16)
// holds token row m of a 16-row group and, for MFMA step s, 8 head-dimension
// values at positions dslot(j, s, 0..7). `load` reads the lane's bytes from
// HBM through a buffer resource whose base is the group's first row (`voff`
// is the lane's fixed offset); `load_lds` reads the same bytes of one row
// staged in LDS (`p` = row start + lane_off(j)).
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
  __device__ static void load_lds(Raw& r, const uint8_t* p) {
#pragma unroll
    for (int s = 0; s < S; ++s) r.c[s] = *reinterpret_cast<const u32x4*>(p + 64 * s);
  }
  __device__ static f16x8 op(const Raw& r, int s, uint32_t, uint32_t) { return bitcast<f16x8>(r.c[s]); }
  __host__ __device__ static constexpr int dslot(int j, int s, int i) { return 32 * s + 8 * j + i; }
  // dslot(j, s, i) = dslot(j, s, 0) + qoff(i): two aligned groups of four
  // positions, the second kQGap past the first (load_q_slots)
  static constexpr int kQGap = 4;
  __host__ __device__ static constexpr int qsel(int i) { return i; }
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
  __device__ static void load_lds(Raw& r, const uint8_t* p) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < NW; ++i) r.w[i] = w[i];
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
  static constexpr int NBL = D / 128;   // ggml blocks per lane
  // step s: block s/4 of the lane, quants 8*(s%4) .. +7, emitted in the order
  // (0,2),(1,3),(4,6),(5,7) by the byte-pair conversion.
  __device__ static f16x8 op(const Raw& r, int s, uint32_t sh, uint32_t mg) {
    const int blk = s / 4, base = 8 * (s % 4);
    const f16x2 d2 = splat2(B::half_at(r, 34 * blk, sh));
    const uint32_t u0 = B::dw(r, 34 * blk + 2 + base, sh) ^ 0x80808080u;
    const uint32_t u1 = B::dw(r, 34 * blk + 2 + base + 4, sh) ^ 0x80808080u;
    return pack8(i8pair_to_f16(u0, d2, mg), i8pair_to_f16(u0 >> 8, d2, mg),
                 i8pair_to_f16(u1, d2, mg), i8pair_to_f16(u1 >> 8, d2, mg));
  }
  __host__ __device__ static constexpr int dslot(int j, int s, int i) {
    constexpr int order[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    return 32 * (j * NBL + s / 4) + 8 * (s % 4) + order[i];
  }
  static constexpr int kQGap = 4;
  __host__ __device__ static constexpr int qsel(int i) {
    constexpr int order[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    return order[i];
  }
};

template <int D> struct KFmt<kQ4_0, D> : KQuantBase<kQ4_0, D> {
  using B = KQuantBase<kQ4_0, D>;
  using typename B::Raw;
  static constexpr int NBL = D / 128;
  __device__ static f16 dscale(const Raw& r, int blk, uint32_t sh) { return B::half_at(r, 18 * blk, sh); }
  // op without the -8 offset and with the high nibbles in the x16 frame (see
  // nd_hi16): slots 0, 1, 4, 5 hold n*d', slots 2, 3, 6, 7 hold 16*n*d', for
  // the same elements as op; d2[blk] = (d', d') the lane's block scale
  // (|d'| < 64, possibly pre-scaled by a power of two), c2[blk] = -1024*d'.
  __device__ static f16x8 op_n16(const Raw& r, int s, uint32_t sh, uint32_t mg, const f16x2* d2,
                                 const f16x2* c2) {
    const int blk = s / 4, c = s % 4;
    const uint32_t w = B::dw(r, 18 * blk + 2 + 4 * c, sh);
    const uint32_t w8 = w >> 8;
    return pack8(nd_lo(w, d2[blk], c2[blk], mg), nd_hi16(w, d2[blk], c2[blk], mg),
                 nd_lo(w8, d2[blk], c2[blk], mg), nd_hi16(w8, d2[blk], c2[blk], mg));
  }
  __host__ __device__ static bool hi_slot(int i) { return (i & 2) != 0; }
  // step s: block s/4, nibble bytes 4c..4c+3 (c = s%4) -> elements
  // 4c, 4c+2, 16+4c, 18+4c, 4c+1, 4c+3, 17+4c, 19+4c.
  __device__ static f16x8 op(const Raw& r, int s, uint32_t sh, uint32_t mg) {
    const int blk = s / 4, c = s % 4;
    const f16x2 d2 = splat2(B::half_at(r, 18 * blk, sh));
    const uint32_t w = B::dw(r, 18 * blk + 2 + 4 * c, sh);
    return pack8(nib_pair_to_f16(w, d2, mg), nib_pair_to_f16(w >> 4, d2, mg),
                 nib_pair_to_f16(w >> 8, d2, mg), nib_pair_to_f16(w >> 12, d2, mg));
  }
  __host__ __device__ static constexpr int dslot(int j, int s, int i) {
    constexpr int order[8] = {0, 2, 16, 18, 1, 3, 17, 19};
    return 32 * (j * NBL + s / 4) + 4 * (s % 4) + order[i];
  }
  static constexpr int kQGap = 16;
  __host__ __device__ static constexpr int qsel(int i) {
    constexpr int sel[8] = {0, 2, 4, 6, 1, 3, 5, 7};
    return sel[i];
  }
};

// The q values at dslot(j, s, 0..7) for every MFMA step s (s < S) of a K
// format, from one fp32 row qw (16-byte aligned): the 8 positions of a step
// are two aligned groups of four floats, at dslot(j, s, 0) and kQGap past it,
// so two 16-byte loads per step.
template <class KF>
__host__ __device__ constexpr bool q_slots_ok(int S) {
  for (int j = 0; j < 4; ++j)
    for (int s = 0; s < S; ++s) {
      if (KF::dslot(j, s, 0) % 4) return false;
      for (int i = 0; i < 8; ++i) {
        const int q = KF::qsel(i);
        if (KF::dslot(j, s, i) != KF::dslot(j, s, 0) + (q < 4 ? q : KF::kQGap + q - 4)) return false;
      }
    }
  return true;
}
template <class KF, int S>
__device__ __forceinline__ void load_q_slots(const float* qw, int j, float (&qv)[S][8]) {
  static_assert(q_slots_ok<KF>(S), "dslot is two aligned groups of four positions per step");
#pragma unroll
  for (int s = 0; s < S; ++s) {
    const float* p = qw + KF::dslot(j, s, 0);
    const float4 A = *reinterpret_cast<const float4*>(p);
    const float4 B = *reinterpret_cast<const float4*>(p + KF::kQGap);
    const float v[8] = {A.x, A.y, A.z, A.w, B.x, B.y, B.z, B.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) qv[s][i] = v[KF::qsel(i)];
  }
}

// ===========================================================================
// V formats: the A operand of the PV MFMA is V^T. Lane (m, j) holds, for
// d-tile e, head-dimension position dv(m, e) of the lane's token rows: 2*NP
// rows, rows 4j..4j+3 of group 0 and (NP = 4) 16+4j..16+4j+3 of group 1.
// `load` names the lane's first row by `voff` (row i of the group is reached
// with the scalar offset i*stride); `load_lds` reads one row staged in LDS
// (`row` = its first byte) at the same in-row offsets.
// ===========================================================================
// Partial rows are stored as binary16 (lucebox PR #555, Summary: normalised
// f16 partials), rounded to nearest even. For every V format below, d-tile
// columns e and e+1 (e even) of a lane sit at adjacent head-dimension
// positions dv(m, e) and dv(m, e) + 1, with dv(m, e) even, so a pair is one
// aligned 4-byte store.
__device__ __forceinline__ void store_f16_pair(f16* row, int d, float x0, float x1) {
  *reinterpret_cast<f16x2*>(row + d) = f16x2{f16(x0), f16(x1)};
}

// The same pair, and one fp32 value, stored device-coherently (sc1: written
// through past this XCD's L2), for partials that workgroups of the same launch
// read back (the single-launch merge); the stored bits are the same.
__device__ __forceinline__ void store_f16_pair_dev(f16* row, int d, float x0, float x1) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(row + d), bitcast<uint32_t>(f16x2{f16(x0), f16(x1)}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes, device-coherent (global_store_dwordx4 sc1; the caller waits for
// it with s_waitcnt vmcnt(0) where the order matters: the compiler does not
// count this store).
__device__ __forceinline__ void store_u32x4_dev(void* p, u32x4 v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_f32_dev(float* p, float x) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), bitcast<uint32_t>(x), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

template <int VT, int D> struct VFmt;

template <int D> struct VFmt<kF16, D> {
  static constexpr int RB = 2 * D;
  static constexpr int E = D / 16;       // d-tiles
  static constexpr int NCH = D / 128;    // 16-byte chunks per row per lane
  static constexpr bool kQuant = false;
  struct Lane { uint32_t voff, sh; };
  struct Raw { u32x4 c[NCH]; };
  // 16 lanes m read 256 contiguous bytes of a row per instruction.
  __device__ static Lane lane(int m, uint32_t row0) { return Lane{row0 + 16u * m, 0}; }
  __device__ static void load(Raw& r, rsrc_t R, const Lane& L, uint32_t soff) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) r.c[c] = buf_u32x4(R, L.voff + 256 * c, soff);
  }
  __device__ static void load_lds(Raw& r, const uint8_t* row, const Lane& L) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) r.c[c] = *reinterpret_cast<const u32x4*>(row + L.voff + 256 * c);
  }
  __device__ static void kill(Raw& r) {
#pragma unroll
    for (int c = 0; c < NCH; ++c) r.c[c] = u32x4{0, 0, 0, 0};
  }
  __host__ __device__ static int dv(int m, int e) { return 8 * (m + 16 * (e / 8)) + e % 8; }
  // Pack half k of chunk e/8 of rows (2p, 2p+1) into dword p.
  template <int NP = 4>
  __device__ static typename OpVec<NP>::type op(const Raw* R, int e) {
    const int c = e / 8, k = e % 8;
    const uint32_t sel = (k & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o = u32x4{0, 0, 0, 0};
#pragma unroll
    for (int p = 0; p < NP; ++p) o[p] = perm_bytes(R[2 * p + 1].c[c][k / 2], R[2 * p].c[c][k / 2], sel);
    return OpVec<NP>::from(o);
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
  __device__ static void load_lds(Raw& r, const uint8_t* row, const Lane& L) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(row + L.voff);
#pragma unroll
    for (int i = 0; i < NW - 1; ++i) r.w[i] = w[i];
    r.w[NW - 1] = *reinterpret_cast<const uint32_t*>(row + L.last);
    r.d = *reinterpret_cast<const f16*>(row + L.doff);
  }
  __device__ static void kill(Raw& r) { r.d = f16(0); }
  __device__ static void realign(const Raw& r, uint32_t sh, uint32_t* q) {
#pragma unroll
    for (int i = 0; i < ND; ++i) q[i] = align_bytes(r.w[i + 1], r.w[i], sh);
  }
};

template <int D> struct VFmt<kQ8_0, D> : VQuantBase<kQ8_0, D> {
  using B = VQuantBase<kQ8_0, D>;
  __host__ __device__ static int dv(int m, int e) { return m * B::EPL + e; }
  // q: realigned quant dwords of the 2*NP rows [row][ND]; dd[p] = (d_2p,
  // d_2p+1). perm gives (q_A, 0, q_B, 0); XOR 0x64806480 flips the sign bits
  // and plants the exponent bytes in one instruction.
  template <int NP = 4>
  __device__ static typename OpVec<NP>::type op_q(const uint32_t (*q)[B::ND], const f16x2* dd, int e,
                                                  uint32_t) {
    const int k = e % 4, i = e / 4;
    const uint32_t sel = uint32_t(k) | (0x0Cu << 8) | (uint32_t(4 + k) << 16) | (0x0Cu << 24);
    f16x2 o[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t x = perm_bytes(q[2 * p + 1][i], q[2 * p][i], sel) ^ 0x64806480u;
      o[p] = (bitcast<f16x2>(x) - f16x2{1152.0f16, 1152.0f16}) * dd[p];
    }
    return OpVec<NP>::pack(o);
  }
};

template <int D> struct VFmt<kQ4_0, D> : VQuantBase<kQ4_0, D> {
  using B = VQuantBase<kQ4_0, D>;
  // op_q without the -8 offset and with the high-nibble columns (e >= QB) in
  // the x16 frame (see nd_hi16); dd[p] = scales with |d'| < 64, cc[p] = -1024*dd[p].
  template <int NP>
  __device__ static typename OpVec<NP>::type op_n16(const uint32_t (*q)[B::ND], const f16x2* dd,
                                                    const f16x2* cc, int e, uint32_t mg) {
    const bool hi = e >= B::QB;
    const int byte = hi ? e - B::QB : e;
    const int k = byte % 4, i = byte / 4;
    const uint32_t sel = uint32_t(k) | (0x0Cu << 8) | (uint32_t(4 + k) << 16) | (0x0Cu << 24);
    f16x2 o[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t x = perm_bytes(q[2 * p + 1][i], q[2 * p][i], sel);
      o[p] = hi ? nd_hi16(x, dd[p], cc[p], mg) : nd_lo(x, dd[p], cc[p], mg);
    }
    return OpVec<NP>::pack(o);
  }
  __host__ __device__ static bool hi_col(int e) { return e >= B::QB; }
  // e < QB: low nibble of quant byte e; e >= QB: high nibble of byte e-QB.
  __host__ __device__ static int dv(int m, int e) {
    const int qidx = m * B::QB;
    const int blk = qidx / 16, st = qidx % 16;
    return 32 * blk + (e < B::QB ? st + e : 16 + st + (e - B::QB));
  }
  template <int NP = 4>
  __device__ static typename OpVec<NP>::type op_q(const uint32_t (*q)[B::ND], const f16x2* dd, int e,
                                                  uint32_t mg) {
    const bool hi = e >= B::QB;
    const int byte = hi ? e - B::QB : e;
    const int k = byte % 4, i = byte / 4;
    const uint32_t sel = uint32_t(k) | (0x0Cu << 8) | (uint32_t(4 + k) << 16) | (0x0Cu << 24);
    f16x2 o[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const uint32_t x = perm_bytes(q[2 * p + 1][i], q[2 * p][i], sel);
      o[p] = nib_pair_to_f16(hi ? (x >> 4) : x, dd[p], mg);
    }
    return OpVec<NP>::pack(o);
  }
};

// ===========================================================================
// Scheduling: live partitions of sequence b are [0, ceil(L_b / psize)). The
// workgroup computes the exclusive prefix unit_start[b] of their counts
// (unit_start[B] = total) and the clamped lengths lens[b] in LDS; `scan` is
// kThreads/64 words of LDS scratch. seq_len outside [0, cap_tokens] sets status
// bit 2 and is clamped.
// ===========================================================================
template <int kThreads>
__device__ __forceinline__ void live_partition_prefix(const DecodeArgs& a, int32_t* lens,
                                                      int32_t* unit_start, int* scan) {
  const int tid = threadIdx.x;
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
  // block-wide inclusive scan of `local`: within each wave by lane shuffles,
  // then the wave totals through LDS (one barrier instead of one per step)
  static_assert(kThreads % 64 == 0, "whole waves");
  const int lane = tid & 63, w = tid >> 6;
  int incl = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) scan[w] = incl;
  __syncthreads();
  for (int k = 0; k < w; ++k) incl += scan[k];
  int run = incl - local;
  for (int b = b0; b < b0 + per && b < a.B; ++b) {
    unit_start[b] = run;
    run += (lens[b] + a.psize - 1) / a.psize;
  }
  if (tid == kThreads - 1) unit_start[a.B] = incl;
  __syncthreads();
}

// Largest b with unit_start[b] <= bp (the sequence of live partition bp).
__device__ __forceinline__ int sequence_of(const int32_t* unit_start, int B, int bp) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (unit_start[mid] <= bp) lo = mid; else hi = mid - 1;
  }
  return __builtin_amdgcn_readfirstlane(lo);
}

// Workgroup -> logical index so that consecutive logical units run on one
// XCD (workgroups are dealt round-robin over the 8 XCDs).
__device__ __forceinline__ int xcd_logical(int block, int G) {
  const int xcd = block % 8, kk = block / 8;
  const int cb = G / 8, rem = G % 8;
  return xcd * cb + (xcd < rem ? xcd : rem) + kk;
}

}  // namespace pa
