// Paged GQA decode attention: the register-streaming partition kernel.
//
// Used for the shapes the LDS-staged kernel (decode_lds.hip) does not take
// (F16 K or V at D=256, Hkv not a multiple of 4, large batches).
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
#include "decode_common.h"

namespace pa {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
// ===========================================================================
// The kernel
// ===========================================================================
// 16-row groups per tile (32 tokens: the PV MFMA contracts over 32 rows).
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
//   unit_start[B+1] | lens[B] | pad | ids[kNid+1] | qs[r*D] | comb[3*(r*D+32)]
// comb doubles as the scratch of the start-up prefix scan (needs kThreads).
constexpr int kNid = 2048;     // block ids staged per segment of a partition

__host__ __device__ inline int lds_words(int B, int r, int D) {
  const int pre = ((2 * B + 1) + 3) & ~3;
  const int ids = (kNid + 1 + 3) & ~3;
  const int comb = 3 * (r * D + 32) > kThreads ? 3 * (r * D + 32) : kThreads;
  return pre + ids + r * D + comb;
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
  float* qs = reinterpret_cast<float*>(ids + ((kNid + 1 + 3) & ~3));
  float* comb = qs + a.r * D;
  const int comb_stride = a.r * D + 32;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int m = lane & 15;
  const int j = lane >> 4;

  // ---- per-workgroup prefix of live partitions per sequence -------------
  live_partition_prefix<kThreads>(a, lens, unit_start, reinterpret_cast<int*>(comb));
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
  const int logical = xcd_logical(blockIdx.x, G);

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
    U.b = sequence_of(unit_start, a.B, bp);
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

    f16x8 qop[S];
    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    int bad = 0;

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
        // Q operand: column n = lane%16 holds head g*r+n (zero when n >= r)
        const int n = m < a.r ? m : a.r - 1;
        const float keep = m < a.r ? 1.0f : 0.0f;
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int i = 0; i < 8; ++i) qop[s][i] = f16(qs[n * D + KF::dslot(j, s, i)] * keep);
      }

      const int ntiles = (seg_t1 - seg_t0 + kTile - 1) / kTile;

      // ---- tile loader (block ids come from LDS, one per 16-row group) ----
      // A tile index past the segment still issues its loads, through a
      // zero-size buffer resource: they return 0 without touching memory, so
      // every path through the loop has the same loads in flight and the
      // compiler's wait counts stay exact.
      auto load_tile = [&](T& t, int kt) __attribute__((always_inline)) {
        const bool valid = kt < ntiles;
        const int t0 = seg_t0 + (valid ? kt : ntiles - 1) * kTile;
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
          const int tg = t0 + 16 * gi;
          const bool live = tg < U.t_end;
          const int tq = live ? tg : U.t_end - 1;
          const int32_t id = __builtin_amdgcn_readfirstlane(ids[(tq >> a.bs_shift) - jb0]);
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
      auto compute_tile = [&](T& t, int t0) __attribute__((always_inline)) {
        const bool full = t0 + kTile <= U.t_end;
        if (!full) {
          // zero V rows past the end so 0 * junk never reaches the PV MFMA
#pragma unroll
          for (int gi = 0; gi < NG; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t0 + 16 * gi + 4 * j + i >= U.t_end) VF::kill(t.v[gi / 2][4 * (gi % 2) + i]);
        }
        f32x4 sc[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) sc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) sc[gi] = mfma(KF::op(t.k[gi], s, ksh, mg), qop[s], sc[gi]);
        if constexpr (NG == 1) mfma_settle(sc[0]);
        else mfma_settle(sc[0], sc[1]);
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
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = mfma(VF::op_q(q, dd, e, mg), pop, acc[e]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = mfma(VF::op(t.v[pp], e), pop, acc[e]);
          }
        }
        l_run += sum_over_rows(ps);
      };

      // ---- wave w streams tiles w, w+4, ... with one tile prefetched ------
      int k = wave;
      if (k < ntiles) {
        T A, Bt;
        load_tile(A, k);
        while (true) {
          load_tile(Bt, k + kWaves);
          compute_tile(A, seg_t0 + k * kTile);
          k += kWaves;
          if (k >= ntiles) break;
          load_tile(A, k + kWaves);
          compute_tile(Bt, seg_t0 + k * kTile);
          k += kWaves;
          if (k >= ntiles) break;
        }
      }
    }

    // ---- combine the four waves through LDS -------------------------------
    mfma_settle(acc);   // the last tile's PV MFMAs wrote it
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
      const float inv = bad ? __builtin_nanf("") : 1.0f / l;
      const int h = U.g * a.r + n;
      if (bad && lane == 0) atomicOr(a.status, 1u);
      // combined, normalised value of d-tile column e, row i of this lane
      auto value = [&](int e, int i) {
        const int d = VF::dv(4 * j + i, e);
        float v = acc[e][i] * c0;
#pragma unroll
        for (int w = 0; w < 3; ++w) v += comb[w * comb_stride + n * D + d] * cwt[w];
        return v * inv;
      };
      if (n < a.r) {
        if (a.direct) {
          float* dst = a.out + (int64_t(U.b) * a.Hq + h) * D;
#pragma unroll
          for (int e = 0; e < E; ++e)
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[VF::dv(4 * j + i, e)] = value(e, i);
        } else {
          const int64_t row = (int64_t(U.b) * a.Hq + h) * a.p_max + U.p;
          f16* dst = reinterpret_cast<f16*>(a.part_o) + row * D;
          if (j == 0) {
            a.part_ml[2 * row] = bad ? __builtin_nanf("") : M;
            a.part_ml[2 * row + 1] = l;
          }
#pragma unroll
          for (int e = 0; e < E; e += 2)
#pragma unroll
            for (int i = 0; i < 4; ++i) store_f16_pair(dst, VF::dv(4 * j + i, e), value(e, i), value(e + 1, i));
        }
      }
    }
    __syncthreads();
  }
}

template <int KT, int VT, int D>
hipError_t launch_typed(const DecodeArgs& a, hipStream_t stream) {
  const size_t lds = size_t(lds_words(a.B, a.r, D)) * 4;
  // Large batches and head groups (e.g. B = 1024, or r = 16 at D = 256) need
  // more than the default 64 KiB of dynamic LDS; a workgroup may use up to
  // the CU's 160 KiB.
  if (lds > 65536) {
    const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_kernel<KT, VT, D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
    if (attr != hipSuccess) return attr;
  }
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

hipError_t launch_decode_regs(const DecodeArgs& a, hipStream_t stream) {
  if (a.D == 256) return launch_d<256>(a, stream);
  if (a.D == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
