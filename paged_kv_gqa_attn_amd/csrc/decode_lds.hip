// Paged GQA decode attention: the LDS-staged partition kernel.
//
// Computes what the register-streaming kernel computes (lucebox PR #555,
// Summary: for each live (sequence, K/V head, context partition) the r query
// heads of the group attend over the partition's tokens and write (m, l, o)
// partials, or the final output in direct mode), organised around how the
// paged pool sits in HBM:
//   * One block of the pool holds block_size token slots of all Hkv heads,
//     so the 16-slot groups of 4 consecutive kv heads are one contiguous run
//     of 16 * 4 * row_bytes bytes when Hkv == 4 (16 runs of 4 rows otherwise).
//     A workgroup (4 wave64s) takes a unit (sequence b, partition p, kv-head
//     quad hg) and wave w serves kv head g = 4*hg + w with its r query heads,
//     so the four waves consume together exactly what one coalesced stream
//     of the block brings in.
//   * K/V bytes move HBM -> LDS with buffer_load_dwordx4 ... lds: every lane
//     fetches one 16-byte chunk and an instruction lands 1 KB of contiguous
//     pool bytes (or of 4-row runs) in LDS, without passing through VGPRs.
//     The block table is resolved once per 16-slot group from an LDS copy of
//     the partition's block ids; the group address is 64-bit (mlxcel issue
//     #2153, Proposed Solution).
//   * A step stages G groups (16*G tokens) of K and V for the four heads; a
//     ring of R step slots keeps the DMA of the next R-1 steps in flight
//     while the current one is computed. One barrier per step separates "my
//     DMA of step s has landed" (every wave waits until only its DMA of the
//     later steps is outstanding) from "the slot of step s-1 is free" (every
//     wave finished computing it).
//   * Each wave reads its head's rows from LDS into the same MFMA operand
//     layouts the register kernel builds from HBM (decode_common.h), then
//     runs the same scores / exp2 online softmax / PV sequence: 16x16x32
//     MFMAs for 32-token steps, 16x16x16 for the PV of 16-token steps.
//   * No cross-wave combine: a wave owns all tokens of its head group, so it
//     writes its partial (or output) rows directly.
//   * Single launch (plan->fused): the merge runs in the same launch (the
//     llama.cpp PR #13 HRX page, Changes: the partials reduced by the decode
//     launch itself, ordered by an atomic count of finished work, with no
//     second dispatch). Workgroups claim items from a counter in the workspace:
//     every decode unit; a workgroup whose claim comes after the last unit
//     turns to its share of the merge slices (a query-head row and 64 output
//     columns, the separate merge's workgroup, same code). A unit stores its
//     partial device-coherently and adds one to its (sequence, head quad)'s
//     done counter; a slice waits for its counter to reach the sequence's
//     partition count. Merging starts only after every unit has been claimed,
//     and a workgroup holding a claimed unit never waits, so every wait ends
//     (each wait is also bounded by one second of the constant clock). The
//     last workgroup to leave zeroes the counters for the next launch. Which
//     workgroup computes a unit does not change its bits.
#include <algorithm>
#include <type_traits>

#include "decode_common.h"
#include "lds_ring.h"
#include "merge_common.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kNidS = 512;     // block ids staged per segment of a partition
constexpr int kIdRegs = (kNidS + 1 + kThreads - 1) / kThreads;   // ids a thread fetches
static_assert(kThreads == kMergeThreads && kMergeCols == kMergeColsHost, "merge slices run on this workgroup");

// Single-launch merge: one claim from the item counter (relaxed: the claim
// itself orders nothing).
__device__ __forceinline__ uint32_t claim_item(uint32_t* work) {
  return __hip_atomic_fetch_add(work, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits (one thread) until *cnt equals `target`, for at most `ticks` of the
// 100 MHz constant clock. 1 when reached; 0 on time-out or when the count has
// passed the target (the counters were not zero at the launch).
__device__ __forceinline__ int wait_count(const uint32_t* cnt, uint32_t target, uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  for (;;) {
    const uint32_t v = __hip_atomic_load(cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (v == target) return 1;
    if (v > target || wall_clock64() - t0 > ticks) return 0;
    // every poll is a device-coherent load of one memory line, so hundreds
    // of waiting workgroups would load the one memory channel that holds it
    // and slow the K/V stream of the units still running: poll sparsely
    __builtin_amdgcn_s_sleep(8);
  }
}

template <int KT, int VT, int D>
__global__ void __launch_bounds__(kThreads, 2) decode_lds_kernel(const DecodeArgs a) {
  using KF = KFmt<KT, D>;
  using VF = VFmt<VT, D>;
  using LY = LdsLayout<KT, VT, D, decode_group_slots(KT, VT, D)>;
  constexpr int S = D / 32;      // score MFMA steps
  constexpr int E = D / 16;      // PV d-tiles
  constexpr int G = LY::G;       // token-slot groups per step, each one 16-row MFMA tile
  constexpr int GS = LY::kGS;    // slots per group: 16, or 8 (tile rows 8..15 masked)
  constexpr int T = GS * G;      // tokens per step
  constexpr int NP = 2 * G;      // V row pairs per lane (4 rows per group)
  constexpr bool kKFold = KT == kQ4_0;   // Q4_0 offsets folded into corrections
  constexpr bool kVFold = VT == kQ4_0;
  constexpr int KF_NBL = kKFold ? D / 128 : 1;   // ggml blocks per K lane window

  unsigned char* const smem = g_lds;
  unsigned char* ring = smem;
  int32_t* unit_start = reinterpret_cast<int32_t*>(smem + a.ring_bytes);
  int32_t* lens = unit_start + (a.B + 1);
  int32_t* ids = unit_start + (((2 * a.B + 1) + 3) & ~3);
  int32_t* bcast = ids + ((kNidS + 1 + 3) & ~3);      // single launch: claimed items, flags

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int m = lane & 15;
  const int j = lane >> 4;

  // single launch: the first claim is in flight while the prefix reads seq_len
  uint32_t first = 0;
  if (a.fused && tid == 0) first = claim_item(a.work);
  live_partition_prefix<kThreads>(a, lens, unit_start, reinterpret_cast<int*>(ring));
  const int n_bp = __builtin_amdgcn_readfirstlane(unit_start[a.B]);
  const int HG = a.Hkv / 4;
  const int n_units = n_bp * HG;
  const int Gd = gridDim.x;

  // In direct mode no merge follows: an empty sequence's rows are zeroed here.
  if (a.direct) {
    for (int b = blockIdx.x; b < a.B; b += Gd) {
      if (lens[b] != 0) continue;
      float* o = a.out + int64_t(b) * a.Hq * D;
      for (int i = tid; i < a.Hq * D; i += kThreads) o[i] = 0.0f;
    }
  }

  const int logical = xcd_logical(blockIdx.x, Gd);
  const int cw = (LY::NI - wave + 3) / 4;              // DMA instructions this wave issues per step
  // LDS offsets (within a group) of the rows this lane reads: K row m, V rows
  // 4j+i, of the wave's head, at their rotated row positions
  // (with 8-slot groups, tile rows 8..15 read rows 0..7 again and are masked)
  const int km = m & (GS - 1);
  const int k_row = km * LY::SPK + ((wave + RowRot<LY::RBK>::k(km)) & 3) * LY::RBK + int(KF::lane_off(j));
  int v_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v_row[i] = ((4 * j + i) & (GS - 1)) * LY::SPV + ((wave + RowRot<LY::RBV>::v((4 * j + i) & (GS - 1))) & 3) * LY::RBV;
  const uint32_t kstride = uint32_t(a.Hkv) * LY::RBK;  // pool bytes between token slots
  const uint32_t vstride = uint32_t(a.Hkv) * LY::RBV;
  const uint32_t ksh = KF::shift(j);
  const auto vl = VF::lane(m, 0u);
  const uint32_t mg = opaque_vgpr(kMagic);
  const int seg_tokens = kNidS << a.bs_shift;

  int u = logical;
  if (a.fused) {
    if (tid == 0) bcast[0] = int(first);
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(bcast[0]);
  }
  while (u < n_units) {
    // ---- locate the unit -----------------------------------------------------
    const int bp = u / HG;
    const int hg = u - bp * HG;
    const int b = sequence_of(unit_start, a.B, bp);
    const int p = bp - __builtin_amdgcn_readfirstlane(unit_start[b]);
    const int t_begin = p * a.psize;
    const int t_end = min(__builtin_amdgcn_readfirstlane(lens[b]), t_begin + a.psize);
    const int g = 4 * hg + wave;                        // this wave's kv head
    const uint32_t khead = uint32_t(4 * hg) * LY::RBK;  // first head's offset in a slot
    const uint32_t vhead = uint32_t(4 * hg) * LY::RBV;
    // this lane's pool offset in each DMA instruction q = wave + 4i of a step
    // (the same for every step: only the group base changes)
    uint32_t dvoff[LY::NIW];
#pragma unroll
    for (int i = 0; i < LY::NIW; ++i) {
      const int q = wave + 4 * i;
      if (q < G * LY::NIK)
        dvoff[i] = chunk_voff<LY::CPK, LY::RBK, GS>(q % LY::NIK, lane, kstride, khead, 16u * kstride,
                                                 RowRot<LY::RBK>::k);
      else
        dvoff[i] = chunk_voff<LY::CPV, LY::RBV, GS>((q - G * LY::NIK) % LY::NIV, lane, vstride, vhead,
                                                 16u * vstride, RowRot<LY::RBV>::v);
    }

    // ---- the first segment's block ids and this lane's q values ------------
    // Both global reads are in flight together; the first steps' DMA is then
    // issued before the Q operand is built, so its latency covers that work.
    int seg_t0 = t_begin;
    int seg_t1 = min(t_end, seg_t0 + seg_tokens);
    int jb0 = seg_t0 >> a.bs_shift;
    int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
    // (every thread reads a live entry, so that the reads need no branch and
    // are all in flight at once; entries past nb are not used)
    int32_t idr[kIdRegs];
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k)
      idr[k] = block_of(a.table, b, a.max_blocks, jb0 + min(tid + k * kThreads, nb - 1));
    // Q operand: column n = lane%16 holds head g*r+n (zero when n >= r)
    float qv[S][8];
    {
      const int n = m < a.r ? m : a.r - 1;
      const float* qw = a.q + (int64_t(b) * a.Hq + int64_t(g) * a.r + n) * D;
      load_q_slots<KF, S>(qw, j, qv);       // q is 16-byte aligned on this path
    }
    __syncthreads();                        // the previous unit is done with the ring and ids[]
    int bad = 0;
    {
      int badl = 0;
#pragma unroll
      for (int k = 0; k < kIdRegs; ++k) {
        const int i = tid + k * kThreads;
        if (i < nb) {
          int32_t id = idr[k];
          if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
          ids[i] = id;
        }
      }
      bad |= __syncthreads_or(badl);        // also publishes ids[]
    }

    // ---- DMA of step s of the current segment into ring slot s % LY::R (each
    // wave its share) -----------------------------------------------------------
    auto issue = [&](int s) __attribute__((always_inline)) {
      issue_step<LY>(wave, a, uint32_t(s % LY::R) * LY::SLOT, seg_t0 + s * T, seg_t1, ids, jb0, kstride,
                     vstride, dvoff);
    };
    int nsteps = (seg_t1 - seg_t0 + T - 1) / T;
    for (int s = 0; s < LY::R - 1 && s < nsteps; ++s) issue(s);

    f16x8 qop[S];
    {
      const float keep = m < a.r ? 1.0f : 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // Q4_0: the high-nibble slots meet K values in the x16 frame
          const float hs = (kKFold && KFmtHi<KT, D>::hi(i)) ? 0.0625f : 1.0f;
          qop[s][i] = f16(qv[s][i] * a.qscale * keep * hs);
        }
    }

    // Q4_0 K: B operand of the per-block offset correction. Column n = head,
    // lane j: for each of the lane's ggml blocks bl, -8 * (sum of the q values
    // its slots carry for that block), in fp32 (a 16x16x4 f32 MFMA per block).
    float kcorr[KF_NBL];
#pragma unroll
    for (int bl = 0; bl < KF_NBL; ++bl) {
      float qsum = 0.0f;
#pragma unroll
      for (int s2 = 4 * bl; s2 < 4 * bl + 4; ++s2)
#pragma unroll
        for (int i = 0; i < 8; ++i) qsum += float(qop[s2][i]) * (KFmtHi<KT, D>::hi(i) ? 16.0f : 1.0f);
      kcorr[bl] = -8.0f * qsum;
    }

    // The reference max of a head column; +inf in the columns past the r
    // heads, so that their p is exactly 0: the PV MFMAs then multiply zeros
    // there, which costs less power (the kernel runs power-limited when HBM
    // and the ALUs are both busy; measured 2-4% faster). Those columns go
    // NaN at the first rescale and are never written.
    // l_lane: this lane's share of the head's sum l (its rows only), summed
    // over the rows once at the end of the unit.
    float m_run = m < a.r ? -INFINITY : INFINITY, l_lane = 0.0f;
    f32x4 acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 vcorr = f32x4{0.f, 0.f, 0.f, 0.f};   // Q4_0 V: sum_t d_t p_t per row block
    int vshift = 0;                            // Q4_0 V: acc holds the sums times 2^-vshift

    for (;;) {
      // ---- compute step s from LDS: scores, online softmax (exp2), PV -------
      auto compute = [&](int s) __attribute__((always_inline)) {
        const unsigned char* slot = ring + (s % LY::R) * LY::SLOT;
        const int t0 = seg_t0 + s * T;
        // (an 8-slot step is never full: its tile rows 8..15 are masked)
        const bool full = GS == 16 && t0 + T <= t_end;
        // tokens of the step left before t_end (wave-uniform): the row tests
        // below compare it, less a constant, with the lane's fixed 4j or m, so
        // that they cost no per-step vector arithmetic
        const int rem = GS == 16 ? t_end - t0 : min(t_end - t0, GS);
        typename KF::Raw kr[G];
        typename VF::Raw vr[2 * NP];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) KF::load_lds(kr[gi], slot + gi * LY::NIK * 1024 + k_row);
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            VF::load_lds(vr[4 * gi + i], slot + LY::VOFF + gi * LY::NIV * 1024 + v_row[i], vl);
        if (!full) {
          // zero V rows past the end so 0 * junk never reaches the PV MFMA
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * j >= rem - 16 * gi - i) VF::kill(vr[4 * gi + i]);
        }
        // The fma form of the Q4_0 conversion needs |d| < 64 (-1024*d finite):
        // a step whose live scales exceed that is converted with d * 2^-k (exact
        // scaling) and the results are scaled back by 2^k in fp32, so every
        // step runs the same code.
        // (the largest |d| of the lane, as an f16 max with the abs modifier -
        // three scales per instruction; a NaN scale does not count, it makes
        // its values NaN whatever the shift; the shift is only worked out when
        // some lane's reaches 64)
        int kk = 0, kv = 0;
        if constexpr (kKFold) {
          f16 dk = f16(0.0f);
          if (full) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
              for (int bl = 0; bl < KF_NBL; ++bl)
                dk = __builtin_fmaxf16(dk, __builtin_fabsf16(KF::dscale(kr[gi], bl, ksh)));
          } else {
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
              const bool live_row = m < rem - 16 * gi;   // dead K rows are masked below
#pragma unroll
              for (int bl = 0; bl < KF_NBL; ++bl)
                if (live_row) dk = __builtin_fmaxf16(dk, __builtin_fabsf16(KF::dscale(kr[gi], bl, ksh)));
            }
          }
          if (__any(dk >= f16(64.0f))) kk = wave_max_shift(scale_shift(dk));
        }
        if constexpr (kVFold) {
          // (dead V rows were killed above: their scale is 0)
          f16 dv = f16(0.0f);
#pragma unroll
          for (int i = 0; i < 2 * NP; ++i) dv = __builtin_fmaxf16(dv, __builtin_fabsf16(vr[i].d));
          if (__any(dv >= f16(64.0f))) kv = wave_max_shift(scale_shift(dv));
        }

        f32x4 sc[G];
#pragma unroll
        for (int gi = 0; gi < G; ++gi) sc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        // ---- scores ------------------------------------------------------
        if constexpr (kKFold) {
          // n*d operands; the -8 offset is added per block by a 16x16x4 f32
          // MFMA of the block scales (A: row m, k = the lane's j) against kcorr
          const f16x2 sk = pow2_neg_f16x2(kk);
#pragma unroll
          for (int gi = 0; gi < G; ++gi) {
            f16x2 d2[KF_NBL], c2[KF_NBL];
#pragma unroll
            for (int bl = 0; bl < KF_NBL; ++bl) {
              d2[bl] = splat2(KF::dscale(kr[gi], bl, ksh)) * sk;
              c2[bl] = d2[bl] * f16x2{-1024.0f16, -1024.0f16};
            }
#pragma unroll
            for (int s2 = 0; s2 < S; ++s2)
              sc[gi] = mfma(KF::op_n16(kr[gi], s2, ksh, mg, d2, c2), qop[s2], sc[gi]);
          }
          if (kk) {
            const float up = __builtin_ldexpf(1.0f, kk);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) sc[gi] *= up;
          }
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int bl = 0; bl < KF_NBL; ++bl)
              sc[gi] = __builtin_amdgcn_mfma_f32_16x16x4f32(float(KF::dscale(kr[gi], bl, ksh)), kcorr[bl],
                                                            sc[gi], 0, 0, 0);
        } else {
#pragma unroll
          for (int s2 = 0; s2 < S; ++s2)
#pragma unroll
            for (int gi = 0; gi < G; ++gi) sc[gi] = mfma(KF::op(kr[gi], s2, ksh, mg), qop[s2], sc[gi]);
        }
        if constexpr (G == 1) mfma_settle(sc[0]);
        else mfma_settle(sc[0], sc[1]);
        if (!full) {
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * j >= rem - 16 * gi - i) sc[gi][i] = -INFINITY;
        }
        // ---- online softmax ------------------------------------------------
        float mx = -INFINITY;
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
          mx = fmaxf(mx, fmaxf(fmaxf(sc[gi][0], sc[gi][1]), fmaxf(sc[gi][2], sc[gi][3])));
        // Lazy rescale: the reference m only moves when some head's max
        // exceeds it by more than kSlack (then p <= 2^kSlack, safe in f16);
        // the lucebox page skips the rescale when the max is unchanged. Each
        // lane tests its own rows; the head's max over all rows is only
        // needed when the reference moves.
        if (__any(mx > m_run + kSlack)) {
          const float m_new = fmaxf(m_run, max_over_rows(mx));
          const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
          l_lane *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] *= alpha;
          vcorr *= alpha;
          m_run = m_new;
        }
        float pr[2 * NP];
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[4 * gi + i] = __builtin_amdgcn_exp2f(sc[gi][i] - m_run);
        float ps = 0.0f;
#pragma unroll
        for (int i = 0; i < 2 * NP; i += 4) ps += (pr[i] + pr[i + 1]) + (pr[i + 2] + pr[i + 3]);
        typename OpVec<NP>::type pop;
#pragma unroll
        for (int i = 0; i < 2 * NP; ++i) pop[i] = f16(pr[i]);
        auto pv = [&](typename OpVec<NP>::type av, f32x4 c) __attribute__((always_inline)) {
          if constexpr (NP == 4) return mfma(av, pop, c);
          else return mfma16(av, pop, c);
        };
        __builtin_amdgcn_s_setprio(1);
        // ---- PV ------------------------------------------------------------
        if constexpr (VF::kQuant) {
          uint32_t q[2 * NP][VF::ND];
          f16x2 dd[NP];
#pragma unroll
          for (int i = 0; i < 2 * NP; ++i) VF::realign(vr[i], vl.sh, q[i]);
#pragma unroll
          for (int qq = 0; qq < NP; ++qq) dd[qq] = f16x2{vr[2 * qq].d, vr[2 * qq + 1].d};
          if constexpr (kVFold) {
            // n*d' operands with d' = d * 2^-kv; acc holds the true sums times
            // 2^-vshift, so a change of shift rescales it once (exact). The sum
            // of d_t p_t (per row block and head) carries the -8 offset, added
            // once at the end of the unit.
            if (kv != vshift) {
              const float f = __builtin_ldexpf(1.0f, vshift - kv);
#pragma unroll
              for (int e = 0; e < E; ++e) acc[e] *= f;
              vshift = kv;
            }
            const f16x2 sv = pow2_neg_f16x2(kv);
            f16x2 ds[NP], cc[NP];
#pragma unroll
            for (int qq = 0; qq < NP; ++qq) {
              ds[qq] = dd[qq] * sv;
              cc[qq] = ds[qq] * f16x2{-1024.0f16, -1024.0f16};
            }
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = pv(VF::template op_n16<NP>(q, ds, cc, e, mg), acc[e]);
            vcorr = pv(OpVec<NP>::pack(dd), vcorr);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) acc[e] = pv(VF::template op_q<NP>(q, dd, e, mg), acc[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = pv(VF::template op<NP>(vr, e), acc[e]);
        }
        l_lane += ps;
      };

      // ---- the ring: steps s+1 .. s+R-2 in flight while step s is computed -
      // (the first R-1 steps of the segment are already issued)
      for (int s = 0; s < nsteps; ++s) {
        // every wave's DMA of step s has landed (this wave may still have the
        // DMA of the later steps outstanding: cw instructions each), and every
        // wave is done with step s-1, whose slot the next issue overwrites
        if constexpr (LY::R == 2) {
          wait_dma_then_barrier(0);
        } else {
          const int later = min(LY::R - 2, nsteps - 1 - s);
          wait_dma_then_barrier(later * cw);
        }
        // Issue priority: the DMA and the score / softmax chain (short,
        // latency bound) go ahead of the other workgroup's wave on this SIMD,
        // whose VALU-heavy PV part then fills the gaps (measured 3-8% faster).
        __builtin_amdgcn_s_setprio(3);
        if (s + LY::R - 1 < nsteps) issue(s + LY::R - 1);
        compute(s);
      }

      // ---- next segment: its block ids, then the first steps' DMA ----------
      seg_t0 = seg_t1;
      if (seg_t0 >= t_end) break;
      seg_t1 = min(t_end, seg_t0 + seg_tokens);
      jb0 = seg_t0 >> a.bs_shift;
      nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
      __syncthreads();                       // ids[] and the ring are free
      int badl = 0;
      for (int i = tid; i < nb; i += kThreads) {
        int32_t id = block_of(a.table, b, a.max_blocks, jb0 + i);
        if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
        ids[i] = id;
      }
      bad |= __syncthreads_or(badl);         // also publishes ids[]
      nsteps = (seg_t1 - seg_t0 + T - 1) / T;
      for (int s = 0; s < LY::R - 1 && s < nsteps; ++s) issue(s);
    }

    mfma_settle(acc, vcorr);   // the last step's PV MFMAs wrote them
    const float l_run = sum_over_rows(l_lane);

    // ---- Q4_0 V: add the -8 offset of every accumulated value -------------
    if constexpr (kVFold) {
      const float f = __builtin_ldexpf(1.0f, vshift);
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float fe = VFmtHi<VT, D>::hi(e) ? f * 0.0625f : f;   // undo the x16 frame
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[e][i] = acc[e][i] * fe - 8.0f * vcorr[i];
      }
    }

    // ---- partial (or final) rows of the wave's r heads --------------------
    // Partials go out as whole rows: every wave stages its r rows (binary16)
    // in the idle ring and copies them with 16-byte stores, so each 512-byte
    // (D = 256) row reaches memory as whole lines. The stores are
    // device-coherent (written through past this XCD's L2) so that a single
    // launch can merge them in the same launch; as whole lines they cost no
    // more than write-back stores.
    const int n = m;
    if (bad && tid == 0) atomicOr(a.status, 1u);
    unsigned char* const stage = ring + wave * (a.r * 2 * D);   // this wave's rows
    if (!a.direct) __syncthreads();      // every wave is done reading the ring
    if (n < a.r) {
      const int h = g * a.r + n;
      const float inv = bad ? __builtin_nanf("") : 1.0f / l_run;
      if (a.direct) {
        float* dst = a.out + (int64_t(b) * a.Hq + h) * D;
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[VF::dv(4 * j + i, e)] = acc[e][i] * inv;
      } else {
        const int64_t row = (int64_t(b) * a.Hq + h) * a.p_max + p;
        if (j == 0) {
          store_f32_dev(a.part_ml + 2 * row, bad ? __builtin_nanf("") : m_run);
          store_f32_dev(a.part_ml + 2 * row + 1, l_run);
        }
        f16* srow = reinterpret_cast<f16*>(stage) + n * D;
#pragma unroll
        for (int e = 0; e < E; e += 2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            store_f16_pair(srow, VF::dv(4 * j + i, e), acc[e][i] * inv, acc[e + 1][i] * inv);
      }
    }
    if (!a.direct) {
      __syncthreads();                   // the staged rows are complete
      constexpr int kRowChunks = D / 8;  // 16-byte chunks of a binary16 row
      const int64_t row0 = (int64_t(b) * a.Hq + g * a.r) * a.p_max + p;
      for (int c = lane; c < a.r * kRowChunks; c += 64) {
        const int n2 = c / kRowChunks, w = c - n2 * kRowChunks;
        const u32x4 v = *reinterpret_cast<const u32x4*>(stage + n2 * (2 * D) + 16 * w);
        store_u32x4_dev(reinterpret_cast<uint8_t*>(a.part_o) + ((row0 + int64_t(n2) * a.p_max) * D) * 2 + 16 * w, v);
      }
    }
    if (!a.fused) {
      u += Gd;
      continue;
    }
    // single launch: publish the partial - every thread waits until its
    // device-coherent stores are performed, then one increment of the unit's
    // done counter (no cache write-back needed: nothing of the partial sits
    // in L2 only) - and claim the next item
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");     // (also the 16-byte asm stores)
    __syncthreads();
    if (tid == 0) {
      __hip_atomic_fetch_add(a.done + (b * HG + hg) * kDoneStride, 1u, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      bcast[0] = int(claim_item(a.work));
    }
    __syncthreads();
    u = __builtin_amdgcn_readfirstlane(bcast[0]);
  }
  if (!a.fused) return;

  // ---- single launch: merge slices, then leave ----------------------------
  // Slice i is query-head row bh = i / (D/64) and output columns
  // 64 * (i % (D/64)) ..; it waits for every partition of the row's
  // (sequence, head quad) and then runs the separate merge's code on them.
  // Slices are dealt by workgroup index (slice blockIdx.x + k * grid): this
  // workgroup got here because its claim came after the last unit, so every
  // unit is already held by a running workgroup that does not wait.
  MergeLds& mlds = *reinterpret_cast<MergeLds*>(ring);   // the ring is idle now
  const int chunks = D / kMergeCols;
  u = n_units + blockIdx.x;
  while (u < n_units + a.merge_items) {
    const int next = u + Gd;
    const int item = u - n_units;
    const int bh = item / chunks;
    const int col0 = (item - bh * chunks) * kMergeCols;
    const int b = bh / a.Hq;
    const int hg = (bh - b * a.Hq) / a.r / 4;
    const int P = (lens[b] + a.psize - 1) / a.psize;
    if (tid == 0) bcast[1] = wait_count(a.done + (b * HG + hg) * kDoneStride, uint32_t(P), a.wait_ticks);
    __syncthreads();
    const int ok = bcast[1];
    u = next;
    float* dst = a.out + int64_t(bh) * D + col0;
    if (ok) {
      // (device-coherent loads: the partials come from this launch)
      merge_slice<true>(reinterpret_cast<const f16*>(a.part_o) + int64_t(bh) * a.p_max * D,
                  a.part_ml + int64_t(bh) * a.p_max * 2, P, D, col0, dst, mlds);
    } else {
      if (tid < kMergeCols) dst[tid] = __builtin_nanf("");
      if (tid == 0) atomicOr(a.status, 4u);
    }
    __syncthreads();                      // bcast and the slice's LDS are free again
  }
  // every workgroup counts itself out; the last one zeroes the counters (all
  // others have made their last claim and increment by then)
  if (tid == 0) {
    const uint32_t n = __hip_atomic_fetch_add(a.leave, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    bcast[2] = n == gridDim.x - 1;
  }
  __syncthreads();
  if (bcast[2]) {
    for (int i = tid; i < a.B * HG; i += kThreads)
      __hip_atomic_store(a.done + i * kDoneStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (tid == 0) {
      __hip_atomic_store(a.work, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(a.leave, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// LDS bytes of a launch: the ring, then unit_start[B+1] | lens[B] | pad |
// ids[kNidS+1] | bcast[4] (a segment of kNidS blocks' worth of tokens that
// starts inside a block touches kNidS+1 blocks).
template <int KT, int VT, int D>
size_t lds_bytes(const DecodeArgs& a, int* ring_bytes) {
  using LY = LdsLayout<KT, VT, D, decode_group_slots(KT, VT, D)>;
  static_assert(size_t(LY::R) * LY::SLOT >= sizeof(MergeLds), "merge slices reuse the ring");
  static_assert(size_t(LY::R) * LY::SLOT >= 4 * 16 * 2 * D, "four waves stage up to 16 binary16 rows each");
  const size_t ring = size_t(LY::R) * LY::SLOT;
  *ring_bytes = int((ring + 15) & ~size_t(15));
  return size_t(*ring_bytes) + 4 * size_t(((2 * a.B + 1) + 3) & ~3) + 4 * size_t((kNidS + 1 + 3) & ~3) + 16;
}

template <int KT, int VT, int D>
hipError_t launch_typed(const DecodeArgs& a0, hipStream_t stream) {
  if constexpr (decode_group_slots(KT, VT, D) == 0) {
    return hipErrorInvalidValue;
  } else {
    DecodeArgs a = a0;
    const size_t lds = lds_bytes<KT, VT, D>(a, &a.ring_bytes);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_lds_kernel<KT, VT, D>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 81920);
    if (attr != hipSuccess) return attr;
    hipLaunchKernelGGL((decode_lds_kernel<KT, VT, D>), dim3(a.grid), dim3(kThreads), lds, stream, a);
    return hipGetLastError();
  }
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

hipError_t launch_decode_lds(const DecodeArgs& a, hipStream_t stream) {
  if (a.Hkv % 4 || a.B > kLdsMaxB) return hipErrorInvalidValue;
  if (a.D == 256) return launch_d<256>(a, stream);
  if (a.D == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
