// Multi-token queries over the paged pool: chunked prefill and verify windows.
//
// What it computes (llama.cpp PR #13 HRX, Roadmap item 3: multi-token queries
// over the preceding paged K/V with causal attention inside the chunk;
// TensorFold PR #1418, What: paged prompt-chunk attention that equals the
// contiguous one bit for bit): q is [B, Tq, Hq, D]; the chunk's Tq tokens are
// the last Tq of each sequence, so chunk token t of sequence b (length L)
// sits at position L - Tq + t and attends to the keys at positions
// 0 .. L - Tq + t of kv head g = h / r.
//
// How it maps onto gfx950:
//   * The Tq*r query rows of one kv head play the part the r heads play in
//     the decode kernels: row n = t*r + (h - g*r), and 16 of them form the N
//     side of the 16x16x32 f16 MFMAs (S^T = K Q^T, O^T += V^T P^T), with the
//     same operand layouts and the same online exp2 softmax.
//   * A workgroup is one wave64 and takes a unit (sequence b, partition p of
//     the keys, kv head g, tile of 16 query rows). Units that differ only in
//     the row tile are adjacent and land on one XCD, so the K/V rows they all
//     stream are read from HBM once and from L2 after that.
//   * K/V stream from the pool straight into registers in MFMA operand order,
//     double-buffered (the next 32-token tile is in flight while the current
//     one is computed), through the block table with 64-bit row addresses
//     (mlxcel issue #2153) - the register path of the decode kernels.
//   * Causal limit: each lane's query row sees keys up to min(its position,
//     partition end - 1); tiles past every row's limit are not read, and only
//     tiles that cross some row's limit are masked.
//   * Partitions of the keys give partials (normalised binary16 o, fp32 m and
//     l) in the decode layout with Tq*Hq rows per sequence, reduced by the
//     same merge kernel; a single partition writes the output directly.
#include "decode_common.h"

namespace pa {
namespace {

constexpr int kThreads = 64;
constexpr int kNid = 512;       // block ids staged per segment of a partition

template <int KT, int VT, int D>
struct CTile {
  using KF = KFmt<KT, D>;
  using VF = VFmt<VT, D>;
  typename KF::Raw k[2];
  typename VF::Raw v[8];        // the lane's 8 token rows of the tile
};

// Waves per SIMD the register allocation is held to (for one-wave
// workgroups the bound counts waves per SIMD): two where the kernel fits in
// 256 registers without spilling, else one.
template <int KT, int VT, int D>
struct CMinBlocks {
  static constexpr int value = (D == 128 || (KT == kQ4_0 && VT == kQ4_0)) ? 2 : 1;
};

template <int KT, int VT, int D>
__global__ void __launch_bounds__(kThreads, (CMinBlocks<KT, VT, D>::value))
chunk_kernel(const ChunkArgs a) {
  using KF = KFmt<KT, D>;
  using VF = VFmt<VT, D>;
  using T = CTile<KT, VT, D>;
  constexpr int S = D / 32;      // score MFMA steps
  constexpr int E = D / 16;      // PV d-tiles
  constexpr int kTile = 32;      // tokens per tile

  __shared__ int32_t ids[kNid + 1];

  const int lane = threadIdx.x;
  const int m = lane & 15;
  const int j = lane >> 4;
  const int R = a.Tq * a.r;                  // query rows per kv head
  const int QT = (R + 15) / 16;              // 16-row tiles
  const int n_units = a.B * a.p_max * a.Hkv * QT;
  const int Gd = gridDim.x;
  const int logical = xcd_logical(blockIdx.x, Gd);

  const uint32_t kstride = uint32_t(a.Hkv) * KF::RB;
  const uint32_t vstride = uint32_t(a.Hkv) * VF::RB;
  const uint32_t ksh = KF::shift(j);
  const uint32_t kvoff = m * kstride + KF::lane_off(j);
  const auto vl = VF::lane(m, 4u * j * vstride);
  const uint32_t mg = opaque_vgpr(kMagic);
  const int bs_mask = (1 << a.bs_shift) - 1;
  const int seg_tokens = kNid << a.bs_shift;

  for (int u = logical; u < n_units; u += Gd) {
    // ---- locate the unit: ((b*p_max + p)*Hkv + g)*QT + qt ------------------
    const int qt = u % QT;
    const int g = (u / QT) % a.Hkv;
    const int bp = u / (QT * a.Hkv);
    const int b = bp / a.p_max;
    const int p = bp - b * a.p_max;
    int L = a.seq_len[b];
    if (L < 0 || L > a.cap_tokens) {
      if (lane == 0 && p == 0 && g == 0 && qt == 0) atomicOr(a.status, 2u);
      L = L < 0 ? 0 : a.cap_tokens;
    }
    if (L > 0 && L < a.Tq) {             // the chunk is longer than the sequence
      if (lane == 0 && p == 0 && g == 0 && qt == 0) atomicOr(a.status, 2u);
      L = 0;
    }
    L = __builtin_amdgcn_readfirstlane(L);
    // this lane's query row (column n = m of every MFMA)
    const int row = qt * 16 + m;
    const bool valid = row < R;
    const int t = valid ? row / a.r : 0;
    const int h = g * a.r + (valid ? row - t * a.r : 0);
    const int64_t orow = (int64_t(b) * a.Tq + t) * a.Hq + h;    // row of out / partials
    if (L == 0) {
      // an empty (or refused) sequence: zero rows in direct mode; the merge
      // writes its zero rows otherwise
      if (a.direct && valid && j == 0)
        for (int d = 0; d < D; ++d) a.out[orow * D + d] = 0.0f;
      continue;
    }
    const int P = (L + a.psize - 1) / a.psize;
    if (p >= P) continue;                 // no such partition: nothing to write
    const int t_begin = p * a.psize;
    const int t_end = min(L, t_begin + a.psize);
    // keys this lane's row sees: [t_begin, lim]
    const int lim = valid ? min(L - a.Tq + t, t_end - 1) : t_begin - 1;
    int lim_max = lim, lim_min = valid ? lim : INT32_MAX;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      lim_max = max(lim_max, __shfl_xor(lim_max, off));
      lim_min = min(lim_min, __shfl_xor(lim_min, off));
    }
    lim_max = __builtin_amdgcn_readfirstlane(lim_max);
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);
    const int t_stop = min(t_end, lim_max + 1);     // no row reads a key past this

    // ---- Q operand: column n holds query row qt*16+n (zero past R) ---------
    f16x8 qop[S];
    {
      const float* qr = a.q + orow * D;
      const float keep = valid ? a.qscale : 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) qop[s][i] = f16(valid ? qr[KF::dslot(j, s, i)] * keep : 0.0f);
    }

    // reference max: +inf in columns past R (their p is exactly 0); -inf
    // until the row has seen a key
    float m_run = valid ? -INFINITY : INFINITY, l_lane = 0.0f;
    f32x4 acc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) acc[e] = f32x4{0.f, 0.f, 0.f, 0.f};
    int bad = 0;

    for (int seg_t0 = t_begin; seg_t0 < t_stop; seg_t0 += seg_tokens) {
      const int seg_t1 = min(t_stop, seg_t0 + seg_tokens);
      const int jb0 = seg_t0 >> a.bs_shift;
      const int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
      __syncthreads();                       // earlier readers of ids[] are done
      int badl = 0;
      for (int i = lane; i < nb; i += kThreads) {
        int32_t id = block_of(a.table, b, a.max_blocks, jb0 + i);
        if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
        ids[i] = id;
      }
      bad |= __syncthreads_or(badl);
      const int ntiles = (seg_t1 - seg_t0 + kTile - 1) / kTile;

      // A tile index past the segment still issues its loads, through a
      // zero-size buffer resource (they return 0 and touch nothing), so every
      // path keeps the same loads in flight.
      auto load_tile = [&](T& tl, int kt) __attribute__((always_inline)) {
        const bool live_tile = kt < ntiles;
        const int t0 = seg_t0 + (live_tile ? kt : ntiles - 1) * kTile;
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const int tg = t0 + 16 * gi;
          const bool live = tg < seg_t1;
          const int tq = live ? tg : seg_t1 - 1;
          const int32_t id = __builtin_amdgcn_readfirstlane(ids[(tq >> a.bs_shift) - jb0]);
          const int slot0 = live ? (tg & bs_mask) : 0;
          const rsrc_t kr = make_rsrc(a.k_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, KF::RB),
                                      live_tile ? 16u * kstride : 0u);
          const rsrc_t vr = make_rsrc(a.v_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, VF::RB),
                                      live_tile ? 16u * vstride : 0u);
          KF::load(tl.k[gi], kr, kvoff);
#pragma unroll
          for (int i = 0; i < 4; ++i) VF::load(tl.v[4 * gi + i], vr, vl, i * vstride);
        }
      };

      auto compute_tile = [&](T& tl, int t0) __attribute__((always_inline)) {
        // rows past the last key any row reads (junk, maybe NaN) never reach
        // the PV MFMA
        if (t0 + kTile > seg_t1) {
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t0 + 16 * gi + 4 * j + i >= seg_t1) VF::kill(tl.v[4 * gi + i]);
        }
        f32x4 sc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) sc[gi] = mfma(KF::op(tl.k[gi], s, ksh, mg), qop[s], sc[gi]);
        // causal and end-of-partition mask, only where some row's limit falls
        // inside the tile
        if (t0 + kTile - 1 > lim_min) {
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (t0 + 16 * gi + 4 * j + i > lim) sc[gi][i] = -INFINITY;
        }
        float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                         fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
        // lazy rescale (lucebox PR #555, Summary: skip the rescale when the
        // max is unchanged): the reference moves only when a row's max exceeds
        // it by more than kSlack. A row whose reference does not move keeps
        // its sums as they are: that also covers rows with no key yet (m =
        // -inf, where exp2(m - m_new) would be exp2(-inf + inf)) and the
        // +inf columns past R.
        if (__any(mx > m_run + kSlack)) {
          const float m_new = fmaxf(m_run, max_over_rows(mx));
          const float alpha = m_new == m_run ? 1.0f : __builtin_amdgcn_exp2f(m_run - m_new);
          l_lane *= alpha;
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] *= alpha;
          m_run = m_new;
        }
        // a row with no key yet keeps m = -inf: its p are exp2(-inf) = 0
        const float m_use = m_run == -INFINITY ? 0.0f : m_run;
        float pr[8];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi)
#pragma unroll
          for (int i = 0; i < 4; ++i) pr[4 * gi + i] = __builtin_amdgcn_exp2f(sc[gi][i] - m_use);
        l_lane += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        f16x8 pop;
#pragma unroll
        for (int i = 0; i < 8; ++i) pop[i] = f16(pr[i]);
        if constexpr (VF::kQuant) {
          uint32_t q[8][VF::ND];
          f16x2 dd[4];
#pragma unroll
          for (int i = 0; i < 8; ++i) VF::realign(tl.v[i], vl.sh, q[i]);
#pragma unroll
          for (int qq = 0; qq < 4; ++qq) dd[qq] = f16x2{tl.v[2 * qq].d, tl.v[2 * qq + 1].d};
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = mfma(VF::op_q(q, dd, e, mg), pop, acc[e]);
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) acc[e] = mfma(VF::op(tl.v, e), pop, acc[e]);
        }
      };

      // ---- stream the tiles with one in flight -------------------------------
      T A, Bt;
      load_tile(A, 0);
      for (int k = 0; k < ntiles; k += 2) {
        load_tile(Bt, k + 1);
        compute_tile(A, seg_t0 + k * kTile);
        if (k + 1 >= ntiles) break;
        load_tile(A, k + 2);
        compute_tile(Bt, seg_t0 + (k + 1) * kTile);
      }
    }

    // ---- partial (or final) rows -------------------------------------------
    const float l_run = sum_over_rows(l_lane);
    if (bad && lane == 0) atomicOr(a.status, 1u);
    if (!valid) continue;
    const float inv = bad ? __builtin_nanf("") : (l_run > 0.0f ? 1.0f / l_run : 0.0f);
    if (a.direct) {
      float* dst = a.out + orow * D;
#pragma unroll
      for (int e = 0; e < E; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[VF::dv(4 * j + i, e)] = acc[e][i] * inv;
    } else {
      const int64_t prow = orow * a.p_max + p;
      f16* dst = reinterpret_cast<f16*>(a.part_o) + prow * D;
      if (j == 0) {
        a.part_ml[2 * prow] = bad ? __builtin_nanf("") : (l_run > 0.0f ? m_run : -INFINITY);
        a.part_ml[2 * prow + 1] = l_run;
      }
#pragma unroll
      for (int e = 0; e < E; e += 2)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          store_f16_pair(dst, VF::dv(4 * j + i, e), acc[e][i] * inv, acc[e + 1][i] * inv);
    }
  }
}

template <int KT, int VT, int D>
hipError_t launch_typed(const ChunkArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL((chunk_kernel<KT, VT, D>), dim3(a.grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const ChunkArgs& a, hipStream_t stream) {
  switch (a.k_type * 3 + a.v_type) {
    case 0: return launch_typed<kF16, kF16, D>(a, stream);
    case 1: return launch_typed<kF16, kQ8_0, D>(a, stream);
    case 2: return launch_typed<kF16, kQ4_0, D>(a, stream);
    case 3: return launch_typed<kQ8_0, kF16, D>(a, stream);
    case 4: return launch_typed<kQ8_0, kQ8_0, D>(a, stream);
    case 5: return launch_typed<kQ8_0, kQ4_0, D>(a, stream);
    case 6: return launch_typed<kQ4_0, kF16, D>(a, stream);
    case 7: return launch_typed<kQ4_0, kQ8_0, D>(a, stream);
    case 8: return launch_typed<kQ4_0, kQ4_0, D>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk(const ChunkArgs& a, hipStream_t stream) {
  if (a.D == 256) return launch_d<256>(a, stream);
  if (a.D == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
