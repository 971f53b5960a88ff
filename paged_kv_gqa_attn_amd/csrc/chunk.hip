// Multi-token queries over the paged pool: chunked prefill and verify windows.
//
// What it computes (lucebox PR #555, Roadmap item 3: several query tokens per
// sequence attend over the K/V already in the pool, causally inside the chunk;
// TensorFold PR #1418, What: paged prompt-chunk attention that equals the
// contiguous one bit for bit): q is [B, Tq, Hq, D]; the chunk's Tq tokens are
// the last Tq of each sequence, so chunk token t of sequence b (length L)
// sits at position L - Tq + t and attends to the keys at positions
// 0 .. L - Tq + t of kv head g = h / r.
//
// How it maps onto gfx950:
//   * The Tq*r query rows of one kv head play the part the r heads play in
//     the decode kernels: row n = t*r + (h - g*r), and 16 of them form the N
//     side of the f16 MFMAs (S^T = K Q^T, O^T += V^T P^T), with the decode
//     kernels' operand layouts and the same online exp2 softmax.
//   * A workgroup is four wave64s and takes a unit (sequence b, partition p of
//     the keys, kv head g, 64*NTW query rows): each wave owns NTW tiles of 16
//     rows. Every K/V row of the unit is converted to f16 once: per 32-token
//     tile, wave w loads and converts one job - K or V (w >= 2) of the
//     16-token group w & 1 - straight from the pool through the block table
//     (64-bit row addresses, mlxcel issue #2153) and writes it to LDS in MFMA
//     operand order; after one barrier every wave reads the operands for its
//     own rows. The next tile's raw rows load while a tile is computed, and
//     the operand buffers alternate, so a tile costs one barrier.
//   * Causal limit: each lane's query row sees keys up to min(its position,
//     partition end - 1); tiles past the workgroup's last row are not read,
//     and only tiles that cross some row's limit are masked.
//   * Partitions of the keys give partials (normalised binary16 o, fp32 m and
//     l) in the decode layout with Tq*Hq rows per sequence, reduced by the
//     same merge kernel; a single partition writes the output directly.
#include <type_traits>

#include "decode_common.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kNid = 512;       // block ids staged per segment of a partition

// One tile (32 tokens) of converted operands in LDS: K as the A operand of
// the score MFMA, [16-row group gi][step s][lane] x 8 f16, then V as the A
// operand of 16-token PV MFMAs, [gi][d-tile e][lane] x 4 f16.
template <int D>
struct OpsLayout {
  static constexpr int S = D / 32, E = D / 16;
  static constexpr int KB = 2 * S * 64 * 16;
  static constexpr int VB = 2 * E * 64 * 8;
  static constexpr int BUF = KB + VB;          // 32 KB at D=256
};

// Raw rows a wave holds for its conversion job: a 16-row group of K (the
// lane's bytes of row m) or of V (the lane's rows 4j .. 4j+3).
template <typename KF, typename VF, bool VJ> struct JobRaw { typename KF::Raw k; };
template <typename KF, typename VF> struct JobRaw<KF, VF, true> { typename VF::Raw v[4]; };

// Workgroups per CU the register allocation is held to: two (two waves per
// SIMD, 256 registers) for one query tile per wave, else one. (F16 K at
// D = 256 spills 6 registers at two, and still measured 2-28% faster than at
// one: B=8 x 32K F16/Q4_0 Tq=8 222 -> 160 us, an F16 prefill chunk of 512
// tokens over 8K 308 -> 226 us.)
template <int KT, int VT, int D, int NTW>
struct CMinBlocks {
  static constexpr int value = NTW == 1 ? 2 : 1;
};

template <int KT, int VT, int D, int NTW>
__global__ void __launch_bounds__(kThreads, (CMinBlocks<KT, VT, D, NTW>::value))
chunk_kernel(const ChunkArgs a) {
  using KF = KFmt<KT, D>;
  using VF = VFmt<VT, D>;
  using OL = OpsLayout<D>;
  constexpr int S = D / 32;      // score MFMA steps
  constexpr int E = D / 16;      // PV d-tiles
  constexpr int kTile = 32;      // tokens per tile
  // raw rows of two tiles in flight where they fit the registers (Q4_0 K and
  // V, or D = 128), else one
  constexpr bool kDeep = (KT == kQ4_0 && VT == kQ4_0) || D == 128;

  extern __shared__ __align__(16) unsigned char c_lds[];
  int32_t* ids = reinterpret_cast<int32_t*>(c_lds + 2 * OL::BUF);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int m = lane & 15;
  const int j = lane >> 4;
  // this wave's conversion job in every tile: K or V of 16-token group gi
  const int job_gi = wave & 1;
  const bool job_v = wave >= 2;
  const int R = a.Tq * a.r;                        // query rows per kv head
  constexpr int kRows = 64 * NTW;                  // query rows per workgroup
  const int QG = (R + kRows - 1) / kRows;
  const int n_units = a.B * a.p_max * a.Hkv * QG;
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
    // ---- locate the unit: ((b*p_max + p)*Hkv + g)*QG + qg ------------------
    const int qg = u % QG;
    const int g = (u / QG) % a.Hkv;
    const int bp = u / (QG * a.Hkv);
    const int b = bp / a.p_max;
    const int p = bp - b * a.p_max;
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
    // this lane's query row in the wave's tile k (column n = m of its MFMAs);
    // the waves' 16-row tiles interleave so a short last block spreads over them
    bool valid[NTW];
    int64_t orow[NTW];
    int lim[NTW];
    int lim_min = INT32_MAX;
    const int P = L > 0 ? (L + a.psize - 1) / a.psize : 0;
    const int t_begin = p * a.psize;
    const int t_end = min(L, t_begin + a.psize);
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const int row = qg * kRows + (k * 4 + wave) * 16 + m;
      valid[k] = row < R;
      const int t = valid[k] ? row / a.r : 0;
      const int h = g * a.r + (valid[k] ? row - t * a.r : 0);
      orow[k] = (int64_t(b) * a.Tq + t) * a.Hq + h;   // row of out / partials
      lim[k] = valid[k] ? min(L - a.Tq + t, t_end - 1) : t_begin - 1;
      if (valid[k]) lim_min = min(lim_min, lim[k]);
    }
    if (L == 0) {
      // an empty (or refused) sequence: zero rows in direct mode; the merge
      // writes its zero rows otherwise
      if (a.direct && j == 0) {
#pragma unroll
        for (int k = 0; k < NTW; ++k)
          if (valid[k])
            for (int d = 0; d < D; ++d) a.out[orow[k] * D + d] = 0.0f;
      }
      continue;
    }
    if (p >= P) continue;                 // no such partition: nothing to write
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);
    const bool wave_rows = __any(valid[0]);
    // last key any row of the workgroup reads: that of its last valid row
    const int row_hi = min(R - 1, qg * kRows + kRows - 1);
    const int t_stop = min(t_end, L - a.Tq + row_hi / a.r + 1);

    // ---- Q operands ------------------------------------------------------------
    f16x8 qop[NTW][S];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const float* qr = a.q + orow[k] * D;
      const float keep = valid[k] ? a.qscale : 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) qop[k][s][i] = f16(valid[k] ? qr[KF::dslot(j, s, i)] * keep : 0.0f);
    }

    // reference max: +inf in columns past R (their p is exactly 0); -inf
    // until the row has seen a key
    float m_run[NTW], l_lane[NTW];
    f32x4 acc[NTW][E];
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      m_run[k] = valid[k] ? -INFINITY : INFINITY;
      l_lane[k] = 0.0f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc[k][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int bad = 0;

    for (int seg_t0 = t_begin; seg_t0 < t_stop; seg_t0 += seg_tokens) {
      const int seg_t1 = min(t_stop, seg_t0 + seg_tokens);
      const int jb0 = seg_t0 >> a.bs_shift;
      const int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
      __syncthreads();                       // ids[] and both operand buffers are free
      int badl = 0;
      for (int i = tid; i < nb; i += kThreads) {
        int32_t id = block_of(a.table, b, a.max_blocks, jb0 + i);
        if (uint32_t(id) >= uint32_t(a.nblocks)) { badl = 1; id = 0; }
        ids[i] = id;
      }
      bad |= __syncthreads_or(badl);
      const int ntiles = (seg_t1 - seg_t0 + kTile - 1) / kTile;

      // ---- this wave's job: raw K (VJ false) or V rows of group job_gi of
      // tile kt (a group past the segment reads through a zero-size buffer:
      // zeros); JobRaw holds only what the job needs
      auto load_job = [&](auto vj, int kt, auto& raw) __attribute__((always_inline)) {
        constexpr bool VJ = decltype(vj)::value;
        const int tg = seg_t0 + kt * kTile + 16 * job_gi;
        const bool live = kt < ntiles && tg < seg_t1;
        const int tq = live ? tg : seg_t0;
        const int32_t id = __builtin_amdgcn_readfirstlane(ids[(tq >> a.bs_shift) - jb0]);
        const int slot0 = live ? (tg & bs_mask) : 0;
        if constexpr (!VJ) {
          const rsrc_t kr = make_rsrc(a.k_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, KF::RB),
                                      live ? 16u * kstride : 0u);
          KF::load(raw.k, kr, kvoff);
        } else {
          const rsrc_t vr = make_rsrc(a.v_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, g, VF::RB),
                                      live ? 16u * vstride : 0u);
#pragma unroll
          for (int i = 0; i < 4; ++i) VF::load(raw.v[i], vr, vl, i * vstride);
        }
      };
      // ---- convert it once into the tile's LDS operand buffer ----------------
      auto convert_job = [&](auto vj, int kt, auto& raw, unsigned char* ops) __attribute__((always_inline)) {
        constexpr bool VJ = decltype(vj)::value;
        if constexpr (!VJ) {
#pragma unroll
          for (int s = 0; s < S; ++s)
            *reinterpret_cast<f16x8*>(ops + ((job_gi * S + s) * 64 + lane) * 16) = KF::op(raw.k, s, ksh, mg);
        } else {
          // rows past the last key any row reads (junk, maybe NaN) are zeroed
          const int t0 = seg_t0 + kt * kTile + 16 * job_gi;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (t0 + 4 * j + i >= seg_t1) VF::kill(raw.v[i]);
          unsigned char* vops = ops + OL::KB;
          if constexpr (VF::kQuant) {
            uint32_t q[4][VF::ND];
            f16x2 dd[2];
#pragma unroll
            for (int i = 0; i < 4; ++i) VF::realign(raw.v[i], vl.sh, q[i]);
#pragma unroll
            for (int qq = 0; qq < 2; ++qq) dd[qq] = f16x2{raw.v[2 * qq].d, raw.v[2 * qq + 1].d};
#pragma unroll
            for (int e = 0; e < E; ++e)
              *reinterpret_cast<f16x4*>(vops + ((job_gi * E + e) * 64 + lane) * 8) =
                  VF::template op_q<2>(q, dd, e, mg);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
              *reinterpret_cast<f16x4*>(vops + ((job_gi * E + e) * 64 + lane) * 8) =
                  VF::template op<2>(raw.v, e);
          }
        }
      };

      // ---- scores, online softmax (exp2) and PV of the wave's query tiles ----
      auto compute_tile = [&](int kt, const unsigned char* ops) __attribute__((always_inline)) {
        const int t0 = seg_t0 + kt * kTile;
        // even and odd steps accumulate apart (four independent MFMA chains
        // per query tile instead of two), summed once
        f32x4 sc[NTW][2], sc2[NTW][2];
#pragma unroll
        for (int k = 0; k < NTW; ++k) sc[k][0] = sc[k][1] = sc2[k][0] = sc2[k][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < S; ++s)
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const f16x8 kop = *reinterpret_cast<const f16x8*>(ops + ((gi * S + s) * 64 + lane) * 16);
#pragma unroll
            for (int k = 0; k < NTW; ++k) {
              if (s & 1) sc2[k][gi] = mfma(kop, qop[k][s], sc2[k][gi]);
              else sc[k][gi] = mfma(kop, qop[k][s], sc[k][gi]);
            }
          }
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
          mfma_settle(sc[k][0], sc[k][1], sc2[k][0], sc2[k][1]);
          sc[k][0] += sc2[k][0];
          sc[k][1] += sc2[k][1];
        }
        // causal and end-of-partition mask, only where some row's limit falls
        // inside the tile
        if (t0 + kTile - 1 > lim_min) {
#pragma unroll
          for (int k = 0; k < NTW; ++k)
#pragma unroll
            for (int gi = 0; gi < 2; ++gi)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (t0 + 16 * gi + 4 * j + i > lim[k]) sc[k][gi][i] = -INFINITY;
        }
        f16x4 pop[NTW][2];
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
          const float mx = fmaxf(fmaxf(fmaxf(sc[k][0][0], sc[k][0][1]), fmaxf(sc[k][0][2], sc[k][0][3])),
                                 fmaxf(fmaxf(sc[k][1][0], sc[k][1][1]), fmaxf(sc[k][1][2], sc[k][1][3])));
          // lazy rescale (lucebox PR #555, Summary: skip the rescale when the
          // max is unchanged): the reference moves only when a row's max
          // exceeds it by more than kSlack. A row whose reference does not
          // move keeps its sums as they are: that also covers rows with no key
          // yet (m = -inf, where exp2(m - m_new) would be exp2(-inf + inf)) and
          // the +inf columns past R.
          if (__any(mx > m_run[k] + kSlack)) {
            const float m_new = fmaxf(m_run[k], max_over_rows(mx));
            const float alpha = m_new == m_run[k] ? 1.0f : __builtin_amdgcn_exp2f(m_run[k] - m_new);
            l_lane[k] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[k][e] *= alpha;
            m_run[k] = m_new;
          }
          // a row with no key yet keeps m = -inf: its p are exp2(-inf) = 0
          const float m_use = m_run[k] == -INFINITY ? 0.0f : m_run[k];
          float pr[8];
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[4 * gi + i] = __builtin_amdgcn_exp2f(sc[k][gi][i] - m_use);
          l_lane[k] += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
#pragma unroll
          for (int gi = 0; gi < 2; ++gi)
            pop[k][gi] = f16x4{f16(pr[4 * gi]), f16(pr[4 * gi + 1]), f16(pr[4 * gi + 2]), f16(pr[4 * gi + 3])};
        }
        const unsigned char* vops = ops + OL::KB;
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int gi = 0; gi < 2; ++gi) {
            const f16x4 vop = *reinterpret_cast<const f16x4*>(vops + ((gi * E + e) * 64 + lane) * 8);
#pragma unroll
            for (int k = 0; k < NTW; ++k) acc[k][e] = mfma16(vop, pop[k][gi], acc[k][e]);
          }
      };

      // ---- the tile loop: one conversion per tile, one barrier per tile; the
      // next tile's raw rows are loaded while this one is computed, and the
      // operand buffers alternate so a tile's buffer is only rewritten after
      // every wave has passed the next barrier. The loop is written once per
      // job so a wave only holds its own job's raw rows (the waves run the
      // same number of barriers either way).
      auto ops_of = [&](int kt) __attribute__((always_inline)) { return c_lds + (kt & 1) * OL::BUF; };
      auto tile_loop = [&](auto vj) __attribute__((always_inline)) {
        using Raw = JobRaw<KF, VF, decltype(vj)::value>;
        if constexpr (kDeep) {
          // three raw tiles: two in flight while one is converted
          Raw r0, r1, r2;
          load_job(vj, 0, r0);
          load_job(vj, 1, r1);
          for (int kt = 0; kt < ntiles; kt += 3) {
            convert_job(vj, kt, r0, ops_of(kt));
            __syncthreads();
            load_job(vj, kt + 2, r2);
            if (wave_rows) compute_tile(kt, ops_of(kt));
            if (kt + 1 >= ntiles) break;
            convert_job(vj, kt + 1, r1, ops_of(kt + 1));
            __syncthreads();
            load_job(vj, kt + 3, r0);
            if (wave_rows) compute_tile(kt + 1, ops_of(kt + 1));
            if (kt + 2 >= ntiles) break;
            convert_job(vj, kt + 2, r2, ops_of(kt + 2));
            __syncthreads();
            load_job(vj, kt + 4, r1);
            if (wave_rows) compute_tile(kt + 2, ops_of(kt + 2));
          }
        } else {
          unsigned char* const ops0 = c_lds;
          unsigned char* const ops1 = c_lds + OL::BUF;
          Raw r0, r1;
          load_job(vj, 0, r0);
          for (int kt = 0; kt < ntiles; kt += 2) {
            convert_job(vj, kt, r0, ops0);
            __syncthreads();
            load_job(vj, kt + 1, r1);
            if (wave_rows) compute_tile(kt, ops0);
            if (kt + 1 >= ntiles) break;
            convert_job(vj, kt + 1, r1, ops1);
            __syncthreads();
            load_job(vj, kt + 2, r0);
            if (wave_rows) compute_tile(kt + 1, ops1);
          }
        }
      };
      if (job_v)
        tile_loop(std::true_type{});
      else
        tile_loop(std::false_type{});
    }

    // ---- partial (or final) rows -------------------------------------------
#pragma unroll
    for (int k = 0; k < NTW; ++k) mfma_settle(acc[k]);   // the last tile's PV MFMAs wrote them
    if (bad && tid == 0) atomicOr(a.status, 1u);
#pragma unroll
    for (int k = 0; k < NTW; ++k) {
      const float l_run = sum_over_rows(l_lane[k]);
      if (!valid[k]) continue;
      const float inv = bad ? __builtin_nanf("") : (l_run > 0.0f ? 1.0f / l_run : 0.0f);
      if (a.direct) {
        float* dst = a.out + orow[k] * D;
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[VF::dv(4 * j + i, e)] = acc[k][e][i] * inv;
      } else {
        const int64_t prow = orow[k] * a.p_max + p;
        f16* dst = reinterpret_cast<f16*>(a.part_o) + prow * D;
        if (j == 0) {
          a.part_ml[2 * prow] = bad ? __builtin_nanf("") : (l_run > 0.0f ? m_run[k] : -INFINITY);
          a.part_ml[2 * prow + 1] = l_run;
        }
#pragma unroll
        for (int e = 0; e < E; e += 2)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            store_f16_pair(dst, VF::dv(4 * j + i, e), acc[k][e][i] * inv, acc[k][e + 1][i] * inv);
      }
    }
  }
}

template <int KT, int VT, int D, int NTW>
hipError_t launch_nt(const ChunkArgs& a, hipStream_t stream) {
  constexpr size_t lds = 2 * OpsLayout<D>::BUF + 4 * ((kNid + 1 + 3) & ~3);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chunk_kernel<KT, VT, D, NTW>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((chunk_kernel<KT, VT, D, NTW>), dim3(a.grid), dim3(kThreads), lds, stream, a);
  return hipGetLastError();
}

template <int KT, int VT, int D>
hipError_t launch_typed(const ChunkArgs& a, hipStream_t stream) {
  if (a.nt == 1) return launch_nt<KT, VT, D, 1>(a, stream);
  if constexpr (D == 128) {
    if (a.nt == 2) return launch_nt<KT, VT, D, 2>(a, stream);
  }
  return hipErrorInvalidValue;
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
