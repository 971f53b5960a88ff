// Multi-token queries with few query rows per kv head: the window kernel.
//
// What it computes is what chunk.hip computes (lucebox PR #555, Roadmap item
// 3: several query tokens per sequence attend over the K/V already in the
// pool, causally inside the chunk; TensorFold PR #1418, What: paged
// prompt-chunk attention): chunk token t of sequence b (length L) sits at position
// L - Tq + t and attends to the keys at positions 0 .. L - Tq + t of kv head
// g = h / r. It serves the chunks whose Tq*r query rows of a kv head fit
// 16*NQ MFMA columns, NQ <= 3 at D = 128, and at D = 256 NQ <= 2, or 3 with
// Q4_0 K and V (at r = 6 a verify window of up to 5 tokens at D = 256, 8 for
// Q4_0 or at D = 128), where
// converting each K/V tile into LDS operands for four waves of 16 rows
// (chunk.hip) costs more LDS traffic than the rows are worth.
//
// It is the decode kernel's LDS ring with the query rows in place of the
// heads: a workgroup of four wave64s takes a unit (sequence b, key partition
// p, group hg of kv heads), the DMA brings each 16-slot group of those
// heads' K and V rows into LDS as 1 KB contiguous instructions, and each
// wave converts the K and V rows it reads from LDS once into MFMA operands
// used for all of its NQ column groups. Two shapes of workgroup:
//  * a quad of kv heads, wave w serving head 4*hg + w over the whole head
//    dimension (one column group: two workgroups per CU, as in decode; two
//    or three at D = 128 with K or V quantised: mostly two per CU as well,
//    chunk_window_wgs_per_cu (Q4_0 B=8 x 32K, Tq=8 at r=4: 145 -> 94 us per
//    step against one); otherwise one workgroup per CU, whose registers
//    hold the NQ*D/16 accumulator tiles and NQ*D/32 Q operands);
//  * two or three column groups at D = 256, where two are already 64 + 128
//    registers and one wave per SIMD leaves the step latency-bound: a pair
//    of kv heads, two waves per head, each taking half of the head
//    dimension (its Q operands, K and V conversion and output columns), the
//    halves' partial scores added through LDS each step; two workgroups per
//    CU. (Measured on the verify window Q4_0 B=8 L=32768 Tq=4: 121 us per
//    step with the quad of whole-dimension waves, 99 us with the pairs;
//    Tq=8, three groups: 120 us against 140 us on the tile kernel. With a
//    Q8_0 side the three-group split measured no faster than the tile
//    kernel, which keeps those.)
// Each lane's row has its own causal limit; only steps that cross some row's
// limit are masked, and a row with no key in the partition writes m = -inf,
// l = 0. Partials use the decode layout with Tq*Hq rows per sequence and go
// through the same merge.
#include <type_traits>

#include "decode_common.h"
#include "lds_ring.h"

namespace pa {
namespace {

constexpr int kNidS = 512;     // block ids staged per segment of a partition
constexpr int kIdsBytes = 4 * ((kNidS + 1 + 3) & ~3);

// The ring of this kernel. WH = 1 (a quad of kv heads, one wave each): where
// the registers fit two workgroups per CU (chunk_window_wgs_per_cu) the ring
// is the decode kernel's; otherwise one workgroup per CU holds the registers
// of two and may use twice the decode kernel's LDS. WH = 2 (a pair of kv heads, two waves each): two workgroups
// per CU, each with 80 KB of LDS for the ring, the block ids and XBYTES for
// the partial scores the waves exchange; steps of two 16-slot groups where
// that leaves two ring slots, else one.
template <int KT, int VT, int D, int NQ, int WH>
struct WinRing {
  static_assert(WH == chunk_window_split(NQ, D), "the split the plan counts units by");
  static constexpr int NH = WH == 2 ? 2 : 4;           // kv heads per workgroup
  static constexpr int kWgsPerCu = chunk_window_wgs_per_cu(NQ, D, KT, VT);
  static constexpr int xbytes(int g) { return WH == 2 ? 4 * NQ * g * 64 * 16 : 0; }
  static constexpr int slot(int g) {
    return g * 1024 * (lds_dma_per_slots(KT, D, 16, NH) + lds_dma_per_slots(VT, D, 16, NH));
  }
  static constexpr int budget(int g) {
    // (1 KB of the 80 is left for the static LDS the compiler may add)
    return WH == 2 ? 79 * 1024 - kIdsBytes - xbytes(g) : (kWgsPerCu == 2 ? kLdsRingBytes : 2 * kLdsRingBytes);
  }
  using LY = LdsLayout<KT, VT, D, 16, NH, WH == 2 ? (2 * slot(2) <= budget(2) ? 2 : 1) : 0>;
  static constexpr int XBYTES = xbytes(LY::G);
  static constexpr int R = budget(LY::G) / LY::SLOT < 4 ? budget(LY::G) / LY::SLOT : 4;
  static constexpr int BYTES = R * LY::SLOT;
  static constexpr int LDS = BYTES + kIdsBytes + XBYTES;
  static_assert(R >= 2, "two ring slots at least");
  static_assert(kWgsPerCu * (LDS + 1024) <= 160 * 1024, "the workgroups of a CU fit its LDS");
};

// WH = 1: wave w serves kv head 4*hg + w with the whole head dimension.
// WH = 2 (D = 256 with two column groups, where one wave's registers cannot
// hold the Q operands and accumulators of 32 rows at two waves per SIMD): a
// workgroup takes a pair of kv heads, waves w and w + 2 serving kv head
// 2*hg + w, wave w + 2h taking head-dimension positions [128h, 128h + 128). A
// D = 256 row of every format is two D = 128 rows back to back, so each wave
// runs the D = 128 operand formats on its half of the row. The two halves'
// partial scores meet through LDS once per step (both waves add them in the
// same order and so hold the same scores, softmax state and p); each wave
// then accumulates its half of the output columns.
template <int KT, int VT, int D, int NQ, int WH>
__global__ void __launch_bounds__(256, chunk_window_wgs_per_cu(NQ, D, KT, VT)) chunk_lds_kernel(const ChunkArgs a) {
  static_assert(WH == 1 || (WH == 2 && D == 256), "the head dimension splits in two at D = 256 only");
  constexpr int kThreads = 256;
  constexpr int kWaves = 4;
  constexpr int NH = WinRing<KT, VT, D, NQ, WH>::NH;
  constexpr int DH = D / WH;     // head-dimension positions of a wave
  constexpr int kIdRegs = (kNidS + 1 + kThreads - 1) / kThreads;   // ids a thread fetches
  using KF = KFmt<KT, DH>;
  using VF = VFmt<VT, DH>;
  using WR = WinRing<KT, VT, D, NQ, WH>;
  using LY = typename WR::LY;
  constexpr int RS = WR::R;      // ring slots
  constexpr int S = DH / 32;     // score MFMA steps
  constexpr int E = DH / 16;     // PV d-tiles
  constexpr int G = LY::G;       // 16-row groups per step
  constexpr int T = 16 * G;      // tokens per step
  constexpr int NP = 2 * G;      // V row pairs per lane (4 rows per group)
  constexpr int NIW = (LY::NI + kWaves - 1) / kWaves;   // DMA instructions per wave and step, at most
  constexpr bool kKFold = KT == kQ4_0;   // Q4_0 offsets folded into corrections
  constexpr bool kVFold = VT == kQ4_0;
  constexpr int KF_NBL = kKFold ? DH / 128 : 1;  // ggml blocks per K lane window

  unsigned char* const ring = g_lds;
  int32_t* ids = reinterpret_cast<int32_t*>(g_lds + WR::BYTES);
  f32x4* xbuf = reinterpret_cast<f32x4*>(g_lds + WR::BYTES + kIdsBytes);   // WH = 2

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform
  const int hw = wave & (NH - 1);                             // the wave's kv head within the quad or pair
  const int hf = wave / NH;                                   // half of the head dimension
  const int m = lane & 15;
  const int j = lane >> 4;
  const int R = a.Tq * a.r;                      // query rows per kv head (<= 16*NQ)
  const int HG = a.Hkv / NH;
  const int n_units = a.B * a.p_max * HG;
  const int Gd = gridDim.x;
  const int logical = xcd_logical(blockIdx.x, Gd);

  const int cw = (LY::NI - wave + kWaves - 1) / kWaves;   // DMA instructions this wave issues per step
  // LDS offsets (within a group) of the rows this lane reads: K row m, V rows
  // 4j+i, of the wave's head, at their rotated row positions (and the wave's
  // half of each row)
  constexpr int kHalfK = row_bytes_of(KT, DH), kHalfV = row_bytes_of(VT, DH);
  const int k_row = m * LY::SPK + ((hw + RowRot<LY::RBK, NH>::k(m)) & (NH - 1)) * LY::RBK + hf * kHalfK +
                    int(KF::lane_off(j));
  int v_row[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    v_row[i] = (4 * j + i) * LY::SPV + ((hw + RowRot<LY::RBV, NH>::v(4 * j + i)) & (NH - 1)) * LY::RBV +
               hf * kHalfV;
  const uint32_t kstride = uint32_t(a.Hkv) * LY::RBK;  // pool bytes between token slots
  const uint32_t vstride = uint32_t(a.Hkv) * LY::RBV;
  const uint32_t ksh = KF::shift(j);
  const auto vl = VF::lane(m, 0u);
  const uint32_t mg = opaque_vgpr(kMagic);
  const int seg_tokens = kNidS << a.bs_shift;

  for (int u = logical; u < n_units; u += Gd) {
    // ---- locate the unit: (b*p_max + p)*HG + hg -------------------------------
    const int hg = u % HG;
    const int bp = u / HG;
    const int b = bp / a.p_max;
    const int p = bp - b * a.p_max;
    int L = a.seq_len[b];
    if (L < 0 || L > a.cap_tokens) {
      if (tid == 0 && p == 0 && hg == 0) atomicOr(a.status, 2u);
      L = L < 0 ? 0 : a.cap_tokens;
    }
    if (L > 0 && L < a.Tq) {             // the chunk is longer than the sequence
      if (tid == 0 && p == 0 && hg == 0) atomicOr(a.status, 2u);
      L = 0;
    }
    L = __builtin_amdgcn_readfirstlane(L);
    const int g = NH * hg + hw;                         // this wave's kv head
    const int P = L > 0 ? (L + a.psize - 1) / a.psize : 0;
    const int t_begin = p * a.psize;
    const int t_end = min(L, t_begin + a.psize);
    // this lane's query row in column group k: row n = 16k + m, i.e. chunk
    // token n / r of head g*r + n % r; its last visible key; rows past R are
    // dead columns (zero q, reference +inf, never written)
    bool valid[NQ];
    int64_t orow[NQ];
    int lim[NQ];
    int lim_min = INT32_MAX;
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const int row = 16 * k + m;
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
        for (int k = 0; k < NQ; ++k)
          if (valid[k])
            for (int d = hf * DH; d < hf * DH + DH; ++d) a.out[orow[k] * D + d] = 0.0f;
      }
      continue;
    }
    if (p >= P) continue;                 // no such partition: nothing to write
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) lim_min = min(lim_min, __shfl_xor(lim_min, off));
    lim_min = __builtin_amdgcn_readfirstlane(lim_min);

    const uint32_t khead = uint32_t(NH * hg) * LY::RBK;   // first head's offset in a slot
    const uint32_t vhead = uint32_t(NH * hg) * LY::RBV;
    // this lane's pool offset in each DMA instruction q = wave + kWaves*i of a step
    uint32_t dvoff[NIW];
#pragma unroll
    for (int i = 0; i < NIW; ++i) {
      const int q = wave + kWaves * i;
      if (q < G * LY::NIK)
        dvoff[i] = chunk_voff<LY::CPK, LY::RBK, 16, NH>(q % LY::NIK, lane, kstride, khead, 16u * kstride,
                                                         RowRot<LY::RBK, NH>::k);
      else
        dvoff[i] = chunk_voff<LY::CPV, LY::RBV, 16, NH>((q - G * LY::NIK) % LY::NIV, lane, vstride, vhead,
                                                         16u * vstride, RowRot<LY::RBV, NH>::v);
    }

    // ---- the first segment's block ids and the first column group's q
    // values, in flight together; the first steps' DMA is issued before the
    // Q operands are built
    int seg_t0 = t_begin;
    int seg_t1 = min(t_end, seg_t0 + seg_tokens);
    int jb0 = seg_t0 >> a.bs_shift;
    int nb = ((seg_t1 - 1) >> a.bs_shift) - jb0 + 1;
    int32_t idr[kIdRegs];
#pragma unroll
    for (int k = 0; k < kIdRegs; ++k)
      idr[k] = block_of(a.table, b, a.max_blocks, jb0 + min(tid + k * kThreads, nb - 1));
    auto load_q = [&](int k, float (&qv)[S][8]) __attribute__((always_inline)) {
      // a dead column reads a live row; q is 16-byte aligned on this path
      load_q_slots<KF, S>(a.q + (valid[k] ? orow[k] : orow[0]) * D + hf * DH, j, qv);
    };
    float qv[S][8];
    load_q(0, qv);
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

    // ---- DMA of step s of the current segment into ring slot s % RS (each
    // wave its share) -----------------------------------------------------------
    auto issue = [&](int s) __attribute__((always_inline)) {
      issue_step<LY>(wave, a, uint32_t(s % RS) * LY::SLOT, seg_t0 + s * T, seg_t1, ids, jb0, kstride,
                     vstride, dvoff);
    };
    int nsteps = (seg_t1 - seg_t0 + T - 1) / T;
    for (int s = 0; s < RS - 1 && s < nsteps; ++s) issue(s);

    // ---- Q operands, column group by column group, and the Q4_0 K offset
    // corrections (the first group's q values are already loaded)
    f16x8 qop[NQ][S];
    float kcorr[NQ][KF_NBL];
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      if (k > 0) load_q(k, qv);
      const float keep = valid[k] ? a.qscale : 0.0f;
#pragma unroll
      for (int s = 0; s < S; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // Q4_0: the high-nibble slots meet K values in the x16 frame
          const float hs = (kKFold && KFmtHi<KT, DH>::hi(i)) ? 0.0625f : 1.0f;
          qop[k][s][i] = f16(qv[s][i] * keep * hs);
        }
#pragma unroll
      for (int bl = 0; bl < KF_NBL; ++bl) {
        float qsum = 0.0f;
#pragma unroll
        for (int s2 = 4 * bl; s2 < 4 * bl + 4; ++s2)
#pragma unroll
          for (int i = 0; i < 8; ++i) qsum += float(qop[k][s2][i]) * (KFmtHi<KT, DH>::hi(i) ? 16.0f : 1.0f);
        kcorr[k][bl] = -8.0f * qsum;
      }
    }

    // reference max: +inf in dead columns (their p is exactly 0), -inf until
    // the row has seen a key
    float m_run[NQ], l_lane[NQ];
    f32x4 acc[NQ][E];
    f32x4 vcorr[NQ];              // Q4_0 V: sum_t d_t p_t per row block
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      m_run[k] = valid[k] ? -INFINITY : INFINITY;
      l_lane[k] = 0.0f;
      vcorr[k] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < E; ++e) acc[k][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    int vshift = 0;               // Q4_0 V: acc holds the sums times 2^-vshift

    for (;;) {
      // ---- compute step s from LDS: scores, online softmax (exp2), PV -------
      auto compute = [&](int s) __attribute__((always_inline)) {
        const unsigned char* slot = ring + (s % RS) * LY::SLOT;
        const int t0 = seg_t0 + s * T;
        const bool full = t0 + T <= t_end;
        const int rem = t_end - t0;
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
          // zero V rows past the partition end so 0 * junk never reaches PV
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * j >= rem - 16 * gi - i) VF::kill(vr[4 * gi + i]);
        }
        // Q4_0 scale range (see the decode kernel): |d| < 64 for the fma form
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
          f16 dv = f16(0.0f);
#pragma unroll
          for (int i = 0; i < 2 * NP; ++i) dv = __builtin_fmaxf16(dv, __builtin_fabsf16(vr[i].d));
          if (__any(dv >= f16(64.0f))) kv = wave_max_shift(scale_shift(dv));
        }

        // ---- scores: each K operand serves the NQ column groups ------------
        f32x4 sc[NQ][G];
#pragma unroll
        for (int k = 0; k < NQ; ++k)
#pragma unroll
          for (int gi = 0; gi < G; ++gi) sc[k][gi] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (kKFold) {
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
            for (int s2 = 0; s2 < S; ++s2) {
              const f16x8 kop = KF::op_n16(kr[gi], s2, ksh, mg, d2, c2);
#pragma unroll
              for (int k = 0; k < NQ; ++k) sc[k][gi] = mfma(kop, qop[k][s2], sc[k][gi]);
            }
          }
          if (kk) {
            const float up = __builtin_ldexpf(1.0f, kk);
#pragma unroll
            for (int k = 0; k < NQ; ++k)
#pragma unroll
              for (int gi = 0; gi < G; ++gi) sc[k][gi] *= up;
          }
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int bl = 0; bl < KF_NBL; ++bl) {
              const float dsc = float(KF::dscale(kr[gi], bl, ksh));
#pragma unroll
              for (int k = 0; k < NQ; ++k)
                sc[k][gi] = __builtin_amdgcn_mfma_f32_16x16x4f32(dsc, kcorr[k][bl], sc[k][gi], 0, 0, 0);
            }
        } else {
#pragma unroll
          for (int s2 = 0; s2 < S; ++s2)
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
              const f16x8 kop = KF::op(kr[gi], s2, ksh, mg);
#pragma unroll
              for (int k = 0; k < NQ; ++k) sc[k][gi] = mfma(kop, qop[k][s2], sc[k][gi]);
            }
        }
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
          if constexpr (G == 1) mfma_settle(sc[k][0]);
          else mfma_settle(sc[k][0], sc[k][1]);
        }
        if constexpr (WH == 2) {
          // the two halves' partial scores: publish, barrier, add the other's
          // (a + b = b + a exactly, so both waves hold the same sums); the
          // next step's ring barrier keeps the buffer until both have read it
          f32x4* mine = xbuf + wave * (NQ * G * 64) + lane;
#pragma unroll
          for (int k = 0; k < NQ; ++k)
#pragma unroll
            for (int gi = 0; gi < G; ++gi) mine[(k * G + gi) * 64] = sc[k][gi];
          lds_barrier();
          const f32x4* other = xbuf + (wave ^ NH) * (NQ * G * 64) + lane;
#pragma unroll
          for (int k = 0; k < NQ; ++k)
#pragma unroll
            for (int gi = 0; gi < G; ++gi) sc[k][gi] += other[(k * G + gi) * 64];
        }
        // causal and end-of-partition mask, only where some row's limit falls
        // inside the step (lim <= t_end - 1 covers the slots past the end)
        if (t0 + T - 1 > lim_min) {
#pragma unroll
          for (int k = 0; k < NQ; ++k)
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
              for (int i = 0; i < 4; ++i)
                if (t0 + 16 * gi + 4 * j + i > lim[k]) sc[k][gi][i] = -INFINITY;
        }
        // ---- online softmax per column group (lazy rescale; a row whose
        // reference does not move keeps its sums, which also covers rows with
        // no key yet and the dead columns)
        typename OpVec<NP>::type pop[NQ];
#pragma unroll
        for (int k = 0; k < NQ; ++k) {
          float mx = -INFINITY;
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
            mx = fmaxf(mx, fmaxf(fmaxf(sc[k][gi][0], sc[k][gi][1]), fmaxf(sc[k][gi][2], sc[k][gi][3])));
          if (__any(mx > m_run[k] + kSlack)) {
            const float m_new = fmaxf(m_run[k], max_over_rows(mx));
            const float alpha = m_new == m_run[k] ? 1.0f : __builtin_amdgcn_exp2f(m_run[k] - m_new);
            l_lane[k] *= alpha;
#pragma unroll
            for (int e = 0; e < E; ++e) acc[k][e] *= alpha;
            vcorr[k] *= alpha;
            m_run[k] = m_new;
          }
          // a row with no key yet keeps m = -inf: its p are exp2(-inf) = 0
          const float m_use = m_run[k] == -INFINITY ? 0.0f : m_run[k];
          float pr[2 * NP];
#pragma unroll
          for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int i = 0; i < 4; ++i) pr[4 * gi + i] = __builtin_amdgcn_exp2f(sc[k][gi][i] - m_use);
          float ps = 0.0f;
#pragma unroll
          for (int i = 0; i < 2 * NP; i += 4) ps += (pr[i] + pr[i + 1]) + (pr[i + 2] + pr[i + 3]);
          l_lane[k] += ps;
#pragma unroll
          for (int i = 0; i < 2 * NP; ++i) pop[k][i] = f16(pr[i]);
        }
        auto pv = [&](typename OpVec<NP>::type av, const typename OpVec<NP>::type& bv, f32x4 c)
            __attribute__((always_inline)) {
          if constexpr (NP == 4) return mfma(av, bv, c);
          else return mfma16(av, bv, c);
        };
        __builtin_amdgcn_s_setprio(1);
        // ---- PV: each V operand serves the NQ column groups -----------------
        if constexpr (VF::kQuant) {
          uint32_t q[2 * NP][VF::ND];
          f16x2 dd[NP];
#pragma unroll
          for (int i = 0; i < 2 * NP; ++i) VF::realign(vr[i], vl.sh, q[i]);
#pragma unroll
          for (int qq = 0; qq < NP; ++qq) dd[qq] = f16x2{vr[2 * qq].d, vr[2 * qq + 1].d};
          if constexpr (kVFold) {
            if (kv != vshift) {
              const float f = __builtin_ldexpf(1.0f, vshift - kv);
#pragma unroll
              for (int k = 0; k < NQ; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e) acc[k][e] *= f;
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
            for (int e = 0; e < E; ++e) {
              const auto vop = VF::template op_n16<NP>(q, ds, cc, e, mg);
#pragma unroll
              for (int k = 0; k < NQ; ++k) acc[k][e] = pv(vop, pop[k], acc[k][e]);
            }
            const auto dop = OpVec<NP>::pack(dd);
#pragma unroll
            for (int k = 0; k < NQ; ++k) vcorr[k] = pv(dop, pop[k], vcorr[k]);
          } else {
#pragma unroll
            for (int e = 0; e < E; ++e) {
              const auto vop = VF::template op_q<NP>(q, dd, e, mg);
#pragma unroll
              for (int k = 0; k < NQ; ++k) acc[k][e] = pv(vop, pop[k], acc[k][e]);
            }
          }
        } else {
#pragma unroll
          for (int e = 0; e < E; ++e) {
            const auto vop = VF::template op<NP>(vr, e);
#pragma unroll
            for (int k = 0; k < NQ; ++k) acc[k][e] = pv(vop, pop[k], acc[k][e]);
          }
        }
      };

      // ---- the ring: steps s+1 .. s+RS-1 in flight while step s is computed
      for (int s = 0; s < nsteps; ++s) {
        if constexpr (RS == 2) {
          wait_dma_then_barrier(0);
        } else {
          const int later = min(RS - 2, nsteps - 1 - s);
          wait_dma_then_barrier(later * cw);
        }
        __builtin_amdgcn_s_setprio(3);
        if (s + RS - 1 < nsteps) issue(s + RS - 1);
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
      for (int s = 0; s < RS - 1 && s < nsteps; ++s) issue(s);
    }

    // ---- partial (or final) rows -------------------------------------------
#pragma unroll
    for (int k = 0; k < NQ; ++k) mfma_settle(acc[k], vcorr[k]);   // the last step's PV MFMAs wrote them
    if (bad && tid == 0) atomicOr(a.status, 1u);
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
      const float l_run = sum_over_rows(l_lane[k]);
      if constexpr (kVFold) {
        // add the -8 offset of every accumulated value, undo the x16 frame
        const float f = __builtin_ldexpf(1.0f, vshift);
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float fe = VFmtHi<VT, DH>::hi(e) ? f * 0.0625f : f;
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[k][e][i] = acc[k][e][i] * fe - 8.0f * vcorr[k][i];
        }
      }
      if (!valid[k]) continue;
      const float inv = bad ? __builtin_nanf("") : (l_run > 0.0f ? 1.0f / l_run : 0.0f);
      if (a.direct) {
        float* dst = a.out + orow[k] * D + hf * DH;
#pragma unroll
        for (int e = 0; e < E; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) dst[VF::dv(4 * j + i, e)] = acc[k][e][i] * inv;
      } else {
        const int64_t prow = orow[k] * a.p_max + p;
        f16* dst = reinterpret_cast<f16*>(a.part_o) + prow * D + hf * DH;
        if (j == 0 && hf == 0) {
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

template <int KT, int VT, int D, int NQ, int WH = 1>
hipError_t launch_nq(const ChunkArgs& a, hipStream_t stream) {
  constexpr size_t lds = size_t(WinRing<KT, VT, D, NQ, WH>::LDS);
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&chunk_lds_kernel<KT, VT, D, NQ, WH>),
      hipFuncAttributeMaxDynamicSharedMemorySize, int(lds));
  if (attr != hipSuccess) return attr;
  hipLaunchKernelGGL((chunk_lds_kernel<KT, VT, D, NQ, WH>), dim3(a.grid), dim3(256), lds, stream, a);
  return hipGetLastError();
}

template <int KT, int VT, int D>
hipError_t launch_typed(const ChunkArgs& a, hipStream_t stream) {
  if constexpr (lds_groups(KT, VT, D) == 0) {
    return hipErrorInvalidValue;
  } else {
    const int nq = (a.Tq * a.r + 15) / 16;
    if (nq == 1) return launch_nq<KT, VT, D, 1>(a, stream);
    if (nq == 2) return launch_nq<KT, VT, D, 2, chunk_window_split(2, D)>(a, stream);
    if (nq == 3) return launch_nq<KT, VT, D, 3, chunk_window_split(3, D)>(a, stream);
    return hipErrorInvalidValue;
  }
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

hipError_t launch_chunk_lds(const ChunkArgs& a, hipStream_t stream) {
  if (a.Hkv % 4) return hipErrorInvalidValue;   // (pairs of heads too: the plan counts units by quads or pairs)
  if (a.D == 256) return launch_d<256>(a, stream);
  if (a.D == 128) return launch_d<128>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
