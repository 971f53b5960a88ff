// The LDS ring shared by the LDS-staged kernels: geometry of a step's slot,
// placement of the head rows (a quad or a pair of kv heads) in LDS, the
// per-lane pool offsets of the 1 KB DMA instructions that fill it, and the
// per-step wait + barrier.
// (Included by one translation unit each; everything is internal.)
#pragma once

#include "decode_common.h"

namespace pa {
namespace {

// GS: token slots per group, 16, or 8 for the decode kernel's rows too large
// for 16 (decode_group_slots). NH: kv heads per slot, 4 (a quad), or 2 for
// the window kernel's half-quad workgroups. GF: groups per step, 0 for the
// default (lds_groups() for 16 slots, else 1).
template <int KT, int VT, int D, int GS = 16, int NH = 4, int GF = 0>
struct LdsLayout {
  static_assert(GS == 16 || GS == 8, "groups of 16 or 8 slots");
  static_assert(NH == 4 || NH == 2, "quads or pairs of kv heads");
  static constexpr int kNH = NH;
  static constexpr int RBK = row_bytes_of(KT, D), RBV = row_bytes_of(VT, D);
  static constexpr int SPK = NH * RBK, SPV = NH * RBV; // one slot's rows of NH heads
  static constexpr int CPK = SPK / 16, CPV = SPV / 16; // 16-byte chunks per slot
  static constexpr int NIK = lds_dma_per_slots(KT, D, GS, NH), NIV = lds_dma_per_slots(VT, D, GS, NH);
  static constexpr int G = GF ? GF : (GS == 16 ? lds_groups(KT, VT, D) : 1);
  static constexpr int VOFF = G * NIK * 1024;          // V groups follow the K groups
  static constexpr int SLOT = G * 1024 * (NIK + NIV);
  static constexpr int R = SLOT == 0 ? 0 : (kLdsRingBytes / SLOT > kLdsMaxSlots ? kLdsMaxSlots
                                                                               : kLdsRingBytes / SLOT);
  static constexpr int NI = G * (NIK + NIV);           // DMA instructions per step
  static constexpr int NIW = (NI + 3) / 4;             // at most this many per wave
  static constexpr int kGS = GS;        // token slots per group
  static_assert(SPK % 16 == 0 && SPV % 16 == 0, "a slot's rows are whole 16-byte chunks");
};

// x16-frame slots / columns of the Q4_0 conversions (none for other formats).
template <int KT, int D> struct KFmtHi {
  __host__ __device__ static constexpr bool hi(int i) { return KT == kQ4_0 && (i & 2) != 0; }
};
template <int VT, int D> struct VFmtHi {
  __host__ __device__ static constexpr bool hi(int e) { return VT == kQ4_0 && e >= (D / 16) / 2; }
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// The workgroup's dynamic LDS (declared at file scope so that the DMA
// destination below is known to be an LDS address).
extern __shared__ __align__(16) unsigned char g_lds[];

// LDS placement of the NH head rows of a slot. Within slot t, head w's row
// is stored at row position (w + rot(t)) mod NH, so that the 64 lanes of a
// wave, which read the same head's K rows from 16 slots at once, spread over
// the LDS banks (a plain copy puts those 16 rows 576 bytes apart on the same
// few banks; measured 5% slower). The V rows a wave reads at once come from 4
// slots and keep their pool order: rotating them measured 0.5-1% slower.
// Only rows made of whole 16-byte chunks can be moved this way
// (row_bytes % 16 == 0); other rows keep rot = 0.
template <int RB, int NH = 4> struct RowRot {
  static constexpr bool on = RB % 16 == 0;
  __device__ static int k(int t) { return on ? (t >> 2) & (NH - 1) : 0; }   // K: 16 slots
  __device__ static int v(int) { return 0; }                               // V: 4 slots
};

// Pool offset of the chunk lane l fetches in the 1 KB DMA instruction `sub`
// of a GS-slot group: LDS chunk 64*sub + l of a group whose slots are CP
// chunks (NH rows of RB bytes) long in LDS and `stride` bytes apart in the
// pool, starting `head_off` bytes into each pool slot, rows placed by `rot`;
// chunks past the group get `oob` (reads as 0).
template <int CP, int RB, int GS = 16, int NH = 4>
__device__ __forceinline__ uint32_t chunk_voff(int sub, int lane, uint32_t stride, uint32_t head_off,
                                               uint32_t oob, int (*rot)(int)) {
  const int c = 64 * sub + lane;
  const int slot = c / CP;
  int within = c - slot * CP;
  if constexpr (RowRot<RB, NH>::on) {
    constexpr int CPR = RB / 16;                       // chunks per row
    const int hp = within / CPR;                       // row position in LDS
    within += (((hp - rot(slot)) & (NH - 1)) - hp) * CPR;   // the pool row stored there
  }
  return c < GS * CP ? uint32_t(slot) * stride + head_off + 16u * within : oob;
}

// One DMA instruction: every lane fetches 16 bytes at its offset and the
// wave lands them as 1 KB at LDS byte dst + 16*lane. With quads of kv heads
// every pool line is read once here (a workgroup owns whole token rows of its
// quad), so the loads carry the non-temporal hint: it raised the streaming
// rate of this pattern from ~5.9 to ~6.7 TB/s when measured on its own. (The
// window kernel's pairs share the line where one pair's rows end and the
// next begin: +10% fetched at Q4_0 D=256; without the hint that kernel ran
// 1% faster and every quad kernel 6-9% slower, so the hint stays.)
constexpr int kDmaNonTemporal = 2;
__device__ __forceinline__ void dma16(rsrc_t R, uint32_t dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(R, (lds_ptr_t)(g_lds + dst), 16, voff, 0, 0, kDmaNonTemporal);
}

// DMA of one step into the ring slot at LDS byte `slot`: the LY::G groups of
// GS token slots of K and V, tokens t0 .. t0 + GS*LY::G - 1 of the current segment
// (block ids[] staged from block jb0; groups at or past seg_t1 get a
// zero-size resource and read nothing). Of the NW issuing waves, wave W
// issues the instructions q with q % NW == W; W is a compile-time constant,
// so the selection costs no branches. dvoff[i] is this lane's pool offset in
// instruction W + NW*i.
template <class LY, int W, class Args, int NW = 4>
__device__ __forceinline__ void issue_step_as(const Args& a, uint32_t slot, int t0, int seg_t1,
                                              const int32_t* ids, int jb0, uint32_t kstride,
                                              uint32_t vstride, const uint32_t* dvoff) {
  constexpr int G = LY::G;
  const int bs_mask = (1 << a.bs_shift) - 1;
#pragma unroll
  for (int gi = 0; gi < G; ++gi) {
    const int tg = t0 + LY::kGS * gi;
    const bool live = tg < seg_t1;
    const int32_t id = live ? __builtin_amdgcn_readfirstlane(ids[(tg >> a.bs_shift) - jb0]) : 0;
    const int slot0 = live ? (tg & bs_mask) : 0;
    const rsrc_t kr = make_rsrc(a.k_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, 0, LY::RBK),
                                live ? uint32_t(LY::kGS) * kstride : 0u);
    const rsrc_t vr = make_rsrc(a.v_pool + row_offset(id, slot0, a.bs_shift, a.Hkv, 0, LY::RBV),
                                live ? uint32_t(LY::kGS) * vstride : 0u);
#pragma unroll
    for (int sub = 0; sub < LY::NIK; ++sub) {
      const int q = gi * LY::NIK + sub;
      if (q % NW == W) dma16(kr, slot + q * 1024, dvoff[q / NW]);
    }
#pragma unroll
    for (int sub = 0; sub < LY::NIV; ++sub) {
      const int q = G * LY::NIK + gi * LY::NIV + sub;
      if (q % NW == W) dma16(vr, slot + LY::VOFF + (gi * LY::NIV + sub) * 1024, dvoff[q / NW]);
    }
  }
}
// The same for the calling wave (one switch on the wave index), NW = 4 or 8
// issuing waves.
template <class LY, class Args, int NW = 4>
__device__ __forceinline__ void issue_step(int wave, const Args& a, uint32_t slot, int t0, int seg_t1,
                                           const int32_t* ids, int jb0, uint32_t kstride,
                                           uint32_t vstride, const uint32_t* dvoff) {
  static_assert(NW == 4 || NW == 8, "four or eight issuing waves");
#define PA_ISSUE_CASE(w) \
  case w: issue_step_as<LY, w, Args, NW>(a, slot, t0, seg_t1, ids, jb0, kstride, vstride, dvoff); break;
  if constexpr (NW == 4) {
    switch (wave) {
      PA_ISSUE_CASE(0) PA_ISSUE_CASE(1) PA_ISSUE_CASE(2)
      default: issue_step_as<LY, 3, Args, NW>(a, slot, t0, seg_t1, ids, jb0, kstride, vstride, dvoff); break;
    }
  } else {
    switch (wave) {
      PA_ISSUE_CASE(0) PA_ISSUE_CASE(1) PA_ISSUE_CASE(2) PA_ISSUE_CASE(3)
      PA_ISSUE_CASE(4) PA_ISSUE_CASE(5) PA_ISSUE_CASE(6)
      default: issue_step_as<LY, 7, Args, NW>(a, slot, t0, seg_t1, ids, jb0, kstride, vstride, dvoff); break;
    }
  }
#undef PA_ISSUE_CASE
}

// s_waitcnt vmcnt(n) (n wave-uniform, at most 15; larger n waits for more
// than needed, which is safe) followed by the workgroup barrier. The asm
// memory clobber keeps every LDS read of the step after the barrier.
__device__ __forceinline__ void wait_dma_then_barrier(int n) {
#define PA_WAIT_CASE(k) \
  case k: asm volatile("s_waitcnt vmcnt(" #k ")\n\ts_barrier" ::: "memory"); break;
  switch (n < 15 ? n : 15) {
    PA_WAIT_CASE(0) PA_WAIT_CASE(1) PA_WAIT_CASE(2) PA_WAIT_CASE(3) PA_WAIT_CASE(4)
    PA_WAIT_CASE(5) PA_WAIT_CASE(6) PA_WAIT_CASE(7) PA_WAIT_CASE(8) PA_WAIT_CASE(9)
    PA_WAIT_CASE(10) PA_WAIT_CASE(11) PA_WAIT_CASE(12) PA_WAIT_CASE(13) PA_WAIT_CASE(14)
    default: asm volatile("s_waitcnt vmcnt(15)\n\ts_barrier" ::: "memory"); break;
  }
#undef PA_WAIT_CASE
}

// Workgroup barrier for data passed through LDS only: the wave's LDS
// accesses complete first, its DMA loads stay in flight (a __syncthreads()
// would also wait for those).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

}  // namespace
}  // namespace pa
