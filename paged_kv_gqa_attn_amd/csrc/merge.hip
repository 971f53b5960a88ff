// Max-shifted merge of the partitions' softmax partials.
//
// For each (sequence b, query head h) over its live partitions
// p < ceil(seq_len[b]/psize), with per-partition base-2 reference m_p, sum
// l_p and normalised output o_p (lucebox PR #555, Summary: partials stored
// normalised in f16, merged across partitions without overflow; llama.cpp PR #13 HRX,
// Changes: per-block normalisation scale):
//     M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
// The rows are (b, h) for decode and (b, t, h) for chunks (Hq then counts
// Tq*Hq rows per sequence); a partition that held no key for a row has
// m = -inf and l = 0 and so weight 0.
// The merge reads every partial byte once, so it is spread wide: a workgroup
// takes one (b, h) and 64 output columns (merge_slice, merge_common.h, which
// the single-launch decode calls too).
// With many rows of few partitions (p_max <= 16 over at least 1024 rows, or
// p_max <= 32 over at least 512, e.g. the Tq*Hq rows of a prefill chunk or
// a verify window) that layout leaves most threads idle and launches
// thousands of workgroups, and merge_rows_kernel is used instead: one thread
// per (row, 8 output columns) reads all of the row's partitions at once and
// sums them in order, 8 rows per workgroup at D=256.
// Loop bounds are the runtime partition count (llama.cpp PR #13, the
// SGPR-exhaustion fix: a constant-folded bound fully unrolled the reduction).
#include "merge_common.h"
#include "pa_host.h"

namespace pa {
namespace {

constexpr int kThreads = kMergeThreads;
constexpr int kCols = kMergeCols;

__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeArgs a) {
  __shared__ MergeLds lds;
  const int chunks = a.D / kCols;
  const int bh = blockIdx.x / chunks;
  const int col0 = (blockIdx.x - bh * chunks) * kCols;
  const int b = bh / a.Hq;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.cap_tokens ? a.cap_tokens : L);
  if (L < a.min_len) L = 0;       // a chunk longer than its sequence (flagged by the chunk kernel)
  const int P = (L + a.psize - 1) / a.psize;
  merge_slice<false>(reinterpret_cast<const f16*>(a.part_o) + int64_t(bh) * a.p_max * a.D,
              a.part_ml + int64_t(bh) * a.p_max * 2, P, a.D, col0, a.out + int64_t(bh) * a.D + col0, lds);
}

// The value that lane (lane ^ MASK) holds, for MASK < 32 (ds_swizzle in its
// bit-mask mode: no LDS memory is touched).
template <int MASK>
__device__ __forceinline__ float lane_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (MASK << 10)));
}

// S adjacent lanes serve one (row, 8 output columns): lane s of the group
// takes partitions s, s + S, s + 2S, ... (NPS of them, the most a row can
// have being NPS*S); the group's max is formed with lane swaps; each lane
// sums its own partitions in order, the 8 column sums are then halved over
// the group by log2(S) swap-and-add rounds, so lane s ends with 8/S columns
// of the row, and the weight sum is added over the group the same way
// (a fixed order: repeated runs give the same bits).
template <int NPS, int S>
__global__ void __launch_bounds__(kThreads) merge_rows_kernel(const MergeArgs a) {
  static_assert(S == 1 || S == 2 || S == 4, "a group of 1, 2 or 4 lanes");
  const int octs = a.D / 8;
  const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t rows = int64_t(a.B) * a.Hq;
  // (rows * octs * S is a multiple of S, so a group is whole or absent)
  if (gid >= rows * octs * S) return;
  const int s = int(gid & (S - 1));
  const int64_t cell = gid / S;
  const int64_t bh = cell / octs;
  const int q = int(cell - bh * octs);
  const int b = int(bh / a.Hq);
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.cap_tokens ? a.cap_tokens : L);
  if (L < a.min_len) L = 0;       // a chunk longer than its sequence (flagged by the chunk kernel)
  const int P = (L + a.psize - 1) / a.psize;
  float* dst = a.out + bh * a.D + 8 * q;
  if (P == 0) {                   // (uniform over the group: one row)
    constexpr int kw = 8 / S;
#pragma unroll
    for (int k = 0; k < kw; ++k) dst[s * kw + k] = 0.0f;
    return;
  }
  const float* ml = a.part_ml + bh * a.p_max * 2;
  const f16* o = reinterpret_cast<const f16*>(a.part_o) + bh * a.p_max * a.D + 8 * q;
  // every load reads a live partition (p clamped to P-1), so that none needs
  // a branch and all are in flight at once; dead slots are then masked (the
  // rows of a wave differ, so a per-row buffer resource would not be uniform)
  f16x8 v[NPS];
  float mp[NPS], lp[NPS];
#pragma unroll
  for (int j = 0; j < NPS; ++j)
    v[j] = *reinterpret_cast<const f16x8*>(o + int64_t(min(s + S * j, P - 1)) * a.D);
#pragma unroll
  for (int j = 0; j < NPS; ++j) {
    const int p = s + S * j;
    const float2 x = *reinterpret_cast<const float2*>(ml + 2 * min(p, P - 1));
    mp[j] = p < P ? x.x : -INFINITY;
    lp[j] = p < P ? x.y : 0.0f;
  }
  // a NaN m (a partition that met a bad block id) makes the row NaN: the
  // lane's weight sum becomes NaN, and so the group's
  float M = -INFINITY;
  bool nan_seen = false;
#pragma unroll
  for (int j = 0; j < NPS; ++j) {
    nan_seen |= mp[j] != mp[j];
    M = fmaxf(M, mp[j]);
  }
  if constexpr (S >= 4) M = fmaxf(M, lane_xor<2>(M));
  if constexpr (S >= 2) M = fmaxf(M, lane_xor<1>(M));
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float W = 0.0f;
  // (a dead slot has weight 2^-inf * 0 = 0 and holds a live partition's
  // finite values, so it adds exactly 0: no branch; a lane with no live
  // partition adds 0 as well)
#pragma unroll
  for (int j = 0; j < NPS; ++j) {
    const float w = __builtin_amdgcn_exp2f(mp[j] - M) * lp[j];
    W += w;
    merge_axpy8(acc, w, v[j]);
  }
  if (nan_seen) W = __builtin_nanf("");
  // halve the columns per round: the lane whose mask bit is 0 keeps the lower
  // half and adds its partner's lower half, the other the upper half
  int off = 0;
  if constexpr (S >= 4) {
    const bool hi = s & 2;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float keep = hi ? acc[4 + k] : acc[k];
      const float give = hi ? acc[k] : acc[4 + k];
      acc[k] = keep + lane_xor<2>(give);
    }
    W += lane_xor<2>(W);
    off += hi ? 4 : 0;
  }
  if constexpr (S >= 2) {
    constexpr int h = 8 / S;        // columns held after this round
    const bool hi = s & 1;
#pragma unroll
    for (int k = 0; k < h; ++k) {
      const float keep = hi ? acc[h + k] : acc[k];
      const float give = hi ? acc[k] : acc[h + k];
      acc[k] = keep + lane_xor<1>(give);
    }
    W += lane_xor<1>(W);
    off += hi ? h : 0;
  }
  constexpr int kw = 8 / S;
  float r[kw];
#pragma unroll
  for (int k = 0; k < kw; ++k) r[k] = acc[k] / W;
  if constexpr (kw == 8) {
    *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(r[4], r[5], r[6], r[7]);
  } else if constexpr (kw == 4) {
    *reinterpret_cast<float4*>(dst + off) = make_float4(r[0], r[1], r[2], r[3]);
  } else {
    *reinterpret_cast<float2*>(dst + off) = make_float2(r[0], r[1]);
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D % kCols) return hipErrorInvalidValue;
  const int64_t rows = int64_t(a.B) * a.Hq;
  if (merge_rows_layout(rows, a.p_max)) {
    // the smallest unrolled partition count that covers p_max (slots past a
    // row's partitions re-read its last one and add 0, so a tight count saves
    // those loads and their arithmetic); past 8 partitions two or four lanes
    // share a row's columns, each reading its share of the partitions
    const int S = a.p_max <= 8 ? 1 : (a.p_max <= 16 ? 2 : 4);
    const int64_t threads = rows * (a.D / 8) * S;
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    const dim3 g{unsigned(blocks)}, t{unsigned(kThreads)};
    if (a.p_max <= 2) hipLaunchKernelGGL((merge_rows_kernel<2, 1>), g, t, 0, stream, a);
    else if (a.p_max <= 4) hipLaunchKernelGGL((merge_rows_kernel<4, 1>), g, t, 0, stream, a);
    else if (a.p_max <= 6) hipLaunchKernelGGL((merge_rows_kernel<6, 1>), g, t, 0, stream, a);
    else if (a.p_max <= 8) hipLaunchKernelGGL((merge_rows_kernel<8, 1>), g, t, 0, stream, a);
    else if (a.p_max <= 12) hipLaunchKernelGGL((merge_rows_kernel<6, 2>), g, t, 0, stream, a);
    else if (a.p_max <= 16) hipLaunchKernelGGL((merge_rows_kernel<8, 2>), g, t, 0, stream, a);
    else if (a.p_max <= 24) hipLaunchKernelGGL((merge_rows_kernel<6, 4>), g, t, 0, stream, a);
    else hipLaunchKernelGGL((merge_rows_kernel<8, 4>), g, t, 0, stream, a);
  } else {
    hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq * (a.D / kCols)), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
