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

// NPM: the most partitions a row has (2 to 32)
template <int NPM>
__global__ void __launch_bounds__(kThreads) merge_rows_kernel(const MergeArgs a) {
  const int octs = a.D / 8;
  const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t rows = int64_t(a.B) * a.Hq;
  if (gid >= rows * octs) return;
  const int64_t bh = gid / octs;
  const int q = int(gid - bh * octs);
  const int b = int(bh / a.Hq);
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.cap_tokens ? a.cap_tokens : L);
  if (L < a.min_len) L = 0;       // a chunk longer than its sequence (flagged by the chunk kernel)
  const int P = (L + a.psize - 1) / a.psize;
  float* dst = a.out + bh * a.D + 8 * q;
  if (P == 0) {
    *reinterpret_cast<float4*>(dst) = make_float4(0.f, 0.f, 0.f, 0.f);
    *reinterpret_cast<float4*>(dst + 4) = make_float4(0.f, 0.f, 0.f, 0.f);
    return;
  }
  const float* ml = a.part_ml + bh * a.p_max * 2;
  const f16* o = reinterpret_cast<const f16*>(a.part_o) + bh * a.p_max * a.D + 8 * q;
  // every load reads a live partition (p clamped to P-1), so that none needs
  // a branch and all are in flight at once; dead slots are then masked (the
  // rows of a wave differ, so a per-row buffer resource would not be uniform)
  f16x8 v[NPM];
  float mp[NPM], lp[NPM];
#pragma unroll
  for (int p = 0; p < NPM; ++p)
    v[p] = *reinterpret_cast<const f16x8*>(o + int64_t(min(p, P - 1)) * a.D);
#pragma unroll
  for (int p = 0; p < NPM; ++p) {
    const float2 x = *reinterpret_cast<const float2*>(ml + 2 * min(p, P - 1));
    mp[p] = p < P ? x.x : -INFINITY;
    lp[p] = p < P ? x.y : 0.0f;
  }
  // a NaN m (a partition that met a bad block id) makes the row NaN
  float M = -INFINITY;
  bool nan_seen = false;
#pragma unroll
  for (int p = 0; p < NPM; ++p) {
    nan_seen |= mp[p] != mp[p];
    M = fmaxf(M, mp[p]);
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float W = 0.0f;
  // (a dead slot has weight 2^-inf * 0 = 0 and holds a live partition's
  // finite values, so it adds exactly 0: no branch)
#pragma unroll
  for (int p = 0; p < NPM; ++p) {
    const float w = __builtin_amdgcn_exp2f(mp[p] - M) * lp[p];
    W += w;
    merge_axpy8(acc, w, v[p]);
  }
  float r[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) r[k] = nan_seen ? __builtin_nanf("") : acc[k] / W;
  *reinterpret_cast<float4*>(dst) = make_float4(r[0], r[1], r[2], r[3]);
  *reinterpret_cast<float4*>(dst + 4) = make_float4(r[4], r[5], r[6], r[7]);
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D % kCols) return hipErrorInvalidValue;
  const int64_t rows = int64_t(a.B) * a.Hq;
  if (merge_rows_layout(rows, a.p_max)) {
    const int64_t threads = rows * (a.D / 8);
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    // the smallest unrolled partition count that covers p_max: slots past a
    // row's partitions re-read its last one and add 0, so a tight count saves
    // those loads and their arithmetic
    const dim3 g{unsigned(blocks)}, t{unsigned(kThreads)};
    if (a.p_max <= 2) hipLaunchKernelGGL(merge_rows_kernel<2>, g, t, 0, stream, a);
    else if (a.p_max <= 4) hipLaunchKernelGGL(merge_rows_kernel<4>, g, t, 0, stream, a);
    else if (a.p_max <= 6) hipLaunchKernelGGL(merge_rows_kernel<6>, g, t, 0, stream, a);
    else if (a.p_max <= 8) hipLaunchKernelGGL(merge_rows_kernel<8>, g, t, 0, stream, a);
    else if (a.p_max <= 12) hipLaunchKernelGGL(merge_rows_kernel<12>, g, t, 0, stream, a);
    else if (a.p_max <= 16) hipLaunchKernelGGL(merge_rows_kernel<16>, g, t, 0, stream, a);
    else if (a.p_max <= 24) hipLaunchKernelGGL(merge_rows_kernel<24>, g, t, 0, stream, a);
    else hipLaunchKernelGGL(merge_rows_kernel<32>, g, t, 0, stream, a);
  } else {
    hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq * (a.D / kCols)), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
