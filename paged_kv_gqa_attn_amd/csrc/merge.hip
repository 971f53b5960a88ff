// Stable split-softmax merge of partition partials.
//
// For each (sequence b, query head h) over its live partitions
// p < ceil(seq_len[b]/psize), with per-partition base-2 reference m_p, sum
// l_p and normalised output o_p (lucebox PR #555, Summary: partials stored
// normalised in f16, stable split-softmax merge; llama.cpp PR #13 HRX,
// Changes: per-block normalisation scale):
//     M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
// The rows are (b, h) for decode and (b, t, h) for chunks (Hq then counts
// Tq*Hq rows per sequence); a partition that held no key for a row has
// m = -inf and l = 0 and so weight 0.
// The merge reads every partial byte once, so it is spread wide: a workgroup
// takes one (b, h) and 64 output columns; its 256 threads are 8 column octets
// x 32 partition classes (p mod 32). A thread reads 8 binary16 columns (16
// bytes) of each of its partitions and accumulates w_p o_p in fp32; the 32
// classes are then summed through LDS in a fixed order. The first kPre
// partitions of every class are loaded before the max is reduced, so their
// latency overlaps the reduction.
// Loop bounds are the runtime partition count (llama.cpp PR #13, the
// SGPR-exhaustion fix: a constant-folded bound fully unrolled the reduction).
#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;                   // output columns per workgroup
constexpr int kOcts = kCols / 8;            // 16-byte loads of 8 binary16 columns
constexpr int kClasses = kThreads / kOcts;  // partition classes
constexpr int kPre = 2;                     // partitions per class loaded ahead of the max

__device__ __forceinline__ void axpy8(float* acc, float w, const f16x8& v) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] += w * float(v[k]);
}

__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeArgs a) {
  __shared__ float red[kThreads];
  __shared__ float part[kClasses][kCols + 1];
  __shared__ float wpart[kClasses];
  const int tid = threadIdx.x;
  const int chunks = a.D / kCols;
  const int bh = blockIdx.x / chunks;
  const int col0 = (blockIdx.x - bh * chunks) * kCols;
  const int b = bh / a.Hq;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.cap_tokens ? a.cap_tokens : L);
  if (L < a.min_len) L = 0;       // a chunk longer than its sequence (flagged by the chunk kernel)
  const int P = (L + a.psize - 1) / a.psize;
  float* dst = a.out + int64_t(bh) * a.D + col0;
  if (P == 0) {
    if (tid < kCols) dst[tid] = 0.0f;
    return;
  }
  const float* ml = a.part_ml + int64_t(bh) * a.p_max * 2;
  const int q = tid % kOcts, c = tid / kOcts;
  const f16* o = reinterpret_cast<const f16*>(a.part_o) + int64_t(bh) * a.p_max * a.D + col0 + 8 * q;

  // the first kPre partitions of this thread's class, loaded ahead
  f16x8 pre[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int p = c + u * kClasses;
    pre[u] = p < P ? *reinterpret_cast<const f16x8*>(o + int64_t(p) * a.D) : f16x8{};
  }

  // pass 1: M = max_p m_p; a NaN m (a partition that met a bad block id)
  // turns into a NaN max through the comparison below
  float mx = -INFINITY;
  bool nan_seen = false;
  for (int p = tid; p < P; p += kThreads) {
    const float mp = ml[2 * p];
    nan_seen |= mp != mp;
    mx = fmaxf(mx, mp);
  }
  red[tid] = nan_seen ? __builtin_nanf("") : mx;
  __syncthreads();
  for (int off = kThreads / 2; off > 0; off >>= 1) {
    if (tid < off) {
      const float x = red[tid], y = red[tid + off];
      red[tid] = (x != x || y != y) ? __builtin_nanf("") : fmaxf(x, y);
    }
    __syncthreads();
  }
  const float M = red[0];

  // pass 2: thread (octet q, class c) sums w_p o_p[8q..8q+7] over p = c mod kClasses
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int p = c + u * kClasses;
    if (p < P) {
      const float w = __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
      wsum += w;
      axpy8(acc, w, pre[u]);
    }
  }
  int p = c + kPre * kClasses;
  for (; p + kClasses < P; p += 2 * kClasses) {
    const f16x8 v0 = *reinterpret_cast<const f16x8*>(o + int64_t(p) * a.D);
    const f16x8 v1 = *reinterpret_cast<const f16x8*>(o + int64_t(p + kClasses) * a.D);
    const float w0 = __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
    const float w1 = __builtin_amdgcn_exp2f(ml[2 * (p + kClasses)] - M) * ml[2 * (p + kClasses) + 1];
    wsum += w0;
    axpy8(acc, w0, v0);
    wsum += w1;
    axpy8(acc, w1, v1);
  }
  if (p < P) {
    const f16x8 v = *reinterpret_cast<const f16x8*>(o + int64_t(p) * a.D);
    const float w = __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
    wsum += w;
    axpy8(acc, w, v);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) part[c][8 * q + k] = acc[k];
  if (q == 0) wpart[c] = wsum;
  __syncthreads();

  // pass 3: sum the classes in a fixed order and normalise
  if (tid < kCols) {
    float s = part[0][tid];
    float W = wpart[0];
    for (int k = 1; k < kClasses; ++k) {
      s += part[k][tid];
      W += wpart[k];
    }
    dst[tid] = M != M ? __builtin_nanf("") : s / W;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D % kCols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq * (a.D / kCols)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
