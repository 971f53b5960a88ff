// Stable split-softmax merge of partition partials.
//
// For each (sequence b, query head h) over its live partitions
// p < ceil(seq_len[b]/psize), with per-partition base-2 reference m_p, sum
// l_p and normalised output o_p (lucebox PR #555, Summary: partials stored
// normalised, stable split-softmax merge; llama.cpp PR #13 HRX, Changes:
// per-block normalisation scale):
//     M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
// The merge reads every partial byte once, so it is spread wide: a workgroup
// takes one (b, h) and 64 output columns; its 256 threads are 16 column
// quads x 16 partition classes (p mod 16), each thread accumulating float4
// columns over its partitions, and the 16 classes are summed through LDS.
// Loop bounds are the runtime partition count (llama.cpp PR #13, the
// SGPR-exhaustion fix: a constant-folded bound fully unrolled the reduction).
#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

constexpr int kThreads = 256;
constexpr int kCols = 64;                 // output columns per workgroup
constexpr int kQuads = kCols / 4;         // float4 column quads
constexpr int kClasses = kThreads / kQuads;

__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeArgs a) {
  __shared__ float red[kThreads];
  __shared__ float4 part[kClasses][kQuads];
  __shared__ float wpart[kClasses];
  const int tid = threadIdx.x;
  const int chunks = a.D / kCols;
  const int bh = blockIdx.x / chunks;
  const int col0 = (blockIdx.x - bh * chunks) * kCols;
  const int b = bh / a.Hq;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.cap_tokens ? a.cap_tokens : L);
  const int P = (L + a.psize - 1) / a.psize;
  float* dst = a.out + int64_t(bh) * a.D + col0;
  if (P == 0) {
    if (tid < kCols) dst[tid] = 0.0f;
    return;
  }
  const float* ml = a.part_ml + int64_t(bh) * a.p_max * 2;
  const float* o = a.part_o + int64_t(bh) * a.p_max * a.D + col0;

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

  // pass 2: thread (quad q, class c) sums w_p o_p[4q..4q+3] over p = c mod kClasses
  const int q = tid % kQuads, c = tid / kQuads;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float wsum = 0.0f;
  int p = c;
  for (; p + 3 * kClasses < P; p += 4 * kClasses) {
    float w[4];
    float4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int pu = p + u * kClasses;
      w[u] = __builtin_amdgcn_exp2f(ml[2 * pu] - M) * ml[2 * pu + 1];
      v[u] = reinterpret_cast<const float4*>(o + int64_t(pu) * a.D)[q];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      wsum += w[u];
      acc.x += w[u] * v[u].x; acc.y += w[u] * v[u].y; acc.z += w[u] * v[u].z; acc.w += w[u] * v[u].w;
    }
  }
  for (; p < P; p += kClasses) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
    const float4 v = reinterpret_cast<const float4*>(o + int64_t(p) * a.D)[q];
    wsum += w;
    acc.x += w * v.x; acc.y += w * v.y; acc.z += w * v.z; acc.w += w * v.w;
  }
  part[c][q] = acc;
  if (q == 0) wpart[c] = wsum;
  __syncthreads();

  // pass 3: sum the classes in a fixed order and normalise
  if (tid < kQuads) {
    float4 s = part[0][tid];
    float W = wpart[0];
    for (int k = 1; k < kClasses; ++k) {
      const float4 t = part[k][tid];
      s.x += t.x; s.y += t.y; s.z += t.z; s.w += t.w;
      W += wpart[k];
    }
    const float inv = 1.0f / W;
    float4 r = make_float4(s.x * inv, s.y * inv, s.z * inv, s.w * inv);
    if (M != M) r = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    reinterpret_cast<float4*>(dst)[tid] = r;
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  if (a.D % kCols) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq * (a.D / kCols)), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
