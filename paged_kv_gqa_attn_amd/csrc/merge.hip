// Stable split-softmax merge of partition partials.
//
// For each (sequence b, query head h) over its live partitions
// p < ceil(seq_len[b]/psize), with per-partition base-2 max m_p, sum l_p and
// normalised output o_p (lucebox PR #555, Summary: partials stored
// normalised, stable split-softmax merge; llama.cpp PR #13 HRX, Changes:
// per-block normalisation scale):
//     M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
// One workgroup of D threads per (b, h); thread d owns output column d, so
// the partial reads are coalesced rows of D floats. The loop bound is the
// runtime partition count (llama.cpp PR #13, the SGPR-exhaustion fix: a
// constant-folded bound fully unrolled the reduction).
#include "pa_device.h"
#include "pa_host.h"

namespace pa {
namespace {

constexpr int kChunk = 256;   // partitions staged in LDS per pass

__global__ void __launch_bounds__(256) merge_kernel(const MergeArgs a) {
  __shared__ float w_s[kChunk];
  __shared__ float red[256];
  __shared__ int nan_flag;
  const int bh = blockIdx.x;
  const int b = bh / a.Hq;
  const int d = threadIdx.x;
  const int nt = blockDim.x;
  int L = a.seq_len[b];
  L = L < 0 ? 0 : (L > a.cap_tokens ? a.cap_tokens : L);
  const int P = (L + a.psize - 1) / a.psize;
  float* dst = a.out + int64_t(bh) * a.D;
  if (P == 0) {
    dst[d] = 0.0f;
    return;
  }
  const float* ml = a.part_ml + int64_t(bh) * a.p_max * 2;
  const float* o = a.part_o + int64_t(bh) * a.p_max * a.D;

  // pass 1: M = max_p m_p, and whether any partition is flagged NaN
  if (d == 0) nan_flag = 0;
  float mx = -INFINITY;
  int has_nan = 0;
  for (int p = d; p < P; p += nt) {
    const float mp = ml[2 * p];
    has_nan |= (mp != mp);
    mx = fmaxf(mx, mp);
  }
  red[d] = mx;
  __syncthreads();
  if (has_nan) nan_flag = 1;
  for (int off = nt / 2; off > 0; off >>= 1) {
    if (d < off) red[d] = fmaxf(red[d], red[d + off]);
    __syncthreads();
  }
  const float M = red[0];
  const bool any_nan = nan_flag != 0;

  // pass 2: weighted sum, partitions staged kChunk at a time
  float acc = 0.0f, wsum = 0.0f;
  for (int p0 = 0; p0 < P; p0 += kChunk) {
    const int n = min(kChunk, P - p0);
    __syncthreads();
    for (int i = d; i < n; i += nt) {
      const int p = p0 + i;
      w_s[i] = __builtin_amdgcn_exp2f(ml[2 * p] - M) * ml[2 * p + 1];
    }
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const float w = w_s[i];
      wsum += w;
      acc += w * o[int64_t(p0 + i) * a.D + d];
    }
  }
  dst[d] = any_nan ? __builtin_nanf("") : acc / wsum;
}

}  // namespace

hipError_t launch_merge(const MergeArgs& a, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq), dim3(a.D), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pa
