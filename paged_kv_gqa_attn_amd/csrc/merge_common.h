// The split-softmax merge of one (row, 64 output columns) slice, shared by the
// merge kernel (merge.hip) and the single-launch decode (decode_lds.hip), so
// that both produce the same bits.
//
// For a row (sequence b, query head h, or chunk row) over its live partitions
// p < P, with per-partition base-2 reference m_p, sum l_p and normalised
// output o_p (lucebox PR #555, Summary: partials stored normalised in f16,
// recombined by a numerically stable merge of the split softmax; llama.cpp
// PR #13 HRX, Changes: per-block normalisation scale):
//     M = max_p m_p,  w_p = 2^(m_p - M) * l_p,  out = sum_p w_p o_p / sum_p w_p
// A partition that held no key for a row has m = -inf and l = 0 and so weight
// 0; a NaN m (a partition that met a bad block id) makes the row NaN; P = 0
// gives zeros.
// The 256 threads of the workgroup are 8 column octets x 32 partition classes
// (p mod 32). A thread reads 8 binary16 columns (16 bytes) of each of its
// partitions and accumulates w_p o_p in fp32; the 32 classes are then summed
// in a fixed order (lane butterflies within a wave, then the four waves
// through LDS). The first kPre partitions of every class are loaded together
// with the m values the max needs, so one memory latency covers both.
// Loop bounds are the runtime partition count (llama.cpp PR #13, the
// SGPR-exhaustion fix: a constant-folded bound fully unrolled the reduction).
#pragma once
#include "pa_device.h"

namespace pa {

constexpr int kMergeThreads = 256;
constexpr int kMergeCols = 64;                          // output columns per slice
constexpr int kMergeOcts = kMergeCols / 8;              // 16-byte loads of 8 binary16 columns
constexpr int kMergeClasses = kMergeThreads / kMergeOcts;  // partition classes
constexpr int kMergePre = 2;                            // partitions per class loaded ahead of the max
constexpr int kMergeBatch = 16;                         // partitions per class per later batch

// LDS the slice needs (kMergeThreads threads, four waves).
struct MergeLds {
  float wmax[4];
  int wnan[4];
  float part[4][kMergeCols];
  float wpart[4];
};

__device__ __forceinline__ void merge_axpy8(float* acc, float w, const f16x8& v) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] += w * float(v[k]);
}

// Merges columns col0 .. col0+63 of one row. o_row / ml_row: the row's
// partials (partition stride D binary16 values / 2 floats), P live partitions,
// dst: the row's output + col0. Every thread of the workgroup calls it.
// kCoherent: the partials were written by other workgroups of the same launch
// (device-coherent stores) and become final during it. The (m, l) pairs of
// several rows can share a cache line, which an earlier slice of another row
// may have brought into this XCD's L2 before this row's pairs were final, so
// they are read device-coherently (sc1: from memory, past L2). An o line
// (128 bytes: 64 binary16 columns of one partition of one row) belongs to
// this slice alone and is read by nothing before it is final, so plain loads
// fetch it fresh. Across a kernel boundary plain loads see everything. The
// values read, and so the result, are the same either way.
template <bool kCoherent>
__device__ __forceinline__ void merge_slice(const f16* o_row, const float* ml_row, int P, int D, int col0,
                                            float* dst, MergeLds& s) {
  constexpr int kPolicy = kCoherent ? 16 : 0;           // cache policy of the (m, l) loads: sc1
  constexpr int kWaves = kMergeThreads / 64;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  if (P == 0) {
    if (tid < kMergeCols) dst[tid] = 0.0f;
    return;
  }
  const int q = tid % kMergeOcts, c = tid / kMergeOcts;

  // Loads in flight together: the first kMergePre partitions of this thread's
  // class with their (m, l), and m of partitions tid and tid + 256. They go through buffer
  // resources that end at the row's last live partition, so a load past it
  // returns 0 without touching memory and none needs a branch.
  const rsrc_t ro = make_rsrc(o_row, uint32_t(P) * uint32_t(D) * 2u);
  const rsrc_t rml = make_rsrc(ml_row, uint32_t(P) * 8u);
  const uint32_t ocol = uint32_t(col0 + 8 * q) * 2u;
  f16x8 pre[kMergePre];
  float2 mlp[kMergePre];
#pragma unroll
  for (int u = 0; u < kMergePre; ++u) {
    const uint32_t pu = uint32_t(c + u * kMergeClasses);
    pre[u] = bitcast<f16x8>(__builtin_amdgcn_raw_buffer_load_b128(ro, pu * uint32_t(D) * 2u + ocol, 0, 0));
    mlp[u] = bitcast<float2>(__builtin_amdgcn_raw_buffer_load_b64(rml, pu * 8u, 0, kPolicy));
  }
  const float m0 = bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(rml, uint32_t(tid) * 8u, 0, kPolicy));
  const float m1 =
      bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(rml, uint32_t(tid + kMergeThreads) * 8u, 0, kPolicy));
  float mx = tid < P ? m0 : -INFINITY;
  bool nan_seen = mx != mx;
  if (tid + kMergeThreads < P) {
    nan_seen |= m1 != m1;
    mx = fmaxf(mx, m1);
  }
  for (int p = tid + 2 * kMergeThreads; p < P; p += kMergeThreads) {
    const float mp = bitcast<float>(__builtin_amdgcn_raw_buffer_load_b32(rml, uint32_t(p) * 8u, 0, kPolicy));
    nan_seen |= mp != mp;
    mx = fmaxf(mx, mp);
  }

  // M = max_p m_p: within the wave by lane shuffles, then over the waves.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  nan_seen = __any(nan_seen);
  if (lane == 0) {
    s.wmax[wave] = mx;
    s.wnan[wave] = nan_seen;
  }
  __syncthreads();
  float M = s.wmax[0];
  int any_nan = s.wnan[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    M = fmaxf(M, s.wmax[k]);
    any_nan |= s.wnan[k];
  }

  // thread (octet q, class c) sums w_p o_p[8q..8q+7] over p = c mod kMergeClasses
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
#pragma unroll
  for (int u = 0; u < kMergePre; ++u) {
    // a slot past the last partition read zeros: weight 0, adds exactly 0
    const float w = c + u * kMergeClasses < P ? __builtin_amdgcn_exp2f(mlp[u].x - M) * mlp[u].y : 0.0f;
    wsum += w;
    merge_axpy8(acc, w, pre[u]);
  }
  // the rest of the class in batches of kMergeBatch partitions, all loads of a
  // batch in flight at once (a row with hundreds of partitions, e.g. one
  // long sequence alone, would otherwise pay one latency per partition pair)
  for (int u0 = kMergePre; u0 * kMergeClasses < P; u0 += kMergeBatch) {
    f16x8 v[kMergeBatch];
    float2 x[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const uint32_t pu = uint32_t(c + (u0 + u) * kMergeClasses);
      v[u] = bitcast<f16x8>(__builtin_amdgcn_raw_buffer_load_b128(ro, pu * uint32_t(D) * 2u + ocol, 0, 0));
      x[u] = bitcast<float2>(__builtin_amdgcn_raw_buffer_load_b64(rml, pu * 8u, 0, kPolicy));
    }
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float w =
          c + (u0 + u) * kMergeClasses < P ? __builtin_amdgcn_exp2f(x[u].x - M) * x[u].y : 0.0f;
      wsum += w;
      merge_axpy8(acc, w, v[u]);
    }
  }

  // sum the classes in a fixed order: the wave's 8 classes (lane bits 3..5)
  // by butterflies, then the waves through LDS
#pragma unroll
  for (int off = kMergeOcts; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], off, 64);
    wsum += __shfl_xor(wsum, off, 64);
  }
  if (lane < kMergeOcts) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s.part[wave][8 * lane + k] = acc[k];
    if (lane == 0) s.wpart[wave] = wsum;
  }
  __syncthreads();
  if (tid < kMergeCols) {
    float sum = s.part[0][tid];
    float W = s.wpart[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
      sum += s.part[k][tid];
      W += s.wpart[k];
    }
    dst[tid] = any_nan ? __builtin_nanf("") : sum / W;
  }
}

}  // namespace pa
