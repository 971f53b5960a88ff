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
// classes are then summed in a fixed order (lane butterflies within a wave,
// then the four waves through LDS). The first kPre partitions of every class
// are loaded together with the m values the max needs, so one memory latency
// covers both, and the max is reduced with lane shuffles and one barrier.
// With many rows of few partitions (p_max <= 16 over at least 1024 rows, or
// p_max <= 32 over at least 512, e.g. the Tq*Hq rows of a prefill chunk or
// a verify window) that layout leaves most threads idle and launches
// thousands of workgroups, and merge_rows_kernel is used instead: one thread
// per (row, 8 output columns) reads all of the row's partitions at once and
// sums them in order, 8 rows per workgroup at D=256.
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
constexpr int kBatch = 8;                   // partitions per class per later batch

__device__ __forceinline__ void axpy8(float* acc, float w, const f16x8& v) {
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] += w * float(v[k]);
}

__global__ void __launch_bounds__(kThreads) merge_kernel(const MergeArgs a) {
  constexpr int kWaves = kThreads / 64;
  __shared__ float wmax[kWaves];
  __shared__ int wnan[kWaves];
  __shared__ float part[kWaves][kCols];
  __shared__ float wpart[kWaves];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  // Loads in flight together: the first kPre partitions of this thread's
  // class with their (m, l), and m of partition tid. They go through buffer
  // resources that end at the row's last live partition, so a load past it
  // returns 0 without touching memory and none needs a branch.
  const rsrc_t ro = make_rsrc(reinterpret_cast<const f16*>(a.part_o) + int64_t(bh) * a.p_max * a.D,
                              uint32_t(P) * uint32_t(a.D) * 2u);
  const rsrc_t rml = make_rsrc(ml, uint32_t(P) * 8u);
  const uint32_t ocol = uint32_t(col0 + 8 * q) * 2u;
  f16x8 pre[kPre];
  float2 mlp[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const uint32_t pu = uint32_t(c + u * kClasses);
    pre[u] = bitcast<f16x8>(buf_u32x4(ro, pu * uint32_t(a.D) * 2u + ocol, 0));
    mlp[u] = bitcast<float2>(buf_u32x2(rml, pu * 8u, 0));
  }
  const float m0 = bitcast<float>(buf_u32(rml, uint32_t(tid) * 8u, 0));
  float mx = tid < P ? m0 : -INFINITY;
  bool nan_seen = mx != mx;
  for (int p = tid + kThreads; p < P; p += kThreads) {
    const float mp = ml[2 * p];
    nan_seen |= mp != mp;
    mx = fmaxf(mx, mp);
  }

  // M = max_p m_p: within the wave by lane shuffles, then over the waves. A
  // NaN m (a partition that met a bad block id) makes the row NaN.
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  nan_seen = __any(nan_seen);
  if (lane == 0) {
    wmax[wave] = mx;
    wnan[wave] = nan_seen;
  }
  __syncthreads();
  float M = wmax[0];
  int any_nan = wnan[0];
#pragma unroll
  for (int k = 1; k < kWaves; ++k) {
    M = fmaxf(M, wmax[k]);
    any_nan |= wnan[k];
  }

  // thread (octet q, class c) sums w_p o_p[8q..8q+7] over p = c mod kClasses
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wsum = 0.0f;
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    // a slot past the last partition read zeros: weight 0, adds exactly 0
    const float w = c + u * kClasses < P ? __builtin_amdgcn_exp2f(mlp[u].x - M) * mlp[u].y : 0.0f;
    wsum += w;
    axpy8(acc, w, pre[u]);
  }
  // the rest of the class in batches of kBatch partitions, all loads of a
  // batch in flight at once (a row with hundreds of partitions, e.g. one
  // long sequence alone, would otherwise pay one latency per partition pair)
  for (int u0 = kPre; u0 * kClasses < P; u0 += kBatch) {
    f16x8 v[kBatch];
    float2 x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t pu = uint32_t(c + (u0 + u) * kClasses);
      v[u] = bitcast<f16x8>(buf_u32x4(ro, pu * uint32_t(a.D) * 2u + ocol, 0));
      x[u] = bitcast<float2>(buf_u32x2(rml, pu * 8u, 0));
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const float w = c + (u0 + u) * kClasses < P ? __builtin_amdgcn_exp2f(x[u].x - M) * x[u].y : 0.0f;
      wsum += w;
      axpy8(acc, w, v[u]);
    }
  }

  // sum the classes in a fixed order: the wave's 8 classes (lane bits 3..5)
  // by butterflies, then the waves through LDS
#pragma unroll
  for (int off = kOcts; off < 64; off <<= 1) {
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += __shfl_xor(acc[k], off, 64);
    wsum += __shfl_xor(wsum, off, 64);
  }
  if (lane < kOcts) {
#pragma unroll
    for (int k = 0; k < 8; ++k) part[wave][8 * lane + k] = acc[k];
    if (lane == 0) wpart[wave] = wsum;
  }
  __syncthreads();
  if (tid < kCols) {
    float s = part[0][tid];
    float W = wpart[0];
#pragma unroll
    for (int k = 1; k < kWaves; ++k) {
      s += part[k][tid];
      W += wpart[k];
    }
    dst[tid] = any_nan ? __builtin_nanf("") : s / W;
  }
}

constexpr int kRowsMergeMinRows = 1024;   // fewer rows: the wide layout has more parallelism
                                          // (half as many when up to 32 partitions per row)

// NPM: the most partitions a row has (8 or 16)
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
    axpy8(acc, w, v[p]);
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
  if ((a.p_max <= 16 && rows >= kRowsMergeMinRows) || (a.p_max <= 32 && rows >= kRowsMergeMinRows / 2)) {
    const int64_t threads = rows * (a.D / 8);
    const int64_t blocks = (threads + kThreads - 1) / kThreads;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidValue;
    if (a.p_max <= 8)
      hipLaunchKernelGGL(merge_rows_kernel<8>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a);
    else if (a.p_max <= 16)
      hipLaunchKernelGGL(merge_rows_kernel<16>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(merge_rows_kernel<32>, dim3(unsigned(blocks)), dim3(kThreads), 0, stream, a);
  } else {
    hipLaunchKernelGGL(merge_kernel, dim3(a.B * a.Hq * (a.D / kCols)), dim3(kThreads), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pa
