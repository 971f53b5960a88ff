// Device-side helpers shared by the decode and gather kernels: vector types,
// the pool row address, and small bit-manipulation wrappers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// 16-byte vector whose address is only guaranteed 4-byte aligned (ggml block
// rows are 2- or 4-byte aligned inside a row).
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

enum : int { kF16 = 0, kQ8_0 = 1, kQ4_0 = 2 };

__host__ __device__ constexpr int row_bytes_of(int type, int D) {
  return type == kF16 ? 2 * D : (type == kQ8_0 ? 34 * (D / 32) : 18 * (D / 32));
}

// Physical block of logical block j of sequence b; a null table is the
// contiguous layout (sequence b's block j is block b*max_blocks + j).
__device__ __forceinline__ int32_t block_of(const int32_t* __restrict__ table, int32_t b,
                                            int32_t max_blocks, int32_t j) {
  const int64_t idx = int64_t(b) * max_blocks + j;
  return table ? table[idx] : int32_t(idx);
}

// Byte offset of the first row of block `id`, slot `slot`, kv head `g` in a
// [nblocks, block_size, Hkv, row_bytes] pool:
//   ((id*block_size + slot)*Hkv + g) * row_bytes
// computed in 64 bits, widened before the first multiply (mlxcel issue #2153,
// Proposed Solution and Implementation Notes).
__device__ __forceinline__ uint64_t row_offset(int32_t id, int32_t slot, int32_t bs_shift,
                                               int32_t Hkv, int32_t g, int32_t row_bytes) {
  const uint64_t row = (uint64_t(uint32_t(id)) << bs_shift) + uint32_t(slot);
  return (row * uint32_t(Hkv) + uint32_t(g)) * uint64_t(uint32_t(row_bytes));
}

__device__ __forceinline__ uint32_t ld_u32(const uint8_t* p) {
  return *reinterpret_cast<const uint32_t*>(p);
}
__device__ __forceinline__ u32x4 ld_u32x4(const uint8_t* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ u32x4 ld_u32x4_a4(const uint8_t* p) {
  u32x4_a4 v = *reinterpret_cast<const u32x4_a4*>(p);
  return u32x4{v[0], v[1], v[2], v[3]};
}
__device__ __forceinline__ uint16_t ld_u16(const uint8_t* p) {
  return *reinterpret_cast<const uint16_t*>(p);
}

// Bytes [sh, sh+4) of the 8-byte value {hi:lo}.
__device__ __forceinline__ uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t sh) {
  return __builtin_amdgcn_alignbyte(hi, lo, sh);
}
// v_perm_b32: byte selectors 0-3 pick bytes of `lo`, 4-7 bytes of `hi`, 12 gives 0x00.
__device__ __forceinline__ uint32_t perm_bytes(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

template <typename T, typename F>
__device__ __forceinline__ T bitcast(F x) {
  return __builtin_bit_cast(T, x);
}

// Raw buffer resource over [base, base + bytes): a scalar base per block, so
// every lane addresses it with a 32-bit offset (loads past `bytes` return 0).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, int(bytes), 0x00020000);
}
// Cache policy of the K/V loads. The non-temporal hint is off: a quantised
// row shares 128-byte lines with the neighbouring kv head, read by another
// workgroup on the same XCD, and streaming those lines out of L2 costs a refetch.
constexpr int kNonTemporal = 0;
__device__ __forceinline__ u32x4 buf_u32x4(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ u32x2 buf_u32x2(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ uint32_t buf_u32(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, kNonTemporal);
}
__device__ __forceinline__ uint16_t buf_u16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, kNonTemporal);
}

// (x & mask) | magic in one v_and_or_b32: gfx9 VOP3 takes no literal, so the
// mask rides in an SGPR and `magic` must already sit in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
  return r;
}
// A value the compiler cannot fold back into a literal operand.
__device__ __forceinline__ uint32_t opaque_vgpr(uint32_t c) {
  uint32_t r;
  asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "s"(c));
  return r;
}

// Wait states after the last MFMA that wrote `a` (and `b`, ...), before any
// later instruction reads them, whatever the branch layout. Reading an MFMA
// result too early returns the old register contents; the compiler pads for
// this, but the padding was observed missing on gfx950 (ROCm 7.2) for a read
// in a block entered by a branch taken right after the MFMA: a partial-step
// mask (`if (!full)`) between the score MFMAs and the softmax then fed stale
// scores to every full step. 16 wait states cover the XDL ops used here (at
// most pass count + 4). The values are asm operands so that every MFMA
// producing them precedes the wait and every read of them follows it.
__device__ __forceinline__ void mfma_settle(f32x4& a) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a));
}
__device__ __forceinline__ void mfma_settle(f32x4& a, f32x4& b) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void mfma_settle(f32x4& a, f32x4& b, f32x4& c, f32x4& d) {
  asm volatile("s_nop 7\n\ts_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}
// The same for a whole accumulator array (8 or 16 tiles) and one more tile,
// at the end of a loop whose last MFMAs wrote them.
__device__ __forceinline__ void mfma_settle(f32x4 (&x)[8], f32x4& c) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7]), "+v"(c));
}
__device__ __forceinline__ void mfma_settle(f32x4 (&x)[8]) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7]));
}
__device__ __forceinline__ void mfma_settle(f32x4 (&x)[16]) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),
                 "+v"(x[13]), "+v"(x[14]), "+v"(x[15]));
}
__device__ __forceinline__ void mfma_settle(f32x4 (&x)[16], f32x4& c) {
  asm volatile("s_nop 7\n\ts_nop 7"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]), "+v"(x[6]),
                 "+v"(x[7]), "+v"(x[8]), "+v"(x[9]), "+v"(x[10]), "+v"(x[11]), "+v"(x[12]),
                 "+v"(x[13]), "+v"(x[14]), "+v"(x[15]), "+v"(c));
}

}  // namespace pa
