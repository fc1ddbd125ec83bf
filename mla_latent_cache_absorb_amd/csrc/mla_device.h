// Device-side building blocks shared by the gfx950 kernels of libmla_absorb.
//
// Matrix-core operand layouts (v_mfma_f32_32x32x16_bf16, wave64), lane l:
//   A (32 x 16, M x K): row l % 32, k = 8 * (l / 32) + e, e = 0..7 (8 bf16, one 16-byte load)
//   B (16 x 32, K x N): col l % 32, k = 8 * (l / 32) + e
//   D (32 x 32, fp32) : col l % 32, row 8 * i + 4 * (l / 32) + j in register 4 * i + j
// LDS transpose read (ds_read_b64_tr_b16), per group of 16 lanes: lanes 4e..4e+3 each name
// 8 bytes, together the 16 consecutive 16-bit values of "row" e (e = 0..3); lane i of the
// group receives column i of that 4 x 16 block, i.e. rows 0..3 of one column.  This feeds an
// operand whose K index runs along rows of a row-major tile (the transpose of the tile).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kLatent = 512;        // R
constexpr int kHeadDim = 256;       // D
constexpr int kRowBytes = kLatent * 2;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte-chunk swizzle for a row of an LDS tile: chunk c of row r lives at slot c ^ swz(r).
// swz is a bijection of r mod 8 onto 0..7, chosen so that (a) eight consecutive rows at one
// chunk hit eight different 16-byte bank groups (row-major operand reads), and (b) four
// consecutive rows (aligned to 4) at two adjacent chunks hit eight different bank groups
// (transpose reads).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

__device__ __forceinline__ s16x4 lds_read_tr16(const void* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ bf16x8 concat_bf16(const s16x4& lo, const s16x4& hi) {
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return (bf16x8)v;
}

// Round-to-nearest-even fp32 -> bf16 bits (gfx950 has a native packed convert; the compiler
// selects it for this pattern).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __builtin_bit_cast(float, ((uint32_t)b) << 16);
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt bits [3:0] and [15:14],
// expcnt [6:4] = 7, lgkmcnt [11:8] = 15 leave the other counters unconstrained).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 32-bit LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// One 1 KiB row, global -> LDS without passing through registers: lane s copies the 16
// bytes at row + voff(s) to lds + 16 * s.  `row` and `lds` are wave-uniform (SGPRs);
// voff is the lane's byte offset inside the row.  Issued from asm so that the compiler does
// not wait for these copies before unrelated LDS reads: the caller waits (vmcnt) itself
// before the copied data is read.  M0 is written one wait state before the copy uses it; the
// kernels that call this use M0 for nothing else (no LDS-DMA builtins, no indirect register
// indexing), so clobbering it is safe.
__device__ __forceinline__ void row_to_lds(const uint8_t* row, uint32_t lds, uint32_t voff) {
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(voff), "s"(row)
      : "memory", "m0");
#pragma clang diagnostic pop
}

// Map the hardware workgroup id to a logical id so that consecutive logical ids run on the
// same XCD: workgroups are dispatched round-robin over the 8 XCDs of an MI355X, so XCD x
// receives hardware ids x, x+8, x+16, ...; those become one contiguous block of logical ids.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
  const int xcd = hw & 7, local = hw >> 3;
  const int per = total >> 3, extra = total & 7;
  return xcd * per + (xcd < extra ? xcd : extra) + local;
}

}  // namespace mla
