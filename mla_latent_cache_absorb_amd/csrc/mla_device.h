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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kLatent = 512;        // R
constexpr int kHeadDim = 256;       // D
constexpr int kRowBytes = kLatent * 2;

__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16-byte-chunk swizzle for a row of an LDS tile: chunk c of row r lives at slot c ^ swz(r).
// gfx950's LDS serves 256 bytes (64 banks x 4 bytes) per cycle, i.e. 16 lanes of a 16-byte
// read or 32 lanes of an 8-byte read.  swz is a bijection of r mod 16 onto 0..15 chosen so
// that (a) sixteen consecutive rows at one chunk hit sixteen different bank groups
// (row-major operand reads), and (b) four consecutive rows (aligned to 4) at four adjacent
// chunks (aligned to 4) hit sixteen different bank groups (transpose reads).  Rows must be a
// multiple of 256 bytes long and hold at least 16 chunks.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

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

// Cache policy of the row copies below: NT marks the copy non-temporal, for a stream whose rows no
// other workgroup of the call reads (they are not kept for reuse in L2 or the Infinity Cache, so
// the stream does not push out data that is read again, and a plain read of 256 MiB ran at 6.8
// against 6.1 TB/s with it).  Rows that several workgroups share through L2 (the queries of one
// sequence on one XCD) take the default policy.
//
// One 1 KiB row, global -> LDS without passing through registers: lane s copies the 16
// bytes at row + (lane16(s) ^ sw) to lds + 16 * s, lane16 = 16 * s.  `row`, `lds` and `sw`
// are wave-uniform (SGPRs).  Issued from asm so that the compiler does not wait for these
// copies before unrelated LDS reads: the caller waits (vmcnt) itself before the copied data
// is read.  The per-row lane offset is formed inside the asm, so no per-row register stays
// live in the caller; the load reads it when it issues.  M0 is written one wait state before
// the copy uses it; the kernels that call this use M0 for nothing else (no LDS-DMA builtins, no
// indirect register indexing), so clobbering it is safe.
template <bool NT>
__device__ __forceinline__ void row_to_lds(const uint8_t* row, uint32_t lds, uint32_t lane16, uint32_t sw) {
  // the operands are wave-uniform by construction; readfirstlane makes them SGPRs for certain
  const uint64_t ra = (uint64_t)(uintptr_t)row;
  const uint64_t rs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ra >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ra);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(lds);
  const uint32_t ss = __builtin_amdgcn_readfirstlane(sw);
  uint32_t voff;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_xor_b32 %0, %2, %3\n\t"
        "global_load_lds_dwordx4 %0, %4 nt"
        : "=&v"(voff)
        : "s"(ls), "s"(ss), "v"(lane16), "s"(rs)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_xor_b32 %0, %2, %3\n\t"
        "global_load_lds_dwordx4 %0, %4"
        : "=&v"(voff)
        : "s"(ls), "s"(ss), "v"(lane16), "s"(rs)
        : "memory", "m0");
#pragma clang diagnostic pop
}

// As row_to_lds, for a row `off` bytes past a wave-uniform `base`: the lane offset is
// (lane16 ^ sw) + off, so consecutive rows share one base address.
template <bool NT>
__device__ __forceinline__ void row_to_lds_at(const uint8_t* base, uint32_t off, uint32_t lds, uint32_t lane16,
                                              uint32_t sw) {
  const uint64_t ra = (uint64_t)(uintptr_t)base;
  const uint64_t rs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(ra >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)ra);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(lds);
  const uint32_t ss = __builtin_amdgcn_readfirstlane(sw);
  const uint32_t os = __builtin_amdgcn_readfirstlane(off);
  uint32_t voff;
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_xor_b32 %0, %2, %3\n\t"
        "v_add_u32 %0, %4, %0\n\t"
        "global_load_lds_dwordx4 %0, %5 nt"
        : "=&v"(voff)
        : "s"(ls), "s"(ss), "v"(lane16), "s"(os), "s"(rs)
        : "memory", "m0");
  else
    asm volatile(
        "s_mov_b32 m0, %1\n\t"
        "v_xor_b32 %0, %2, %3\n\t"
        "v_add_u32 %0, %4, %0\n\t"
        "global_load_lds_dwordx4 %0, %5"
        : "=&v"(voff)
        : "s"(ls), "s"(ss), "v"(lane16), "s"(os), "s"(rs)
        : "memory", "m0");
#pragma clang diagnostic pop
}

// Lane-addressed copy of 16 bytes from `src` (any per-lane address) to lds + 16 * lane, `lds`
// wave-uniform, without passing through registers.  Issued from asm so that the compiler does not
// wait for it before unrelated LDS reads: the caller waits (vmcnt) before reading the copy.  M0 is
// clobbered, as in row_to_lds.
__device__ __forceinline__ void copy16_to_lds(const void* src, uint32_t lds) {
  const uint32_t ls = __builtin_amdgcn_readfirstlane(lds);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off" : : "s"(ls), "v"(src) : "memory", "m0");
#pragma clang diagnostic pop
}

// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned
__device__ __forceinline__ void wait_lds_reads() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// A copy of x that the compiler cannot see through.  Address arithmetic derived from it inside
// a loop stays in the loop (recomputed with a VALU op or two per use) instead of being hoisted
// into loop-invariant registers, which the big kernels cannot spare.
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Combine a value with the one in the other half of the wave (lane l and l ^ 32):
// v_permlane32_swap(x, x) returns x's lanes 0-31 in both halves of its first result and lanes
// 32-63 in both halves of the second, so one VALU op pairs every lane with its partner.
__device__ __forceinline__ float half_swap_max(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Log-sum-exp merge of split-K attention partials.  A split's partial is (m, l, u): m a running
// maximum in log2 units, l = sum 2^(score - m) and u = o / l its normalised weighted sum of latents
// (o the unnormalised sum), stored in fp16: u is a convex combination of cached latents, so its
// magnitude is at most theirs, and fp16 keeps it to 2^-11 relative; 0 when the split saw nothing.
// The merged row is sum_s 2^(m_s - M) l_s u_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.  The splits
// are taken in groups of eight, every load of a group issued together.  A group is first reduced
// on its own, relative to its own maximum Mg (splits that saw no position, l = 0, weigh nothing),
// and the group results are then folded in order into a running (M, L, o), rescaling what was
// accumulated by 2^(M_old - M_new) and the group by 2^(Mg - M_new).  The sequential form below
// (merge_splits8) and the wide merge kernel (groups reduced by different threads, folded in the
// same order) give identical bits.  With one group the fold multiplies by one and adds zero, so it is exact.
struct MergeGroup {
  float mm[8], ll[8];
  f32x4 v[8];
};
struct MergePartial {
  float M, L;
  f32x4 acc;
};

// A slot past the last split weighs nothing: merge_group's condition skips it in the maximum, and
// its weight is zero in the sums.  Its values only have to be finite; with them zero the sums take
// exactly the same values as with any other finite values (an accumulator that starts at +0 and
// gains a +0 or -0 term stays +0 under round-to-nearest, and a nonzero one is unchanged).
__device__ __forceinline__ void merge_slot_empty(MergeGroup& g, int k) {
  g.mm[k] = 0.f;
  g.ll[k] = 0.f;
  g.v[k] = (f32x4){0.f, 0.f, 0.f, 0.f};
}

// The partials of one group of splits, s0 .. s0 + 7, for eight adjacent latents (two blocks of
// four): part_o holds the row's eight latents (of this thread, fp16) in split 0 and part_ml the
// row's (m, l) in split 0; split s lies o_step (ml_step) elements further on.  NS (2, 4 or 8)
// slots are loaded, unconditionally, so that the group's loads all issue before the first one is
// waited for (one memory round trip; a conditional load per slot makes the compiler wait before
// each branch).  Callers pick NS >= the splits left (NS < 8 only with a single group); a loaded
// slot past the last split reloads the last split (in bounds, a cache hit), the others are filled
// by merge_slot_empty.
template <int NS = 8>
__device__ __forceinline__ void merge_load8(MergeGroup (&g)[2], const uint16_t* part_o, const float* part_ml,
                                            size_t o_step, size_t ml_step, int S, int s0) {
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    if (k >= NS) {
      merge_slot_empty(g[0], k);
      merge_slot_empty(g[1], k);
      continue;
    }
    const size_t s = (size_t)min(s0 + k, S - 1);
    const float2 ml = *(const float2*)(part_ml + s * ml_step);
    const f16x8 x = *(const f16x8*)(part_o + s * o_step);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      g[h].mm[k] = ml.x;
      g[h].ll[k] = ml.y;
      g[h].v[k] = __builtin_convertvector((f16x4){x[4 * h], x[4 * h + 1], x[4 * h + 2], x[4 * h + 3]}, f32x4);
    }
  }
}

// one group reduced relative to its own maximum; false when none of its splits saw a position
__device__ __forceinline__ bool merge_group(const MergeGroup& g, int S, int s0, MergePartial& r) {
  float Mg = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (s0 + k < S && g.ll[k] > 0.f) Mg = fmaxf(Mg, g.mm[k]);
  if (Mg == -INFINITY) return false;
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const float w = (s0 + k < S && g.ll[k] > 0.f) ? __builtin_amdgcn_exp2f(g.mm[k] - Mg) : 0.f;
    const float wl = w * g.ll[k];  // the split's weight: its sum rescaled to the group's maximum
    L = __builtin_fmaf(w, g.ll[k], L);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(wl, g.v[k][e], acc[e]);
  }
  r.M = Mg;
  r.L = L;
  r.acc = acc;
  return true;
}

// every product and sum is written out as one fused multiply-add so that each kernel that folds
// rounds the same way (the compiler may otherwise contract the two forms differently)
__device__ __forceinline__ void merge_fold(float& M, float& L, f32x4& acc, const MergePartial& r) {
  const float Mn = fmaxf(M, r.M);
  const float a = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
  const float b = __builtin_amdgcn_exp2f(r.M - Mn);
  L = __builtin_fmaf(r.L, b, __builtin_fmaf(L, a, 0.f));
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(r.acc[e], b, __builtin_fmaf(acc[e], a, 0.f));
  M = Mn;
}

// The whole merge for the eight latents a thread owns, as two blocks of four, each through its
// own (M, L, o): *lse2 = M + log2(L) (log2 units).  NS as in merge_load8.
template <int NS = 8>
__device__ __forceinline__ void merge_splits8(const uint16_t* part_o, const float* part_ml, size_t o_step,
                                              size_t ml_step, int S, float* lse2, f32x4 (&out)[2]) {
  float M[2] = {-INFINITY, -INFINITY}, L[2] = {0.f, 0.f};
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int s0 = 0; s0 < S; s0 += 8) {
    MergeGroup g[2];
    merge_load8<NS>(g, part_o, part_ml, o_step, ml_step, S, s0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      MergePartial r;
      if (merge_group(g[h], S, s0, r)) merge_fold(M[h], L[h], acc[h], r);
    }
  }
  // __builtin_amdgcn_logf is the hardware base-2 logarithm
  *lse2 = M[0] + __builtin_amdgcn_logf(L[0]);
#pragma unroll
  for (int h = 0; h < 2; ++h) out[h] = acc[h] * (1.0f / L[h]);
}

// merge_splits8's steps for one group of slots already loaded (at most eight splits), for NB
// blocks of four latents whose splits share their (m, l) (the blocks of one row): merge_group's
// steps, then merge_fold into the empty state, for each block, with the split weights computed
// once instead of once a block.  Each value goes through the same operations in the same order
// as in merge_splits8, so the bits are its bits.
template <int NB>
__device__ __forceinline__ void merge_one_group8_blocks(const float (&mm)[8], const float (&ll)[8],
                                                        const f32x4 (&v)[NB][8], int S, float* lse2,
                                                        f32x4 (&out)[NB]) {
  float Mg = -INFINITY;
#pragma unroll
  for (int k = 0; k < 8; ++k)
    if (k < S && ll[k] > 0.f) Mg = fmaxf(Mg, mm[k]);
  float M = -INFINITY, L = 0.f;
  f32x4 acc[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) acc[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
  if (Mg != -INFINITY) {
    float wl[8], Lg = 0.f;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const float w = (k < S && ll[k] > 0.f) ? __builtin_amdgcn_exp2f(mm[k] - Mg) : 0.f;
      wl[k] = w * ll[k];
      Lg = __builtin_fmaf(w, ll[k], Lg);
    }
    // merge_fold of (Mg, Lg, group sum) into (M, L, acc) = (-inf, 0, 0)
    const float Mn = fmaxf(M, Mg);
    const float bw = __builtin_amdgcn_exp2f(Mg - Mn);
    L = __builtin_fmaf(Lg, bw, __builtin_fmaf(L, 0.f, 0.f));
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      f32x4 g = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < 8; ++k)
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = __builtin_fmaf(wl[k], v[b][k][e], g[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[b][e] = __builtin_fmaf(g[e], bw, __builtin_fmaf(acc[b][e], 0.f, 0.f));
    }
    M = Mn;
  }
  // __builtin_amdgcn_logf is the hardware base-2 logarithm
  *lse2 = M + __builtin_amdgcn_logf(L);
#pragma unroll
  for (int b = 0; b < NB; ++b) out[b] = acc[b] * (1.0f / L);
}

// merge slots to load for S splits in one group (2, 4 or 8)
__host__ __device__ constexpr int merge_slots(int S) { return S <= 2 ? 2 : S <= 4 ? 4 : 8; }

// Map the hardware workgroup id to a logical id so that consecutive logical ids run on the
// same XCD: workgroups are dispatched round-robin over the 8 XCDs of an MI355X, so XCD x
// receives hardware ids x, x+8, x+16, ...; those become one contiguous block of logical ids.
__device__ __forceinline__ int xcd_remap(int hw, int total) {
  const int xcd = hw & 7, local = hw >> 3;
  const int per = total >> 3, extra = total & 7;
  return xcd * per + (xcd < extra ? xcd : extra) + local;
}

}  // namespace mla
