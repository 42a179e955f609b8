// Matrix-core helpers for gfx950 (CDNA4): operand types, MFMA wrappers,
// int4 unpacking and direct global->LDS loads.
#pragma once
#include "common.h"
#include "kernels.h"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

// 8 int4 values (one word of the storage layout) -> bf16 (136 + q), in k order:
// nibble u ^ 8 (= q + 8) placed in the mantissa of 128.0 (0x4300) is exactly
// 136 + q.
DEV uint4 unpack_offset8(uint32_t w) {
  const uint32_t t = w ^ 0x88888888u;
  uint4 r;
  r.x = (t & 0x000F000Fu) | 0x43004300u;
  r.y = ((t >> 4) & 0x000F000Fu) | 0x43004300u;
  r.z = ((t >> 8) & 0x000F000Fu) | 0x43004300u;
  r.w = ((t >> 12) & 0x000F000Fu) | 0x43004300u;
  return r;
}

// Signed int4 of element j (0..7) of a storage word.
DEV int int4_of_word(uint32_t w, int j) {
  const int slot = (j >> 1) + ((j & 1) << 2);
  return __builtin_amdgcn_sbfe(w, 4 * slot, 4);
}

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
DEV uint32_t cvt_pk_bf16(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// silu(z) = z / (1 + e^-z) with the hardware reciprocal (about 1 ulp): +-inf
// limits come out as 0 and z.
DEV float silu_rcp(float z) { return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }
DEV float sigmoid_rcp(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

DEV bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// XOR swizzle of the 16-byte chunks of 128-byte LDS rows: chunk c of row r
// is stored at position c ^ row_swz(r).  A 16-byte read by 16 lanes of rows
// r0 .. r0+15 (one chunk index each) then touches every 16-byte bank group
// of 256 bytes once: rows r and r + 8 share a bank group under r & 7 alone.
DEV int row_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

// Output-column permutation of the int4 products: matrix-instruction row j
// (0..15) of column fragment nf holds column 32 (nf >> 1) + 8 (j >> 2) +
// 4 (nf & 1) + (j & 3) of the fragments' span, so that a lane's four values
// of fragment 2t and four of 2t + 1 are 8 adjacent columns (16-byte accesses
// in an epilogue).  Rows of 32 bytes per column in LDS (the int4 words of a
// stage, adapter rows) then sit at position gt_pos(c) = c ^ (4 bit3(c)), the
// two 16-byte halves swapped when bit 4 of c is set (gt_half): the 16 columns
// one fragment reads, 8 bytes a lane, touch every bank once per half wave.
DEV constexpr int gt_col(int nf, int j) { return 32 * (nf >> 1) + 8 * (j >> 2) + 4 * (nf & 1) + (j & 3); }
DEV constexpr int gt_pos(int c) { return c ^ (4 * ((c >> 3) & 1)); }
DEV constexpr int gt_half(int c) { return (c >> 4) & 1; }

// D = A(16x32) B(32x16) + C.  Lane l holds A row l%16 / B column l%16 with 8
// consecutive K values of lane group l/16; D lane l holds column l%16, rows
// 4*(l/16) .. 4*(l/16)+3.
DEV f32x4_t mfma32(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
// Same with K = 16 (4 values per lane).
DEV f32x4_t mfma16(short4_t a, short4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 16 bytes per lane from global memory straight into LDS: lane i of the wave
// writes lds_wave_base + 16 i.
DEV void load_lds16(const void *gsrc, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void *)lds_wave_base, 16, 0, 0);
}

// 4 bytes per lane straight into LDS: lane i writes lds_wave_base + 4 i
// (only the active lanes write).
DEV void load_lds4(const void *gsrc, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void *)lds_wave_base, 4, 0, 0);
}

// 2 bytes per lane straight into LDS, zero-extended into a 4-byte slot: lane i
// writes lds_wave_base + 4 i (only the active lanes write).
DEV void load_lds2(const void *gsrc, void *lds_wave_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void *)lds_wave_base, 2, 0, 0);
}

// The same transfers issued from inline asm, addressed as a wave-uniform
// 64-bit base (SGPRs) plus a 32-bit per-lane byte offset.  The compiler then
// does not know that they write LDS, so it adds none of its own waits before
// LDS reads (its tracking of LDS-DMA is conservative across loop back-edges
// and would drain a deep prefetch); callers wait explicitly (s_waitcnt
// vmcnt) and synchronise before reading what these wrote.  They read their
// operands at issue and write no registers.  The base must be the same in
// every lane of the wave: values derived from lane-dependent ones go through
// uniform_ptr (readfirstlane) first.
DEV uint32_t lds_addr(const void *p) {   // 32-bit LDS byte address of a __shared__ pointer
  return (uint32_t)(uintptr_t)(const lds_void *)p;
}
// Load a T from LDS byte address `addr`.  With `addr` = an opaque per-lane
// base + a compile-time constant, the constant becomes the instruction's
// 16-bit offset (the base should then already include the array's address).
// T should be a scalar or an ext_vector type: those carry their natural
// alignment, so 8- and 16-byte reads stay single instructions.
template <typename T> DEV T lds_ld(uint32_t addr) {
  return *(const __attribute__((address_space(3))) T *)(uintptr_t)addr;
}
template <typename T> DEV void lds_st(uint32_t addr, T v) {
  *(__attribute__((address_space(3))) T *)(uintptr_t)addr = v;
}
DEV uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}
DEV const void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
}
// lds: wave-uniform LDS byte address where lane i's data lands (+ size * i).
// Each transfer sets M0 itself and declares it clobbered: the statement is
// then recorded as defining M0, so the compiler re-initialises M0 before any
// later instruction of its own that reads it.  (The compiler warns that a
// reserved register in a clobber list is not saved and restored around the
// statement; nothing here needs it restored, so that warning is silenced.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
DEV void dma16(const void *sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
DEV void dma4(const void *sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
DEV void dma2(const void *sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_ushort %0, %1" ::"v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// s_waitcnt immediates (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt
// 6:4, lgkmcnt 11:8).  vmcnt_imm(n): at most n vector memory operations
// (loads, LDS-DMA, stores) of this wave outstanding; kWaitAll: none, and no
// LDS operation either.
constexpr int vmcnt_imm(int n) { return 0x0f70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitAll = 0x0070;
// every vector memory operation of this wave done (LDS untouched).  The
// LDS-DMA pipelines wait with this rather than with a count of the newest
// loads: LDS-DMA loads of one wave were observed to complete out of issue
// order (a count-based wait let a stage be read before all of it had
// landed), and waiting for all of them costs nothing measurable here.
constexpr int kWaitVm = vmcnt_imm(0);

// Next item of a persistent launch whose `total` items are split into eight
// contiguous ranges, one per XCD, range r with the zeroed counter
// ctr[r * kCtrStride]: a block draws from range *rng (its own XCD's first)
// and, once that range is used up, from the following ranges in turn, so
// that no XCD idles while another still has items (the ranges hold equal
// numbers of items, not equal work).
// -1 when every range is used up.  One thread calls it; the counters only
// choose which block computes an item.  (steal = false: the own range only.)
DEV int draw_item(int *ctr, int total, int &rng, int xcd, bool steal = true) {
  for (; rng < xcd + (steal ? 8 : 1); ++rng) {
    const int r = rng & 7;
    const int end = (int)(((long long)total * (r + 1)) >> 3);
    const int w = (int)(((long long)total * r) >> 3) + atomicAdd(&ctr[r * kCtrStride], 1);
    if (w < end) return w;
  }
  return -1;
}

// Workgroup barrier without the memory fence of __syncthreads(): the fence
// would make the compiler drain every outstanding load, including LDS-DMA
// that is deliberately left in flight.  Callers wait (s_waitcnt) for the
// data they need before calling it; the empty asm statements keep the
// compiler from moving memory operations across it.
DEV void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace moe
