// LDS staging helpers shared by the gfx950 kernels: the 16-byte-chunk XOR
// swizzle of K/V tiles, bounds-checked buffer loads straight into LDS, waits
// and barriers around them, and LDS reads through 32-bit byte addresses
// (including the transposing ds_read_b64_tr_b16).
#pragma once

#include "device_common.h"

namespace attn {

// 16-byte chunk swizzle: physical chunk = logical chunk ^ swz<D>(row).  The
// LDS serves 256 bytes (64 banks) per cycle: 16 lanes of a ds_read_b128 or 32
// lanes of a ds_read_b64_tr_b16.  The K operand read has 16 consecutive rows
// at one logical chunk; the transposed V read has 4 consecutive rows (first
// row a multiple of 4) times 4 consecutive chunks (first a multiple of 4).
// Both must land on 16 distinct 16-byte bank groups:
//  d = 128 (256-byte rows): swz = 4*(row%4) + (row/4)%4 is a permutation of
//    0..15 over 16 consecutive rows, and over 4 consecutive rows its top two
//    bits take 4 distinct values;
//  d = 64 (128-byte rows, two per bank row): swz = 4*((row/2)%2) + (row/4)%4
//    permutes 0..7 over the 8 rows of one parity, and rows 2 apart differ in
//    bit 2;
//  d = 32 (64-byte rows, four per bank row): swz = (row/4)%4 permutes 0..3
//    over the 4 rows of one residue mod 4 among 16 consecutive rows; 4
//    consecutive rows fill one bank row whatever the swizzle;
//  d = 256 (512-byte rows, two bank rows each): the d = 128 swizzle on the
//    low four chunk bits (a chunk's bank group is its index mod 16), so both
//    reads see the same bank groups as at d = 128.
template <int D>
__device__ __forceinline__ int swz(int row) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dims with a swizzle");
  if constexpr (D == 128 || D == 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  else if constexpr (D == 64) return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
  else return (row >> 2) & 3;
}

// Buffer descriptor over one (batch, kv head) slice of K or V: base address,
// stride 0 (raw buffer), size in bytes, gfx9 word 3.  Offsets at or past the
// size read as zero, so rows past M come back as zeros.  The host guarantees
// that the rows a kernel may address past M (up to one tile) stay below 2^32
// bytes, so the per-lane offsets never wrap around.
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 make_desc(const uint16_t* base, int64_t row_stride, int M, int D) {
  const int64_t bytes = ((int64_t)(M - 1) * row_stride + D) * 2;
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  return (i32x4){(int)(uint32_t)addr, (int)((uint32_t)(addr >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
// The same with the row stride and length in bytes (8-bit elements).
__device__ __forceinline__ i32x4 make_desc_bytes(const uint8_t* base, int64_t row_stride_bytes, int M, int row_bytes) {
  const int64_t bytes = (int64_t)(M - 1) * row_stride_bytes + row_bytes;
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  return (i32x4){(int)(uint32_t)addr, (int)((uint32_t)(addr >> 32) & 0xffffu), (int)bytes, 0x00020000};
}
// The same over M >= 0 rows: with M == 0 the size is 0 and every offset reads as zero.
__device__ __forceinline__ i32x4 make_desc_rows(const uint16_t* base, int64_t row_stride, int M, int D) {
  const int64_t bytes = M > 0 ? ((int64_t)(M - 1) * row_stride + D) * 2 : 0;
  const uint64_t addr = (uint64_t)(uintptr_t)base;
  return (i32x4){(int)(uint32_t)addr, (int)((uint32_t)(addr >> 32) & 0xffffu), (int)bytes, 0x00020000};
}

// One buffer_load_dwordx4 ... lds: lane L's 16 bytes at byte offset voff of the
// buffer go to LDS byte address lds + 16 * L (M0 holds lds).  Inline asm, so
// that the compiler does not see an LDS write: it would otherwise wait for
// every outstanding tile fetch (vmcnt(0)) before the next LDS read.  Each tile
// is instead waited for explicitly (vmcnt) by the fetching wave before the
// barrier that publishes it.  s_nop: one wait state between the M0 write and
// its use.  M0 is listed as clobbered (nothing else in these kernels keeps a
// value in M0).  kStream adds the nontemporal hint for data read exactly once
// (it then neither displaces nor hits cached lines in L2 and the MALL).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
template <bool kStream = false>
__device__ __forceinline__ void dma16(i32x4 desc, uint32_t lds, uint32_t voff) {
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(desc)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(desc)
                 : "memory", "m0");
}
// The same with a uniform byte offset soff in the instruction's scalar offset
// operand: the bounds check covers voff + soff (measured on gfx950: bytes at
// or past the buffer's size read as zero also when soff takes them there), so
// a tile's row offset needs no per-lane add.
template <bool kStream = false>
__device__ __forceinline__ void dma16_so(i32x4 desc, uint32_t lds, uint32_t voff, uint32_t soff) {
  if constexpr (kStream)
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(desc),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :
                 : "s"(__builtin_amdgcn_readfirstlane(lds)), "v"(voff), "s"(desc),
                   "s"(__builtin_amdgcn_readfirstlane(soff))
                 : "memory", "m0");
}
#pragma clang diagnostic pop

__device__ __forceinline__ void wait_tile_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector memory operations are outstanding
// (they complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory"); }

// Workgroup barrier: this wave's LDS reads are complete (lgkmcnt(0)) so the
// buffers they read can be refilled after it.  The asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void kv_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS access through 32-bit byte addresses; constant parts of an address
// (tile, 32-key block, k-step) become the instruction's offset field.
typedef __attribute__((address_space(3))) s16x8 lds_s16x8;
typedef __attribute__((address_space(3))) uint16_t lds_u16;
__device__ __forceinline__ s16x8 lds_read_b128(uint32_t addr) { return *(const lds_s16x8*)(uintptr_t)addr; }
__device__ __forceinline__ s16x4 lds_read_tr16_b64(uint32_t addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)addr);
}
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
__device__ __forceinline__ void lds_write_b64(uint32_t addr, u32x2 v) { *(lds_u32x2*)(uintptr_t)addr = v; }
// Orders this wave's LDS accesses when lanes exchange data through LDS: the
// wait completes the writes, and the memory clobber stops the compiler from
// reusing values read before it (to the compiler, lanes are separate threads,
// so without it another lane's write is invisible).
__device__ __forceinline__ void lds_lane_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace attn
