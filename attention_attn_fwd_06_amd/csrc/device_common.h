// Device-side helpers shared by the gfx950 attention kernels: vector types,
// MFMA wrappers, 16-bit conversions, lane exchanges and the XCD-aware
// workgroup remap.  CDNA4 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D[32x32] += A[32x16] * B[16x32] in fp32.  Lane l supplies row (l % 32) of A
// and column (l % 32) of B, each as 8 consecutive contraction slots; the two
// lane halves (l / 32) hold slots 0-7 and 8-15.  Accumulator element i of lane l
// is D[8*(i/4) + 4*(l/32) + i%4][l % 32].
template <bool BF16>
__device__ __forceinline__ f32x16 mfma32x32x16(s16x8 a, s16x8 b, f32x16 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// D[16x16] += A[16x32] * B[32x16] in fp32.  Lane l supplies row (l % 16) of A
// and column (l % 16) of B, each as 8 consecutive contraction slots; lane group
// l / 16 holds slots 8*(l/16) .. +7.  Accumulator element i of lane l is
// D[4*(l/16) + i][l % 16].
template <bool BF16>
__device__ __forceinline__ f32x4 mfma16x16x32(s16x8 a, s16x8 b, f32x4 c) {
  if constexpr (BF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                   __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// Two fp32 values to one packed 16-bit pair (round to nearest even).
template <bool BF16>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (BF16) {
    bf16x2 v = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, v);
  } else {
    f16x2 v = __builtin_convertvector((f32x2){lo, hi}, f16x2);
    return __builtin_bit_cast(uint32_t, v);
  }
}

// A packed 16-bit pair back to fp32 (exact).
template <bool BF16>
__device__ __forceinline__ f32x2 unpack2(uint32_t u) {
  if constexpr (BF16) {
    return (f32x2){__uint_as_float(u << 16), __uint_as_float(u & 0xffff0000u)};
  } else {
    f16x2 h = __builtin_bit_cast(f16x2, u);
    return (f32x2){(float)h[0], (float)h[1]};
  }
}

// This lane's index in the wave, read afresh at each call (asm volatile, so
// neither hoisted nor merged with another read): a value the compiler would
// otherwise keep in a register for the whole kernel is recomputed where it is
// needed, in two instructions.
__device__ __forceinline__ uint32_t lane_id_now() {
  uint32_t l;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
  return l;
}

// x, hidden from the optimiser: values computed from the result inside a loop
// cannot be hoisted out of it, so a loop-invariant per-lane base plus several
// per-iteration offsets costs one register instead of one per offset.
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}

// Value held by lane l ^ 32 (one v_permlane32_swap).
__device__ __forceinline__ float xor32(float x) {
  int xi = __float_as_int(x);
  auto pr = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  // lanes 0-31 receive (own, partner); lanes 32-63 receive (partner, own)
  int partner = (__lane_id() < 32) ? pr[1] : pr[0];
  return __int_as_float(partner);
}

// max / sum over lanes l and l ^ 32 (the result is the same in both).
__device__ __forceinline__ float max_xor32(float x) {
  int xi = __float_as_int(x);
  auto pr = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return fmaxf(__int_as_float(pr[0]), __int_as_float(pr[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  int xi = __float_as_int(x);
  auto pr = __builtin_amdgcn_permlane32_swap(xi, xi, false, false);
  return __int_as_float(pr[0]) + __int_as_float(pr[1]);
}

// DPP lane moves inside rows of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

// Sum over each aligned group of 16 lanes, result in every lane of the group.
__device__ __forceinline__ float sum16(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x;
}
// Sum over each aligned group of 8 lanes.
__device__ __forceinline__ float sum4(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  return x;
}
__device__ __forceinline__ float sum8(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  return x;
}

// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i runs on
// XCD i % 8, measured on MI355X).  This bijection gives each XCD one contiguous
// range of logical tile ids, so tiles that share K/V share an L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  constexpr int kXcd = 8;
  const int xcd = id % kXcd, local = id / kXcd;
  const int per = total / kXcd, rem = total % kXcd;
  // XCDs below rem own per + 1 ids, the others per (no branch, so that the
  // kernel's argument loads are not split around one)
  return xcd * per + min(xcd, rem) + local;
}

}  // namespace attn
