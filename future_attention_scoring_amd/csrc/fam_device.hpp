// Device-side helpers shared by the score kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fam {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kInf = __builtin_huge_valf();

struct Bf16 {};
struct Fp16 {};

// One 32x32x16 MFMA on raw 16-byte operand fragments (8 two-byte elements per
// lane). Lane l supplies row l%32 of A (or column l%32 of B) and 8 entries of
// the contraction axis; A and B must use the same assignment of the
// contraction axis to (lane/32, element), which the callers guarantee by
// loading both from the same head-dim offsets.
template <typename T> struct Mma;
template <> struct Mma<Bf16> {
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
};
template <> struct Mma<Fp16> {
  static __device__ __forceinline__ f32x16_t run(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
};

// Row of accumulator entry v held by a lane in the 32x32 MFMA output; the
// column is lane % 32. Verified on gfx950 for v_mfma_f32_32x32x16_{bf16,f16}.
__device__ __forceinline__ int acc_row(int v, int lane) {
  return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ u32x4_t load16(const uint16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ void store16(uint16_t* p, u32x4_t v) {
  *reinterpret_cast<u32x4_t*>(p) = v;
}
__device__ __forceinline__ u32x4_t zero16() { return u32x4_t{0u, 0u, 0u, 0u}; }

// Sum of squares of the 8 two-byte elements of a 16-byte fragment, in fp32.
template <typename T> __device__ float sumsq8(u32x4_t v);
template <> __device__ __forceinline__ float sumsq8<Bf16>(u32x4_t v) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = __uint_as_float(v[w] << 16), hi = __uint_as_float(v[w] & 0xffff0000u);
    s = fmaf(lo, lo, fmaf(hi, hi, s));
  }
  return s;
}
template <> __device__ __forceinline__ float sumsq8<Fp16>(u32x4_t v) {
  float s = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float lo = (float)__builtin_bit_cast(_Float16, (unsigned short)(v[w] & 0xffffu));
    const float hi = (float)__builtin_bit_cast(_Float16, (unsigned short)(v[w] >> 16));
    s = fmaf(lo, lo, fmaf(hi, hi, s));
  }
  return s;
}

// Order-preserving u32 key of a score: larger scores give larger keys, -0.0
// maps like +0.0, NaN maps to 1 (below every number; 0 stays free as a
// "no entry" marker).
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (f != f) return 1u;
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVm0 = 0x0F70;
typedef __attribute__((address_space(3))) void lds_void;

// 16 bytes per lane from global memory (uniform base + per-lane byte
// offset) into LDS at lds + 16 * lane (gfx950 global_load_lds_dwordx4;
// M0 holds the LDS address). Written as assembly so that the compiler's
// wait analysis does not take it for a store that may alias every LDS read
// (it would wait for it before each read of the other buffer); the caller
// waits for it (vmcnt) before the barrier that publishes the tile.
// M0 is named as clobbered (nothing else in these kernels keeps a value in
// it; the compiler warns that it reserves M0, hence the local pragma).
// Used by the score passes to stage their streamed tiles.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(off), "s"(base), "s"(lds)
      : "memory", "m0");
}
#pragma clang diagnostic pop

// Pairwise sum of the 16 accumulator-shaped values.
__device__ __forceinline__ float sum16(const float (&e)[16]) {
  float a0 = e[0] + e[1], a1 = e[2] + e[3], a2 = e[4] + e[5], a3 = e[6] + e[7];
  float a4 = e[8] + e[9], a5 = e[10] + e[11], a6 = e[12] + e[13], a7 = e[14] + e[15];
  return ((a0 + a1) + (a2 + a3)) + ((a4 + a5) + (a6 + a7));
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS round trips).
__device__ __forceinline__ int wave_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 into rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 into rows 2 and 3
  return v;
}

}  // namespace fam
