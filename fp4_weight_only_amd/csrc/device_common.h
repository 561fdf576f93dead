// Device helpers shared by the gfx950 kernels: codec bit assembly, bf16
// rounding, wave64 cross-lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// float32 -> bf16 bits, round to nearest even, NaN kept quiet.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  uint32_t r = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  return ((u & 0x7FFFFFFFu) > 0x7F800000u) ? ((u >> 16) | 0x40u) : r;
}

// E2M1 code (low 4 bits of c) -> float32, exact.  The code's exponent and
// mantissa bits are placed at the bottom of the float32 exponent field, which
// gives value * 2^-126 (code 1 lands on the subnormal 2^-127); one multiply by
// 2^126 (subnormal inputs are preserved in this kernel mode) restores the value.
// The sign bit is moved to bit 31.
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
  float mag = __uint_as_float((c & 7u) << 22) * 0x1p126f;
  return __uint_as_float(__float_as_uint(mag) | ((c & 8u) << 28));
}

// E8M0 byte -> float32: 2^(b-127); b = 0 is the subnormal 2^-127, b = 255 NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  uint32_t bits = (b == 0u) ? 0x00400000u : (b << 23);
  return __uint_as_float(b == 255u ? 0x7FC00000u : bits);
}

// E4M3FN byte `sel` of word w -> float32 (hardware OCP fp8 conversion).
template <int SEL>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
  return __builtin_amdgcn_cvt_f32_fp8((int)w, SEL);
}

// Two E2M1 words A (row k) and B (row k+1), each holding 8 columns (low
// nibble first), become 8 bf16x2 registers: column c as {lo: A.c, hi: B.c},
// the K-pair a dot2 consumes.  Each bf16 is assembled directly from the code
// bits: sign to bit 15, exponent+mantissa bits to bits 8..6, so the value is
// e2m1 * 2^-126 (code 1 is the bf16 subnormal 2^-127).  The caller folds the
// 2^126 into a power-of-two pre-scale of the activations.
__device__ __forceinline__ void e2m1_kpair_to_bf16x2(uint32_t a, uint32_t b, uint32_t (&w)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // bytes [a.j, 0, b.j, 0]: each 16-bit half holds one byte (two codes).
    const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
    const uint32_t q = __builtin_amdgcn_perm(b, a, sel);
    const uint32_t ev_code = q << 6;                  // even code -> bits 8..6 / 24..22
    const uint32_t ev_sign = (q << 12) & 0x80008000u;  // even sign -> bits 15 / 31
    const uint32_t od_code = q << 2;                  // odd code  -> bits 8..6 / 24..22
    const uint32_t od_sign = (q << 8) & 0x80008000u;   // odd sign  -> bits 15 / 31
    w[2 * j] = (ev_code & 0x01C001C0u) | ev_sign;
    w[2 * j + 1] = (od_code & 0x01C001C0u) | od_sign;
  }
}

// The same K pairs from gfx950's FP4 conversion: one instruction turns byte j
// of a word (codes of columns 2j and 2j+1) into two bf16 (scale 1: the exact
// code values), and a byte permute pairs row k with row k+1 of each column.
// Four VALU instructions per 8 codes, against about nine for bit assembly.
template <int J>
__device__ __forceinline__ void e2m1_kpair_cvt_byte(uint32_t a, uint32_t b, uint32_t &even, uint32_t &odd) {
  const uint32_t pa = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(a, 1.0f, J));
  const uint32_t pb = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(b, 1.0f, J));
  even = __builtin_amdgcn_perm(pb, pa, 0x05040100u);  // {pa.lo, pb.lo}
  odd = __builtin_amdgcn_perm(pb, pa, 0x07060302u);   // {pa.hi, pb.hi}
}

__device__ __forceinline__ void e2m1_kpair_cvt(uint32_t a, uint32_t b, uint32_t (&w)[8]) {
  e2m1_kpair_cvt_byte<0>(a, b, w[0], w[1]);
  e2m1_kpair_cvt_byte<1>(a, b, w[2], w[3]);
  e2m1_kpair_cvt_byte<2>(a, b, w[4], w[5]);
  e2m1_kpair_cvt_byte<3>(a, b, w[6], w[7]);
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// DPP moves inside a wave64 (all lanes active).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

// ds_swizzle bit-mask mode: lane ^ 16 inside each 32-lane half.
__device__ __forceinline__ uint32_t swz_xor16(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}
__device__ __forceinline__ uint32_t bperm_xor32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_ds_bpermute((lane_id() ^ 32) << 2, (int)v);
}

}  // namespace qmoe
