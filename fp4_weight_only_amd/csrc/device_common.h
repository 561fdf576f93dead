// Device helpers shared by the gfx950 kernels: codec bit assembly, bf16
// rounding, wave64 cross-lane moves.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qmoe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats -> packed bf16 pair (first in the low half), each rounded to
// nearest even by the hardware conversion.
__device__ __forceinline__ uint32_t pack_bf16x2_rne(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

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

// Two E2M1 words A (row k) and B (row k+1), 8 columns each (low nibble
// first), become 8 bf16x2 K pairs, column c as {lo: A.c, hi: B.c}, the pair
// a dot2 consumes.  A nibble zip puts the codes of one column's two rows into
// one byte (even columns from the low nibbles, odd columns from the high
// nibbles: two shifts and two bit-field inserts), and gfx950's FP4
// conversion turns each byte into its two exact bf16 values (scale 1).
// Twelve VALU instructions per 16 codes, no table, no branch.
template <int J>
__device__ __forceinline__ uint32_t fp4_byte_to_bf16x2(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, 1.0f, J));
}

__device__ __forceinline__ void e2m1_kpair_cvt(uint32_t a, uint32_t b, uint32_t (&w)[8]) {
  const uint32_t ev = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
  const uint32_t od = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  w[0] = fp4_byte_to_bf16x2<0>(ev);
  w[1] = fp4_byte_to_bf16x2<0>(od);
  w[2] = fp4_byte_to_bf16x2<1>(ev);
  w[3] = fp4_byte_to_bf16x2<1>(od);
  w[4] = fp4_byte_to_bf16x2<2>(ev);
  w[5] = fp4_byte_to_bf16x2<2>(od);
  w[6] = fp4_byte_to_bf16x2<3>(ev);
  w[7] = fp4_byte_to_bf16x2<3>(od);
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

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active): a
// Hillis-Steele scan inside each 16-lane row (row shifts by 1, 2, 4, 8;
// lanes shifted in from outside the row read 0), then the last lane of row
// 0 is added to rows 1 and 3 and the last lane of row 1 to rows 2 and 3
// (row broadcasts; rows masked off add 0).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
  return v;
}

// Finds the expert holding the s-th non-empty row range, with its first row
// and row count.  Every lane gets the same answer; returns -1 if fewer than
// s+1 experts have rows.
__device__ __forceinline__ int find_slot_expert(const int32_t *__restrict__ off, int E, int s, int &row0, int &m) {
  const int lane = lane_id();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = 4 * lane + i;
    o[i] = (e <= E) ? off[e] : 0;
  }
  int before = 0;
  bool ne[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ne[i] = (4 * lane + i < E) && (o[i + 1] > o[i]);
    before += __popcll(__ballot(ne[i]) & lt);
  }
  int found = -1, r0 = 0, cnt = 0;
  int run = before;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (ne[i] && run == s) {
      found = 4 * lane + i;
      r0 = o[i];
      cnt = o[i + 1] - o[i];
    }
    run += ne[i] ? 1 : 0;
  }
  const unsigned long long fb = __ballot(found >= 0);
  if (fb == 0ull) return -1;
  const int src = __ffsll((long long)fb) - 1;
  row0 = __builtin_amdgcn_readlane(r0, src);
  m = __builtin_amdgcn_readlane(cnt, src);
  return __builtin_amdgcn_readlane(found, src);
}

// Slot s when every expert's rows are dealt out in groups of at most G: an
// expert with m rows owns ceil(m / G) consecutive slots (experts in
// ascending order, its groups in row order).  Returns the expert, the
// group's first row and row count (every lane the same answer), or -1 when
// s is past the last group.  A lane covers experts 4*lane .. 4*lane + 3
// (E <= 256); a wave prefix sum of the per-lane group counts locates s.
// G is a power of two (the pass sizes 1, 2 and 4).
__device__ __forceinline__ int find_slot_group(const int32_t *__restrict__ off, int E, int s, int G, int &row0,
                                               int &m) {
  const int lane = lane_id();
  const int gsh = __builtin_ctz((unsigned)G);
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = 4 * lane + i;
    o[i] = (e <= E) ? off[e] : 0;
  }
  int cnt[4], grp[4], local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cnt[i] = (4 * lane + i < E) ? o[i + 1] - o[i] : 0;
    grp[i] = (cnt[i] + G - 1) >> gsh;
    local += grp[i];
  }
  const int incl = wave_inclusive_sum(local);
  int found = -1, r0 = 0, rc = 0;
  int run = incl - local;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (found < 0 && s >= run && s < run + grp[i]) {
      const int q = s - run;
      found = 4 * lane + i;
      r0 = o[i] + q * G;
      rc = (cnt[i] - q * G) < G ? (cnt[i] - q * G) : G;
    }
    run += grp[i];
  }
  const unsigned long long fb = __ballot(found >= 0);
  if (fb == 0ull) return -1;
  const int src = __ffsll((long long)fb) - 1;
  row0 = __builtin_amdgcn_readlane(r0, src);
  m = __builtin_amdgcn_readlane(rc, src);
  return __builtin_amdgcn_readlane(found, src);
}

// SwiGLU(G, L) = G * sigmoid(alpha G) * (L + beta), G = min(gate, limit),
// L = clamp(lin, -limit, limit) (operator documentation section 8).
__device__ __forceinline__ float swiglu(float gate, float lin, float alpha, float beta, float limit) {
  const float G = fminf(gate, limit);
  const float L = fminf(fmaxf(lin, -limit), limit);
  return G / (1.0f + expf(-alpha * G)) * (L + beta);
}

// Finds the s-th (expert, m tile) item: experts in ascending order, each with
// ceil(rows/BM) tiles.  Returns the expert (-1 past the last item) and the
// tile index inside it.  Every lane gets the same answer.
template <int BM>
__device__ __forceinline__ int find_mtile(const int32_t *__restrict__ off, int E, int s, int &mt) {
  const int lane = lane_id();
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = 4 * lane + i;
    o[i] = (e <= E) ? off[e] : 0;
  }
  int cnt[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    cnt[i] = (4 * lane + i < E) ? (o[i + 1] - o[i] + BM - 1) / BM : 0;
    sum += cnt[i];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  int run = incl - sum;
  int found = -1, tile = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (s >= run && s < run + cnt[i]) {
      found = 4 * lane + i;
      tile = s - run;
    }
    run += cnt[i];
  }
  const unsigned long long fb = __ballot(found >= 0);
  if (fb == 0ull) return -1;
  const int src = __ffsll((long long)fb) - 1;
  mt = __builtin_amdgcn_readlane(tile, src);
  return __builtin_amdgcn_readlane(found, src);
}

// A wave-uniform pointer, moved to scalar registers (a buffer resource built
// from it stays scalar; otherwise the compiler wraps every buffer load in a
// waterfall loop).
__device__ __forceinline__ void *uniform_ptr(const void *p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (void *)(((uint64_t)hi << 32) | lo);
}

// Workgroup barrier that orders LDS accesses only: __syncthreads() also
// waits for the wave's outstanding global loads (its fence covers every
// address space), which would stall on loads meant to stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

}  // namespace qmoe
