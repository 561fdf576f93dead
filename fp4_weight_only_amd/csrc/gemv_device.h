// Building blocks of the FP4 decode GEMV shared by the per-call GEMV
// kernels (gemv.hip) and the single-launch decode layer (layer.hip): block
// scale decode, the LDS layout of one pass, and the per-lane decode + dot2
// over a lane's 32 k rows (operator documentation sections 9b.2-9b.3; PR
// 31159: K-paired accumulation, the block scale applied to the block's
// partial sum).
#pragma once

#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kMaxChunkK = kGemvMaxWaves * kGemvWaveK;
constexpr uint32_t kOutOfRange = 0x80000000u;  // buffer offset past any resource: loads return 0
constexpr int kBufNontemporal = 2;            // cache policy: streaming (nt)

template <int FMT>
__device__ __forceinline__ void decode_scales(u32x2_t sb, float (&sc)[8]) {
  if constexpr (FMT == 0) {
    sc[0] = e4m3_to_f32<0>(sb.x);
    sc[1] = e4m3_to_f32<1>(sb.x);
    sc[2] = e4m3_to_f32<2>(sb.x);
    sc[3] = e4m3_to_f32<3>(sb.x);
    sc[4] = e4m3_to_f32<0>(sb.y);
    sc[5] = e4m3_to_f32<1>(sb.y);
    sc[6] = e4m3_to_f32<2>(sb.y);
    sc[7] = e4m3_to_f32<3>(sb.y);
  } else {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      sc[c] = e8m0_to_f32((sb.x >> (8 * c)) & 0xFFu);
      sc[c + 4] = e8m0_to_f32((sb.y >> (8 * c)) & 0xFFu);
    }
  }
}


// Lower + upper half-wave sums of two values at once: v_permlane32_swap
// exchanges lanes 32..63 of a with lanes 0..31 of b, so lanes 0..31 end up
// with a's lower + upper halves and lanes 32..63 with b's (both sums taken
// lower half first, as a lane swap with __shfl_xor would give).
__device__ __forceinline__ float half_sum_pair(float a, float b) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

template <int MRMAX>
struct Smem {
  uint16_t xs[MRMAX][kMaxChunkK];                 // activations of the chunk
  float red[kGemvMaxWaves][MRMAX][kGemvTileN];    // per-wave partial sums
};

// Decode + dot2 over the lane's 32 k rows for MR staged rows r0 .. r0 +
// MR - 1; the wave's partial (the two halves added) goes to LDS.  A row's
// arithmetic does not depend on MR or r0.
template <int FMT, int MR, int MRMAX>
__device__ __forceinline__ void lane_dot(Smem<MRMAX> &sm, const uint32_t (&A)[kGemvLaneK], const u32x2_t (&SB)[2],
                                         int g, int wave, int lane, int r0 = 0) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int NBLK = kGemvLaneK / B;
  float acc[MR][8];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    // One row: the activation K pairs of this scale block are read once up
    // front.  Two rows: read per K pair (a preload would cost ~100 VGPRs).
    constexpr bool kPre = (MR == 1);
    uint32_t xq[kPre ? B / 2 : 1];
    if constexpr (kPre) {
#pragma unroll
      for (int q = 0; q < B / 8; ++q) {
        const u32x4_t v = *(const u32x4_t *)&sm.xs[r0][g * kGemvLaneK + b * B + q * 8];
        xq[4 * q + 0] = v.x;
        xq[4 * q + 1] = v.y;
        xq[4 * q + 2] = v.z;
        xq[4 * q + 3] = v.w;
      }
    }
    float bs[MR][8];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) bs[r][c] = 0.f;
    // More rows: the activation K pairs are read one K pair ahead, so the
    // LDS latency hides behind the current pair's decode and dot2s.
    uint32_t xn[MR];
    if constexpr (!kPre) {
#pragma unroll
      for (int r = 0; r < MR; ++r) xn[r] = *(const uint32_t *)&sm.xs[r0 + r][g * kGemvLaneK + b * B];
    }
#pragma unroll
    for (int kp = 0; kp < B / 2; ++kp) {
      uint32_t xc[MR];
      if constexpr (!kPre) {
#pragma unroll
        for (int r = 0; r < MR; ++r) {
          xc[r] = xn[r];
          if (kp + 1 < B / 2) xn[r] = *(const uint32_t *)&sm.xs[r0 + r][g * kGemvLaneK + b * B + 2 * (kp + 1)];
        }
      }
      uint32_t w[8];
      e2m1_kpair_cvt(A[b * B + 2 * kp], A[b * B + 2 * kp + 1], w);
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const uint32_t xp = kPre ? xq[kPre ? kp : 0] : xc[r];
#pragma unroll
        for (int c = 0; c < 8; ++c) bs[r][c] = dot2_bf16(xp, w[c], bs[r][c]);
      }
      // Keep each K pair's decode next to its dot2s (bounds the live decoded
      // weights to 8 registers): the empty asm pins the partial sums here so
      // no dot2 is sunk towards its later use, and the barrier stops the
      // scheduler from hoisting the next decode.
#pragma unroll
      for (int r = 0; r < MR; ++r)
#pragma unroll
        for (int c = 0; c < 8; ++c) asm volatile("" : "+v"(bs[r][c]));
      __builtin_amdgcn_sched_barrier(0);
    }
    float sc[8];
    decode_scales<FMT>(SB[b], sc);
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(sc[c], bs[r][c], acc[r][c]);
  }
  const int nl = lane & 31;
  // columns c and c + 4 paired: lanes 0..31 store columns 0..3 of their
  // eight, lanes 32..63 columns 4..7
  const int half = lane >> 5;
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    float v[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) v[c] = half_sum_pair(acc[r][c], acc[r][c + 4]);
    *(float4 *)&sm.red[wave][r0 + r][nl * 8 + 4 * half] = make_float4(v[0], v[1], v[2], v[3]);
  }
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Columns 4 GRP .. 4 GRP + 3 of two E2M1 rows as bf16 K pairs (the
// matching half of e2m1_kpair_cvt's output).
template <int GRP>
__device__ __forceinline__ void e2m1_kpair_cvt_half(uint32_t a, uint32_t b, uint32_t (&w)[4]) {
  const uint32_t ev = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
  const uint32_t od = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  w[0] = fp4_byte_to_bf16x2<2 * GRP>(ev);
  w[1] = fp4_byte_to_bf16x2<2 * GRP>(od);
  w[2] = fp4_byte_to_bf16x2<2 * GRP + 1>(ev);
  w[3] = fp4_byte_to_bf16x2<2 * GRP + 1>(od);
}

// Two to four staged rows r0 .. r0 + mr - 1 through the matrix cores, over
// the same lane layout as lane_dot: 4x4x4 bf16 blocks, sixteen per
// instruction.  Block b is lanes 4b .. 4b + 3; lane 4b + i brings activation
// row r0 + i and lane 4b + j one of its own weight columns,
// each over a k quad (4 of the lane's 32 k rows); the result is the lane's
// column for all four rows.  Per column and scale block the k quads
// accumulate in fp32 from +0, and the block scale multiplies the block sum
// into the lane's running sum (fma), the dot2 path's order of operations.
// Columns go in two groups of four to bound the live accumulators.
// MASKX: lanes past the mr rows read zeros (a masked read per k quad);
// otherwise they read a staged row, which is as good: a block's output row i
// depends on activation row i alone, and rows past mr are never stored.  The
// per-call GEMV reads unmasked (MXFP4 hidden-4096 T=8 layer 170.8 -> 164.5 us
// with the shift-based slot lookup); the single-launch layer keeps the
// masked read (T=4 25.7 against 26.5 us unmasked).
template <int FMT, int MRMAX, int GRP, bool MASKX>
__device__ __forceinline__ void lane_mfma_group(Smem<MRMAX> &sm, const uint32_t (&A)[kGemvLaneK],
                                                const u32x2_t (&SB)[2], int g, int wave, int lane, int r0, int mr) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int NBLK = kGemvLaneK / B;
  constexpr int QPB = B / 4;  // k quads per scale block
  const int i = lane & 3;
  const bool xon = !MASKX || i < mr;
  const uint16_t *xrow = &sm.xs[MASKX ? (xon ? r0 + i : 0) : (r0 + i < MRMAX ? r0 + i : MRMAX - 1)][g * kGemvLaneK];
  float acc[4][4];
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[c][r] = 0.f;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    f32x4_t bacc[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) bacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < QPB; ++q) {
      const int kq = b * QPB + q;
      const u32x2_t xa = xon ? *(const u32x2_t *)(xrow + 4 * kq) : u32x2_t{0u, 0u};
      uint32_t w0[4], w1[4];
      e2m1_kpair_cvt_half<GRP>(A[4 * kq], A[4 * kq + 1], w0);
      e2m1_kpair_cvt_half<GRP>(A[4 * kq + 2], A[4 * kq + 3], w1);
#pragma unroll
      for (int c = 0; c < 4; ++c)
        bacc[c] = __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(__builtin_bit_cast(s16x4_t, xa),
                                                        __builtin_bit_cast(s16x4_t, u32x2_t{w0[c], w1[c]}),
                                                        bacc[c], 0, 0, 0);
    }
    float sc[8];
    decode_scales<FMT>(SB[b], sc);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[c][r] = fmaf(sc[4 * GRP + c], bacc[c][r], acc[c][r]);
  }
  const int nl = lane & 31;
  if constexpr (FMT == 0) {
    // rows rp and rp + 1 paired: lanes 0..31 store row rp, lanes 32..63 row
    // rp + 1 (NVFP4 T=4 single-launch layer 25.7 -> 25.4 us, T=8 separate
    // calls 38.5 -> 37.8 us)
    const int half = lane >> 5;
#pragma unroll
    for (int rp = 0; rp < 4; rp += 2) {
      if (rp < mr) {  // uniform
        float v[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = half_sum_pair(acc[c][rp], acc[c][rp + 1]);
        const int r = rp + half;
        if (r < mr)
          *(float4 *)&sm.red[wave][r0 + r][nl * 8 + 4 * GRP] = make_float4(v[0], v[1], v[2], v[3]);
      }
    }
  } else {
    // MXFP4: a lane swap per value (the paired form measured slower here:
    // hidden-4096 T=8 layer 164.3 -> 165.9 us)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (r < mr) {  // uniform
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c][r] = acc[c][r] + __shfl_xor(acc[c][r], 32);  // lower half + upper half
        if (lane < 32)
          *(float4 *)&sm.red[wave][r0 + r][nl * 8 + 4 * GRP] = make_float4(acc[0][r], acc[1][r], acc[2][r], acc[3][r]);
      }
    }
  }
}

// One pass over mr <= MRMAX staged rows starting at r0: two to four rows on
// the matrix cores; one row on the dot2 path for NVFP4 and on the matrix
// cores for MXFP4 (a quarter of each 4x4x4 block used, the dot products off
// the VALU: the MXFP4 hidden-4096 decode layer, whose GEMV is VALU-bound,
// 182.7 -> 169.8 us on MI355X; the NVFP4 single-launch layers, bound by
// each item's latency, ran 0.3-0.5 us slower that way).
template <int FMT, int MRMAX, bool MASKX = true>
__device__ __forceinline__ void lane_pass(Smem<MRMAX> &sm, const uint32_t (&A)[kGemvLaneK], const u32x2_t (&SB)[2],
                                          int g, int wave, int lane, int r0, int mr) {
  if (FMT == 0 && (MRMAX == 1 || mr == 1)) {
    lane_dot<FMT, 1, MRMAX>(sm, A, SB, g, wave, lane, r0);
  } else {
    lane_mfma_group<FMT, MRMAX, 0, MASKX>(sm, A, SB, g, wave, lane, r0, mr);
    lane_mfma_group<FMT, MRMAX, 1, MASKX>(sm, A, SB, g, wave, lane, r0, mr);
  }
}

}  // namespace qmoe
