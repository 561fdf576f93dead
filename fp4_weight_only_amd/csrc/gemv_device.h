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
#pragma unroll
  for (int r = 0; r < MR; ++r) {
#pragma unroll
    for (int c = 0; c < 8; ++c)
      acc[r][c] = acc[r][c] + __shfl_xor(acc[r][c], 32);  // lower half + upper half, same order in every lane pair
    if (lane < 32) {
      *(float4 *)&sm.red[wave][r0 + r][nl * 8] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
      *(float4 *)&sm.red[wave][r0 + r][nl * 8 + 4] = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
    }
  }
}

}  // namespace qmoe
