// FP4 (E2M1) weight-only decode GEMV over routed MoE rows, gfx950.
//
// What it computes (PR 31159 "[CUDA] Speed up the NVFP4 QMoE decode GEMV and
// enable it for MTP verify"; operator documentation sections 8, 9b.2, 12.1):
// for every permuted row p of expert e,
//   u[p][n] = g[e] * sum_b scale[e][b][n] * sum_{k in block b} a[p][k] * e2m1(code[e][k][n])
// then FC1 applies interleaved SwiGLU on (u[2j], u[2j+1]) and writes bf16 h,
// FC2 writes float32 y.
//
// gfx950 design:
// * A workgroup is 4 waves on one 256-column tile and a 256-row k chunk of
//   one routed expert.  In a wave, lanes 0..31 each own 8 consecutive columns
//   (one dword per k row, so 32 lanes read one 128-byte line of the row) and
//   the two 32-lane halves own different 32-row k ranges.  All 32 dword loads
//   of a lane are issued before any decode so the weight stream has many
//   requests in flight.
// * Decode: two k rows of one dword each become K-paired bf16x2 registers by
//   bit assembly (no table); v_dot2c_f32_bf16 multiplies a K pair of
//   activations by a K pair of weights.  Products are summed per scale block
//   and the block scale is applied once per (row, column, block).
// * The bf16 weights carry a factor 2^-126 (the code bits sit at the bottom
//   of the exponent field).  The staged activations are pre-scaled by a
//   power of two P chosen per row and 32-wide k group from the group's
//   largest |a|, which keeps every product a normal float32; the group's
//   partial is multiplied back by 2^(126-P).  Power-of-two scaling commutes
//   with rounding, so this changes no result.
// * The 8 k groups of a workgroup reduce through LDS in a fixed order.  When
//   K spans several chunks (split-K) each workgroup writes g * partial to the
//   workspace and a second, small kernel sums the chunks in order and runs
//   the epilogue (the two-pass split-K SwiGLU of section 12.1).  Kernel
//   boundaries order the passes: no fences, no atomics, deterministic sums.
// * Work items (expert slot, column tile) are spread round-robin over the 8
//   XCDs and all k chunks of an item land on the same XCD.
// * The routed experts are found on the device from expert_offsets (wave
//   ballots); grids are sized for the worst case and idle slots exit.  Rows
//   of an expert are processed in passes of one or two rows.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kThreads = 256;
constexpr int kKGroups = 8;  // 4 waves x 2 halves

// Finds the expert holding the s-th non-empty row range.  Every lane gets
// the same answer; returns -1 if fewer than s+1 experts have rows.
__device__ __forceinline__ int find_slot_expert(const int32_t *__restrict__ off, int E, int s) {
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
  int found = -1;
  int run = before;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (ne[i] && run == s) found = 4 * lane + i;
    run += ne[i] ? 1 : 0;
  }
  const unsigned long long fb = __ballot(found >= 0);
  if (fb == 0ull) return -1;
  const int src = __ffsll((long long)fb) - 1;
  return __builtin_amdgcn_readlane(found, src);
}

template <int FMT>
__device__ __forceinline__ void decode_scales(uint2 sb, float (&sc)[8]) {
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

__device__ __forceinline__ float swiglu(float gate, float lin, float alpha, float beta, float limit) {
  const float G = fminf(gate, limit);
  const float L = fminf(fmaxf(lin, -limit), limit);
  return G / (1.0f + expf(-alpha * G)) * (L + beta);
}

template <int MRMAX>
struct Smem {
  uint16_t xs[MRMAX][kGemvChunkK];
  int pexp[MRMAX][kKGroups];
  float red[kKGroups][MRMAX][kGemvTileN];
};

// Decode + dot2 over the lane's 32 k rows for MR staged rows; leaves the
// group partials (already multiplied back by 2^(126-P)) in LDS.
template <int FMT, int MR, int MRMAX>
__device__ __forceinline__ void lane_dot(Smem<MRMAX> &sm, const uint32_t (&A)[kGemvLaneK], const uint2 (&SB)[2], int g,
                                         int nl) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int NBLK = kGemvLaneK / B;
  float acc[MR][8];
#pragma unroll
  for (int r = 0; r < MR; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = 0.f;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    float bs[MR][8];
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) bs[r][c] = 0.f;
#pragma unroll
    for (int kp = 0; kp < B / 2; ++kp) {
      uint32_t w[8];
      e2m1_kpair_to_bf16x2(A[b * B + 2 * kp], A[b * B + 2 * kp + 1], w);
      const int kloc = g * kGemvLaneK + b * B + 2 * kp;
#pragma unroll
      for (int r = 0; r < MR; ++r) {
        const uint32_t xp = *(const uint32_t *)&sm.xs[r][kloc];
#pragma unroll
        for (int c = 0; c < 8; ++c) bs[r][c] = dot2_bf16(xp, w[c], bs[r][c]);
      }
      // keep each K pair's decode next to its dot2s: bounds the live weights to 8 registers
      __builtin_amdgcn_sched_barrier(0);
    }
    float sc[8];
    decode_scales<FMT>(SB[b], sc);
#pragma unroll
    for (int r = 0; r < MR; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[r][c] = fmaf(sc[c], bs[r][c], acc[r][c]);
  }
#pragma unroll
  for (int r = 0; r < MR; ++r) {
    const int sh = 126 - sm.pexp[r][g];
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = ldexpf(acc[r][c], sh);
    *(float4 *)&sm.red[g][r][nl * 8] = make_float4(acc[r][0], acc[r][1], acc[r][2], acc[r][3]);
    *(float4 *)&sm.red[g][r][nl * 8 + 4] = make_float4(acc[r][4], acc[r][5], acc[r][6], acc[r][7]);
  }
}

// FC1 epilogue of one column: even threads write h[p][col/2].
__device__ __forceinline__ void store_fc1(const GemvArgs &a, int p, int col, float u) {
  const float partner = __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(u)));
  if (col < a.N && (threadIdx.x & 1) == 0)
    a.out_bf16[(size_t)p * (a.N >> 1) + (col >> 1)] = (uint16_t)bf16_rne(swiglu(u, partner, a.alpha, a.beta, a.limit));
}

template <int FMT, int MRMAX>
__global__ __launch_bounds__(kThreads) void fp4_gemv_kernel(GemvArgs a) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int NBLK = kGemvLaneK / B;
  __shared__ __attribute__((aligned(16))) Smem<MRMAX> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  // Work item: XCD-aware decode of the linear workgroup id.
  const int L = blockIdx.x;
  const int j = L >> 3;
  const int item = (j / a.nchunks) * 8 + (L & 7);
  const int kc = j % a.nchunks;
  if (item >= a.nslots * a.ntiles) return;
  const int slot = item / a.ntiles;
  const int tile = item - slot * a.ntiles;

  const int e = find_slot_expert(a.offsets, a.E, slot);
  if (e < 0) return;  // uniform over the workgroup
  const int row0 = a.offsets[e];
  const int m = a.offsets[e + 1] - row0;

  // ---- issue the weight and scale loads of this lane -----------------------
  const int nl = lane & 31;
  const int kh = lane >> 5;
  const int g = wave * 2 + kh;  // k group 0..7
  const int col0 = tile * kGemvTileN + nl * 8;
  const int klane = kc * kGemvChunkK + g * kGemvLaneK;
  const bool col_ok = col0 < a.N;
  const size_t rowbytes = (size_t)(a.N >> 1);
  const uint8_t *wp = a.w + ((size_t)e * a.K + klane) * rowbytes + (col0 >> 1);
  // Branch-free loads: rows past K (or columns past N) read row/column 0 of
  // the expert and are masked to code 0 afterwards.
  uint32_t A[kGemvLaneK];
  const uint8_t *wbase = a.w + (size_t)e * a.K * rowbytes;
#pragma unroll
  for (int i = 0; i < kGemvLaneK; ++i) {
    const bool ok = col_ok && (klane + i < a.K);
    const uint8_t *src = ok ? (wp + (size_t)i * rowbytes) : wbase;
    A[i] = __builtin_nontemporal_load((const uint32_t *)src);
    A[i] = ok ? A[i] : 0u;
  }
  uint2 SB[2] = {make_uint2(0u, 0u), make_uint2(0u, 0u)};
  const int KB = a.K / B;
#pragma unroll
  for (int b = 0; b < NBLK; ++b) {
    const int kb = klane / B + b;
    if (col_ok && klane + b * B < a.K) SB[b] = *(const uint2 *)(a.scales + ((size_t)e * KB + kb) * a.N + col0);
  }
  const float gs = a.gscale ? a.gscale[e] : 1.0f;
  const int col = tile * kGemvTileN + tid;  // column of this thread in the reduction

  // ---- passes of up to MRMAX rows ---------------------------------------------
#pragma nounroll
  for (int rbase = 0; rbase < m; rbase += MRMAX) {
    // Opaque to the optimiser: keeps the weight decode inside the pass (a
    // decode hoisted out of this loop would hold 128 registers live).
#pragma unroll
    for (int i = 0; i < kGemvLaneK; ++i) asm volatile("" : "+v"(A[i]));
    const int rem = m - rbase;
    const int mr = rem < MRMAX ? rem : MRMAX;
    // Stage mr activation rows of this k chunk, pre-scaled per (row, k group).
    {
      const int r = tid >> 5;         // up to 8 rows x 32 threads, 8 values each
      const int kk = (tid & 31) * 8;  // k offset inside the chunk
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      const int kabs = kc * kGemvChunkK + kk;
      if (r < mr && kabs < a.K) {
        const int p = row0 + rbase + r;
        const int src = a.fc1 ? (a.p2e[p] / a.topk) : p;
        v = *(const uint4 *)(a.act + (size_t)src * a.K + kabs);
      }
      uint32_t mx = 0;
      const uint32_t wv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        mx = max(mx, wv[q] & 0x7FFFu);
        mx = max(mx, (wv[q] >> 16) & 0x7FFFu);
      }
      // the 4 threads of a 32-wide k group share one exponent
      mx = max(mx, dpp_u32<kDppXor1>(mx));
      mx = max(mx, dpp_u32<kDppXor2>(mx));
      const int ef = (int)(mx >> 7);  // biased exponent of max |a| (0: zero/subnormal)
      const int P = (mx == 0u) ? 0 : 252 - (ef < 1 ? 1 : ef);
      uint32_t o[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = ldexpf(__uint_as_float(wv[q] << 16), P);
        const float hi = ldexpf(__uint_as_float(wv[q] & 0xFFFF0000u), P);
        o[q] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
      }
      if (r < MRMAX) {
        *(uint4 *)&sm.xs[r][kk] = make_uint4(o[0], o[1], o[2], o[3]);
        if ((tid & 3) == 0) sm.pexp[r][(tid & 31) >> 2] = P;
      }
    }
    __syncthreads();

    if (MRMAX == 1 || mr == 1)
      lane_dot<FMT, 1, MRMAX>(sm, A, SB, g, nl);
    else
      lane_dot<FMT, MRMAX, MRMAX>(sm, A, SB, g, nl);
    __syncthreads();

    // ---- reduce the 8 k groups (fixed order); thread = column ---------------
    for (int r = 0; r < mr; ++r) {
      float s = sm.red[0][r][tid];
#pragma unroll
      for (int q = 1; q < kKGroups; ++q) s += sm.red[q][r][tid];
      const int p = row0 + rbase + r;
      const float u = gs * s;
      if (a.nchunks > 1) {
        if (col < a.N) a.partials[((size_t)kc * a.rows + p) * a.N + col] = u;
      } else if (a.fc1) {
        store_fc1(a, p, col, u);
      } else if (col < a.N) {
        a.out_f32[(size_t)p * a.N + col] = u;
      }
    }
    __syncthreads();
  }
}

// Split-K epilogue: sums the k-chunk partials of every (row, column) in chunk
// order, then SwiGLU -> bf16 h (FC1) or float32 y (FC2).
__global__ __launch_bounds__(kThreads) void splitk_epilogue_kernel(GemvArgs a) {
  const int p = blockIdx.y;
  const int col = blockIdx.x * kThreads + threadIdx.x;
  float s = 0.f;
  if (col < a.N) {
    s = a.partials[(size_t)p * a.N + col];
    for (int q = 1; q < a.nchunks; ++q) s += a.partials[((size_t)q * a.rows + p) * a.N + col];
  }
  if (a.fc1)
    store_fc1(a, p, col, s);
  else if (col < a.N)
    a.out_f32[(size_t)p * a.N + col] = s;
}

size_t gemv_workspace_bytes(int32_t rows, int32_t E, int32_t K, int32_t N) {
  (void)E;
  const int nchunks = (K + kGemvChunkK - 1) / kGemvChunkK;
  const size_t part = nchunks > 1 ? (size_t)nchunks * rows * N * sizeof(float) : 0;
  return part > 256 ? part : 256;
}

void gemv_plan(GemvArgs &a, void *ws) {
  a.nslots = a.rows < a.E ? a.rows : a.E;
  a.ntiles = (a.N + kGemvTileN - 1) / kGemvTileN;
  a.nchunks = (a.K + kGemvChunkK - 1) / kGemvChunkK;
  a.partials = (float *)ws;
}

hipError_t launch_fp4_gemv(const GemvArgs &a, int fmt, int max_rows_per_expert, hipStream_t s) {
  const int items = a.nslots * a.ntiles;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8 * a.nchunks));
  // One row per pass when no expert can hold more than one row (one token),
  // else two: the 2-row body needs 120 VGPRs, 4 rows would need ~170.
  if (fmt == 0) {
    if (max_rows_per_expert <= 1)
      fp4_gemv_kernel<0, 1><<<grid, kThreads, 0, s>>>(a);
    else
      fp4_gemv_kernel<0, 2><<<grid, kThreads, 0, s>>>(a);
  } else {
    if (max_rows_per_expert <= 1)
      fp4_gemv_kernel<1, 1><<<grid, kThreads, 0, s>>>(a);
    else
      fp4_gemv_kernel<1, 2><<<grid, kThreads, 0, s>>>(a);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.nchunks == 1) return err;
  const dim3 g2((unsigned)((a.N + kThreads - 1) / kThreads), (unsigned)a.rows);
  splitk_epilogue_kernel<<<g2, kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qmoe
