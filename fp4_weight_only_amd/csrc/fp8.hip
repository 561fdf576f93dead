// FP8 E4M3 weight-only (W8A16) decode GEMV and dequant for gfx950.
//
// Weights are raw E4M3FN bytes laid out [E][N][K] (each output column's K
// weights contiguous) with one float32 global scale per expert and no block
// scales ("MoE and QMoE -- CUDA Operator Documentation", sections 6.4 and
// 10: the product is scaled by the expert's global scale in the epilogue).
//
// GEMV: a column's K bytes are contiguous, so 16 lanes (one DPP row) share a
// column and each lane loads 16 consecutive k with one 16-byte load.  A lane
// row covers CPR columns (1 for K >= 1536, 2 for K >= 768, else 4, so a lane
// keeps up to 8 loads in flight even for short K), a wave 4 * CPR columns, a
// workgroup of 8 waves 32 * CPR, over the whole K in passes (8 loads per lane
// per pass): there is no split-K and no second launch.  Rows go in passes of
// up to 8 per workgroup, so any batch works; a prefill batch re-reads an
// expert's columns (from L2) once per 8 rows.
// The hardware FP8 -> bf16 conversion is exact; the k pairs meet the
// activation pairs in dot2 instructions.  The 16 per-lane partial sums of a
// column are added with a symmetric DPP butterfly inside the row, which
// leaves the same value in all 16 lanes.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kF8Waves = 8;
constexpr int kF8Loads = 8;                          // 16-byte loads per lane per pass
constexpr int kF8PassK = 16 * 16 * kF8Loads;         // 2048 k per pass (CPR = 1)
constexpr int kF8TileN1 = kF8Waves * 4;              // 32 columns per workgroup and column per lane row
constexpr uint32_t kF8OutOfRange = 0x80000000u;

__device__ __forceinline__ float row16_sum(float v) {
  auto add = [](float x, uint32_t y) { return x + __uint_as_float(y); };
  v = add(v, dpp_u32<kDppXor1>(__float_as_uint(v)));
  v = add(v, dpp_u32<kDppXor2>(__float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowHalfMirror>(__float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowMirror>(__float_as_uint(v)));
  return v;
}

__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true));
}

template <int MRMAX, int CPR>
__global__ __launch_bounds__(kF8Waves * 64) void fp8_gemv_kernel(GemvArgs a) {
  constexpr int PASSK = kF8PassK / CPR;       // k per pass: CPR columns x PASSK / 256 loads per lane
  constexpr int NLD = PASSK / 256;
  __shared__ __attribute__((aligned(16))) uint16_t xs[MRMAX][PASSK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  // Work item: consecutive column tiles of one slot on one XCD (its
  // activation rows stay in that XCD's L2; the expert's columns are
  // contiguous in memory).
  const int per = gridDim.x >> 3;
  const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (item >= a.nslots * a.ntiles) return;
  const int slot = item / a.ntiles;
  const int tile = item - slot * a.ntiles;

  int row0 = 0, m = 0;
  const int e = find_slot_expert(a.offsets, a.E, slot, row0, m);
  if (e < 0) return;  // uniform over the workgroup

  // lane row rr of the wave takes columns base + 4 j + rr (j < CPR): an
  // interleaved gate / linear pair sits in lane rows 2i, 2i+1 for every j
  const int col0 = (tile * kF8Waves + wave) * 4 * CPR + (lane >> 4);
  const int q = lane & 15;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.w + (size_t)e * a.N * a.K), (short)0, (int)((uint32_t)a.N * (uint32_t)a.K), 0x00020000);
  const float gs = a.gscale[e];

#pragma nounroll
  for (int rbase = 0; rbase < m; rbase += MRMAX) {
    const int rem = m - rbase;
    const int mr = rem < MRMAX ? rem : MRMAX;
    float acc[CPR][MRMAX];
#pragma unroll
    for (int j = 0; j < CPR; ++j)
#pragma unroll
      for (int r = 0; r < MRMAX; ++r) acc[j][r] = 0.f;

#pragma nounroll
    for (int k0 = 0; k0 < a.K; k0 += PASSK) {
      // activation rows of the pass first (memory returns in issue order),
      // then this lane's weight bytes
      const int kx = k0 + tid * 8;
      u32x4_t xv[MRMAX];
#pragma unroll
      for (int r = 0; r < MRMAX; ++r) {
        const int p = row0 + rbase + r;
        xv[r] = u32x4_t{0u, 0u, 0u, 0u};
        if (r < mr && tid * 8 < PASSK && kx < a.K) {
          const int src = a.fc1 ? a.p2e[p] / a.topk : p;  // FC1 gathers x rows by token
          xv[r] = *(const u32x4_t *)(a.act + (size_t)src * a.K + kx);
        }
      }
      u32x4_t W[CPR][NLD];
#pragma unroll
      for (int j = 0; j < CPR; ++j)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int col = col0 + 4 * j;
          const int kk = k0 + i * 256 + q * 16;
          const uint32_t voff =
              (col < a.N && kk < a.K) ? (uint32_t)col * (uint32_t)a.K + (uint32_t)kk : kF8OutOfRange;
          W[j][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, 0, 2));
        }
      if (tid * 8 < PASSK) {
#pragma unroll
        for (int r = 0; r < MRMAX; ++r) *(u32x4_t *)&xs[r][tid * 8] = xv[r];
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
          uint32_t w2[8];
          w2[0] = fp8x2_lo(W[j][i].x);
          w2[1] = fp8x2_hi(W[j][i].x);
          w2[2] = fp8x2_lo(W[j][i].y);
          w2[3] = fp8x2_hi(W[j][i].y);
          w2[4] = fp8x2_lo(W[j][i].z);
          w2[5] = fp8x2_hi(W[j][i].z);
          w2[6] = fp8x2_lo(W[j][i].w);
          w2[7] = fp8x2_hi(W[j][i].w);
#pragma unroll
          for (int r = 0; r < MRMAX; ++r) {
            if (MRMAX > 1 && r >= mr) break;  // uniform
            const u32x4_t x0 = *(const u32x4_t *)&xs[r][i * 256 + q * 16];
            const u32x4_t x1 = *(const u32x4_t *)&xs[r][i * 256 + q * 16 + 8];
            float v = acc[j][r];
            v = dot2_bf16(x0.x, w2[0], v);
            v = dot2_bf16(x0.y, w2[1], v);
            v = dot2_bf16(x0.z, w2[2], v);
            v = dot2_bf16(x0.w, w2[3], v);
            v = dot2_bf16(x1.x, w2[4], v);
            v = dot2_bf16(x1.y, w2[5], v);
            v = dot2_bf16(x1.z, w2[6], v);
            v = dot2_bf16(x1.w, w2[7], v);
            acc[j][r] = v;
          }
        }
      }
      lds_barrier();  // the next pass overwrites xs
    }

    // column sums, global scale, outputs
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      const int col = col0 + 4 * j;
      const bool col_ok = col < a.N;
#pragma unroll
      for (int r = 0; r < MRMAX; ++r) {
        if (MRMAX > 1 && r >= mr) break;  // uniform
        const float u = gs * row16_sum(acc[j][r]);
        const int p = row0 + rbase + r;
        if (a.fc1 && !a.concat) {
          // gate (even) columns in lane rows 0 / 2 meet their linear values
          // in lane rows 1 / 3
          const float partner = __shfl_xor(u, 16, 64);
          if (q == 0 && ((lane >> 4) & 1) == 0 && col_ok)
            a.out_bf16[(size_t)p * (a.N >> 1) + (col >> 1)] =
                (uint16_t)bf16_rne(swiglu(u, partner, a.alpha, a.beta, a.limit));
        } else if (q == 0 && col_ok) {
          a.out_f32[(size_t)p * a.N + col] = u;  // FC2 y, or FC1 u for the concatenated layout
        }
      }
    }
  }
}

size_t fp8_workspace_bytes(int32_t rows, int32_t N, bool concat) {
  const size_t u = concat ? (size_t)rows * N * sizeof(float) : 0;
  return u > 256 ? u : 256;
}

hipError_t launch_fp8_gemv(GemvArgs &a, int max_rows_per_expert, void *ws, hipStream_t s) {
  const int cpr = a.K >= 1536 ? 1 : (a.K >= 768 ? 2 : 4);
  a.nslots = a.rows < a.E ? a.rows : a.E;
  a.ntiles = (a.N + kF8TileN1 * cpr - 1) / (kF8TileN1 * cpr);
  const int items = a.nslots * a.ntiles;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));
  const dim3 block(kF8Waves * 64);
  if (a.concat) a.out_f32 = (float *)ws;
  const int mr = max_rows_per_expert <= 1 ? 1 : (max_rows_per_expert <= 4 ? 4 : 8);
#define QMOE_F8_LAUNCH(MR)                                                   \
  if (cpr == 1)                                                              \
    fp8_gemv_kernel<MR, 1><<<grid, block, 0, s>>>(a);                        \
  else if (cpr == 2)                                                         \
    fp8_gemv_kernel<MR, 2><<<grid, block, 0, s>>>(a);                        \
  else                                                                       \
    fp8_gemv_kernel<MR, 4><<<grid, block, 0, s>>>(a);
  if (mr == 1) {
    QMOE_F8_LAUNCH(1)
  } else if (mr == 4) {
    QMOE_F8_LAUNCH(4)
  } else {
    QMOE_F8_LAUNCH(8)
  }
#undef QMOE_F8_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !a.concat) return err;
  a.partials = (float *)ws;
  a.nchunks = 1;
  return launch_splitk_epilogue(a, s);
}

// Dequant: out[e][n][k] = bf16(float32(e4m3(w[e][n][k]) * g[e])), the same
// [E][N][K] layout as the input, so a thread converts 16 consecutive bytes
// into 32 consecutive output bytes.
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint8_t *__restrict__ w,
                                                          const float *__restrict__ g, size_t per_expert,
                                                          uint16_t *__restrict__ out) {
  const int e = blockIdx.y;
  const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 16;
  if (i >= per_expert) return;
  const float ge = g[e];
  const size_t off = (size_t)e * per_expert + i;
  const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)(w + off));
  const uint32_t vs[4] = {v.x, v.y, v.z, v.w};
  uint32_t o[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vs[j], 1.0f, false);
    const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vs[j], 1.0f, true);
    o[2 * j] = pack_bf16x2_rne(lo.x * ge, lo.y * ge);
    o[2 * j + 1] = pack_bf16x2_rne(hi.x * ge, hi.y * ge);
  }
  u32x4_t* dst = (u32x4_t *)(out + off);
  __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, dst);
  __builtin_nontemporal_store(u32x4_t{o[4], o[5], o[6], o[7]}, dst + 1);
}

hipError_t launch_fp8_dequant(const uint8_t *w, const float *g, int32_t E, int32_t K, int32_t N, uint16_t *out,
                              hipStream_t s) {
  const size_t per = (size_t)N * K;
  const dim3 grid((unsigned)((per / 16 + 255) / 256), (unsigned)E);
  fp8_dequant_kernel<<<grid, 256, 0, s>>>(w, g, per, out);
  return hipGetLastError();
}

}  // namespace qmoe
