// Prefill path: grouped GEMM over routed rows with bf16 MFMA, FP4 weights
// dequantised into LDS tiles, gfx950.
//
// What it computes (operator documentation section 4.3, the dequant-to-A16
// path for shapes outside the decode GEMV; section 9b.1/9b.5, prefill-sized
// batches go to a grouped GEMM): for every routed row p of expert e,
//   u[p][n] = g[e] * sum_k a[p][k] * (e2m1(code[e][k][n]) * scale[e][k/B][n])
// FC1: a = x[token(p)], then interleaved SwiGLU -> bf16 h.  FC2: a = h[p],
// float32 y.  Same outputs as the decode GEMV.
//
// gfx950 design:
// * Work item = (expert, 64-row m tile, 128-column n tile); a workgroup of 4
//   waves (2 x 2) computes 64 x 128 with v_mfma_f32_16x16x32_bf16, each wave
//   32 rows x 64 columns (2 x 4 MFMA tiles, 32 float32 accumulators).
// * The k loop steps 64 rows.  Per step the activation tile (64 rows x 64 k,
//   rows gathered through the permutation for FC1) and the packed weight
//   tile (64 k x 128 columns, 4 KB) are loaded to registers one step ahead,
//   then written to a double-buffered LDS tile; the weight tile is
//   dequantised on the way into LDS, stored transposed ([n][k]) so each lane
//   reads its MFMA operand (8 consecutive k of one column) as one 16-byte
//   read.  One barrier per step.
// * Dequant: the product code * block scale is exact in bf16 (2 significant
//   bits times a power of two, or times E4M3's 4 bits), so the MFMA operand
//   is the exact weight without the global scale; g is applied to the float32
//   accumulator in the epilogue.  MXFP4 tiles use the gfx950 scaled FP4->bf16
//   conversion (the scale's exponent is the E8M0 block scale), one per column
//   per K pair, plus one byte permute to pair k and k+1.  NVFP4 tiles are
//   dequantised through float32 (code value times the E4M3 scale).
// * 16-row MFMA sub-tiles with no routed rows are skipped, so a small expert
//   costs one 16-row MFMA tile, not 64.
// * Work items: the (expert, m tile) list is found on the device from
//   expert_offsets; the grid covers the worst case (rows/64 + experts tiles)
//   and idle items exit.  The m tiles of one expert for one n tile land on
//   the same XCD, so repeated weight tiles of hot experts meet in one L2.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kBM = 64, kBN = 128, kBK = 64;
constexpr int kLdA = kBK + 8;  // bf16 per LDS row of the activation tile (padding against bank conflicts)
constexpr int kLdB = kBK + 8;  // bf16 per LDS row of the transposed weight tile (16-byte aligned rows)

struct GroupedSmem {
  uint16_t a[2][kBM][kLdA];
  uint16_t b[2][kBN][kLdB];
};

// Finds the s-th (expert, m tile) item: experts in ascending order, each with
// ceil(rows/64) tiles.  Returns the expert (-1 past the last item) and the
// tile index inside it.  Every lane gets the same answer.
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
    cnt[i] = (4 * lane + i < E) ? (o[i + 1] - o[i] + kBM - 1) / kBM : 0;
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

__device__ __forceinline__ float grouped_swiglu(float gate, float lin, float alpha, float beta, float limit) {
  const float G = fminf(gate, limit);
  const float L = fminf(fmaxf(lin, -limit), limit);
  return G / (1.0f + expf(-alpha * G)) * (L + beta);
}

// Dequantises 16 columns x one K pair (rows k, k+1 as two 8-byte words) into
// 16 bf16x2 registers: column c as {lo: w(k, c), hi: w(k+1, c)}.
template <int FMT>
__device__ __forceinline__ void dequant_kpair16(u32x2_t r0, u32x2_t r1, u32x4_t sb, uint32_t (&out)[16]) {
#pragma unroll
  for (int c = 0; c < 16; ++c) {
    const uint32_t sbyte = (sb[c >> 2] >> (8 * (c & 3))) & 0xFFu;
    const int wd = c >> 3;          // dword holding column c
    const int byte = (c >> 1) & 3;  // byte inside it
    if constexpr (FMT == 1) {
      const float sf = e8m0_to_f32(sbyte);
      // two codes -> two bf16 per conversion; keep the half of column c
      uint32_t p0, p1;
      switch (byte) {
        case 0:
          p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r0[wd], sf, 0));
          p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r1[wd], sf, 0));
          break;
        case 1:
          p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r0[wd], sf, 1));
          p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r1[wd], sf, 1));
          break;
        case 2:
          p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r0[wd], sf, 2));
          p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r1[wd], sf, 2));
          break;
        default:
          p0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r0[wd], sf, 3));
          p1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(r1[wd], sf, 3));
          break;
      }
      // bytes of {p1, p0}: take half (c & 1) of each
      const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
      out[c] = __builtin_amdgcn_perm(p1, p0, sel);
    } else {
      const float sf = __builtin_amdgcn_cvt_f32_fp8((int)sbyte, 0);
      const float v0 = e2m1_to_f32(r0[wd] >> (4 * (c & 7))) * sf;  // exact
      const float v1 = e2m1_to_f32(r1[wd] >> (4 * (c & 7))) * sf;
      out[c] = (__float_as_uint(v0) >> 16) | (__float_as_uint(v1) & 0xFFFF0000u);
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void grouped_gemm_kernel(GemvArgs a) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  __shared__ __attribute__((aligned(16))) GroupedSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  // XCD-aware decode: consecutive logical items share an XCD.
  const int G = gridDim.x;
  const int per = G >> 3;
  const int q = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
  const int ntile = q / a.nslots;
  const int slot = q - ntile * a.nslots;
  if (ntile >= a.ntiles) return;
  int mt = 0;
  const int e = find_mtile(a.offsets, a.E, slot, mt);
  if (e < 0) return;  // uniform over the workgroup
  const int row0 = a.offsets[e] + mt * kBM;
  const int mrows = min(kBM, a.offsets[e + 1] - row0);
  const int n0 = ntile * kBN;

  // ---- loader roles ----------------------------------------------------------
  // activation tile: thread -> (row, 16 k)
  const int ar = tid >> 2;
  const int ak = (tid & 3) * 16;
  const uint16_t *arow = nullptr;
  if (ar < mrows) {
    const int p = row0 + ar;
    const int src = a.fc1 ? (a.p2e[p] / a.topk) : p;
    arow = a.act + (size_t)src * a.K;
  }
  // weight tile: thread -> (K pair kp, 16 columns cg*16)
  const int cg = tid >> 5;  // 0..7
  const int kp = tid & 31;  // 0..31
  const uint32_t rowbytes = (uint32_t)(a.N >> 1);
  const int KB = a.K / B;
  const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.w + (size_t)e * a.K * rowbytes), (short)0, (int)((uint32_t)a.K * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void *)(a.scales + (size_t)e * KB * a.N), (short)0, (int)((uint32_t)KB * a.N), 0x00020000);
  const int bcol = n0 + cg * 16;
  const uint32_t woff = (uint32_t)(2 * kp) * rowbytes + (uint32_t)(bcol >> 1);

  u32x4_t ra0, ra1;
  u32x2_t rb0, rb1;
  u32x4_t rs;
  auto load_step = [&](int k0) {
    if (arow) {
      ra0 = *(const u32x4_t *)(arow + k0 + ak);
      ra1 = *(const u32x4_t *)(arow + k0 + ak + 8);
    } else {
      ra0 = u32x4_t{0u, 0u, 0u, 0u};
      ra1 = ra0;
    }
    const uint32_t o = woff + (uint32_t)k0 * rowbytes;
    rb0 = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, o, 0, 2);
    rb1 = __builtin_amdgcn_raw_buffer_load_b64(wrsrc, o + rowbytes, 0, 2);
    rs = __builtin_amdgcn_raw_buffer_load_b128(srsrc, (uint32_t)((k0 + 2 * kp) / B) * (uint32_t)a.N + (uint32_t)bcol, 0, 0);
  };
  auto store_step = [&](int buf) {
    *(u32x4_t *)&sm.a[buf][ar][ak] = ra0;
    *(u32x4_t *)&sm.a[buf][ar][ak + 8] = ra1;
    uint32_t d[16];
    dequant_kpair16<FMT>(rb0, rb1, rs, d);
#pragma unroll
    for (int c = 0; c < 16; ++c) *(uint32_t *)&sm.b[buf][cg * 16 + c][2 * kp] = d[c];
  };

  // ---- MFMA roles: wave (wr, wc) computes rows wr*32.., columns wc*64.. ------
  const int wr = wave >> 1;
  const int wc = wave & 1;
  const int li = lane & 15;
  const int lk = (lane >> 4) * 8;
  const bool sub_live[2] = {wr * 32 < mrows, wr * 32 + 16 < mrows};
  f32x4_t acc[2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int steps = a.K / kBK;
  load_step(0);
  for (int s = 0; s < steps; ++s) {
    const int buf = s & 1;
    store_step(buf);
    __syncthreads();
    if (s + 1 < steps) load_step((s + 1) * kBK);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 32) {
      bf16x8_t bv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bv[j] = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)&sm.b[buf][wc * 64 + j * 16 + li][kk + lk]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if (!sub_live[i]) continue;  // wave-uniform
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, *(const u32x4_t *)&sm.a[buf][wr * 32 + i * 16 + li][kk + lk]);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[j], acc[i][j], 0, 0, 0);
      }
    }
  }

  // ---- epilogue: lane holds rows 4*(lane/16)+q, column lane%16 of each tile --
  const float gs = a.gscale ? a.gscale[e] : 1.0f;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (!sub_live[i]) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wc * 64 + j * 16 + li;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const int r = wr * 32 + i * 16 + (lane >> 4) * 4 + qd;
        const float u = gs * acc[i][j][qd];
        if (a.fc1) {
          const float partner = __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(u)));
          if (r < mrows && (lane & 1) == 0)
            a.out_bf16[(size_t)(row0 + r) * (a.N >> 1) + (col >> 1)] =
                (uint16_t)bf16_rne(grouped_swiglu(u, partner, a.alpha, a.beta, a.limit));
        } else if (r < mrows) {
          a.out_f32[(size_t)(row0 + r) * a.N + col] = u;
        }
      }
    }
  }
}

size_t grouped_workspace_bytes() { return 256; }

hipError_t launch_grouped(GemvArgs &a, int fmt, hipStream_t s) {
  const int erows = a.rows < a.E ? a.rows : a.E;
  a.nslots = (a.rows + kBM - 1) / kBM + erows;  // worst-case (expert, m tile) count
  a.ntiles = a.N / kBN;
  const int items = a.nslots * a.ntiles;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));
  if (fmt == 0)
    grouped_gemm_kernel<0><<<grid, 256, 0, s>>>(a);
  else
    grouped_gemm_kernel<1><<<grid, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qmoe
