// Weighted un-permute (finalize) for gfx950.
//
// out[t][n] = bf16_rne( sum_{j<k} w[t][j] * y[e2p[t*k+j]][n] ), j ascending,
// float32 (operator documentation section 1; PR 31156: the routing metadata
// of a token is read once per workgroup so the k row loads are independent,
// and the columns are split over many workgroups).
//
// One thread owns 8 consecutive columns: two 16-byte loads per expanded row
// and one 16-byte bf16 store.  The token's k row indices and weights are
// uniform across the workgroup and live in scalar registers.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

template <int KMAX>
__global__ __launch_bounds__(256) void finalize_kernel(const float *__restrict__ y, const float *__restrict__ w,
                                                       const int32_t *__restrict__ e2p, int k, int H,
                                                       uint16_t *__restrict__ out) {
  const int t = blockIdx.y;
  const int col = (blockIdx.x * 256 + threadIdx.x) * 8;
  int rows[KMAX];
  float wt[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    rows[j] = (j < k) ? e2p[(size_t)t * k + j] : 0;
    wt[j] = (j < k) ? w[(size_t)t * k + j] : 0.f;
  }
  if (col >= H) return;
  float4 v0[KMAX], v1[KMAX];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      const float *src = y + (size_t)rows[j] * H + col;
      v0[j] = *(const float4 *)src;
      v1[j] = *(const float4 *)(src + 4);
    }
  }
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    if (j < k) {
      acc[0] = fmaf(wt[j], v0[j].x, acc[0]);
      acc[1] = fmaf(wt[j], v0[j].y, acc[1]);
      acc[2] = fmaf(wt[j], v0[j].z, acc[2]);
      acc[3] = fmaf(wt[j], v0[j].w, acc[3]);
      acc[4] = fmaf(wt[j], v1[j].x, acc[4]);
      acc[5] = fmaf(wt[j], v1[j].y, acc[5]);
      acc[6] = fmaf(wt[j], v1[j].z, acc[6]);
      acc[7] = fmaf(wt[j], v1[j].w, acc[7]);
    }
  }
  uint4 o;
  o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
  o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
  o.z = bf16_rne(acc[4]) | (bf16_rne(acc[5]) << 16);
  o.w = bf16_rne(acc[6]) | (bf16_rne(acc[7]) << 16);
  *(uint4 *)(out + (size_t)t * H + col) = o;
}

hipError_t launch_finalize(const float *y, const float *w, const int32_t *e2p, int32_t T, int32_t k, int32_t H,
                           uint16_t *out, hipStream_t s) {
  const dim3 grid((unsigned)((H / 8 + 255) / 256), (unsigned)T);
  finalize_kernel<8><<<grid, 256, 0, s>>>(y, w, e2p, k, H, out);
  return hipGetLastError();
}

}  // namespace qmoe
