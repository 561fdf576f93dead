// Weighted un-permute (finalize) for gfx950.
//
// out[t][n] = bf16_rne( sum_{j<k} w[t][j] * y[e2p[t*k+j]][n] ), j ascending,
// float32 (operator documentation section 1; PR 31156: the routing metadata
// of a token is read once per workgroup so the k row loads are independent,
// and the columns are split over many workgroups).
//
// One thread owns 4 consecutive columns, one wave 256 columns of one token:
// T x H/256 waves, so a decode step's few tokens still spread over many CUs.
// The token's k row indices and weights are uniform across the wave and live
// in scalar registers; the loads of up to kPlaneGroup split-K planes for all
// k rows are issued together before any is summed.  k is a template
// argument (1..8), so no load sits behind a branch.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kPlaneGroup = 4;

// Adds G consecutive split-K planes, starting at plane c, to the k rows'
// running sums.  Every load is unconditional (the counts are template
// arguments), so all G*K loads are in flight before the first add.
template <int K, int G>
__device__ __forceinline__ void add_planes(const float *__restrict__ y, size_t plane, int c, const int (&rows)[K],
                                           int H, int col, float4 (&v)[K]) {
  float4 a[G][K];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < K; ++j)
      a[g][j] = *(const float4 *)(y + (size_t)(c + g) * plane + (size_t)rows[j] * H + col);
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int j = 0; j < K; ++j) {
      v[j].x += a[g][j].x;
      v[j].y += a[g][j].y;
      v[j].z += a[g][j].z;
      v[j].w += a[g][j].w;
    }
}

// y holds nsplit planes of [rows][H] partial sums (nsplit = 1: the rows
// themselves); a routed row's value is the planes' sum in plane order, the
// same float32 additions the split-K epilogue of FC2 performs (starting from
// -0 so that the first plane passes through unchanged, signed zeros included).
template <int K>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(1, 2))) void finalize_kernel(const float *__restrict__ y, int nsplit, size_t plane,
                                                      const float *__restrict__ w, const int32_t *__restrict__ e2p,
                                                      int H, uint16_t *__restrict__ out) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * 64 + threadIdx.x) * 4;
  int rows[K];
  float wt[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    rows[j] = e2p[(size_t)t * K + j];
    wt[j] = w[(size_t)t * K + j];
  }
  if (col >= H) return;
  float4 v[K];
#pragma unroll
  for (int j = 0; j < K; ++j) v[j] = make_float4(-0.f, -0.f, -0.f, -0.f);
  int c = 0;
  for (; c + kPlaneGroup <= nsplit; c += kPlaneGroup) add_planes<K, kPlaneGroup>(y, plane, c, rows, H, col, v);
  switch (nsplit - c) {
    case 3:
      add_planes<K, 3>(y, plane, c, rows, H, col, v);
      break;
    case 2:
      add_planes<K, 2>(y, plane, c, rows, H, col, v);
      break;
    case 1:
      add_planes<K, 1>(y, plane, c, rows, H, col, v);
      break;
    default:
      break;
  }
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < K; ++j) {
    acc[0] = fmaf(wt[j], v[j].x, acc[0]);
    acc[1] = fmaf(wt[j], v[j].y, acc[1]);
    acc[2] = fmaf(wt[j], v[j].z, acc[2]);
    acc[3] = fmaf(wt[j], v[j].w, acc[3]);
  }
  uint2 o;
  o.x = bf16_rne(acc[0]) | (bf16_rne(acc[1]) << 16);
  o.y = bf16_rne(acc[2]) | (bf16_rne(acc[3]) << 16);
  *(uint2 *)(out + (size_t)t * H + col) = o;
}

hipError_t launch_finalize(const float *y, int nsplit, size_t plane, const float *w, const int32_t *e2p, int32_t T,
                           int32_t k, int32_t H, uint16_t *out, hipStream_t s) {
  const dim3 grid((unsigned)T, (unsigned)((H / 4 + 63) / 64));
  switch (k) {
#define QMOE_FINALIZE_CASE(KK) \
  case KK:                     \
    finalize_kernel<KK><<<grid, 64, 0, s>>>(y, nsplit, plane, w, e2p, H, out); \
    break;
    QMOE_FINALIZE_CASE(1)
    QMOE_FINALIZE_CASE(2)
    QMOE_FINALIZE_CASE(3)
    QMOE_FINALIZE_CASE(4)
    QMOE_FINALIZE_CASE(5)
    QMOE_FINALIZE_CASE(6)
    QMOE_FINALIZE_CASE(7)
    QMOE_FINALIZE_CASE(8)
#undef QMOE_FINALIZE_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace qmoe
