// FP4 -> bf16 weight dequant, [E][K][N/2] -> [E][N][K], gfx950.
//
// What it computes ("[CUDA] Coalesce QMoE MXFP4/NVFP4 weight dequantization",
// PR 31349; operator documentation section 6.5):
//   out[e][n][k] = bf16_rne( f32_rne( e2m1(code) * scale(e, k/B, n) ) * g[e] )
// with E4M3 block-16 scales and a global scale for NVFP4, E8M0 block-32
// scales for MXFP4; one kernel serves both codecs.
//
// gfx950 layout: a workgroup covers 64 k x 256 n of one expert.  Thread t
// owns 8 k (a 16-byte output segment) of 8 columns: ks = t % 8 picks the k
// segment, cg = t / 8 the column group.  It loads the 8 packed dwords
// (8 k rows x 8 columns), transposes them in registers and writes 8 stores
// of 16 bytes; the 8 threads sharing a column group write one contiguous
// 128-byte output row segment per store.  The block-scale byte of each
// (column, 8-k segment) is read once.  The grid is (K/64, N/256, E): all
// index arithmetic is grid arithmetic, no integer division.  Stores are
// non-temporal (the output is written once and not re-read here).
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

template <int FMT>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ s,
                                                      const float *__restrict__ g, int K, int N,
                                                      uint16_t *__restrict__ out) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  const int e = blockIdx.z;
  const int ks = threadIdx.x & 7;
  const int cg = threadIdx.x >> 3;
  const int k0 = blockIdx.x * 64 + ks * 8;
  const int n0 = blockIdx.y * 256 + cg * 8;
  const size_t rowbytes = (size_t)(N >> 1);
  const uint8_t *wp = w + ((size_t)e * K + k0) * rowbytes + (n0 >> 1);
  uint32_t A[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) A[i] = __builtin_nontemporal_load((const uint32_t *)(wp + (size_t)i * rowbytes));
  const uint2 sb = *(const uint2 *)(s + ((size_t)e * (K / B) + k0 / B) * N + n0);
  const bool has_g = g != nullptr;
  const float gs = has_g ? g[e] : 1.0f;
  uint16_t *op = out + ((size_t)e * N + n0) * K + k0;
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sbyte = ((c < 4 ? sb.x : sb.y) >> (8 * (c & 3))) & 0xFFu;
    float sf;
    if constexpr (FMT == 0)
      sf = __builtin_amdgcn_cvt_f32_fp8((int)sbyte, 0);
    else
      sf = e8m0_to_f32(sbyte);
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float v = e2m1_to_f32(A[i] >> (4 * c)) * sf;  // exact
      if (has_g) v *= gs;                           // one float32 rounding
      h[i] = bf16_rne(v);
    }
    u32x4_t o;
    o.x = h[0] | (h[1] << 16);
    o.y = h[2] | (h[3] << 16);
    o.z = h[4] | (h[5] << 16);
    o.w = h[6] | (h[7] << 16);
    __builtin_nontemporal_store(o, (u32x4_t *)(op + (size_t)c * K));
  }
}

hipError_t launch_dequant(const uint8_t *w, const uint8_t *scales, const float *g, int32_t E, int32_t K, int32_t N,
                          int fmt, uint16_t *out, hipStream_t s) {
  const dim3 grid((unsigned)(K / 64), (unsigned)(N / 256), (unsigned)E);
  if (fmt == 0)
    dequant_kernel<0><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
  else
    dequant_kernel<1><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
  return hipGetLastError();
}

}  // namespace qmoe
