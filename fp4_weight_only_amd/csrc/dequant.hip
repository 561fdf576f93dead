// FP4 -> bf16 weight dequant, [E][K][N/2] -> [E][N][K], gfx950.
//
// What it computes ("[CUDA] Coalesce QMoE MXFP4/NVFP4 weight dequantization",
// PR 31349; operator documentation section 6.5):
//   out[e][n][k] = bf16_rne( f32_rne( e2m1(code) * scale(e, k/B, n) ) * g[e] )
// with E4M3 block-16 scales and a global scale for NVFP4, E8M0 block-32
// scales for MXFP4; one kernel serves both codecs.
//
// gfx950 layout: a workgroup covers KT k rows of one expert (128 when K
// allows); a thread owns 8 k rows (a 16-byte output segment per column) of
// CW consecutive columns, loading CW/2 bytes of each of its 8 packed rows.
// The KT/8 threads sharing a column block write KT/8 * 16 contiguous bytes
// of each output row per store.  The block-scale bytes of each (column,
// 8-k segment) are read once.  The grid is (K/KT, N/NT, E): all index
// arithmetic is grid arithmetic, no integer division.  Stores are
// non-temporal (the output is written once and not re-read here).
//
// Transpose and decode in one step: a nibble zip puts one column's codes of
// rows k and k+1 into one byte, and gfx950's FP4 conversions turn that byte
// into the (k, k+1) pair of the output row.  MXFP4 without a global scale
// converts straight to bf16 with the block scale as the conversion's
// exponent (exact); otherwise the conversion yields float32 codes, the block
// scale multiplies exactly, the global scale rounds once, and the hardware
// float32 -> bf16 pack rounds to nearest even.
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {


// One output column c (8 consecutive k) of a thread: z holds the nibble-
// zipped row pairs (0,1), (2,3), (4,5), (6,7); byte c/2 of the even (c even)
// or odd (c odd) words holds that column's two codes of each pair.
template <int C, int FMT, bool POW2>
__device__ __forceinline__ u32x4_t dequant_col(const uint32_t (&ev)[4], const uint32_t (&od)[4], uint32_t sbyte,
                                               float gs, bool has_g) {
  constexpr int J = C >> 1;
  u32x4_t o;
  if constexpr (POW2) {
    // E8M0 without a global scale: the output is bf16_rne(code * 2^(b-127)),
    // which the scaled FP4 -> bf16 conversion computes for every byte: it
    // takes the scale operand's exponent field as an E8M0 value (field 0 is
    // 2^-127, giving bf16 subnormals; 255 is NaN; past bf16's range +-inf),
    // checked for all 256 bytes x 16 codes.
    const float sc = __uint_as_float(sbyte << 23);
#pragma unroll
    for (int q = 0; q < 4; ++q)
      o[q] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4((C & 1) ? od[q] : ev[q], sc, J));
    return o;
  }
  float sf;
  if constexpr (FMT == 0)
    sf = __builtin_amdgcn_cvt_f32_fp8((int)sbyte, 0);
  else
    sf = e8m0_to_f32(sbyte);
  const bool nan = sf != sf;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    f32x2_t f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4((C & 1) ? od[q] : ev[q], 1.0f, J);
    if (!has_g) {
      f.x *= sf;  // exact: 2 x 4 significant bits, or times a power of two
      f.y *= sf;
    } else {
      // One float32 rounding of code * scale * g.  An E4M3 scale and an E8M0
      // scale below 2^1 keep code * scale exact, so it goes first; a larger
      // E8M0 scale (a power of two) goes last, where it is exact too but
      // code * scale alone could overflow before g brings it back in range.
      const bool big = FMT == 1 && sbyte >= 128u;
      const float m1 = big ? gs : sf;
      const float m2 = big ? sf : gs;
      f.x = (f.x * m1) * m2;
      f.y = (f.y * m1) * m2;
    }
    if (!nan)
      o[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));  // round to nearest even
    else
      o[q] = bf16_rne(f.x) | (bf16_rne(f.y) << 16);
  }
  return o;
}

// KT k rows per workgroup; a thread owns 8 k rows of CW columns (CW/8
// packed dwords per row, CW/8 groups of 8 output columns).  KT/8 threads
// share a column block and together write KT/8 * 16 contiguous bytes of
// each output row.
template <int FMT, bool POW2, int KT, int CW>
__global__ __launch_bounds__(256) void dequant_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ s,
                                                      const float *__restrict__ g, int K, int N,
                                                      uint16_t *__restrict__ out) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int KS = KT / 8;          // threads along k
  constexpr int NT = CW * 256 / KS;  // columns per workgroup
  constexpr int D = CW / 8;           // packed dwords per row and thread
  const int e = blockIdx.z;
  const int ks = threadIdx.x % KS;
  const int cb = threadIdx.x / KS;
  const int k0 = blockIdx.x * KT + ks * 8;
  const int n0 = blockIdx.y * NT + cb * CW;
  const size_t rowbytes = (size_t)(N >> 1);
  const uint8_t *wp = w + ((size_t)e * K + k0) * rowbytes + (n0 >> 1);
  uint32_t A[8][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint8_t *rp = wp + (size_t)i * rowbytes;
    if constexpr (D == 1) {
      A[i][0] = __builtin_nontemporal_load((const uint32_t *)rp);
    } else if constexpr (D == 2) {
      const u32x2_t v = __builtin_nontemporal_load((const u32x2_t *)rp);
      A[i][0] = v.x;
      A[i][1] = v.y;
    } else {
#pragma unroll
      for (int j = 0; j < D; j += 4) {
        const u32x4_t v = __builtin_nontemporal_load((const u32x4_t *)rp + j / 4);
        A[i][j] = v.x;
        A[i][j + 1] = v.y;
        A[i][j + 2] = v.z;
        A[i][j + 3] = v.w;
      }
    }
  }
  const uint8_t *sp = s + ((size_t)e * (K / B) + k0 / B) * N + n0;
  uint32_t S[2 * D];
#pragma unroll
  for (int j = 0; j < 2 * D; j += 2) {
    const uint2 v = *(const uint2 *)(sp + 4 * j);
    S[j] = v.x;
    S[j + 1] = v.y;
  }
  const bool has_g = g != nullptr;
  const float gs = has_g ? g[e] : 1.0f;
#pragma unroll
  for (int j = 0; j < D; ++j) {
    // Nibble zip of row pairs: byte b of ev[q] holds column 2b of rows
    // (2q, 2q+1), byte b of od[q] column 2b+1.
    uint32_t ev[4], od[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ev[q] = (A[2 * q][j] & 0x0F0F0F0Fu) | ((A[2 * q + 1][j] << 4) & 0xF0F0F0F0u);
      od[q] = ((A[2 * q][j] >> 4) & 0x0F0F0F0Fu) | (A[2 * q + 1][j] & 0xF0F0F0F0u);
    }
    const uint32_t s0 = S[2 * j], s1 = S[2 * j + 1];
    uint16_t *op = out + ((size_t)e * N + n0 + 8 * j) * K + k0;
#define QMOE_DQ_COL(C)                                                                                     \
  __builtin_nontemporal_store(                                                                             \
      dequant_col<C, FMT, POW2>(ev, od, ((C < 4 ? s0 : s1) >> (8 * (C & 3))) & 0xFFu, gs, has_g),         \
      (u32x4_t *)(op + (size_t)(C)*K))
    QMOE_DQ_COL(0);
    QMOE_DQ_COL(1);
    QMOE_DQ_COL(2);
    QMOE_DQ_COL(3);
    QMOE_DQ_COL(4);
    QMOE_DQ_COL(5);
    QMOE_DQ_COL(6);
    QMOE_DQ_COL(7);
#undef QMOE_DQ_COL
  }
}

// Staged variant for K % 256 == 0 and N % 256 == 0: a workgroup first
// copies a 256 k x 256 n packed tile into LDS with full-line reads (8
// threads per 128-byte row; 4-byte units XOR-swizzled by row / 8 so the
// k-major reads below spread over the banks), then its lanes run along k: 32
// lanes x 8 k cover one column block's 256 k, so every store instruction
// writes 512 contiguous bytes of an output row (the direct kernel's stores
// write 256-byte runs of four rows).  Same decode and rounding per column.
constexpr int kLdsKT = 256, kLdsNT = 256;

template <int FMT, bool POW2>
__global__ __launch_bounds__(256) void dequant_lds_kernel(const uint8_t *__restrict__ w, const uint8_t *__restrict__ s,
                                                          const float *__restrict__ g, int K, int N,
                                                          uint16_t *__restrict__ out) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int KL = kLdsKT / 8;        // lanes along k per column block
  constexpr int BPW = 64 / KL;           // column blocks per wave and pass
  constexpr int PASSES = (kLdsNT / 8) / (4 * BPW);
  __shared__ uint32_t tile[kLdsKT * 32];  // 256 rows x 128 bytes
  const int e = blockIdx.z;
  const int k0 = blockIdx.x * kLdsKT;
  const int n0 = blockIdx.y * kLdsNT;
  const int tid = threadIdx.x;
  const size_t rowbytes = (size_t)(N >> 1);
  {
    const int c = tid & 7;
#pragma unroll
    for (int i = 0; i < kLdsKT / 32; ++i) {
      const int r = (tid >> 3) + 32 * i;
      const u32x4_t v = __builtin_nontemporal_load(
          (const u32x4_t *)(w + ((size_t)e * K + k0 + r) * rowbytes + (n0 >> 1) + 16 * c));
      const int sw = (r >> 3) & 31;
      tile[r * 32 + ((4 * c + 0) ^ sw)] = v.x;
      tile[r * 32 + ((4 * c + 1) ^ sw)] = v.y;
      tile[r * 32 + ((4 * c + 2) ^ sw)] = v.z;
      tile[r * 32 + ((4 * c + 3) ^ sw)] = v.w;
    }
  }
  __syncthreads();
  const bool has_g = g != nullptr;
  const float gs = has_g ? g[e] : 1.0f;
  const int wave = tid >> 6, lane = tid & 63;
  const int kl = lane % KL;
  const int sub = lane / KL;
  const int kk = k0 + 8 * kl;  // this lane's 8 k rows (inside one scale block)
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int cb = (p * 4 + wave) * BPW + sub;  // block of 8 columns = dword cb of a packed row
    uint32_t A[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * kl + i;
      A[i] = tile[r * 32 + (cb ^ ((r >> 3) & 31))];
    }
    const uint2 sv = *(const uint2 *)(s + ((size_t)e * (K / B) + kk / B) * N + n0 + 8 * cb);
    uint32_t ev[4], od[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ev[q] = (A[2 * q] & 0x0F0F0F0Fu) | ((A[2 * q + 1] << 4) & 0xF0F0F0F0u);
      od[q] = ((A[2 * q] >> 4) & 0x0F0F0F0Fu) | (A[2 * q + 1] & 0xF0F0F0F0u);
    }
    uint16_t *op = out + ((size_t)e * N + n0 + 8 * cb) * K + kk;
#define QMOE_DQL_COL(C)                                                                                  \
  __builtin_nontemporal_store(                                                                           \
      dequant_col<C, FMT, POW2>(ev, od, (((C) < 4 ? sv.x : sv.y) >> (8 * ((C) & 3))) & 0xFFu, gs, has_g), \
      (u32x4_t *)(op + (size_t)(C)*K))
    QMOE_DQL_COL(0);
    QMOE_DQL_COL(1);
    QMOE_DQL_COL(2);
    QMOE_DQL_COL(3);
    QMOE_DQL_COL(4);
    QMOE_DQL_COL(5);
    QMOE_DQL_COL(6);
    QMOE_DQL_COL(7);
#undef QMOE_DQL_COL
  }
}

template <int KT, int CW>
static void launch_shape(const uint8_t *w, const uint8_t *scales, const float *g, int32_t E, int32_t K, int32_t N,
                         int fmt, uint16_t *out, hipStream_t s) {
  static_assert(CW == 8 || CW == 16 || CW % 32 == 0, "columns per thread");
  const dim3 grid((unsigned)(K / KT), (unsigned)(N / (CW * 256 / (KT / 8))), (unsigned)E);
  if (fmt == 0)
    dequant_kernel<0, false, KT, CW><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
  else if (g == nullptr)
    dequant_kernel<1, true, KT, CW><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
  else
    dequant_kernel<1, false, KT, CW><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
}

hipError_t launch_dequant(const uint8_t *w, const uint8_t *scales, const float *g, int32_t E, int32_t K, int32_t N,
                          int fmt, uint16_t *out, hipStream_t s) {
  // Measured on E=32, K=2048, N=1536 (MXFP4): 128 k x 512 n tiles with 32
  // columns per thread (a thread loads 16 bytes per packed row; 16 threads
  // write 256 contiguous bytes of an output row) ran 48.7 us against 61 us
  // for 64 x 256 with 8 columns per thread.  Smaller shapes cover K or N
  // that the large tile does not divide.
  // Staged through LDS when the 256 x 256 tile divides the shape (MXFP4,
  // E=32, K=2048, N=1536: 43.7 us against 49.6 us for the direct kernel).
  if (K % kLdsKT == 0 && N % kLdsNT == 0) {
    const dim3 grid((unsigned)(K / kLdsKT), (unsigned)(N / kLdsNT), (unsigned)E);
    if (fmt == 0)
      dequant_lds_kernel<0, false><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
    else if (g == nullptr)
      dequant_lds_kernel<1, true><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
    else
      dequant_lds_kernel<1, false><<<grid, 256, 0, s>>>(w, scales, g, K, N, out);
  } else if (K % 128 == 0 && N % 512 == 0)
    launch_shape<128, 32>(w, scales, g, E, K, N, fmt, out, s);
  else if (N % 512 == 0)
    launch_shape<64, 16>(w, scales, g, E, K, N, fmt, out, s);
  else if (K % 128 == 0)
    launch_shape<128, 16>(w, scales, g, E, K, N, fmt, out, s);
  else
    launch_shape<64, 8>(w, scales, g, E, K, N, fmt, out, s);
  return hipGetLastError();
}

}  // namespace qmoe
