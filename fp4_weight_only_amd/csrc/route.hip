// Softmax top-k routing and expert maps for gfx950.
//
// Top-k follows the register-only design of "[CUDA] Cut the MoE routing
// prologue/epilogue cost for small-batch decode" (PR 31156): one token per
// wave, every key in registers, each lane sorts its own keys and the wave
// runs a butterfly of bitonic top-N merges, C[i] = max(A[i], B[N-1-i]),
// which is symmetric so both partners keep the same list; no LDS and no
// barrier.  On wave64 the partner moves are DPP (quad_perm, row half-mirror,
// row mirror), ds_swizzle (lane ^ 16) and ds_bpermute (lane ^ 32).  The key
// is 64-bit: an order-preserving image of the exact float32 logit (with -0
// folded onto +0) above the complemented expert index, so equal logits
// select the lower expert and the selection is exact.
//
// The expert maps rank the T*k expanded rows by expert with wave ballots
// (8 ballots match the expert-id bits, popcount below the lane gives the
// rank), the ballot-based ranking the same PR adopts.  For up to 16 tokens
// both steps run in one workgroup (one launch, selections passed in LDS).
#include "device_common.h"
#include "qmoe_internal.h"

namespace qmoe {

__device__ __forceinline__ uint64_t make_key(float v, int e) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
}
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t ord = (uint32_t)(key >> 32);
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ void cswap_desc(uint64_t &a, uint64_t &b) {
  const uint64_t hi = a > b ? a : b;
  const uint64_t lo = a > b ? b : a;
  a = hi;
  b = lo;
}

template <int STEP>
__device__ __forceinline__ uint64_t partner(uint64_t v) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  if constexpr (STEP == 0) {
    lo = dpp_u32<kDppXor1>(lo);
    hi = dpp_u32<kDppXor1>(hi);
  } else if constexpr (STEP == 1) {
    lo = dpp_u32<kDppXor2>(lo);
    hi = dpp_u32<kDppXor2>(hi);
  } else if constexpr (STEP == 2) {
    lo = dpp_u32<kDppRowHalfMirror>(lo);
    hi = dpp_u32<kDppRowHalfMirror>(hi);
  } else if constexpr (STEP == 3) {
    lo = dpp_u32<kDppRowMirror>(lo);
    hi = dpp_u32<kDppRowMirror>(hi);
  } else if constexpr (STEP == 4) {
    lo = swz_xor16(lo);
    hi = swz_xor16(hi);
  } else {
    lo = bperm_xor32(lo);
    hi = bperm_xor32(hi);
  }
  return ((uint64_t)hi << 32) | lo;
}

// Merge this lane's descending top-NP list with its partner group's list.
template <int NP, int STEP>
__device__ __forceinline__ void merge_step(uint64_t (&L)[NP]) {
  uint64_t B[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) B[i] = partner<STEP>(L[i]);
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    const uint64_t o = B[NP - 1 - i];
    L[i] = L[i] > o ? L[i] : o;  // bitonic: top NP of the union
  }
#pragma unroll
  for (int d = NP / 2; d >= 1; d /= 2) {
#pragma unroll
    for (int i = 0; i < NP; ++i)
      if ((i & d) == 0) cswap_desc(L[i], L[i + d]);
  }
}

// Top-k of one token by one wave; E <= 256 (4 keys per lane), k <= NP.
// Lanes j < k return the j-th selected expert and its softmax weight.
template <int NP>
__device__ __forceinline__ void topk_token(const float *__restrict__ row, int E, int k, int lane, int &sel,
                                           float &wsel) {
  uint64_t key[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    key[i] = (e < E) ? make_key(row[e], e) : 0ull;
  }
  cswap_desc(key[0], key[1]);
  cswap_desc(key[2], key[3]);
  cswap_desc(key[0], key[2]);
  cswap_desc(key[1], key[3]);
  cswap_desc(key[1], key[2]);
  uint64_t L[NP];
#pragma unroll
  for (int i = 0; i < NP; ++i) L[i] = (i < 4) ? key[i] : 0ull;
  merge_step<NP, 0>(L);
  merge_step<NP, 1>(L);
  merge_step<NP, 2>(L);
  merge_step<NP, 3>(L);
  merge_step<NP, 4>(L);
  merge_step<NP, 5>(L);
  // Every lane now holds the token's top-NP, largest first.
  const float lmax = key_value(L[0]);
  float ex[NP];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    ex[i] = (i < k) ? expf(key_value(L[i]) - lmax) : 0.f;
    sum += ex[i];
  }
  uint64_t mine = 0;
  float mine_ex = 0.f;
#pragma unroll
  for (int i = 0; i < NP; ++i) {
    if (lane == i) {
      mine = L[i];
      mine_ex = ex[i];
    }
  }
  sel = key_index(mine);
  wsel = mine_ex / sum;
}

// One wave per token.
template <int NP>
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                         int32_t *__restrict__ idx, float *__restrict__ wts) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // wave-uniform
  int sel;
  float wsel;
  topk_token<NP>(logits + (size_t)t * E, E, k, lane, sel, wsel);
  if (lane < k) {
    idx[(size_t)t * k + lane] = sel;
    wts[(size_t)t * k + lane] = wsel;
  }
}

// Stable counting sort of the expanded rows by expert, by one workgroup of
// NW waves: NW*64 rows are ranked per round with ballots; E <= 256.  idx
// may point to global or LDS memory.
template <int NW>
__device__ __forceinline__ void build_maps(const int32_t *idx, int R, int E, int32_t *__restrict__ offsets,
                                           int32_t *__restrict__ p2e, int32_t *__restrict__ e2p) {
  __shared__ int cnt[256];
  __shared__ int base[256];
  __shared__ int wc[NW][256];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  for (int e = tid; e < 256; e += NW * 64) cnt[e] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += NW * 64) atomicAdd(&cnt[idx[r]], 1);
  __syncthreads();
  if (wave == 0) {
    // exclusive scan of cnt[0..E) : lane owns entries 4*lane .. 4*lane+3
    int c[4];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      c[i] = (e < E) ? cnt[e] : 0;
      s += c[i];
    }
    int incl = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int o = __shfl_up(incl, d, 64);
      if (lane >= d) incl += o;
    }
    int run = incl - s;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = 4 * lane + i;
      if (e < E) {
        base[e] = run;
        offsets[e] = run;
      }
      run += c[i];
    }
    if (lane == 63) offsets[E] = incl;
  }
  __syncthreads();
  const unsigned long long lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int r0 = 0; r0 < R; r0 += NW * 64) {
    for (int e = lane; e < 256; e += 64) wc[wave][e] = 0;
    const int r = r0 + wave * 64 + lane;
    const bool valid = r < R;
    const int e = valid ? idx[r] : 0;
    unsigned long long match = __ballot(valid);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const bool bit = (e >> b) & 1;
      const unsigned long long m = __ballot(bit);
      match &= bit ? m : ~m;
    }
    const int rank = __popcll(match & lt);
    __syncthreads();
    if (valid && rank == 0) wc[wave][e] = __popcll(match);
    __syncthreads();
    for (int x = tid; x < E; x += NW * 64) {
      int run = base[x];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const int c = wc[w][x];
        wc[w][x] = run;
        run += c;
      }
      base[x] = run;
    }
    __syncthreads();
    if (valid) {
      const int p = wc[wave][e] + rank;
      p2e[p] = r;
      e2p[r] = p;
    }
    __syncthreads();
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void expert_maps_kernel(const int32_t *__restrict__ idx, int R, int E,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ p2e,
                                                              int32_t *__restrict__ e2p) {
  build_maps<NW>(idx, R, E, offsets, p2e, e2p);
}

// Decode-sized batches (T <= NW): top-k and maps in one workgroup, the
// selections handed over through LDS.
template <int NP, int NW>
__global__ __launch_bounds__(NW * 64) void route_fused_kernel(const float *__restrict__ logits, int T, int E, int k,
                                                              int32_t *__restrict__ idx, float *__restrict__ wts,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ p2e,
                                                              int32_t *__restrict__ e2p) {
  __shared__ int32_t sidx[NW * 8];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (wave < T) {  // wave-uniform
    int sel;
    float wsel;
    topk_token<NP>(logits + (size_t)wave * E, E, k, lane, sel, wsel);
    if (lane < k) {
      idx[(size_t)wave * k + lane] = sel;
      wts[(size_t)wave * k + lane] = wsel;
      sidx[wave * k + lane] = sel;
    }
  }
  __syncthreads();
  build_maps<NW>(sidx, T * k, E, offsets, p2e, e2p);
}

template <int NP>
static void launch_fused(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *idx, float *w,
                         int32_t *offsets, int32_t *p2e, int32_t *e2p, hipStream_t s) {
  if (T <= 4)
    route_fused_kernel<NP, 4><<<1, 256, 0, s>>>(logits, T, E, k, idx, w, offsets, p2e, e2p);
  else if (T <= 8)
    route_fused_kernel<NP, 8><<<1, 512, 0, s>>>(logits, T, E, k, idx, w, offsets, p2e, e2p);
  else
    route_fused_kernel<NP, 16><<<1, 1024, 0, s>>>(logits, T, E, k, idx, w, offsets, p2e, e2p);
}

hipError_t launch_route(const float *logits, int32_t T, int32_t E, int32_t k, int32_t *idx, float *w,
                        int32_t *offsets, int32_t *p2e, int32_t *e2p, hipStream_t s) {
  if (T <= 16) {  // one launch: top-k and maps in one workgroup
    if (k <= 1)
      launch_fused<1>(logits, T, E, k, idx, w, offsets, p2e, e2p, s);
    else if (k <= 2)
      launch_fused<2>(logits, T, E, k, idx, w, offsets, p2e, e2p, s);
    else if (k <= 4)
      launch_fused<4>(logits, T, E, k, idx, w, offsets, p2e, e2p, s);
    else
      launch_fused<8>(logits, T, E, k, idx, w, offsets, p2e, e2p, s);
    return hipGetLastError();
  }
  const dim3 grid((T + 3) / 4);
  if (k <= 1)
    route_topk_kernel<1><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else if (k <= 2)
    route_topk_kernel<2><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else if (k <= 4)
    route_topk_kernel<4><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  else
    route_topk_kernel<8><<<grid, 256, 0, s>>>(logits, T, E, k, idx, w);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int R = T * k;
  if (R <= 256)
    expert_maps_kernel<4><<<1, 256, 0, s>>>(idx, R, E, offsets, p2e, e2p);
  else
    expert_maps_kernel<16><<<1, 1024, 0, s>>>(idx, R, E, offsets, p2e, e2p);
  return hipGetLastError();
}

}  // namespace qmoe
