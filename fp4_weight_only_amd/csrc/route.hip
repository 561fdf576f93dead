// Softmax top-k routing and expert maps for gfx950.
//
// Top-k keeps the register-only shape of "[CUDA] Cut the MoE routing
// prologue/epilogue cost for small-batch decode" (PR 31156): one token per
// wave, every logit in registers (4 per lane for E <= 256), no LDS and no
// barrier.  The selection itself is k rounds of a wave-wide argmax rather
// than a merge network: each round takes the maximum of an order-preserving
// 32-bit image of the exact float32 logits (-0 folded onto +0) with four DPP
// max steps inside each 16-lane row and four lane reads, then four ballots
// find the lowest expert index holding that maximum, which leaves the round.
// The selection is exact and equal logits select the lower expert; the
// winners come out largest first.
//
// The expert maps rank the T*k expanded rows by expert with wave ballots
// (8 ballots match the expert-id bits, popcount below the lane gives the
// rank), the ballot-based ranking the same PR adopts.  For up to 16 tokens
// both steps run in one workgroup (one launch, selections passed in LDS);
// up to 64 expanded rows the maps take a single wave and no barrier.
#include "device_common.h"
#include "qmoe_internal.h"
#include "route_device.h"

namespace qmoe {

// One wave per token.
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         const float *__restrict__ rw, int T, int E, int k,
                                                         int32_t *__restrict__ idx, float *__restrict__ wts) {
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;  // wave-uniform
  int sel;
  float wsel;
  topk_token(logits + (size_t)t * E, rw ? rw + (size_t)t * E : nullptr, E, k, lane, sel, wsel);
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
template <int NW>
__global__ __launch_bounds__(NW * 64) void route_fused_kernel(const float *__restrict__ logits,
                                                              const float *__restrict__ rw, int T, int E, int k,
                                                              int32_t *__restrict__ idx, float *__restrict__ wts,
                                                              int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ p2e,
                                                              int32_t *__restrict__ e2p) {
  __shared__ int32_t sidx[NW * 8];
  __shared__ __attribute__((aligned(16))) int32_t cnt[256];
  const int wave = threadIdx.x >> 6;
  const int lane = lane_id();
  if (wave < T) {  // wave-uniform
    int sel;
    float wsel;
    topk_token(logits + (size_t)wave * E, rw ? rw + (size_t)wave * E : nullptr, E, k, lane, sel, wsel);
    if (lane < k) {
      idx[(size_t)wave * k + lane] = sel;
      wts[(size_t)wave * k + lane] = wsel;
      sidx[wave * k + lane] = sel;
    }
  }
  __syncthreads();
  if (T * k <= 64) {  // uniform
    if (wave == 0) build_maps_wave(sidx, T * k, E, offsets, p2e, e2p, cnt);
  } else {
    build_maps<NW>(sidx, T * k, E, offsets, p2e, e2p);
  }
}

hipError_t launch_route(const float *logits, const float *rw, int32_t T, int32_t E, int32_t k, int32_t *idx, float *w,
                        int32_t *offsets, int32_t *p2e, int32_t *e2p, hipStream_t s) {
  if (T <= 16) {  // one launch: top-k and maps in one workgroup
    if (T <= 4)
      route_fused_kernel<4><<<1, 256, 0, s>>>(logits, rw, T, E, k, idx, w, offsets, p2e, e2p);
    else if (T <= 8)
      route_fused_kernel<8><<<1, 512, 0, s>>>(logits, rw, T, E, k, idx, w, offsets, p2e, e2p);
    else
      route_fused_kernel<16><<<1, 1024, 0, s>>>(logits, rw, T, E, k, idx, w, offsets, p2e, e2p);
    return hipGetLastError();
  }
  const dim3 grid((T + 3) / 4);
  route_topk_kernel<<<grid, 256, 0, s>>>(logits, rw, T, E, k, idx, w);
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
