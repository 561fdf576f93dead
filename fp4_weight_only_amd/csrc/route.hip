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

namespace qmoe {

__device__ __forceinline__ uint32_t ord_key(float v) {
  uint32_t u = __float_as_uint(v);
  u = (u == 0x80000000u) ? 0u : u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float ord_value(uint32_t ord) {
  return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

// Maximum / minimum over the wave; the result is uniform.
template <bool MAX>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? max(a, b) : min(a, b); };
  v = op(v, dpp_u32<kDppXor1>(v));
  v = op(v, dpp_u32<kDppXor2>(v));
  v = op(v, dpp_u32<kDppRowHalfMirror>(v));
  v = op(v, dpp_u32<kDppRowMirror>(v));  // every lane holds its 16-lane row's result
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(a, b), op(c, d));
}

constexpr uint32_t kNoExpert = 0xFFFFu;  // padding / consumed slot: loses every tie

// Top-k of one token by one wave; E <= 256 (expert lane + 64 i in key i of
// a lane), 1 <= k <= 8, k <= E.  Lanes j < k return the j-th selected expert
// and its weight: the softmax over the selected logits, or, given the
// token's router_weights row rw (DeepSeek-style routing, operator
// documentation section 2, input 14), rw at the selected expert as it is.
//
// Each lane first sorts its four keys (value descending, lower expert first
// on equal values), so a round only compares the lanes' heads: the wave
// maximum of the heads, the one lane holding it (a wave minimum of the
// expert index breaks the rare tie between lanes), and that lane drops its
// head.
__device__ __forceinline__ void topk_token(const float *__restrict__ row, const float *__restrict__ rw, int E, int k,
                                           int lane, int &sel, float &wsel) {
  uint32_t kv[4], ex[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    kv[i] = (e < E) ? ord_key(row[e]) : 0u;
    ex[i] = (e < E) ? (uint32_t)e : kNoExpert;
  }
  auto order = [&](int a, int b) {  // slot a before slot b
    const bool sw = kv[b] > kv[a] || (kv[b] == kv[a] && ex[b] < ex[a]);
    const uint32_t ka = kv[a], xa = ex[a];
    kv[a] = sw ? kv[b] : ka;
    ex[a] = sw ? ex[b] : xa;
    kv[b] = sw ? ka : kv[b];
    ex[b] = sw ? xa : ex[b];
  };
  order(0, 1);
  order(2, 3);
  order(0, 2);
  order(1, 3);
  order(1, 2);
  uint32_t top0 = 0u, mine_key = 0u;
  int mine = 0;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    if (r < k) {  // uniform
      const uint32_t M = wave_reduce_u32<true>(kv[0]);
      const uint64_t hit = __ballot(kv[0] == M);
      int wl = __builtin_ctzll(hit);
      if (__popcll(hit) != 1) {  // equal heads in several lanes: lowest expert index
        const uint32_t cand = (kv[0] == M) ? ex[0] : 0xFFFFFFFFu;
        const uint32_t emin = wave_reduce_u32<false>(cand);
        wl = __builtin_ctzll(__ballot(cand == emin));
      }
      const int e = __builtin_amdgcn_readlane((int)ex[0], wl);
      if (r == 0) top0 = M;
      if (lane == r) {
        mine = e;
        mine_key = M;
      }
      if (lane == wl) {
        kv[0] = kv[1];
        ex[0] = ex[1];
        kv[1] = kv[2];
        ex[1] = ex[2];
        kv[2] = kv[3];
        ex[2] = ex[3];
        kv[3] = 0u;
        ex[3] = kNoExpert;
      }
    }
  }
  sel = mine;
  if (rw) {  // uniform
    wsel = (lane < k) ? rw[mine] : 0.f;
    return;
  }
  // softmax over the selected logits, largest first: lane j < k owns exp of
  // the j-th; the sum is taken in selection order
  const float lmax = ord_value(top0);
  const float mine_ex = (lane < k) ? expf(ord_value(mine_key) - lmax) : 0.f;
  float sum = 0.f;
#pragma unroll
  for (int r = 0; r < 8; ++r) sum += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mine_ex), r));
  wsel = mine_ex / sum;
}

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

// The same maps for R <= 64 rows by one wave, with no barrier: row r sits in
// lane r.  Matching the expert-id bits from the most significant down, a row
// also counts the rows whose id first differs by a 0 where its own has a 1,
// i.e. the rows of smaller experts, so its position is that count plus its
// rank among equal ids.  The offsets come from per-expert counts in LDS
// (written by the first row of each expert; one wave's LDS accesses complete
// in program order) and a wave prefix sum.
__device__ __forceinline__ void build_maps_wave(const int32_t *idx, int R, int E, int32_t *__restrict__ offsets,
                                                int32_t *__restrict__ p2e, int32_t *__restrict__ e2p,
                                                int32_t (&cnt)[256]) {
  const int lane = lane_id();
  const bool valid = lane < R;
  const int e = valid ? idx[lane] : 0;
  *(int4 *)&cnt[4 * lane] = make_int4(0, 0, 0, 0);
  uint64_t match = __ballot(valid);
  int less = 0;
#pragma unroll
  for (int b = 7; b >= 0; --b) {
    const uint64_t m = __ballot(valid && ((e >> b) & 1));
    if ((e >> b) & 1) {
      less += __popcll(match & ~m);
      match &= m;
    } else {
      match &= ~m;
    }
  }
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank = __popcll(match & lt);
  __builtin_amdgcn_wave_barrier();
  if (valid && rank == 0) cnt[e] = __popcll(match);
  __builtin_amdgcn_wave_barrier();
  if (valid) {
    const int p = less + rank;
    p2e[p] = lane;
    e2p[lane] = p;
  }
  // exclusive scan of the counts: lane owns experts 4*lane .. 4*lane+3
  const int4 c4 = *(const int4 *)&cnt[4 * lane];
  const int c[4] = {c4.x, c4.y, c4.z, c4.w};
  const int s = c[0] + c[1] + c[2] + c[3];
  int incl = s;  // inclusive prefix inside each 16-lane row, then across rows
  incl += (int)__builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, true);  // row_shr:1
  incl += (int)__builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, true);  // row_shr:2
  incl += (int)__builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, true);  // row_shr:4
  incl += (int)__builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, true);  // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(incl, 15);
  const int r1 = __builtin_amdgcn_readlane(incl, 31);
  const int r2 = __builtin_amdgcn_readlane(incl, 47);
  const int row = lane >> 4;
  incl += (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
  int run = incl - s;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * lane + i < E) offsets[4 * lane + i] = run;
    run += c[i];
  }
  if (lane == 0) offsets[E] = R;
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
