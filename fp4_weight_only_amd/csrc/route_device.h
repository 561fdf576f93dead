// Routing building blocks shared by the routing kernels and the GEMV's
// fused routing prologue (gfx950, wave64): exact top-k of one token by one
// wave, and the expert maps of up to 64 expanded rows by one wave.
#pragma once
#include "device_common.h"

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
  // all four loads unconditional (a lane past E reads expert E - 1 and
  // drops it), so they are in flight together: written as conditional
  // loads, each sat in its own branch with a wait behind it, four memory
  // round trips in a row
  float lv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) lv[i] = row[min(lane + 64 * i, E - 1)];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    kv[i] = (e < E) ? ord_key(lv[i]) : 0u;
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

}  // namespace qmoe
