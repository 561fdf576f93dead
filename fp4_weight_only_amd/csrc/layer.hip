// The whole FP4 decode MoE layer in one launch, gfx950: softmax top-k
// routing, the expert maps, FC1 with fused SwiGLU, FC2 and the weighted
// un-permute.
//
// What it computes (operator documentation section 1: router -> permute ->
// GEMM1 -> SwiGLU -> GEMM2 -> un-permute -> weighted sum; sections 8, 9b.2
// and 12.1 for the FP4 GEMV and the split-K SwiGLU; PR 31159 for the decode
// GEMV up to 64 expanded rows; PR 31156 / 29919 for routing fused into the
// path): the same values, bit for bit, as qmoe_route_topk followed by the
// GEMV FC1 call and the fused FC2 + finalize call -- every partial sum, every
// summation order and every rounding is theirs.
//
// gfx950 design:
// * Every workgroup runs the routing of all T tokens (one wave per token, the
//   exact top-k of the routing kernels) and ranks the T*k <= 64 rows by
//   expert with one wave, in LDS; workgroup 0 writes the routing outputs.
//   It then lists the live (expert, row group) slots: an expert's rows in
//   groups of at most one pass (1, 2 or 4 rows), as the per-call GEMV does.
// * Work items are the per-call GEMV's workgroups: (slot, 256-column tile,
//   256-row k chunk), FC1's first, then FC2's, each streaming 32 KB of packed
//   weights (plus scales) with the same loads, decode and dot products.  A
//   workgroup takes items g, g + G, g + 2G, ... (G workgroups, no more than
//   fit on the chip at once), so every item an FC2 item waits for belongs to
//   a resident workgroup that reached it first and never waits itself.
// * Hand-offs go through the workspace with device-coherent stores and loads
//   (buffer cache policy sc1: written through / read past the XCD's L2) and
//   relaxed device-scope atomic counters, one per 64-byte segment; a wave
//   waits for its own stores (s_waitcnt vmcnt(0)) before its workgroup
//   counts.  No release/acquire fences: measured on MI355X, an agent-scope
//   release fence costs about 100 ns of serialised L2 write-back per
//   workgroup (a release atomic 19-30 ns), this scheme about nothing;
//   counters are spread so that no address takes many increments
//   (same-address atomics serialise at about 10 ns each).
//   - FC1 item: writes its g * partial plane and counts on (slot, h chunk)
//     without waiting for the counter's value.
//   - FC2 item: issues its weight loads, waits until the 2 x nch1 FC1 items
//     of its h chunk have counted, forms its h rows from their planes (summed
//     in chunk order from -0, SwiGLU, bf16: the split-K epilogue's
//     arithmetic), writes its g * partial plane and counts on its column
//     tile; the last item of a tile runs the finalize for that tile (FC2
//     planes summed in order, weighted sum over j in order, bf16), then
//     counts on a done counter whose last arrival zeroes every counter for
//     the next call.
// * Every wait is bounded (max_polls); a wait that runs out sets the error
//   word and ends, so the grid always drains.
#include "device_common.h"
#include "gemv_device.h"
#include "qmoe_internal.h"
#include "route_device.h"

namespace qmoe {

namespace {

constexpr int kThreads = 256;
constexpr int kKC = kMaxChunkK;        // 256 k rows per chunk
constexpr int kCoherent = 16;          // buffer cache policy sc1 (device scope)
constexpr int kFinPlanes = 3;          // FC2 planes per load round of the finalize

// Arguments only the rare paths use (h reduction, finalize, routing
// outputs), kept in LDS so they do not occupy scalar registers across the
// item loop.
struct LayerCold {
  int32_t *idx;
  float *wts;
  int32_t *offsets;
  int32_t *p2e, *e2p;
  uint16_t *out;
  float alpha, beta, limit;
  int32_t E, T;
};

template <int MRMAX>
struct LayerSmem {
  LayerCold cold;
  Smem<MRMAX> g;                       // one GEMV pass
  int32_t sidx[64];                    // selected expert of expanded row t*k + j
  float swt[64];                       // its mixing weight
  int32_t off[260];                    // expert offsets [E+1]
  int32_t p2e[64];
  int32_t e2p[64];
  int32_t cnt[256];
  int32_t rinfo[64];                   // permuted row p: expert | rank in expert << 8 | expert's rows << 16
  int32_t slot_e[64], slot_r0[64], slot_m[64];
  int32_t nlive;
  int32_t flag;
};

__device__ __forceinline__ int32_t *sync_err(const LayerArgs &a) { return a.sync; }
__device__ __forceinline__ int32_t *sync_done(const LayerArgs &a) { return a.sync + kLayerSyncStride; }
__device__ __forceinline__ int32_t *sync_tile(const LayerArgs &a, int t) { return a.sync + (2 + t) * kLayerSyncStride; }
__device__ __forceinline__ int32_t *sync_hchunk(const LayerArgs &a, int s, int hc) {
  return a.sync + (2 + kLayerMaxTiles2 + s * kLayerMaxHChunks + hc) * kLayerSyncStride;
}

// Waits until this thread's stores have completed (device-coherent stores
// are then visible device-wide); the clobber keeps the compiler from moving
// memory accesses across it.
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ int count(int32_t *c) {
  return __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FC1 items feeding h chunk hc (256 h values): two 256-column tiles (the
// gate/linear pairs of interleaved columns 512 hc .. 512 hc + 511, or gate
// tile hc and linear tile nhc + hc when concatenated) times the k chunks.
__device__ __forceinline__ int hchunk_items(const LayerArgs &a, int hc) {
  const int tiles = a.concat ? 2 : min(2, a.ntiles1 - 2 * hc);
  return tiles * a.nch1;
}

// Routing of all T tokens (one wave per token: the routing kernels' exact
// top-k), then one wave ranks the T*k <= 64 expanded rows by expert with
// ballots (a row's permuted position is the number of rows of smaller experts
// plus its rank among its expert's rows) and lists the live slots: an
// expert's rows in groups of at most MR, experts in ascending order (the
// per-call GEMV's row split).  The expert offsets themselves are not needed
// here; workgroup 0 writes every routing output after its work items.
template <int MR, class S>
__device__ __forceinline__ void route_and_slots(const LayerArgs &a, S &sm, int wave, int lane) {
  const int E = a.E, k = a.k, T = a.T, R = a.rows;
  for (int t = wave; t < T; t += kThreads / 64) {  // wave-uniform
    int sel;
    float wsel;
    topk_token(a.logits + (size_t)t * E, a.rw ? a.rw + (size_t)t * E : nullptr, E, k, lane, sel, wsel);
    if (lane < k) {
      sm.sidx[t * k + lane] = sel;
      sm.swt[t * k + lane] = wsel;
    }
  }
  lds_barrier();
  if (wave == 0) {
    const bool valid = lane < R;
    const int e = valid ? sm.sidx[lane] : 0;
    uint64_t match = __ballot(valid);
    int less = 0;
#pragma unroll
    for (int b = 7; b >= 0; --b) {
      const uint64_t mb = __ballot(valid && ((e >> b) & 1));
      if ((e >> b) & 1) {
        less += __popcll(match & ~mb);
        match &= mb;
      } else {
        match &= ~mb;
      }
    }
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int rank = __popcll(match & lt);
    const int cnt = __popcll(match);
    if (valid) {
      const int p = less + rank;
      sm.p2e[p] = lane;
      sm.e2p[lane] = p;
      sm.rinfo[p] = e | (rank << 8) | (cnt << 16);
    }
    __builtin_amdgcn_wave_barrier();
    const int info = valid ? sm.rinfo[lane] : 0;  // lane = permuted row now
    const int re = info & 0xFF, rr = (info >> 8) & 0xFF, rc = info >> 16;
    const bool start = valid && (rr % MR) == 0;
    const uint64_t sb = __ballot(start);
    if (start) {
      const int slot = __popcll(sb & lt);
      sm.slot_e[slot] = re;
      sm.slot_r0[slot] = lane;
      sm.slot_m[slot] = min(MR, rc - rr);
    }
    if (lane == 0) sm.nlive = __popcll(sb);
  }
  lds_barrier();
}

// Workgroup 0, after its items: topk_idx, topk_w, the maps and the expert
// offsets (an exclusive scan of the per-expert row counts).
template <class S>
__device__ __forceinline__ void write_routing(const LayerArgs &a, S &sm, int tid) {
  const int E = sm.cold.E, R = a.rows;
  for (int i = tid; i < R; i += kThreads) {
    sm.cold.idx[i] = sm.sidx[i];
    sm.cold.wts[i] = sm.swt[i];
    sm.cold.p2e[i] = sm.p2e[i];
    sm.cold.e2p[i] = sm.e2p[i];
  }
  // rows of experts below e: the permuted position of the first row of an
  // expert at or above e, i.e. a count over the rows' experts
  for (int e = tid; e <= E; e += kThreads) {
    int below = 0;
    for (int r = 0; r < R; ++r) below += sm.sidx[r] < e ? 1 : 0;
    sm.cold.offsets[e] = below;
  }
}

// One GEMV item's weight and scale loads (the per-call GEMV's loads): lane
// (wave, half, nl) holds k rows kc*256 + 32*(2 wave + half) .. +31 of columns
// tile*256 + 8 nl .. +7 of expert e, one dword per row.
template <int FMT>
struct ItemLoads {
  uint32_t A[kGemvLaneK];
  u32x2_t SB[2];
  float gs;
};

template <int FMT>
__device__ __forceinline__ void issue_loads(const uint8_t *w, const uint8_t *scales, const float *gscale, int e, int K,
                                            int N, int tile, int kc, int wave, int lane, ItemLoads<FMT> &L) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int NBLK = kGemvLaneK / B;
  const int nl = lane & 31;
  const int g = wave * 2 + (lane >> 5);
  const int col0 = tile * kGemvTileN + nl * 8;
  const int kl = kc * kKC + g * kGemvLaneK;
  const uint32_t rowbytes = (uint32_t)(N >> 1);
  const int KB = K / B;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(w + (size_t)e * K * rowbytes), (short)0, (int)((uint32_t)K * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(scales + (size_t)e * KB * N), (short)0, (int)((uint32_t)KB * N), 0x00020000);
  const bool col_ok = col0 < N;
  const uint32_t woff = col_ok ? (uint32_t)kl * rowbytes + (uint32_t)(col0 >> 1) : kOutOfRange;
  const uint32_t soff = col_ok ? (uint32_t)(kl / B) * (uint32_t)N + (uint32_t)col0 : kOutOfRange;
#pragma unroll
  for (int b = 0; b < 2; ++b)
    L.SB[b] = (b < NBLK) ? __builtin_amdgcn_raw_buffer_load_b64(sr, soff, b * N, 0) : u32x2_t{0u, 0u};
#pragma unroll
  for (int i = 0; i < kGemvLaneK; ++i)
    L.A[i] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff, i * (int)rowbytes, kBufNontemporal);
  L.gs = gscale ? gscale[e] : 1.0f;
}

// Decode + dot products of a pass over mr <= MRMAX staged rows, then the
// waves' partial sums added in wave order (over the W waves the per-call
// GEMV launches for this K) and g * sum stored to plane kc of a partial-sum
// array [planes][rows][N] with device-coherent stores.
template <int FMT, int MRMAX, class S>
__device__ __forceinline__ void item_dot_store(const LayerArgs &a, S &sm, const ItemLoads<FMT> &L, int m, int row0,
                                               int tile, int kc, int K, int N, float *part, int tid, int wave,
                                               int lane) {
  const int g = wave * 2 + (lane >> 5);
  lane_pass<FMT, MRMAX>(sm.g, L.A, L.SB, g, wave, lane, 0, m);
  lds_barrier();
  const int W = K >= kKC ? kGemvMaxWaves : (K + kGemvWaveK - 1) / kGemvWaveK;
  const uint32_t plane = (uint32_t)a.rows * (uint32_t)N * 4u;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(part), (short)0, (int)(plane * (uint32_t)(kc + 1)), 0x00020000);
  const int cl = tid;  // one column per thread
  const int col = tile * kGemvTileN + cl;
  for (int r = 0; r < m; ++r) {
    float s = sm.g.red[0][r][cl];
    for (int q = 1; q < W; ++q) s += sm.g.red[q][r][cl];
    const float u = L.gs * s;
    const uint32_t off = (uint32_t)kc * plane + ((uint32_t)(row0 + r) * (uint32_t)N + (uint32_t)col) * 4u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(u), pr, col < N ? off : kOutOfRange, 0, kCoherent);
  }
}

// FC2's activations for h chunk hc of slot rows row0 .. row0 + m - 1, formed
// from FC1's partial planes: summed in chunk order from -0, SwiGLU, bf16
// round to nearest even (the split-K epilogue's arithmetic).  A thread forms
// 4 h values of one row (64 threads per row) and writes them to the pass's
// activation tile in LDS.
template <class S>
__device__ __forceinline__ void stage_h(const LayerArgs &a, S &sm, int row0, int m, int hc, int tid, int mrmax) {
  const int I = a.I, N1 = 2 * a.I;
  const int r = tid >> 6;
  const int jl = 4 * (tid & 63);
  const int j0 = hc * kKC + jl;
  const bool on = r < m && j0 < I;
  const uint32_t plane = (uint32_t)a.rows * (uint32_t)N1 * 4u;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.part1), (short)0, (int)(plane * (uint32_t)a.nch1), 0x00020000);
  const uint32_t row = (uint32_t)(row0 + r) * (uint32_t)N1 * 4u;
  const uint32_t o0 = row + 4u * (uint32_t)(a.concat ? j0 : 2 * j0);
  const uint32_t o1 = row + 4u * (uint32_t)(a.concat ? I + j0 : 2 * j0 + 4);
  float4 s0 = make_float4(-0.f, -0.f, -0.f, -0.f), s1 = s0;
  constexpr int G = 8;
  for (int c0 = 0; c0 < a.nch1; c0 += G) {
    float4 v0[G], v1[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const bool ld = on && c0 + gi < a.nch1;
      const uint32_t base = (uint32_t)(c0 + gi) * plane;
      v0[gi] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(pr, ld ? base + o0 : kOutOfRange, 0,
                                                                                 kCoherent));
      v1[gi] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(pr, ld ? base + o1 : kOutOfRange, 0,
                                                                                 kCoherent));
    }
#pragma unroll
    for (int gi = 0; gi < G; ++gi) {
      const bool live = c0 + gi < a.nch1;
      s0.x += live ? v0[gi].x : -0.f;
      s0.y += live ? v0[gi].y : -0.f;
      s0.z += live ? v0[gi].z : -0.f;
      s0.w += live ? v0[gi].w : -0.f;
      s1.x += live ? v1[gi].x : -0.f;
      s1.y += live ? v1[gi].y : -0.f;
      s1.z += live ? v1[gi].z : -0.f;
      s1.w += live ? v1[gi].w : -0.f;
    }
  }
  float gt[4], ln[4];
  if (a.concat) {
    gt[0] = s0.x; gt[1] = s0.y; gt[2] = s0.z; gt[3] = s0.w;
    ln[0] = s1.x; ln[1] = s1.y; ln[2] = s1.z; ln[3] = s1.w;
  } else {
    gt[0] = s0.x; ln[0] = s0.y; gt[1] = s0.z; ln[1] = s0.w;
    gt[2] = s1.x; ln[2] = s1.y; gt[3] = s1.z; ln[3] = s1.w;
  }
  uint32_t h[4];
  const float alpha = sm.cold.alpha, beta = sm.cold.beta, limit = sm.cold.limit;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = bf16_rne(swiglu(gt[i], ln[i], alpha, beta, limit));
  if (r < mrmax) *(u32x2_t *)&sm.g.xs[r][jl] = on ? u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)} : u32x2_t{0u, 0u};
}

// out[t][n] for the 256 columns of FC2 tile n2 and every token: FC2's planes
// of each routed row summed in plane order from -0, then the weighted sum
// over j in ascending order from +0 (the fused FC2 + finalize call's
// arithmetic), bf16.  A thread owns 4 columns of one token (four tokens per
// round); every plane load of a round is in flight at once.
template <class S>
__device__ __forceinline__ void finalize_tile(const LayerArgs &a, S &sm, int n2, int tid) {
  const int H = a.H, k = a.k;
  const int col = n2 * kGemvTileN + 4 * (tid & 63);
  const uint32_t plane = (uint32_t)a.rows * (uint32_t)H * 4u;
  const __amdgpu_buffer_rsrc_t pr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.part2), (short)0, (int)(plane * (uint32_t)a.nch2), 0x00020000);
  const int T = __builtin_amdgcn_readfirstlane(sm.cold.T);
  uint16_t *out = (uint16_t *)uniform_ptr(sm.cold.out);
  for (int t = tid >> 6; t < T; t += kThreads / 64) {  // wave-uniform
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    if (a.nch2 <= kFinPlanes) {  // uniform: one round, every plane of every row in flight
      float4 ld[kFinPlanes][8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t roff = j < k ? (uint32_t)sm.e2p[t * k + j] * (uint32_t)H * 4u + (uint32_t)col * 4u : 0u;
#pragma unroll
        for (int gi = 0; gi < kFinPlanes; ++gi) {
          const bool on = j < k && gi < a.nch2 && col < H;
          ld[gi][j] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                     pr, on ? (uint32_t)gi * plane + roff : kOutOfRange, 0, kCoherent));
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < k) {  // uniform
          float4 v = make_float4(-0.f, -0.f, -0.f, -0.f);
#pragma unroll
          for (int gi = 0; gi < kFinPlanes; ++gi) {
            const bool live = gi < a.nch2;
            v.x += live ? ld[gi][j].x : -0.f;
            v.y += live ? ld[gi][j].y : -0.f;
            v.z += live ? ld[gi][j].z : -0.f;
            v.w += live ? ld[gi][j].w : -0.f;
          }
          const float w = sm.swt[t * k + j];
          acc.x = fmaf(w, v.x, acc.x);
          acc.y = fmaf(w, v.y, acc.y);
          acc.z = fmaf(w, v.z, acc.z);
          acc.w = fmaf(w, v.w, acc.w);
        }
      }
    } else {  // more planes: each routed row's planes in rounds of 8, rows in j order
      for (int j = 0; j < k; ++j) {
        const uint32_t roff = (uint32_t)sm.e2p[t * k + j] * (uint32_t)H * 4u + (uint32_t)col * 4u;
        float4 v = make_float4(-0.f, -0.f, -0.f, -0.f);
        for (int c0 = 0; c0 < a.nch2; c0 += 8) {
          float4 ld[8];
#pragma unroll
          for (int gi = 0; gi < 8; ++gi) {
            const bool on = c0 + gi < a.nch2 && col < H;
            ld[gi] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                    pr, on ? (uint32_t)(c0 + gi) * plane + roff : kOutOfRange, 0,
                                                    kCoherent));
          }
#pragma unroll
          for (int gi = 0; gi < 8; ++gi) {
            const bool live = c0 + gi < a.nch2;
            v.x += live ? ld[gi].x : -0.f;
            v.y += live ? ld[gi].y : -0.f;
            v.z += live ? ld[gi].z : -0.f;
            v.w += live ? ld[gi].w : -0.f;
          }
        }
        const float w = sm.swt[t * k + j];
        acc.x = fmaf(w, v.x, acc.x);
        acc.y = fmaf(w, v.y, acc.y);
        acc.z = fmaf(w, v.z, acc.z);
        acc.w = fmaf(w, v.w, acc.w);
      }
    }
    if (col < H) {
      uint2 o;
      o.x = bf16_rne(acc.x) | (bf16_rne(acc.y) << 16);
      o.y = bf16_rne(acc.z) | (bf16_rne(acc.w) << 16);
      *(uint2 *)(out + (size_t)t * H + col) = o;
    }
  }
}

// One work item: FC1 (slot, tile, k chunk) or FC2 (slot, k chunk = h chunk,
// tile), with its expert and rows.
struct ItemInfo {
  int fc2, s, kc, tile, hc, e, row0, m, K, N;
};

// Items: every FC1 item, then every FC2 item; an FC2 item depends only on
// FC1 items, all of which come before it.  Inside each GEMM the slot is the
// fastest-moving index (FC1: then k chunk, then tile in h-chunk order; FC2:
// then tile, then k chunk = h chunk), so the workgroups the dispatcher puts
// side by side on one compute unit hold different slots: the four-row passes
// of hot experts spread over the chip instead of queueing on a few SIMDs.
template <class S>
__device__ __forceinline__ ItemInfo decode_item(const LayerArgs &a, S &sm, int i, int ni1, int nlive) {
  ItemInfo it;
  const int nhc = a.nch2;
  it.fc2 = i >= ni1;
  const int q1 = it.fc2 ? i - ni1 : i;
  const int q0 = q1 / nlive;
  it.s = q1 - q0 * nlive;
  if (!it.fc2) {
    const int qt = q0 / a.nch1;
    it.kc = q0 - qt * a.nch1;
    it.hc = qt >> 1;
    it.tile = a.concat ? ((qt & 1) ? nhc + it.hc : it.hc) : qt;
  } else {
    it.kc = q0 / a.ntiles2;
    it.tile = q0 - it.kc * a.ntiles2;
    it.hc = it.kc;
  }
  it.e = __builtin_amdgcn_readfirstlane(sm.slot_e[it.s]);
  it.row0 = __builtin_amdgcn_readfirstlane(sm.slot_r0[it.s]);
  it.m = __builtin_amdgcn_readfirstlane(sm.slot_m[it.s]);
  it.K = it.fc2 ? a.I : a.H;
  it.N = it.fc2 ? a.H : 2 * a.I;
  return it;
}

// FC1's activation rows of an item (8 values per thread, 32 threads per
// row): x rows of the slot's tokens, loaded ahead of the weights.
template <int MRMAX, class S>
__device__ __forceinline__ u32x4_t load_x(const LayerArgs &a, S &sm, const ItemInfo &it, int tid) {
  const int per_row = kKC / 8;
  const bool xon = tid < MRMAX * per_row;
  const int xr = xon ? tid / per_row : 0;
  const int xk = (tid - xr * per_row) * 8;
  const int kabs = it.kc * kKC + xk;
  u32x4_t xv = {0u, 0u, 0u, 0u};
  if (!it.fc2 && xon && xr < it.m && kabs < it.K) {
    const int tok = sm.p2e[it.row0 + xr] / a.k;
    xv = *(const u32x4_t *)(a.x + (size_t)tok * it.K + kabs);
  }
  return xv;
}

template <int FMT>
__device__ __forceinline__ void issue_item(const LayerArgs &a, const ItemInfo &it, int wave, int lane,
                                           ItemLoads<FMT> &L) {
  issue_loads<FMT>(it.fc2 ? a.w2 : a.w1, it.fc2 ? a.s2 : a.s1, it.fc2 ? a.g2 : a.g1, it.e, it.K, it.N, it.tile,
                   it.kc, wave, lane, L);
}

// Stages the item's activations (FC1: its x rows; FC2: waits for its h chunk,
// then forms h from FC1's planes), runs the pass, stores the partial plane
// and counts; the last FC2 item of a column tile finalizes that tile, and the
// last finalize zeroes the counters.
template <int FMT, int MRMAX, class S>
__device__ __forceinline__ void run_item(const LayerArgs &a, S &sm, const ItemInfo &it, const ItemLoads<FMT> &L,
                                         u32x4_t xv, int nlive, int tid, int wave, int lane) {
  const int nhc = a.nch2;
  if (it.fc2) {
    if (tid == 0) {  // wait for h chunk hc of this slot (bounded)
      int32_t *c = sync_hchunk(a, it.s, it.hc);
      const int ready = hchunk_items(a, it.hc);
      int polls = 0;
      int ok = 1;
      while (__hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < ready) {
        if (++polls > a.max_polls) {
          __hip_atomic_fetch_or(sync_err(a), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ok = 0;
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      sm.flag = ok;
    }
    lds_barrier();
    asm volatile("" ::: "memory");
    stage_h(a, sm, it.row0, sm.flag >= 0 ? it.m : 0, it.hc, tid, MRMAX);
  } else {
    const int per_row = kKC / 8;
    if (tid < MRMAX * per_row) {
      const int xr = tid / per_row;
      *(u32x4_t *)&sm.g.xs[xr][(tid - xr * per_row) * 8] = xv;
    }
  }
  lds_barrier();
  item_dot_store<FMT, MRMAX>(a, sm, L, it.m, it.row0, it.tile, it.kc, it.K, it.N, it.fc2 ? a.part2 : a.part1, tid,
                             wave, lane);
  stores_done();
  lds_barrier();
  if (!it.fc2) {
    if (tid == 0)  // no value returned: the workgroup moves on at once
      __hip_atomic_fetch_add(sync_hchunk(a, it.s, it.hc), 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (tid == 0) sm.flag = count(sync_tile(a, it.tile)) == nlive * nhc - 1;
  lds_barrier();
  if (sm.flag) {  // uniform: the last FC2 item of this column tile finalizes it
    finalize_tile(a, sm, it.tile, tid);
    stores_done();
    lds_barrier();
    if (tid == 0) sm.flag = count(sync_done(a)) == a.ntiles2 - 1;
    lds_barrier();
    if (sm.flag) {  // uniform: every tile is final; zero the counters for the next call
      for (int x = tid; x < nlive * kLayerMaxHChunks; x += kThreads)
        if ((x & (kLayerMaxHChunks - 1)) < nhc)
          __hip_atomic_store(sync_hchunk(a, x / kLayerMaxHChunks, x & (kLayerMaxHChunks - 1)), 0, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
      for (int x = tid; x < a.ntiles2; x += kThreads)
        __hip_atomic_store(sync_tile(a, x), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (tid == 0) __hip_atomic_store(sync_done(a), 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

}  // namespace

// A workgroup takes items g, g + G, g + 2G, ... in order.  Every FC1 item
// an FC2 item waits for has a lower index: it belongs to this workgroup and
// already ran, or to another resident workgroup whose earlier items are FC1
// items (no wait) or FC2 items of earlier slots (by induction, they finish).
template <int FMT, int MRMAX>
__device__ __forceinline__ void layer_body(const LayerArgs &a) {
  __shared__ __attribute__((aligned(16))) LayerSmem<MRMAX> sm;
  const int tid0 = threadIdx.x;

  if (tid0 == 0) {
    sm.cold.idx = a.idx;
    sm.cold.wts = a.wts;
    sm.cold.offsets = a.offsets;
    sm.cold.p2e = a.p2e;
    sm.cold.e2p = a.e2p;
    sm.cold.out = a.out;
    sm.cold.alpha = a.alpha;
    sm.cold.beta = a.beta;
    sm.cold.limit = a.limit;
    sm.cold.E = a.E;
    sm.cold.T = a.T;
  }
  route_and_slots<MRMAX>(a, sm, tid0 >> 6, lane_id());
  const int nlive = __builtin_amdgcn_readfirstlane(sm.nlive);
  const int per1 = a.ntiles1 * a.nch1;
  const int per2 = a.nch2 * a.ntiles2;
  const int ni1 = nlive * per1;
  const int ni = ni1 + nlive * per2;

  for (int i = blockIdx.x; i < ni; i += gridDim.x) {  // uniform
    // thread-index-derived offsets are recomputed per item from an opaque
    // copy of the index: hoisted out of the loop they would stay live through
    // the dot products and push the four-row pass past 128 registers
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const ItemInfo it = decode_item(a, sm, i, ni1, nlive);
    const u32x4_t xv = load_x<MRMAX>(a, sm, it, tid);
    ItemLoads<FMT> L;
    issue_item<FMT>(a, it, wave, lane, L);
    run_item<FMT, MRMAX>(a, sm, it, L, xv, nlive, tid, wave, lane);
  }
  if (blockIdx.x == 0) write_routing(a, sm, tid0);
}

// Three workgroups per CU (168 VGPRs): with four (128 VGPRs) the body
// spilled and ran slower at every token count measured on MI355X (NVFP4
// E=256, H=2048, I=768: T=1 17.4 -> 16.5 us, T=2 21.7 -> 20.5, T=4 26.8 ->
// 25.6 with four-row passes, T=8 40.9 -> 39.8).
template <int FMT, int MRMAX>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void fp4_layer_kernel(LayerArgs a) {
  layer_body<FMT, MRMAX>(a);
}

// Rows per pass: one at one token, two at two, else four (an expert holds at
// most T rows).  At four tokens four-row passes (the hot experts' weights
// read once) ran 25.6 us against 27.3 us for two-row passes (MI355X, three
// workgroups per CU).
int layer_rows_per_pass(int T) { return T <= 1 ? 1 : (T <= 2 ? 2 : 4); }

int layer_max_items(const LayerArgs &a) {
  const int mr = layer_rows_per_pass(a.T);
  const int nexp = a.rows < a.E ? a.rows : a.E;
  const int nslots = a.T > mr ? (a.rows + nexp * (mr - 1)) / mr : nexp;
  return nslots * (a.ntiles1 * a.nch1 + a.nch2 * a.ntiles2);
}

namespace {

typedef void (*LayerKernel)(LayerArgs);

template <int FMT>
LayerKernel layer_kernel_fmt(int mr) {
  return mr == 1 ? fp4_layer_kernel<FMT, 1> : (mr == 2 ? fp4_layer_kernel<FMT, 2> : fp4_layer_kernel<FMT, 4>);
}

LayerKernel layer_kernel(int fmt, int mr) { return fmt == 0 ? layer_kernel_fmt<0>(mr) : layer_kernel_fmt<1>(mr); }

}  // namespace

hipError_t launch_fp4_layer(const LayerArgs &a, int fmt, hipStream_t s) {
  const int mr = layer_rows_per_pass(a.T);
  LayerKernel kern = layer_kernel(fmt, mr);
  // no more workgroups than fit on the chip at once: an FC2 item waits only
  // for items of workgroups that are resident
  int dev = 0, cus = 0, per_cu = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err == hipSuccess)
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kern), kThreads, 0);
  if (err != hipSuccess) return err;
  if (per_cu < 1 || cus < 1) return hipErrorInvalidConfiguration;
  const int items = layer_max_items(a);
  int grid = per_cu * cus;
  if (grid > items) grid = items;
  kern<<<dim3((unsigned)grid), dim3(kThreads), 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qmoe
