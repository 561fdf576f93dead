// FP4 (E2M1) weight-only decode GEMV over routed MoE rows, gfx950.
//
// What it computes (PR 31159 "[CUDA] Speed up the NVFP4 QMoE decode GEMV and
// enable it for MTP verify"; operator documentation sections 8, 9b.2, 12.1):
// for every permuted row p of expert e,
//   u[p][n] = g[e] * sum_b scale[e][b][n] * sum_{k in block b} a[p][k] * e2m1(code[e][k][n])
// then FC1 applies interleaved SwiGLU on (u[2j], u[2j+1]) and writes bf16 h,
// FC2 writes float32 y.
//
// gfx950 design:
// * A workgroup covers one 256-column tile of one routed expert and a k
//   chunk of W*64 rows (W = 4 waves; fewer when K is shorter).  In a wave, lanes 0..31 each own 8 consecutive
//   columns (one dword per k row: 32 lanes read one 128-byte line of a row)
//   and the two 32-lane halves own consecutive 32-row k ranges.
// * Weights and scales are read with buffer loads from a per-expert buffer
//   resource: the row offset is a scalar (no per-load vector address math)
//   and rows past K or columns past N fall outside the resource and read
//   as zero.  All 32 loads of a lane are issued before any decode.
// * Decode: a nibble zip and gfx950's FP4 -> bf16 conversion turn two k rows
//   of a lane's 8 columns into 8 K-paired bf16x2 registers (twelve VALU
//   instructions per 16 codes, no table, no branch); v_dot2c_f32_bf16 multiplies a K pair of
//   activations by a K pair of weights (one NVFP4 row), or 4x4x4 bf16 MFMA
//   blocks take four k of a column for up to four rows (several rows, and
//   one MXFP4 row).  Products are summed per scale block and the block scale
//   is applied once per (row, column, block).
// * Split-K inside the workgroup: the two halves of a wave add through a
//   lane swap, then the W waves through LDS, in a fixed order.  When K spans
//   several chunks each workgroup writes g * partial to the workspace and a
//   second, small kernel sums the chunks in order and runs the epilogue (the
//   two-pass split-K SwiGLU of section 12.1); kernel boundaries order the
//   passes: no fences, no atomics, deterministic sums.
// * Work items (expert slot, column tile) are spread round-robin over the 8
//   XCDs and all k chunks of an item land on the same XCD.
// * The routed experts are found on the device from expert_offsets (wave
//   ballots); grids are sized for the worst case and idle slots exit.  A
//   workgroup runs one pass over at most one row (single-token batches), two
//   rows (up to 3 tokens) or four rows; an expert holding more rows is dealt
//   out over several slots of at most a pass each (a wave prefix sum of the
//   per-expert group counts), so no workgroup runs longer than one pass.
// * Two fused modes (template MODE): 1, every workgroup of an FC1 launch
//   first runs the routing of all tokens (top-k per wave, one-wave expert
//   maps in LDS) and takes its expert from LDS; 2, FC2 stages its bf16
//   activations from FC1's split-K partial sums (planes in order, SwiGLU,
//   round to nearest even), so FC1 needs no epilogue launch.
#include "device_common.h"
#include "gemv_device.h"
#include "qmoe_internal.h"
#include "route_device.h"

namespace qmoe {

// FC1 epilogue of one column: even threads write h[p][col/2].
__device__ __forceinline__ void store_fc1(const GemvArgs &a, int p, int col, float u) {
  const float partner = __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(u)));
  if (col < a.N && (threadIdx.x & 1) == 0)
    a.out_bf16[(size_t)p * (a.N >> 1) + (col >> 1)] = (uint16_t)bf16_rne(swiglu(u, partner, a.alpha, a.beta, a.limit));
}

// Every row mode uses the same workgroup size.
template <int MRMAX>
constexpr int max_waves() { return kGemvMaxWaves; }

// Routing state of the fused prologue (up to 64 expanded rows).
struct RouteSmem {
  int32_t sidx[64];   // selected expert of expanded row t*k + j
  int32_t off[260];   // expert_offsets [E+1]
  int32_t p2e[64];
  int32_t e2p[64];
  int32_t cnt[256];
};

// Fused routing prologue (operator documentation section 2; the pages'
// fused routing + expert-map kernel, extended here to E <= 256 and up to 64
// expanded rows): the waves take the tokens in turn (one wave per token, the
// exact top-k of the routing kernels), then wave 0 ranks the rows by expert.
// Every workgroup computes the same maps; workgroup 0 writes them out for
// the later calls.
__device__ __forceinline__ void route_prologue(const GemvArgs &a, RouteSmem &rs, int W, int wave, int lane) {
  const int E = a.E, k = a.topk, T = a.route_T, R = a.rows;
  const bool writer = blockIdx.x == 0 && blockIdx.y == 0;
  for (int t = wave; t < T; t += W) {  // wave-uniform
    int sel;
    float wsel;
    topk_token(a.route_logits + (size_t)t * E, a.route_rw ? a.route_rw + (size_t)t * E : nullptr, E, k, lane, sel,
               wsel);
    if (lane < k) {
      rs.sidx[t * k + lane] = sel;
      if (writer) {
        a.route_idx[t * k + lane] = sel;
        a.route_w[t * k + lane] = wsel;
      }
    }
  }
  lds_barrier();
  if (wave == 0) build_maps_wave(rs.sidx, R, E, rs.off, rs.p2e, rs.e2p, rs.cnt);
  lds_barrier();
  if (writer) {
    for (int i = threadIdx.x; i <= E; i += W * 64) a.route_offsets[i] = rs.off[i];
    for (int i = threadIdx.x; i < R; i += W * 64) {
      a.route_p2e[i] = rs.p2e[i];
      a.route_e2p[i] = rs.e2p[i];
    }
  }
}

// FC1's SwiGLU folded into FC2's staging: a thread forms 4 h values of one
// row from the FC1 partial planes it holds (8 floats per plane: the gate and
// linear values), summing the planes in order from -0 as the split-K epilogue
// does (planes past h_nchunks add -0), then SwiGLU and bf16 RNE.
constexpr int kHPlanes = 8;  // planes loaded per round

struct HPart {
  float4 v[kHPlanes][2];
};

__device__ __forceinline__ void load_h_planes(const GemvArgs &a, int c0, int p, int kabs, bool live_row,
                                              HPart &hp) {
  // buffer loads: rows past the expert's count and planes past h_nchunks use
  // an out-of-range offset (no memory access, zeros) while every load is
  // still issued unconditionally
  const uint32_t plane = (uint32_t)a.rows * (uint32_t)(2 * a.K) * 4u;
  const __amdgpu_buffer_rsrc_t hr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.h_partials), (short)0, (int)(plane * (uint32_t)a.h_nchunks), 0x00020000);
  const uint32_t row = (uint32_t)p * (uint32_t)(2 * a.K) * 4u;
  const uint32_t o0 = row + 4u * (uint32_t)(a.h_concat ? kabs : 2 * kabs);
  const uint32_t o1 = row + 4u * (uint32_t)(a.h_concat ? a.K + kabs : 2 * kabs + 4);
#pragma unroll
  for (int g = 0; g < kHPlanes; ++g) {
    const bool on = live_row && c0 + g < a.h_nchunks;
    const uint32_t base = (uint32_t)(c0 + g) * plane;
    hp.v[g][0] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(hr, on ? base + o0 : kOutOfRange, 0, 0));
    hp.v[g][1] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(hr, on ? base + o1 : kOutOfRange, 0, 0));
  }
}

__device__ __forceinline__ void add_h_planes(const GemvArgs &a, int c0, const HPart &hp, float4 &s0, float4 &s1) {
#pragma unroll
  for (int g = 0; g < kHPlanes; ++g) {
    const bool live = c0 + g < a.h_nchunks;
    s0.x += live ? hp.v[g][0].x : -0.f;
    s0.y += live ? hp.v[g][0].y : -0.f;
    s0.z += live ? hp.v[g][0].z : -0.f;
    s0.w += live ? hp.v[g][0].w : -0.f;
    s1.x += live ? hp.v[g][1].x : -0.f;
    s1.y += live ? hp.v[g][1].y : -0.f;
    s1.z += live ? hp.v[g][1].z : -0.f;
    s1.w += live ? hp.v[g][1].w : -0.f;
  }
}

// Four bf16 h values (packed) from the summed planes.
__device__ __forceinline__ u32x2_t h_from_sums(const GemvArgs &a, float4 s0, float4 s1) {
  float gt[4], ln[4];
  if (a.h_concat) {
    gt[0] = s0.x; gt[1] = s0.y; gt[2] = s0.z; gt[3] = s0.w;
    ln[0] = s1.x; ln[1] = s1.y; ln[2] = s1.z; ln[3] = s1.w;
  } else {
    gt[0] = s0.x; ln[0] = s0.y; gt[1] = s0.z; ln[1] = s0.w;
    gt[2] = s1.x; ln[2] = s1.y; gt[3] = s1.z; ln[3] = s1.w;
  }
  uint32_t h[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = bf16_rne(swiglu(gt[i], ln[i], a.h_alpha, a.h_beta, a.h_limit));
  return u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
}

// MODE 0: plain; 1: fused routing prologue (FC1); 2: h formed from FC1's
// partials while staging (FC2).  The plain single-pass variants are held to
// 128 VGPRs (four waves per SIMD), which the four-row body fits without
// spilling once its weight registers may die as they are decoded (FC1 call
// at T=4 16.1 -> 15.5 us); the other variants would spill under that cap.
// A workgroup runs one pass of at most MRMAX rows: an expert with more rows
// is dealt out over several slots (gemv_plan), so the weight registers die
// as they are decoded.
template <int FMT, int MRMAX, int MODE>
__global__ __launch_bounds__(max_waves<MRMAX>() * 64) __attribute__((amdgpu_waves_per_eu(MODE == 0 ? 4 : 1))) void fp4_gemv_kernel(GemvArgs a) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  constexpr int NBLK = kGemvLaneK / B;
  __shared__ __attribute__((aligned(16))) Smem<MRMAX> sm;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  const int W = a.waves;
  const int KC = W * kGemvWaveK;

  // Work item: XCD-aware grid (x = k chunk * 8 + XCD, y = group of 8
  // items); the linear dispatch order (x fastest) deals consecutive
  // workgroups round-robin over the 8 XCDs, so item 8y + x % 8 runs on XCD
  // x % 8 with all its k chunks.
  const int kc = (int)blockIdx.x >> 3;
  const int item = (int)blockIdx.y * 8 + ((int)blockIdx.x & 7);
  if (item >= a.nslots * a.ntiles) return;
  const int slot = item / a.ntiles;
  const int tile = item - slot * a.ntiles;

  // Routing: from the maps in memory, or computed here (fused prologue).
  const int32_t *offs = a.offsets;
  const int32_t *p2e = a.p2e;
  if constexpr (MODE == 1) {
    __shared__ __attribute__((aligned(16))) RouteSmem rs;
    route_prologue(a, rs, W, wave, lane);
    offs = rs.off;
    p2e = rs.p2e;
  }

  // FC1 gathers its x rows through perm_to_expanded (at most 64 rows on this
  // path): fetch it together with the offsets, one lane per row.
  const int p2e_l = (a.fc1 && lane < a.rows) ? p2e[lane] : 0;
  int row0 = 0, m = 0;
  const int e = a.split_rows > 0 ? find_slot_group(offs, a.E, slot, a.split_rows, row0, m)
                                 : find_slot_expert(offs, a.E, slot, row0, m);
  if (e < 0) return;  // uniform over the workgroup

  // ---- activation rows of the first pass, then the weights ---------------------
  // The activation load goes out before the 32 weight loads: memory returns in
  // issue order, so staging then waits for x alone, and the dot products can
  // start on the first weight rows while the rest are still arriving.
  // MRMAX * KC / 8 <= W * 64, so one 16-byte load per thread covers a pass.
  static_assert(MRMAX <= 8, "one staging load per thread per pass");
  const int per_row = KC / 8;
  const int mr0 = m < MRMAX ? m : MRMAX;
  u32x4_t xv0 = {0u, 0u, 0u, 0u};
  int xr0 = 0, xk0 = 0;
  const bool xon0 = tid < MRMAX * per_row;
  {
    const int r = xon0 ? tid / per_row : 0;
    const int kk = (tid - r * per_row) * 8;
    const int kabs = kc * KC + kk;
    const int p = row0 + r;
    const int tok = __shfl(p2e_l, p & 63, 64) / a.topk;
    if (MODE != 2 && xon0 && r < mr0 && kabs < a.K) {
      const int src = a.fc1 ? tok : p;
      xv0 = *(const u32x4_t *)(a.act + (size_t)src * a.K + kabs);
    }
    xr0 = r;
    xk0 = kk;
  }
  // MODE 2: this thread's FC1 partial planes of the first pass (4 h values of
  // one row), issued before the weights
  const int per_row4 = KC / 4;
  const bool hon0 = MODE == 2 && tid < MRMAX * per_row4;
  const int hr0 = hon0 ? tid / per_row4 : 0;
  const int hk0 = (tid - hr0 * per_row4) * 4;
  HPart hp0;
  if constexpr (MODE == 2) {
    const int kabs = kc * KC + hk0;
    load_h_planes(a, 0, row0 + hr0, kabs, hon0 && hr0 < mr0 && kabs < a.K, hp0);
  }

  // ---- weight and scale loads of this lane ----------------------------------
  const int nl = lane & 31;
  const int g = wave * 2 + (lane >> 5);  // 32-row k group inside the chunk
  const int col0 = tile * kGemvTileN + nl * 8;
  const int kl = kc * KC + g * kGemvLaneK;  // first k row of this lane
  const uint32_t rowbytes = (uint32_t)(a.N >> 1);
  const int KB = a.K / B;
  // uniform_ptr keeps the descriptors in scalar registers: the compiler may
  // otherwise form the expert's base address on the vector ALU and wrap each
  // load in a readfirstlane loop
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.w + (size_t)e * a.K * rowbytes), (short)0, (int)((uint32_t)a.K * rowbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t sr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.scales + (size_t)e * KB * a.N), (short)0, (int)((uint32_t)KB * a.N), 0x00020000);
  const bool col_ok = col0 < a.N;
  const uint32_t woff = col_ok ? (uint32_t)kl * rowbytes + (uint32_t)(col0 >> 1) : kOutOfRange;
  const uint32_t soff = col_ok ? (uint32_t)(kl / B) * (uint32_t)a.N + (uint32_t)col0 : kOutOfRange;
  // scales first: their decode does not wait for the weight rows
  u32x2_t SB[2];
#pragma unroll
  for (int b = 0; b < 2; ++b)
    SB[b] = (b < NBLK) ? __builtin_amdgcn_raw_buffer_load_b64(sr, soff, b * a.N, 0) : u32x2_t{0u, 0u};
  uint32_t A[kGemvLaneK];
#pragma unroll
  for (int i = 0; i < kGemvLaneK; ++i)
    A[i] = __builtin_amdgcn_raw_buffer_load_b32(wr, woff, i * (int)rowbytes, kBufNontemporal);
  const float gs = a.gscale ? a.gscale[e] : 1.0f;

  // ---- the pass over the slot's rows (at most MRMAX) ----------------------------
  // Straight-line code: each dot product waits only for its own weight rows.
  // The body stays a lambda taking the first row (called once, with 0): the
  // same body written inline compiled to a slower schedule (T=4 decode layer
  // 30.8 -> 32.4 us, measured A/B on one box).
  auto pass = [&](const int rbase) {
    const int rem = m - rbase;
    const int mr = rem < MRMAX ? rem : MRMAX;
    // Stage the chunk's activation rows (rows past mr as zeros): one thread
    // per 8 values; the first pass's load was issued with the weights.
    if constexpr (MODE == 2) {
      // h from FC1's partial planes (rows past mr and columns past K: zeros)
      const int r = hr0;
      const int kabs = kc * KC + hk0;
      const bool on = hon0 && r < mr && kabs < a.K;
      float4 s0 = make_float4(-0.f, -0.f, -0.f, -0.f), s1 = s0;
      for (int c0 = 0; c0 < a.h_nchunks; c0 += kHPlanes) {
        HPart hp;
        if (rbase == 0 && c0 == 0) {
          hp = hp0;
        } else {
          load_h_planes(a, c0, row0 + rbase + r, kabs, on, hp);
        }
        add_h_planes(a, c0, hp, s0, s1);
      }
      if (hon0) *(u32x2_t *)&sm.xs[r][hk0] = on ? h_from_sums(a, s0, s1) : u32x2_t{0u, 0u};
    } else if (rbase == 0) {
      if (xon0) *(u32x4_t *)&sm.xs[xr0][xk0] = xv0;
    } else {
      const int i = tid;
      const bool on = i < MRMAX * per_row;
      const int r = on ? i / per_row : 0;
      const int kk = (i - r * per_row) * 8;
      const int kabs = kc * KC + kk;
      const int p = row0 + rbase + r;
      const int tok = __shfl(p2e_l, p & 63, 64) / a.topk;
      u32x4_t v = {0u, 0u, 0u, 0u};
      if (on && r < mr && kabs < a.K) {
        const int src = a.fc1 ? tok : p;
        v = *(const u32x4_t *)(a.act + (size_t)src * a.K + kabs);
      }
      if (on) *(u32x4_t *)&sm.xs[r][kk] = v;
    }
    lds_barrier();

    lane_pass<FMT, MRMAX, false>(sm, A, SB, g, wave, lane, 0, mr);
    lds_barrier();

    // ---- reduce the W waves (fixed order); one thread per column ------------
    for (int cl = tid; cl < kGemvTileN; cl += W * 64) {
      const int col = tile * kGemvTileN + cl;
      for (int r = 0; r < mr; ++r) {
        float s = sm.red[0][r][cl];
        for (int q = 1; q < W; ++q) s += sm.red[q][r][cl];
        const int p = row0 + rbase + r;
        const float u = gs * s;
        if (a.nchunks > 1 || a.force_partials || a.concat) {
          if (col < a.N) a.partials[((size_t)kc * a.rows + p) * a.N + col] = u;
        } else if (a.fc1) {
          store_fc1(a, p, col, u);
        } else if (col < a.N) {
          a.out_f32[(size_t)p * a.N + col] = u;
        }
      }
    }
  };
  pass(0);
}

// Split-K epilogue: sums the k-chunk partials of every (row, column) in chunk
// order, then SwiGLU -> bf16 h (FC1) or float32 y (FC2).  One thread owns 4
// output columns (FC1 interleaved: two gate/linear pairs; FC1 concatenated:
// four h columns, their gates at j and linear values at N/2 + j), one wave
// 256 of one row; rows in grid x.  Chunks are read kEpiGroup at a time with
// every load unconditional (indices past the last chunk re-read it and
// contribute -0, which leaves any float sum unchanged), so a row's partials
// are in flight together rather than one memory round trip per chunk.
constexpr int kEpiGroup = 8;

__device__ __forceinline__ float4 sum_chunks(const float *src, size_t plane, int nchunks) {
  float4 s = make_float4(-0.f, -0.f, -0.f, -0.f);
  for (int c = 0; c < nchunks; c += kEpiGroup) {
    float4 v[kEpiGroup];
#pragma unroll
    for (int g = 0; g < kEpiGroup; ++g) {
      const int q = c + g < nchunks ? c + g : nchunks - 1;
      v[g] = *(const float4 *)(src + (size_t)q * plane);
    }
#pragma unroll
    for (int g = 0; g < kEpiGroup; ++g) {
      const bool live = c + g < nchunks;
      s.x += live ? v[g].x : -0.f;
      s.y += live ? v[g].y : -0.f;
      s.z += live ? v[g].z : -0.f;
      s.w += live ? v[g].w : -0.f;
    }
  }
  return s;
}

__global__ __launch_bounds__(64) void splitk_epilogue_kernel(GemvArgs a) {
  const int p = blockIdx.x;
  const int col = (blockIdx.y * 64 + threadIdx.x) * 4;
  const size_t plane = (size_t)a.rows * a.N;
  const float *row = a.partials + (size_t)p * a.N;
  if (a.concat) {
    const int I = a.N >> 1;
    if (col >= I) return;
    const float4 gt = sum_chunks(row + col, plane, a.nchunks);
    const float4 ln = sum_chunks(row + I + col, plane, a.nchunks);
    uint2 o;
    o.x = bf16_rne(swiglu(gt.x, ln.x, a.alpha, a.beta, a.limit)) |
          (bf16_rne(swiglu(gt.y, ln.y, a.alpha, a.beta, a.limit)) << 16);
    o.y = bf16_rne(swiglu(gt.z, ln.z, a.alpha, a.beta, a.limit)) |
          (bf16_rne(swiglu(gt.w, ln.w, a.alpha, a.beta, a.limit)) << 16);
    *(uint2 *)(a.out_bf16 + (size_t)p * I + col) = o;
    return;
  }
  if (col >= a.N) return;
  const float4 s = sum_chunks(row + col, plane, a.nchunks);
  if (a.fc1) {
    const uint32_t h0 = bf16_rne(swiglu(s.x, s.y, a.alpha, a.beta, a.limit));
    const uint32_t h1 = bf16_rne(swiglu(s.z, s.w, a.alpha, a.beta, a.limit));
    *(uint32_t *)(a.out_bf16 + (size_t)p * (a.N >> 1) + (col >> 1)) = h0 | (h1 << 16);
  } else {
    *(float4 *)(a.out_f32 + (size_t)p * a.N + col) = s;
  }
}

hipError_t launch_splitk_epilogue(const GemvArgs &a, hipStream_t s) {
  const int cols = a.concat ? (a.N >> 1) : a.N;
  const dim3 g2((unsigned)a.rows, (unsigned)((cols / 4 + 63) / 64));
  splitk_epilogue_kernel<<<g2, 64, 0, s>>>(a);
  return hipGetLastError();
}

// Four waves (a 256-row k chunk) per workgroup: the kernel is bound by VALU
// issue (bit-assembled decode), so many small workgroups balance the CUs
// best; measured against 2, 8 and 16 waves on the decode and MTP layers.
// Shorter K uses fewer waves.
static void plan_chunks(int items, int K, int maxw, int &nchunks, int &waves) {
  (void)items;
  const int slabs = (K + kGemvWaveK - 1) / kGemvWaveK;
  const int w = maxw < 4 ? maxw : 4;
  waves = slabs < w ? slabs : w;
  nchunks = (slabs + waves - 1) / waves;
}

static int plan_max_waves(int max_rows_per_expert) {
  (void)max_rows_per_expert;
  return kGemvMaxWaves;
}

size_t gemv_workspace_bytes(int32_t rows, int32_t max_rows_per_expert, int32_t E, int32_t K, int32_t N,
                            bool force_partials) {
  const int nslots = rows < E ? rows : E;
  const int ntiles = (N + kGemvTileN - 1) / kGemvTileN;
  int nchunks, waves;
  plan_chunks(nslots * ntiles, K, plan_max_waves(max_rows_per_expert), nchunks, waves);
  const size_t part = (nchunks > 1 || force_partials) ? (size_t)nchunks * rows * N * sizeof(float) : 0;
  return part > 256 ? part : 256;
}

// Rows per pass: one when no expert can hold more than one row (one
// token), two for up to three tokens, else four.
static int rows_per_pass(int max_rows_per_expert) {
  return max_rows_per_expert <= 1 ? 1 : (max_rows_per_expert <= 3 ? 2 : 4);
}

void gemv_plan(GemvArgs &a, int max_rows_per_expert, void *ws) {
  // An expert that may hold more rows than a pass is dealt out over several
  // slots of at most a pass each (workgroups of equal length; no pass loop).
  // Slots needed: sum_e ceil(m_e / G) <= (rows + min(E, rows) * (G - 1)) / G.
  const int mr = rows_per_pass(max_rows_per_expert);  // 1, 2 or 4: find_slot_group takes a power of two
  const int nexp = a.rows < a.E ? a.rows : a.E;
  a.split_rows = max_rows_per_expert > mr ? mr : 0;
  a.nslots = a.split_rows ? (a.rows + nexp * (mr - 1)) / mr : nexp;
  a.ntiles = (a.N + kGemvTileN - 1) / kGemvTileN;
  plan_chunks(a.nslots * a.ntiles, a.K, plan_max_waves(max_rows_per_expert), a.nchunks, a.waves);
  a.partials = (float *)ws;
}

hipError_t launch_fp4_gemv(const GemvArgs &a, int fmt, int max_rows_per_expert, hipStream_t s) {
  const int items = a.nslots * a.ntiles;
  const dim3 grid((unsigned)(8 * a.nchunks), (unsigned)((items + 7) / 8));
  const dim3 block((unsigned)(a.waves * 64));
  // one pass of at most mr rows per workgroup: an expert holding more rows
  // (a token selects an expert at most once, so at most max_rows_per_expert)
  // was split over slots by gemv_plan
  const int mr = rows_per_pass(max_rows_per_expert);
#define QMOE_GEMV_LAUNCH(F, M)                               \
  if (mr == 1)                                               \
    fp4_gemv_kernel<F, 1, M><<<grid, block, 0, s>>>(a);      \
  else if (mr == 2)                                          \
    fp4_gemv_kernel<F, 2, M><<<grid, block, 0, s>>>(a);      \
  else                                                       \
    fp4_gemv_kernel<F, 4, M><<<grid, block, 0, s>>>(a);
  const int mode = a.route_logits ? 1 : (a.h_partials ? 2 : 0);
  if (fmt == 0) {
    if (mode == 1) {
      QMOE_GEMV_LAUNCH(0, 1)
    } else if (mode == 2) {
      QMOE_GEMV_LAUNCH(0, 2)
    } else {
      QMOE_GEMV_LAUNCH(0, 0)
    }
  } else {
    if (mode == 1) {
      QMOE_GEMV_LAUNCH(1, 1)
    } else if (mode == 2) {
      QMOE_GEMV_LAUNCH(1, 2)
    } else {
      QMOE_GEMV_LAUNCH(1, 0)
    }
  }
#undef QMOE_GEMV_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || a.force_partials || (a.nchunks == 1 && !a.concat)) return err;
  return launch_splitk_epilogue(a, s);
}

}  // namespace qmoe
