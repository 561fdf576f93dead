// FP8 E4M3 weight-only (W8A16) decode GEMV and dequant for gfx950.
//
// Weights are raw E4M3FN bytes laid out [E][N][K] (each output column's K
// weights contiguous) with one float32 global scale per expert and no block
// scales ("MoE and QMoE -- CUDA Operator Documentation", sections 6.4 and
// 10: the product is scaled by the expert's global scale in the epilogue).
//
// GEMV: a column's K bytes are contiguous, so 16 lanes (one DPP row) share a
// column and each lane loads 16 consecutive k with one 16-byte load.  A lane
// row covers CPR columns (1 for K >= 1536, 2 for K >= 768, else 4, so a lane
// keeps up to 8 loads in flight even for short K), a wave 4 * CPR columns, a
// workgroup of 4 waves 16 * CPR, over the whole K in passes (8 loads per lane
// per pass): there is no split-K and no second launch.  Rows go in passes of
// up to 8 per workgroup, so any batch works; a prefill batch re-reads an
// expert's columns (from L2) once per 8 rows.
// The hardware FP8 -> bf16 conversion is exact; the k pairs meet the
// activation pairs in dot2 instructions.  The 16 per-lane partial sums of a
// column are added with a symmetric DPP butterfly inside the row, which
// leaves the same value in all 16 lanes.
#include "device_common.h"
#include "qmoe_internal.h"
#include "grouped_sched.h"

namespace qmoe {

constexpr int kF8Waves = 4;                          // measured against 8 and 16 (fewer, larger workgroups: slower)
constexpr int kF8Loads = 8;                          // 16-byte loads per lane per pass
constexpr int kF8PassK = 16 * 16 * kF8Loads;         // 2048 k per pass (CPR = 1)
constexpr int kF8TileN1 = kF8Waves * 4;              // 16 columns per workgroup and column per lane row
static_assert(kF8Waves * 64 * 8 >= kF8PassK, "one 8-value staging load per thread covers a pass");
constexpr uint32_t kF8OutOfRange = 0x80000000u;

__device__ __forceinline__ float row16_sum(float v) {
  auto add = [](float x, uint32_t y) { return x + __uint_as_float(y); };
  v = add(v, dpp_u32<kDppXor1>(__float_as_uint(v)));
  v = add(v, dpp_u32<kDppXor2>(__float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowHalfMirror>(__float_as_uint(v)));
  v = add(v, dpp_u32<kDppRowMirror>(__float_as_uint(v)));
  return v;
}

__device__ __forceinline__ uint32_t fp8x2_lo(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, false));
}
__device__ __forceinline__ uint32_t fp8x2_hi(uint32_t v) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, true));
}

template <int MRMAX, int CPR>
__global__ __launch_bounds__(kF8Waves * 64) void fp8_gemv_kernel(GemvArgs a) {
  constexpr int PASSK = kF8PassK / CPR;       // k per pass: CPR columns x PASSK / 256 loads per lane
  constexpr int NLD = PASSK / 256;
  __shared__ __attribute__((aligned(16))) uint16_t xs[MRMAX][PASSK];
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  // Work item: items are dealt to the 8 XCDs round-robin (workgroup order),
  // so the idle slots past the batch's distinct-expert count, which sit at the
  // end of the item range, are spread over all XCDs.
  const int item = blockIdx.x;
  if (item >= a.nslots * a.ntiles) return;
  const int slot = item / a.ntiles;
  const int tile = item - slot * a.ntiles;

  int row0 = 0, m = 0;
  const int e = find_slot_expert(a.offsets, a.E, slot, row0, m);
  if (e < 0) return;  // uniform over the workgroup

  // lane row rr of the wave takes columns base + 4 j + rr (j < CPR): an
  // interleaved gate / linear pair sits in lane rows 2i, 2i+1 for every j
  const int col0 = (tile * kF8Waves + wave) * 4 * CPR + (lane >> 4);
  const int q = lane & 15;
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      uniform_ptr(a.w + (size_t)e * a.N * a.K), (short)0, (int)((uint32_t)a.N * (uint32_t)a.K), 0x00020000);
  const float gs = a.gscale[e];

#pragma nounroll
  for (int rbase = 0; rbase < m; rbase += MRMAX) {
    const int rem = m - rbase;
    const int mr = rem < MRMAX ? rem : MRMAX;
    // source rows of the pass: FC1 gathers x by token through
    // perm_to_expanded, one lane per row, one memory round trip
    const int pl = row0 + rbase + (lane < mr ? lane : 0);
    const int srcl = a.fc1 ? a.p2e[pl] / a.topk : pl;
    int src[MRMAX];
#pragma unroll
    for (int r = 0; r < MRMAX; ++r) src[r] = __shfl(srcl, r < mr ? r : 0, 64);
    float acc[CPR][MRMAX];
#pragma unroll
    for (int j = 0; j < CPR; ++j)
#pragma unroll
      for (int r = 0; r < MRMAX; ++r) acc[j][r] = 0.f;

#pragma nounroll
    for (int k0 = 0; k0 < a.K; k0 += PASSK) {
      // activation rows of the pass first (memory returns in issue order),
      // then this lane's weight bytes
      // every load unconditional (clamped address; rows past mr and k past
      // K zeroed afterwards), so none waits for another
      const int kx = k0 + tid * 8;
      const bool xon = tid * 8 < PASSK && kx < a.K;
      const int kxc = kx < a.K ? kx : a.K - 8;
      u32x4_t xv[MRMAX];
#pragma unroll
      for (int r = 0; r < MRMAX; ++r) xv[r] = *(const u32x4_t *)(a.act + (size_t)src[r] * a.K + kxc);
#pragma unroll
      for (int r = 0; r < MRMAX; ++r)
        if (!(xon && r < mr)) xv[r] = u32x4_t{0u, 0u, 0u, 0u};
      // keep the activation loads ahead of the weights: staging then waits
      // for them alone
      __builtin_amdgcn_sched_barrier(0);
      u32x4_t W[CPR][NLD];
#pragma unroll
      for (int j = 0; j < CPR; ++j)
#pragma unroll
        for (int i = 0; i < NLD; ++i) {
          const int col = col0 + 4 * j;
          const int kk = k0 + i * 256 + q * 16;
          const uint32_t voff =
              (col < a.N && kk < a.K) ? (uint32_t)col * (uint32_t)a.K + (uint32_t)kk : kF8OutOfRange;
          W[j][i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wr, voff, 0, 2));
        }
      if (tid * 8 < PASSK) {
#pragma unroll
        for (int r = 0; r < MRMAX; ++r) *(u32x4_t *)&xs[r][tid * 8] = xv[r];
      }
      lds_barrier();
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
#pragma unroll
        for (int j = 0; j < CPR; ++j) {
          uint32_t w2[8];
          w2[0] = fp8x2_lo(W[j][i].x);
          w2[1] = fp8x2_hi(W[j][i].x);
          w2[2] = fp8x2_lo(W[j][i].y);
          w2[3] = fp8x2_hi(W[j][i].y);
          w2[4] = fp8x2_lo(W[j][i].z);
          w2[5] = fp8x2_hi(W[j][i].z);
          w2[6] = fp8x2_lo(W[j][i].w);
          w2[7] = fp8x2_hi(W[j][i].w);
#pragma unroll
          for (int r = 0; r < MRMAX; ++r) {
            if (MRMAX > 1 && r >= mr) break;  // uniform
            const u32x4_t x0 = *(const u32x4_t *)&xs[r][i * 256 + q * 16];
            const u32x4_t x1 = *(const u32x4_t *)&xs[r][i * 256 + q * 16 + 8];
            float v = acc[j][r];
            v = dot2_bf16(x0.x, w2[0], v);
            v = dot2_bf16(x0.y, w2[1], v);
            v = dot2_bf16(x0.z, w2[2], v);
            v = dot2_bf16(x0.w, w2[3], v);
            v = dot2_bf16(x1.x, w2[4], v);
            v = dot2_bf16(x1.y, w2[5], v);
            v = dot2_bf16(x1.z, w2[6], v);
            v = dot2_bf16(x1.w, w2[7], v);
            acc[j][r] = v;
          }
        }
      }
      lds_barrier();  // the next pass overwrites xs
    }

    // column sums, global scale, outputs
#pragma unroll
    for (int j = 0; j < CPR; ++j) {
      const int col = col0 + 4 * j;
      const bool col_ok = col < a.N;
#pragma unroll
      for (int r = 0; r < MRMAX; ++r) {
        if (MRMAX > 1 && r >= mr) break;  // uniform
        const float u = gs * row16_sum(acc[j][r]);
        const int p = row0 + rbase + r;
        if (a.fc1 && !a.concat) {
          // gate (even) columns in lane rows 0 / 2 meet their linear values
          // in lane rows 1 / 3
          const float partner = __shfl_xor(u, 16, 64);
          if (q == 0 && ((lane >> 4) & 1) == 0 && col_ok)
            a.out_bf16[(size_t)p * (a.N >> 1) + (col >> 1)] =
                (uint16_t)bf16_rne(swiglu(u, partner, a.alpha, a.beta, a.limit));
        } else if (q == 0 && col_ok) {
          a.out_f32[(size_t)p * a.N + col] = u;  // FC2 y, or FC1 u for the concatenated layout
        }
      }
    }
  }
}

// ---- prefill: grouped GEMM with bf16 MFMA ------------------------------------
// Work item = (expert, 64-row m tile, 256-column n tile) as on the FP4
// grouped path; 8 waves, wave w owns columns 32w..32w+31 (two 16-column MFMA
// tiles) for every live 16-row sub-tile, v_mfma_f32_16x16x32_bf16, K in
// 128-k slices.  The [N][K] layout gives each MFMA B operand (8 consecutive
// k of one column) as 8 contiguous bytes: a column's 128 bytes of a slice
// are copied into LDS (8-byte units XOR-swizzled by column), read back with
// one ds_read_b64 per operand and converted with four exact FP8 -> bf16
// conversions.  Global loads run two slices ahead in registers, LDS is
// double buffered; the global scale multiplies the accumulator.  Persistent
// workgroups (one per CU) stream fixed item lists as on the FP4 path
// (grouped_sched.h): the next item's loads overlap the current item's tail.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kF8BM = 64;
constexpr int kF8BK = 128;                          // k per slice: one 128-byte line of a column
constexpr int kF8CWaves = 8;                        // consumer waves, 32 columns each
constexpr int kF8LWaves = 4;                        // loader waves
constexpr int kF8BN = kF8CWaves * 32;               // columns per work item
constexpr int kF8GThreads = (kF8CWaves + kF8LWaves) * 64;
constexpr int kF8LThreads = kF8LWaves * 64;
constexpr int kF8Units = kF8BK / 8;                 // 8-k units per slice (B: 8 bytes, A: 16 bytes)
constexpr int kF8ALoads = kF8BM * kF8Units / kF8LThreads;  // 16-byte A loads per loader thread
constexpr int kF8LPC = kF8BK / 16;                  // lanes per column (16 bytes each)
constexpr int kF8CPP = kF8LThreads / kF8LPC;        // columns per load pass
constexpr int kF8BLoads = kF8BN / kF8CPP;           // 16-byte B loads per loader thread
static_assert(kF8ALoads * kF8LThreads == kF8BM * kF8Units && kF8BN % kF8CPP == 0 &&
                  (kF8Units & (kF8Units - 1)) == 0, "tile shape");
static_assert(kF8BM == kGBM, "m tile of the item lists");

struct F8GroupedSmem {
  u32x4_t a[2][kF8BM][kF8Units];    // activations, 16-byte chunk c of row r at c ^ (r % units)
  uint8_t b[2][kF8BN][kF8BK];       // weight bytes, 8-byte unit u of column n at u ^ (n % units)
  GroupedPre pre;                   // set-up only
  GroupedItems it;                  // this workgroup's items
  uint32_t ready[2];                // per buffer: loader-wave stores of its slices (4 per slice)
  uint32_t done[2];                 // per buffer: consumer-wave reads of its slices (8 per slice)
  uint32_t abort;                   // set when a wait ran past its bound
};

struct F8SliceRegs {
  u32x4_t A[kF8ALoads];   // activation chunks
  u32x4_t B[kF8BLoads];   // columns cb + j * kF8CPP, bytes 16 * bq .. +15 of the slice
};

__device__ __forceinline__ bf16x8_t fp8_operand(u32x2_t d) {
  u32x4_t o;
  o.x = fp8x2_lo(d.x);
  o.y = fp8x2_hi(d.x);
  o.z = fp8x2_lo(d.y);
  o.w = fp8x2_hi(d.y);
  return __builtin_bit_cast(bf16x8_t, o);
}

__global__ __launch_bounds__(kF8GThreads) __attribute__((amdgpu_waves_per_eu(3))) void fp8_grouped_kernel(GemvArgs a) {
  __shared__ __attribute__((aligned(16))) F8GroupedSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();

  const int nt = build_items(a, sm.pre, sm.it, kF8BN, kF8GThreads, tid, wave, lane);
  if (nt == 0) return;  // uniform
  const int steps = (a.K + kF8BK - 1) / kF8BK;  // K % 64 == 0: the last slice of an item may be half
  const int ktail = a.K - (steps - 1) * kF8BK;  // k in the last slice
  const int total = nt * steps;
  if (tid == 0) {
    sm.ready[0] = sm.ready[1] = 0u;
    sm.done[0] = sm.done[1] = 0u;
    sm.abort = 0u;
  }
  __syncthreads();

  // Loader and consumer wave groups hand slices over through per-buffer
  // counts in LDS, as on the FP4 path (grouped.hip).
  if (wave >= kF8CWaves) {
    // ---- loaders (buffer loads; the item-dependent vector offsets formed once
    // per item, the slice in the scalar offset; chunks past K in a half last
    // slice load as zero; slices past the last item load nothing) -------------
    const int lt_id = tid - kF8CWaves * 64;
    const int act_rows = a.fc1 ? a.rows / a.topk : a.rows;
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(a.act), (short)0, (int)((uint32_t)act_rows * (uint32_t)a.K * 2u), 0x00020000);
    int ar[kF8ALoads], aq[kF8ALoads];
    uint32_t atail[kF8ALoads];
#pragma unroll
    for (int i = 0; i < kF8ALoads; ++i) {
      const int c = lt_id + i * kF8LThreads;
      ar[i] = c / kF8Units;
      aq[i] = c % kF8Units;
      atail[i] = aq[i] * 8 >= ktail ? kF8OutOfRange : 0u;
    }
    const int cb = lt_id / kF8LPC, bq = lt_id % kF8LPC;  // columns cb + j * kF8CPP; 16 bytes bq of the slice
    const uint32_t btail = bq * 16 >= ktail ? kF8OutOfRange : 0u;
    int lt = 0, lks = 0, e = 0;
    uint32_t avoff[kF8ALoads], bvoff[kF8BLoads];
#pragma unroll
    for (int i = 0; i < kF8ALoads; ++i) avoff[i] = kF8OutOfRange;
#pragma unroll
    for (int j = 0; j < kF8BLoads; ++j) bvoff[j] = kF8OutOfRange;
    // Every loader thread issues the same loads for every slice, also past
    // the last one, with no branch around a load, so the compiler's wait
    // counts stay exact.
    auto load_slice = [&](F8SliceRegs &r) {
      const bool dead = lt >= nt;  // uniform
      if (lks == 0 && !dead) {     // uniform
        e = __builtin_amdgcn_readfirstlane(sm.it.item[lt][0]);
        const int n0 = __builtin_amdgcn_readfirstlane(sm.it.item[lt][3]);
#pragma unroll
        for (int i = 0; i < kF8ALoads; ++i) {
          const int srow = sm.it.src[lt][ar[i]];
          avoff[i] = srow >= 0 ? (uint32_t)srow * (uint32_t)a.K * 2u + (uint32_t)(aq[i] * 16) : kF8OutOfRange;
        }
#pragma unroll
        for (int j = 0; j < kF8BLoads; ++j) {
          const int col = n0 + cb + kF8CPP * j;
          bvoff[j] = col < a.N ? (uint32_t)col * (uint32_t)a.K + (uint32_t)(bq * 16) : kF8OutOfRange;
        }
      }
      const int k0 = lks * kF8BK;
      const uint32_t kill = dead ? kF8OutOfRange : 0u;                      // uniform
      const uint32_t halfm = (lks == steps - 1 && ktail < kF8BK) ? ~0u : 0u;  // uniform
      const int ao = __builtin_amdgcn_readfirstlane(k0 * 2), bo = __builtin_amdgcn_readfirstlane(k0);
#pragma unroll
      for (int i = 0; i < kF8ALoads; ++i)
        r.A[i] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(arsrc, avoff[i] | kill | (atail[i] & halfm), ao, 0));
      const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(a.w + (size_t)e * a.N * a.K), (short)0, (int)((uint32_t)a.N * (uint32_t)a.K), 0x00020000);
#pragma unroll
      for (int j = 0; j < kF8BLoads; ++j)
        r.B[j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(wrsrc, bvoff[j] | kill | (btail & halfm), bo, 2));
      if (++lks == steps) {
        lks = 0;
        ++lt;
      }
    };
    auto store_slice = [&](int buf, const F8SliceRegs &r) {
#pragma unroll
      for (int i = 0; i < kF8ALoads; ++i) sm.a[buf][ar[i]][aq[i] ^ (ar[i] & (kF8Units - 1))] = r.A[i];
#pragma unroll
      for (int j = 0; j < kF8BLoads; ++j) {
        const int n = cb + kF8CPP * j;
        *(u32x2_t *)&sm.b[buf][n][8 * ((2 * bq) ^ (n & (kF8Units - 1)))] = u32x2_t{r.B[j].x, r.B[j].y};
        *(u32x2_t *)&sm.b[buf][n][8 * ((2 * bq + 1) ^ (n & (kF8Units - 1)))] = u32x2_t{r.B[j].z, r.B[j].w};
      }
    };
    // slice s: wait until every consumer wave is done with slice s - 2 (the
    // buffer's previous slice, its (s / 2)-th use), store, count.  A wait past
    // its bound lets the loader go on (results then wrong, every wave ends).
    auto put = [&](int s, int buf, F8SliceRegs &r) {
      if (s >= 2 && (lane == 0)) (void)wait_count(lds_cnt(sm.done[buf]), (uint32_t)(kF8CWaves * (s >> 1)), lds_cnt(sm.abort));
      asm volatile("" ::: "memory");
      store_slice(buf, r);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's stores are in LDS
      if (lane == 0) __hip_atomic_fetch_add(lds_cnt(sm.ready[buf]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    F8SliceRegs r0, r1;
    load_slice(r0);
    // slice 0's loads stay ahead of slice 1's: each store waits for the older
    // register set only (memory returns in issue order)
    __builtin_amdgcn_sched_barrier(0);
    load_slice(r1);
    // One exit, at the bottom: a break between the halves makes the compiler
    // wait for both register sets at the top of the loop.
    for (int s = 0; s < total; s += 2) {
      put(s, 0, r0);
      load_slice(r0);
      if (s + 1 < total) put(s + 1, 1, r1);
      load_slice(r1);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    return;
  }

  // ---- consumers: lane (lk, li) -> column li of a 16-column tile, k 8 lk .. +7
  // of a 32-k group; wave w owns columns 32w..32w+31 ---------------------------
  const int li = lane & 15, lk = lane >> 4;
  // the item being computed: (ct, cks) is its next slice
  int ct = 0, cks = 0;
  int c_live = 0, c_row0 = 0, c_mrows = 0, c_n0 = 0;
  auto load_citem = [&]() {
    c_row0 = __builtin_amdgcn_readfirstlane(sm.it.item[ct][1]);
    c_mrows = __builtin_amdgcn_readfirstlane(sm.it.item[ct][2]);
    c_n0 = __builtin_amdgcn_readfirstlane(sm.it.item[ct][3]);
    c_live = (c_mrows + 15) >> 4;  // 16-row sub-tiles holding routed rows
  };
  load_citem();
  f32x4_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute_slice = [&](int buf) {
    if (c_n0 + wave * 32 >= a.N) return;  // uniform (N % 32 == 0): this wave's columns do not exist
#pragma unroll
    for (int kg = 0; kg < kF8BK / 32; ++kg) {
      const int unit = kg * 4 + lk;  // 8-k unit of the slice
      // both column tiles' operands first: one activation read feeds two MFMAs
      bf16x8_t bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int n = wave * 32 + t * 16 + li;
        bv[t] = fp8_operand(*(const u32x2_t *)&sm.b[buf][n][8 * (unit ^ (n & (kF8Units - 1)))]);
      }
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= c_live) break;  // uniform
        const int r = ms * 16 + li;
        const bf16x8_t av = __builtin_bit_cast(bf16x8_t, sm.a[buf][r][unit ^ (r & (kF8Units - 1))]);
        acc[ms][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[0], acc[ms][0], 0, 0, 0);
        acc[ms][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[1], acc[ms][1], 0, 0, 0);
      }
    }
  };

  // epilogue of the item being computed (lane holds rows 4 lk + i, column li
  // of each 16-column tile; no global load); then the accumulators restart
  auto finish_item = [&]() {
    if (c_n0 + wave * 32 < a.N) {  // uniform
      const float gs = sm.it.gsc[ct];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= c_live) break;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          const int col = c_n0 + wave * 32 + t * 16 + li;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = ms * 16 + lk * 4 + i;
            const float u = gs * acc[ms][t][i];
            if (a.fc1 && !a.concat) {
              const float partner = __uint_as_float(dpp_u32<kDppXor1>(__float_as_uint(u)));
              if (r < c_mrows && (lane & 1) == 0)
                a.out_bf16[(size_t)(c_row0 + r) * (a.N >> 1) + (col >> 1)] =
                    (uint16_t)bf16_rne(swiglu(u, partner, a.alpha, a.beta, a.limit));
            } else if (r < c_mrows) {
              a.out_f32[(size_t)(c_row0 + r) * a.N + col] = u;  // FC2 y, or FC1 u for the concatenated layout
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (++ct < nt) load_citem();
  };

  // slice s: wait until the four loader waves have stored it, compute, count
  // this wave's reads done (they have returned: lgkmcnt 0).  Unrolled by two
  // so each buffer's LDS offsets are constants.
  auto take = [&](int s, int buf) {
    bool ok = true;
    if (lane == 0) ok = wait_count(lds_cnt(sm.ready[buf]), (uint32_t)(kF8LWaves * ((s >> 1) + 1)), lds_cnt(sm.abort));
    ok = __builtin_amdgcn_readfirstlane((int)ok) != 0;
    if (!ok) return false;  // uniform: a wait ran past its bound
    asm volatile("" ::: "memory");
    compute_slice(buf);
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) __hip_atomic_fetch_add(lds_cnt(sm.done[buf]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if (++cks == steps) {  // uniform: the item's last slice is done
      cks = 0;
      finish_item();
    }
    return true;
  };
  for (int s = 0; s < total; s += 2) {
    if (!take(s, 0)) break;
    if (s + 1 < total && !take(s + 1, 1)) break;
  }
}

hipError_t launch_fp8_grouped(GemvArgs &a, void *ws, hipStream_t s) {
  const int erows = a.rows < a.E ? a.rows : a.E;
  a.nslots = (a.rows + kF8BM - 1) / kF8BM + erows;  // worst-case (expert, m tile) count
  a.ntiles = (a.N + kF8BN - 1) / kF8BN;
  unsigned grid = 0;
  const hipError_t gerr = grouped_grid(a, &grid);
  if (gerr != hipSuccess) return gerr;
  if (a.concat) a.out_f32 = (float *)ws;
  fp8_grouped_kernel<<<dim3(grid), kF8GThreads, 0, s>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !a.concat) return err;
  a.partials = (float *)ws;
  a.nchunks = 1;
  return launch_splitk_epilogue(a, s);
}

size_t fp8_workspace_bytes(int32_t rows, int32_t N, bool concat) {
  const size_t u = concat ? (size_t)rows * N * sizeof(float) : 0;
  return u > 256 ? u : 256;
}

hipError_t launch_fp8_gemv(GemvArgs &a, int max_rows_per_expert, void *ws, hipStream_t s) {
  const int cpr = a.K >= 1536 ? 1 : (a.K >= 768 ? 2 : 4);
  a.nslots = a.rows < a.E ? a.rows : a.E;
  a.ntiles = (a.N + kF8TileN1 * cpr - 1) / (kF8TileN1 * cpr);
  const int items = a.nslots * a.ntiles;
  const dim3 grid((unsigned)(((items + 7) / 8) * 8));
  const dim3 block(kF8Waves * 64);
  if (a.concat) a.out_f32 = (float *)ws;
  const int mr = max_rows_per_expert <= 1 ? 1 : (max_rows_per_expert <= 4 ? 4 : 8);
#define QMOE_F8_LAUNCH(MR)                                                   \
  if (cpr == 1)                                                              \
    fp8_gemv_kernel<MR, 1><<<grid, block, 0, s>>>(a);                        \
  else if (cpr == 2)                                                         \
    fp8_gemv_kernel<MR, 2><<<grid, block, 0, s>>>(a);                        \
  else                                                                       \
    fp8_gemv_kernel<MR, 4><<<grid, block, 0, s>>>(a);
  if (mr == 1) {
    QMOE_F8_LAUNCH(1)
  } else if (mr == 4) {
    QMOE_F8_LAUNCH(4)
  } else {
    QMOE_F8_LAUNCH(8)
  }
#undef QMOE_F8_LAUNCH
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || !a.concat) return err;
  a.partials = (float *)ws;
  a.nchunks = 1;
  return launch_splitk_epilogue(a, s);
}

// Dequant: out[e][n][k] = bf16(float32(e4m3(w[e][n][k]) * g[e])), the same
// [E][N][K] layout as the input.  A wave converts 1 KB of input as two
// 512-byte halves, 8 bytes per lane each, so every load instruction reads
// and every store instruction writes one contiguous run (a lane's 16 output
// bytes sit next to its neighbours').
__global__ __launch_bounds__(256) void fp8_dequant_kernel(const uint8_t *__restrict__ w,
                                                          const float *__restrict__ g, size_t per_expert,
                                                          uint16_t *__restrict__ out) {
  const int e = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const size_t base = (size_t)blockIdx.x * 4096 + (size_t)(threadIdx.x >> 6) * 1024 + (size_t)lane * 8;
  const float ge = g[e];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const size_t i = base + (size_t)h * 512;
    if (i >= per_expert) continue;  // per_expert % 16 == 0: a lane's 8 bytes are all in or all out
    const size_t off = (size_t)e * per_expert + i;
    const u32x2_t v = __builtin_nontemporal_load((const u32x2_t *)(w + off));
    const uint32_t vs[2] = {v.x, v.y};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const f32x2_t lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vs[j], 1.0f, false);
      const f32x2_t hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(vs[j], 1.0f, true);
      o[2 * j] = pack_bf16x2_rne(lo.x * ge, lo.y * ge);
      o[2 * j + 1] = pack_bf16x2_rne(hi.x * ge, hi.y * ge);
    }
    __builtin_nontemporal_store(u32x4_t{o[0], o[1], o[2], o[3]}, (u32x4_t *)(out + off));
  }
}

hipError_t launch_fp8_dequant(const uint8_t *w, const float *g, int32_t E, int32_t K, int32_t N, uint16_t *out,
                              hipStream_t s) {
  const size_t per = (size_t)N * K;
  const dim3 grid((unsigned)((per + 4095) / 4096), (unsigned)E);
  fp8_dequant_kernel<<<grid, 256, 0, s>>>(w, g, per, out);
  return hipGetLastError();
}

}  // namespace qmoe
