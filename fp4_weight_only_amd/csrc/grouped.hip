// Prefill path: grouped GEMM over routed rows with bf16 MFMA, FP4 weights
// kept packed in LDS and decoded straight into MFMA operands, gfx950.
//
// What it computes (operator documentation section 4.3, the dequant-to-A16
// path for shapes outside the decode GEMV; section 9b.1/9b.5, prefill-sized
// batches go to a grouped GEMM): for every routed row p of expert e,
//   u[p][n] = g[e] * sum_k a[p][k] * (e2m1(code[e][k][n]) * scale[e][k/B][n])
// FC1: a = x[token(p)], then interleaved SwiGLU -> bf16 h.  FC2: a = h[p],
// float32 y.  Same outputs as the decode GEMV.
//
// gfx950 design:
// * Work item = (expert, 64-row m tile, 512-column n tile), K in 128-k
//   slices.  A workgroup has two wave groups: four loader waves move each
//   slice from memory into LDS, eight consumer waves compute; consumer wave w
//   owns columns 64w..64w+63 (four 16-column MFMA tiles) for every live
//   16-row sub-tile of the m tile, with v_mfma_f32_16x16x32_bf16.  Most
//   experts of a prefill batch hold a handful of rows, so the cost is
//   streaming and decoding weights.
// * Weights stay packed in LDS, copied as loaded: 128 k rows x 256 bytes per
//   slice (sixteen lanes load a row's two 128-byte lines; 8-byte units
//   XOR-swizzled by row in LDS).  gfx950's 4-bit transpose read
//   (ds_read_b64_tr_b4) hands each lane of a 16-lane group one column's 16
//   consecutive k codes from the rows its group points at, which is two
//   K-paired MFMA B operands (k 16g..16g+7 and 16g+8..16g+15 of a 64-k
//   group, g = lane / 16).  The k order inside an MFMA is free as long as
//   both operands share it, so the activation operand reads the matching
//   16-byte chunks.  No VALU work transposes the weights.
// * Decode on read: four gfx950 FP4 -> bf16 conversions per operand.  A
//   lane's 16 k lie in one block, so the block scale is per lane: for MXFP4
//   the E8M0 scale is the conversion's exponent (exact); for NVFP4 the codes
//   convert to float32, the E4M3 scale multiplies exactly and the hardware
//   pack to bf16 is exact (2 x 4 significant bits).  The global scale
//   multiplies the float32 accumulator in the epilogue.
// * Activations: 64 rows x 128 k bf16 per slice (rows gathered through the
//   permutation for FC1), 16-byte chunks XOR-swizzled by row so the operand
//   reads are conflict free.
// * Pipeline: the loaders keep two slices of loads in flight in registers
//   (52 KB per workgroup per slice at most) and store each slice into one of
//   two LDS buffers; the groups hand slices over through per-buffer counts
//   in LDS (no workgroup barrier in the loop), so the loaders' stores and
//   waits overlap the consumers' reads, conversions and MFMAs.  With every
//   wave doing both in turn (one barrier per slice), the kernel was bound by
//   its in-CU work per slice rather than by HBM.  One workgroup (12 waves,
//   at most 168 VGPRs each) per CU.  The 512-column tile halves the
//   activation re-reads of the n tiles (measured against 256 columns).
//   16-row sub-tiles with no routed rows are skipped.  No weight element is
//   decoded or read from LDS by more than one wave.
// * Persistent work items: one workgroup per CU takes a fixed list of
//   (expert, 64-row m tile, n tile) items and streams their slices as one
//   sequence, so the next item's first loads are in flight while the
//   current one finishes and writes its tile (with one workgroup per item,
//   a CU idled about 3 us between items and again while its first slices
//   arrived).  The lists are built on the device from expert_offsets: m
//   tiles ordered by class (live 16-row sub-tiles, heaviest first), dealt
//   over the workgroups in a snake so the per-workgroup work evens out; the
//   n tiles of one m tile land on one XCD (its activation rows stay in that
//   L2).  Each slice's loads are branch-free (item-dependent offsets formed
//   once per item) so the compiler waits for exactly the older register set.
#include "grouped_sched.h"

namespace qmoe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kBM = 64, kBN = 512, kBK = 128;
constexpr int kCT = 4;                      // 16-column MFMA tiles per consumer wave
constexpr int kCWaves = kBN / (16 * kCT);   // consumer wave w owns columns 16 kCT w .. 16 kCT (w + 1) - 1
constexpr int kLWaves = 4;                  // loader waves
constexpr int kThreads = (kCWaves + kLWaves) * 64;
constexpr int kLThreads = kLWaves * 64;
constexpr int kALoads = kBM * (kBK / 8) / kLThreads;  // 16-byte activation chunks per loader thread per slice
constexpr int kBLoads = kBK * 16 / kLThreads;         // 16-byte weight chunks per loader thread per slice
constexpr int kARowStep = kLThreads / 16;             // rows between a loader thread's activation chunks
constexpr int kBRowStep = kLThreads / 16;             // k rows between a loader thread's weight chunks
static_assert(kALoads >= 1 && kBLoads >= 1 && kBN % (16 * kCT) == 0 && kCWaves == 8, "tile shape");
constexpr int kAChunks = kBK / 8;    // 16-byte chunks per activation row of a slice
constexpr int kBRow = kBN / 2;       // packed bytes per weight row of a slice (two 128-byte lines)
constexpr uint32_t kGOutOfRange = 0x80000000u;

static_assert(kBM == kGBM, "m tile of the item lists");

struct GroupedSmem {
  u32x4_t a[2][kBM][kAChunks];      // activations, chunk c of row r at c ^ (r & 15)
  uint8_t b[2][kBK][kBRow];         // packed codes, 8-byte unit u of row r at u ^ (r & 31)
  uint8_t sc[2][kBK / 16][kBN + 16];  // block scales of the slice (B = 32 uses 4 rows); the pad
                                      // puts neighbouring block rows on other banks
  GroupedPre pre;                     // set-up only
  GroupedItems it;                    // this workgroup's items
  uint32_t ready[2];                  // per buffer: loader-wave stores of its slices (4 per slice)
  uint32_t done[2];                   // per buffer: consumer-wave reads of its slices (8 per slice)
  uint32_t abort;                     // set when a wait ran past its bound
};

// One slice's global loads for one loader thread.
template <int NS>
struct SliceRegs {
  u32x4_t A[kALoads];
  u32x4_t B[kBLoads];
  uint32_t S[NS];
};

// MFMA B operand of one lane: 8 consecutive k codes of its column (one
// dword, low nibble first), decoded to bf16 with the block scale.  The
// weights are bf16 values code * scale, rounded to nearest even: exact for
// every finite E4M3 byte and for E8M0 bytes 0..252 (bf16 subnormals at 0
// and 1); at E8M0 bytes 253 and 254 a product past bf16's range is +-inf,
// and byte 255 (NaN) gives NaN.  The scaled FP4 conversion takes the
// scale operand's exponent field as an E8M0 value (field 0 is 2^-127, 255
// NaN): checked for all 256 bytes x 16 codes against round-to-nearest-even
// of the exact product, so the byte shifted into the exponent field is the
// whole decode.
template <int FMT>
__device__ __forceinline__ bf16x8_t decode_operand(uint32_t d, uint32_t sbyte) {
  u32x4_t o;
  if constexpr (FMT == 1) {
    const float sc = __uint_as_float(sbyte << 23);  // E8M0 byte as the conversion's scale exponent
    o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 0));
    o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 1));
    o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 2));
    o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, sc, 3));
  } else {
    const float sf = __builtin_amdgcn_cvt_f32_fp8((int)sbyte, 0);
    const f32x2_t f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 0) * sf;
    const f32x2_t f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 1) * sf;
    const f32x2_t f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 2) * sf;
    const f32x2_t f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(d, 1.0f, 3) * sf;
    o.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(f0, bf16x2_t));
    o.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(f1, bf16x2_t));
    o.z = __builtin_bit_cast(uint32_t, __builtin_convertvector(f2, bf16x2_t));
    o.w = __builtin_bit_cast(uint32_t, __builtin_convertvector(f3, bf16x2_t));
  }
  return __builtin_bit_cast(bf16x8_t, o);
}

// Persistent grouped GEMM: G workgroups (one per CU or as many as the item
// tables need), workgroup g takes the items at positions g, 2G - 1 - g,
// 2G + g, ... of the class order (a snake over the rounds, so the heavy
// items spread evenly), and streams them as one sequence of 128-k slices: the
// loads for the next item's first slices are in flight while the current
// item finishes and writes its tile.
template <int FMT>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(3))) void grouped_gemm_kernel(GemvArgs a) {
  constexpr int B = (FMT == 0) ? 16 : 32;
  __shared__ __attribute__((aligned(16))) GroupedSmem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = lane_id();
  // ---- this workgroup's items -------------------------------------------------
  const int nt = build_items(a, sm.pre, sm.it, kBN, kThreads, tid, wave, lane);
  if (nt == 0) return;  // uniform

  const int steps = (a.K + kBK - 1) / kBK;
  const bool ragged = (a.K % kBK) != 0;  // the last slice of an item holds 64 valid k rows
  const int total = nt * steps;
  if (tid == 0) {
    sm.ready[0] = sm.ready[1] = 0u;
    sm.done[0] = sm.done[1] = 0u;
    sm.abort = 0u;
  }
  __syncthreads();

  // Two wave groups, no workgroup barrier in the loop: four loader waves
  // move each slice from memory into an LDS buffer (two buffers) and count
  // it in the buffer's ready count; eight consumer waves wait for that count,
  // read, convert and multiply the slice, and count their reads in the
  // buffer's done count, which frees the buffer for the loaders.  So the
  // stores, the waits and the compute of different slices overlap instead of
  // alternating in step.  The counts are per buffer: a wave cannot count a
  // buffer's next slice before the other group has passed it, so a count of
  // (waves x uses) means every wave is through; one count over both buffers
  // could be reached while a wave two slices behind still reads.
  if (wave >= kCWaves) {
    // ---- loaders ---------------------------------------------------------------
    const int lt_id = tid - kCWaves * 64;
    const uint32_t rowbytes = (uint32_t)(a.N >> 1);
    const int KB = a.K / B;
    // activations: thread -> 16-byte chunk aq (8 k) of m-tile rows ra[i]
    const int aq = lt_id & 15;
    int ra[kALoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i) ra[i] = (lt_id >> 4) + i * kARowStep;
    const int act_rows = a.fc1 ? a.rows / a.topk : a.rows;
    const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
        uniform_ptr(a.act), (short)0, (int)((uint32_t)act_rows * (uint32_t)a.K * 2u), 0x00020000);
    // weights: thread -> 16 bytes bq of k rows rb + j * kBRowStep; sixteen
    // lanes read a row's 256 bytes (two 128-byte lines)
    const int rb = lt_id >> 4;
    const int bq = lt_id & 15;
    constexpr int kSBlocks = kBK / B;
    constexpr int kSLoads = (kSBlocks * (kBN / 4) + kLThreads - 1) / kLThreads;
    const int sq = lt_id & 127;  // scales: thread -> 4 columns sq of block rows sb[i]
    uint32_t btail[kBLoads], stail[kSLoads];  // rows past the first 64 k of a ragged slice
#pragma unroll
    for (int j = 0; j < kBLoads; ++j) btail[j] = (rb + j * kBRowStep >= kBK / 2) ? kGOutOfRange : 0u;
#pragma unroll
    for (int i = 0; i < kSLoads; ++i)
      stail[i] = ((lt_id >> 7) + i * (kLThreads / 128) >= kSBlocks / 2) ? kGOutOfRange : 0u;
    // The item-dependent part of the offsets is formed once per item; a
    // slice's loads then differ only by uniform masks, so the load sequence
    // has no branches (a branch around a load leaves the compiler's wait
    // counts conservative).  Out-of-range offsets stay out of range when a
    // row step is added.
    int lt = 0, lks = 0;
    int e = 0;
    uint32_t avoff[kALoads], boff = kGOutOfRange, soff[kSLoads];
#pragma unroll
    for (int i = 0; i < kALoads; ++i) avoff[i] = kGOutOfRange;
#pragma unroll
    for (int i = 0; i < kSLoads; ++i) soff[i] = kGOutOfRange;
    using Regs = SliceRegs<kSLoads>;
    auto load_slice = [&](Regs &r) {
      const bool dead = lt >= nt;  // uniform
      if (lks == 0 && !dead) {     // uniform
        e = __builtin_amdgcn_readfirstlane(sm.it.item[lt][0]);
        const int n0 = __builtin_amdgcn_readfirstlane(sm.it.item[lt][3]);
#pragma unroll
        for (int i = 0; i < kALoads; ++i) {
          const int srow = sm.it.src[lt][ra[i]];
          avoff[i] = srow >= 0 ? (uint32_t)srow * (uint32_t)a.K * 2u + (uint32_t)(aq * 16) : kGOutOfRange;
        }
        // a partial last tile (N % 512 != 0) reads nothing past N
        boff = n0 + 32 * bq + 32 <= a.N ? (uint32_t)rb * rowbytes + (uint32_t)(n0 >> 1) + (uint32_t)(bq * 16)
                                        : kGOutOfRange;
#pragma unroll
        for (int i = 0; i < kSLoads; ++i) {
          const int sb = (lt_id >> 7) + i * (kLThreads / 128);
          soff[i] = (n0 + sq * 4 + 4 <= a.N && sb < kSBlocks) ? (uint32_t)sb * (uint32_t)a.N + (uint32_t)(n0 + sq * 4)
                                                             : kGOutOfRange;
        }
      }
      const int k0 = lks * kBK;
      const uint32_t tailm = (ragged && lks + 1 == steps) ? ~0u : 0u;  // uniform
      const uint32_t kill = dead ? kGOutOfRange : 0u;                  // uniform
      const int ao = __builtin_amdgcn_readfirstlane(k0 * 2);
#pragma unroll
      for (int i = 0; i < kALoads; ++i) r.A[i] = __builtin_amdgcn_raw_buffer_load_b128(arsrc, avoff[i] | kill, ao, 0);
      const __amdgpu_buffer_rsrc_t wrsrc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(a.w + (size_t)e * a.K * rowbytes), (short)0, (int)((uint32_t)a.K * rowbytes), 0x00020000);
      const int so = __builtin_amdgcn_readfirstlane((int)((uint32_t)k0 * rowbytes));
#pragma unroll
      for (int j = 0; j < kBLoads; ++j)
        r.B[j] = __builtin_amdgcn_raw_buffer_load_b128(
            wrsrc, (boff + (uint32_t)(j * kBRowStep) * rowbytes) | kill | (btail[j] & tailm), so, 2);
      const __amdgpu_buffer_rsrc_t srsrc = __builtin_amdgcn_make_buffer_rsrc(
          uniform_ptr(a.scales + (size_t)e * KB * a.N), (short)0, (int)((uint32_t)KB * a.N), 0x00020000);
      const int sso = __builtin_amdgcn_readfirstlane((int)((uint32_t)(k0 / B) * (uint32_t)a.N));
#pragma unroll
      for (int i = 0; i < kSLoads; ++i)
        r.S[i] = __builtin_amdgcn_raw_buffer_load_b32(srsrc, soff[i] | kill | (stail[i] & tailm), sso, 0);
      if (++lks == steps) {
        lks = 0;
        ++lt;
      }
    };
    // LDS positions of this thread's stores (unit u of weight row r sits at
    // u ^ (r & 31): the two 8-byte halves of a loaded chunk land separately;
    // the transpose reads of lane groups 16 rows apart then hit opposite bank
    // halves)
    int bpos[kBLoads][2];
#pragma unroll
    for (int j = 0; j < kBLoads; ++j)
#pragma unroll
      for (int h = 0; h < 2; ++h) bpos[j][h] = 8 * ((2 * bq + h) ^ ((rb + j * kBRowStep) & 31));
    auto store_slice = [&](int buf, const Regs &r) {
#pragma unroll
      for (int i = 0; i < kALoads; ++i) sm.a[buf][ra[i]][aq ^ (ra[i] & 15)] = r.A[i];
#pragma unroll
      for (int j = 0; j < kBLoads; ++j) {
        const int row = rb + j * kBRowStep;
        *(u32x2_t *)&sm.b[buf][row][bpos[j][0]] = u32x2_t{r.B[j].x, r.B[j].y};
        *(u32x2_t *)&sm.b[buf][row][bpos[j][1]] = u32x2_t{r.B[j].z, r.B[j].w};
      }
#pragma unroll
      for (int i = 0; i < kSLoads; ++i) {
        const int sb = (lt_id >> 7) + i * (kLThreads / 128);
        if (sb < kSBlocks) *(uint32_t *)&sm.sc[buf][sb][sq * 4] = r.S[i];
      }
    };
    // slice s: wait until every consumer wave is done with slice s - 2 (the
    // buffer's previous slice, its (s / 2)-th use), store, count
    // (A wait past its bound lets the loader go on: the results are then
    // wrong but every wave still ends.  Control flow that depends on the wait's
    // outcome made the compiler's waits for the in-flight loads conservative.)
    auto put = [&](int s, int buf, Regs &r) {
      if (s >= 2 && (lane == 0)) (void)wait_count(lds_cnt(sm.done[buf]), (uint32_t)(kCWaves * (s >> 1)), lds_cnt(sm.abort));
      asm volatile("" ::: "memory");
      store_slice(buf, r);
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // this wave's stores are in LDS
      if (lane == 0) __hip_atomic_fetch_add(lds_cnt(sm.ready[buf]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    };
    Regs r0, r1;
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

  // ---- consumers: wave w owns units T = kCT w + t of a packed row (16
  // columns each; the row swizzle permutes the row's 32 units) ---------------
  const int li = lane & 15;
  const int lk = lane >> 4;
  // the item being computed: (ct, cks) is its next slice
  int ct = 0, cks = 0;
  int c_live = 0, c_row0 = 0, c_mrows = 0, c_n0 = 0;
  // the epilogue makes no global load
  auto load_citem = [&]() {
    c_row0 = __builtin_amdgcn_readfirstlane(sm.it.item[ct][1]);
    c_mrows = __builtin_amdgcn_readfirstlane(sm.it.item[ct][2]);
    c_n0 = __builtin_amdgcn_readfirstlane(sm.it.item[ct][3]);
    c_live = (c_mrows + 15) >> 4;  // 16-row sub-tiles holding routed rows
  };
  load_citem();
  f32x4_t acc[4][kCT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < kCT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto compute_slice = [&](int buf) {
    if (c_n0 + wave * 16 * kCT >= a.N) return;  // uniform: this wave's columns do not exist
    const int nkg = (ragged && cks + 1 == steps) ? 1 : 2;  // 64-k groups below K
#pragma unroll
    for (int kg = 0; kg < 2; ++kg) {
      if (kg >= nkg) break;
      // lane (lk, li) points at weight row kg*64 + 16*lk + li of its N tile;
      // the transpose returns column li's codes of rows kg*64 + 16*lk + 0..15
      const int row = kg * 64 + lk * 16 + li;
      const int blk = (kg * 64 + lk * 16) / B;
      // every column tile's operands of this k group first, so one
      // activation read feeds kCT MFMAs
      typedef int v2i_t __attribute__((ext_vector_type(2)));
      v2i_t v[kCT];
      uint32_t sbyte[kCT];
#pragma unroll
      for (int t = 0; t < kCT; ++t) {
        const int T = wave * kCT + t;
        v[t] = __builtin_amdgcn_ds_read_tr4_b64_v2i32(
            (__attribute__((address_space(3))) v2i_t *)(&sm.b[buf][row][8 * (T ^ (row & 31))]));
        sbyte[t] = sm.sc[buf][blk][T * 16 + li];
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        // decoded just before their MFMAs: kCT operands live at a time
        bf16x8_t bv[kCT];
#pragma unroll
        for (int t = 0; t < kCT; ++t) bv[t] = decode_operand<FMT>(h ? (uint32_t)v[t].y : (uint32_t)v[t].x, sbyte[t]);
        const int chunk = kg * 8 + lk * 2 + h;  // k = kg*64 + 16*lk + 8*h .. +7
#pragma unroll
        for (int ms = 0; ms < 4; ++ms) {
          if (ms >= c_live) break;  // uniform
          const int r = ms * 16 + li;
          const bf16x8_t av = __builtin_bit_cast(bf16x8_t, sm.a[buf][r][chunk ^ (r & 15)]);
#pragma unroll
          for (int t = 0; t < kCT; ++t)
            acc[ms][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[t], acc[ms][t], 0, 0, 0);
        }
      }
    }
  };

  // ---- epilogue of the item being computed: lane holds rows 4*(lane/16)+i,
  // column lane%16 of each tile; then the accumulators restart for the next
  auto finish_item = [&]() {
    if (c_n0 + wave * 16 * kCT < a.N) {  // uniform
      const float gs = sm.it.gsc[ct];
#pragma unroll
      for (int ms = 0; ms < 4; ++ms) {
        if (ms >= c_live) break;
#pragma unroll
        for (int t = 0; t < kCT; ++t) {
          const int col = c_n0 + wave * 16 * kCT + t * 16 + li;
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
              a.out_f32[(size_t)(c_row0 + r) * a.N + col] = u;
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < kCT; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (++ct < nt) load_citem();
  };

  // slice s: wait until the four loader waves have stored it, compute,
  // count this wave's reads done (they have returned: lgkmcnt 0).  Unrolled
  // by two so each buffer's LDS offsets are constants.
  auto take = [&](int s, int buf) {
    bool ok = true;
    if (lane == 0) ok = wait_count(lds_cnt(sm.ready[buf]), (uint32_t)(kLWaves * ((s >> 1) + 1)), lds_cnt(sm.abort));
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

// The concatenated SwiGLU layout pairs columns from different tiles: FC1
// then writes g * u as float32 rows to the workspace and the split-K
// epilogue (one chunk) forms h.
size_t grouped_workspace_bytes(int32_t rows, int32_t N, bool concat) {
  const size_t u = concat ? (size_t)rows * N * sizeof(float) : 0;
  return u > 256 ? u : 256;
}

hipError_t launch_grouped(GemvArgs &a, int fmt, hipStream_t s) {
  const int erows = a.rows < a.E ? a.rows : a.E;
  a.nslots = (a.rows + kBM - 1) / kBM + erows;  // worst-case (expert, m tile) count
  a.ntiles = (a.N + kBN - 1) / kBN;  // N % 128 == 0: a partial last tile (whole 16 kCT-column waves)
  unsigned grid = 0;
  const hipError_t err = grouped_grid(a, &grid);
  if (err != hipSuccess) return err;
  if (fmt == 0)
    grouped_gemm_kernel<0><<<dim3(grid), kThreads, 0, s>>>(a);
  else
    grouped_gemm_kernel<1><<<dim3(grid), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace qmoe
