// Work-item lists of the persistent grouped GEMMs (the FP4 and FP8 prefill
// paths).  A slot is one (expert, 64-row m tile); its class is the number of
// 16-row sub-tiles holding routed rows (1..4), which sets its MFMA and LDS
// work.  An expert with R rows has R / 64 full tiles (class 4) and, when
// R % 64 != 0, one tile of class ceil((R % 64) / 16).  Slots are ordered by
// class, heaviest first (experts ascending within a class); a work item is
// (slot, n tile).  One workgroup per CU takes a fixed list of items and
// streams them as one sequence of k slices, so the next item's first loads
// are in flight while the current one finishes and writes its tile.
#pragma once
#include "device_common.h"
#include "qmoe.h"
#include "qmoe_internal.h"

namespace qmoe {

constexpr int kGMaxItems = 32;  // work items per workgroup (LDS tables)
constexpr int kGClasses = 4;
constexpr int kGBM = 64;        // rows per m tile
constexpr int kGPreE = QMOE_MAX_EXPERTS;

// pre[w][e]: the class-(4 - w) slots of the experts before e (set-up only)
typedef int32_t GroupedPre[kGClasses][kGPreE + 1];

// A workgroup's item list in LDS, in the order it runs them.
struct GroupedItems {
  int32_t item[kGMaxItems][4];   // expert, first row, rows, first column
  int32_t src[kGMaxItems][kGBM];  // activation row of each m-tile row, -1 past the expert's rows
  float gsc[kGMaxItems];          // the expert's global scale (1 without one)
};

// Waves 0..3 each count one class: wave prefix sums over the experts.
__device__ __forceinline__ void class_prefix(const int32_t *__restrict__ off, int E, GroupedPre &pre, int wave,
                                             int lane) {
  if (wave >= kGClasses) return;  // uniform
  const int c = kGClasses - wave;
  int o[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int e = 4 * lane + i;
    o[i] = (e <= E) ? off[e] : 0;
  }
  int cnt[4], sum = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int R = (4 * lane + i < E) ? o[i + 1] - o[i] : 0;
    cnt[i] = (((R & (kGBM - 1)) + 15) >> 4) == c ? 1 : 0;
    if (c == kGClasses) cnt[i] += R / kGBM;
    sum += cnt[i];
  }
  int incl = sum;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d, 64);
    if (lane >= d) incl += v;
  }
  int run = incl - sum;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    pre[wave][4 * lane + i] = run;
    run += cnt[i];
  }
  if (lane == 63) pre[wave][kGPreE] = run;
}

// Slot q of the class order -> expert and m tile.
__device__ __forceinline__ void slot_of(const int32_t *__restrict__ off, int E, const GroupedPre &pre, int q, int &e,
                                        int &mt) {
  int w = 0, base = 0;
  while (w < kGClasses - 1 && q >= base + pre[w][kGPreE]) {
    base += pre[w][kGPreE];
    ++w;
  }
  const int u = q - base;
  int lo = 0, hi = E;  // pre[w][lo] <= u < pre[w][hi]
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (pre[w][mid] <= u)
      lo = mid;
    else
      hi = mid;
  }
  e = lo;
  mt = (w == 0) ? u - pre[0][lo] : (off[lo + 1] - off[lo]) / kGBM;
}

// This workgroup's items: positions g, 2G - 1 - g, 2G + g, ... of the class
// order (a snake over the rounds, so the heavy items spread evenly over the
// workgroups).  The items of one slot sit 8 positions apart (blocks of 8
// slots x NT tiles), so they run on one XCD and share its L2 copy of the
// activation rows; workgroups start their lists at an offset set by the XCD,
// so at any time each XCD works on a different mix of classes.  Returns the
// item count (uniform); every thread of the workgroup calls it.
__device__ __forceinline__ int build_items(const GemvArgs &a, GroupedPre &pre, GroupedItems &it, int BN, int nthreads,
                                           int tid, int wave, int lane) {
  const int G = gridDim.x;
  const int g = blockIdx.x;
  const int NT = a.ntiles;
  class_prefix(a.offsets, a.E, pre, wave, lane);
  __syncthreads();
  int S = 0;
#pragma unroll
  for (int w = 0; w < kGClasses; ++w) S += pre[w][kGPreE];
  const int NI = S * NT;
  int nt = 0;
  while (nt < kGMaxItems) {
    const int j = nt * G + ((nt & 1) ? G - 1 - g : g);
    if (j >= NI) break;
    ++nt;
  }
  if (nt == 0) return 0;  // uniform
  const int rot = ((g & 7) * nt) >> 3;
  if (tid < nt) {
    const int t = tid;
    const int j = t * G + ((t & 1) ? G - 1 - g : g);
    const int bsz = 8 * NT;
    const int b = j / bsz;
    const int p = j - b * bsz;
    const int sb = min(8, S - 8 * b);
    const int q = 8 * b + p % sb;
    const int ntile = p / sb;
    int e, mt;
    slot_of(a.offsets, a.E, pre, q, e, mt);
    const int row0 = a.offsets[e] + mt * kGBM;
    int tt = t - rot;
    if (tt < 0) tt += nt;
    it.item[tt][0] = e;
    it.item[tt][1] = row0;
    it.item[tt][2] = min(kGBM, a.offsets[e + 1] - row0);
    it.item[tt][3] = ntile * BN;
    it.gsc[tt] = a.gscale ? a.gscale[e] : 1.0f;
  }
  __syncthreads();
  for (int x = tid; x < nt * kGBM; x += nthreads) {
    const int t = x / kGBM, r = x - (x / kGBM) * kGBM;
    const int row0 = it.item[t][1], mrows = it.item[t][2];
    int src = -1;
    if (r < mrows) src = a.fc1 ? a.p2e[row0 + r] / a.topk : row0 + r;
    it.src[t][r] = src;
  }
  __syncthreads();
  return nt;
}

// ---- hand-off between the loader and consumer wave groups -------------------
constexpr int kMaxPolls = 1 << 22;  // bound of every wait on the other wave group (a fault, not a slow load)

// The wave groups' counters, addressed as LDS: through a generic pointer the
// compiler would make them flat accesses, which it also waits for with the
// global-load counter (a loader's wait would then drain its loads).
typedef __attribute__((address_space(3))) volatile uint32_t lds_cnt_t;
__device__ __forceinline__ lds_cnt_t *lds_cnt(uint32_t &x) { return (lds_cnt_t *)&x; }

// Waits (the calling lane polling LDS, sleeping between polls) until
// *c >= target; past the poll bound it sets *abort and returns false.  One
// loop with one exit and nothing else in it; a loader ignores the result:
// control flow that depends on it made the compiler's waits for the
// loader's in-flight loads conservative (they waited for the next slice's
// loads too).
__device__ __forceinline__ bool wait_count(lds_cnt_t *c, uint32_t target, lds_cnt_t *abort) {
  uint32_t polls = 0;
  while (*c < target && polls < (uint32_t)kMaxPolls) {
    __builtin_amdgcn_s_sleep(1);
    ++polls;
  }
  if (polls >= (uint32_t)kMaxPolls) {
    *abort = 1u;
    return false;
  }
  return true;
}

// Grid of a persistent grouped GEMM: one workgroup per CU (a multiple of 8,
// the XCD count), more when a workgroup's item table would overflow; a.nslots
// and a.ntiles set (the worst-case item count is their product).
inline hipError_t grouped_grid(const GemvArgs &a, unsigned *grid) {
  int dev = 0, cus = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (err != hipSuccess) return err;
  if (cus < 1) return hipErrorInvalidConfiguration;
  const long items = (long)a.nslots * a.ntiles;
  long g = (cus + 7) / 8 * 8;
  const long need = (items + kGMaxItems - 1) / kGMaxItems;
  if (g < need) g = (need + 7) / 8 * 8;
  *grid = (unsigned)g;
  return hipSuccess;
}

}  // namespace qmoe
