// Internal host-side launch interface between the C ABI (abi.hip) and the
// kernels.  Arguments are validated by the ABI before any launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qmoe {

constexpr int kGemvTileN = 256;    // output columns per GEMV block (32 lanes x 8 columns)
constexpr int kGemvLaneK = 32;     // k rows per lane
constexpr int kGemvWaveK = 64;     // k rows per wave (two 32-lane halves)
constexpr int kGemvMaxWaves = 4;   // waves per GEMV block (k chunk of 256 rows)

struct GemvArgs {
  const uint16_t *act;     // FC1: x [T][K]; FC2: h [rows][K]
  const int32_t *p2e;      // FC1 only: permuted row -> expanded row
  const int32_t *offsets;  // [E+1]
  const uint8_t *w;
  const uint8_t *scales;
  const float *gscale;     // may be null
  int32_t E, K, N, topk, rows;
  int32_t nslots, ntiles, nchunks;
  int32_t split_rows;      // 0: a slot is one routed expert; G > 0: a group of at most G rows of one expert
  int32_t waves;           // waves per block; the k chunk is waves * 64 rows
  int32_t fc1;             // 1: act rows gathered by token, SwiGLU epilogue, bf16 out
  int32_t force_partials;  // GEMV: write g * partial sums even for one k chunk, run no epilogue
  int32_t concat;          // FC1: gate = column j, linear = column N/2 + j (else 2j, 2j+1)
  float alpha, beta, limit;
  uint16_t *out_bf16;      // FC1: h [rows][N/2]
  float *out_f32;          // FC2: y [rows][N]
  float *partials;         // [nchunks][rows][N] split-K partials (nchunks > 1)
  // FC1 GEMV with fused routing (route_logits set, rows <= 64): every
  // workgroup selects the top-k experts of all route_T tokens and builds the
  // expert maps in LDS (offsets and p2e above are then not read); workgroup 0
  // also writes them to the route_* outputs.
  const float *route_logits;  // [route_T][E]
  const float *route_rw;      // [route_T][E] router_weights, or null: softmax weights
  int32_t route_T;
  int32_t *route_idx;         // [route_T][topk]
  float *route_w;             // [route_T][topk]
  int32_t *route_offsets;     // [E+1]
  int32_t *route_p2e;         // [rows]
  int32_t *route_e2p;         // [rows]
  // FC2 with FC1's SwiGLU folded into the activation staging (h_partials
  // set): h[p][j] is formed from FC1's split-K partials exactly as the FC1
  // epilogue forms it (planes summed in order from -0, SwiGLU, bf16 RNE);
  // act is not read.
  const float *h_partials;    // [h_nchunks][rows][2*K] FC1 u (g applied)
  int32_t h_nchunks;
  int32_t h_concat;           // FC1 pairing: gate j / linear K + j (else 2j, 2j + 1)
  float h_alpha, h_beta, h_limit;
};

// The whole decode layer in one launch (layer.hip): routing, FC1 + SwiGLU,
// FC2 and the weighted un-permute, workgroups handing results to each other
// through the workspace and counters.
struct LayerArgs {
  const float *logits;      // [T][E]
  const float *rw;          // [T][E] router_weights, or null: softmax weights
  const uint16_t *x;        // [T][H] bf16
  const uint8_t *w1, *s1;   // FC1: K = H, N = N1 = 2I
  const float *g1;          // may be null (MXFP4)
  const uint8_t *w2, *s2;   // FC2: K = I, N = H
  const float *g2;
  int32_t T, E, k, H, I;
  int32_t concat;           // FC1 pairing: gate j / linear I + j (else 2j, 2j + 1)
  float alpha, beta, limit;
  int32_t *idx;             // [T][k]
  float *wts;               // [T][k]
  int32_t *offsets;         // [E+1]
  int32_t *p2e, *e2p;       // [T*k]
  uint16_t *out;            // [T][H] bf16
  int32_t *sync;            // counters (zero on entry, zero again on exit) and the error word
  float *part1;             // [nch1][rows][2I] FC1 split-K partial sums (g applied)
  float *part2;             // [nch2][rows][H] FC2 split-K partial sums (g applied)
  int32_t rows;             // T*k (<= 64)
  int32_t nch1, nch2;       // k chunks of 256 rows: ceil(H / 256), ceil(I / 256)
  int32_t ntiles1, ntiles2; // 256-column tiles: ceil(2I / 256), ceil(H / 256)
  int32_t max_polls;        // bound on every wait (then the error word is set and the wait ends)
};

constexpr int kLayerMaxHChunks = 16;   // I <= 4096
constexpr int kLayerMaxTiles2 = 64;    // H <= 16384
constexpr int kLayerSyncStride = 16;   // int32 per counter: one 64-byte segment each
constexpr size_t kLayerSyncBytes =
    (size_t)(2 + kLayerMaxTiles2 + 64 * kLayerMaxHChunks) * kLayerSyncStride * sizeof(int32_t);
// rows per workgroup pass of the layer (1 for one token, 2 for two, else 4)
int layer_rows_per_pass(int T);
// upper bound of the work items of one call (every slot live)
int layer_max_items(const LayerArgs &a);
hipError_t launch_fp4_layer(const LayerArgs &a, int fmt, hipStream_t s);

size_t gemv_workspace_bytes(int32_t rows, int32_t max_rows_per_expert, int32_t E, int32_t K, int32_t N,
                            bool force_partials = false);
void gemv_plan(GemvArgs &a, int max_rows_per_expert, void *ws);
hipError_t launch_fp4_gemv(const GemvArgs &a, int fmt, int max_rows_per_expert, hipStream_t s);

// Sums a.nchunks planes of a.partials per (row, column) and writes SwiGLU ->
// bf16 h (a.fc1) or float32 y.
hipError_t launch_splitk_epilogue(const GemvArgs &a, hipStream_t s);

size_t grouped_workspace_bytes(int32_t rows, int32_t N, bool concat);
hipError_t launch_grouped(GemvArgs &a, int fmt, hipStream_t s);

// FP8 E4M3 weight-only GEMV ([E][N][K] bytes, a.gscale required; a.concat
// uses ws for float32 u rows) and dequant.
size_t fp8_workspace_bytes(int32_t rows, int32_t N, bool concat);
hipError_t launch_fp8_gemv(GemvArgs &a, int max_rows_per_expert, void *ws, hipStream_t s);
hipError_t launch_fp8_grouped(GemvArgs &a, void *ws, hipStream_t s);  // K % 64 == 0
hipError_t launch_fp8_dequant(const uint8_t *w, const float *g, int32_t E, int32_t K, int32_t N, uint16_t *out,
                              hipStream_t s);

hipError_t launch_route(const float *logits, const float *rw, int32_t T, int32_t E, int32_t k, int32_t *idx, float *w,
                        int32_t *offsets, int32_t *p2e, int32_t *e2p, hipStream_t s);

hipError_t launch_finalize(const float *y, int nsplit, size_t plane, const float *w, const int32_t *e2p, int32_t T,
                           int32_t k, int32_t H, uint16_t *out, hipStream_t s);

hipError_t launch_dequant(const uint8_t *w, const uint8_t *scales, const float *g, int32_t E, int32_t K,
                          int32_t N, int fmt, uint16_t *out, hipStream_t s);

}  // namespace qmoe
