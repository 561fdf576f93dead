/*
 * qmoe.h -- C ABI of the FP4 weight-only MoE expert path for AMD MI355X (gfx950).
 *
 * The path is the one of "MoE and QMoE -- CUDA Operator Documentation",
 * section 1: router (top-k softmax) -> permute by expert -> GEMM1 ->
 * SwiGLU -> GEMM2 -> un-permute -> weighted sum, with FP4 (E2M1) weights and
 * bf16 activations (W4A16).  Five calls cover it:
 *
 *   qmoe_route_topk           softmax top-k routing + expert maps
 *                             (qmoe_route_topk_router_weights: DeepSeek-style
 *                             mixing weights from a second tensor)
 *   qmoe_fp4_gemv_fc1_swiglu  FC1 over the routed rows, fused SwiGLU
 *   qmoe_fp4_gemv_fc2         FC2 over the routed rows
 *   qmoe_finalize             weighted un-permute
 *   qmoe_dequant_fp4          standalone FP4 -> bf16 weight dequant
 *
 * FP8 E4M3 weight-only (W8A16) layers have their own calls:
 *
 *   qmoe_fp8_gemv_fc1_swiglu, qmoe_fp8_gemv_fc2, qmoe_dequant_fp8
 *
 * Fused calls for decode-sized batches (bit-identical to the calls they
 * replace):
 *
 *   qmoe_fp4_gemv_fc2_finalize  FC2 + weighted un-permute without y_rows
 *   qmoe_fp4_route_fc1_swiglu   routing inside the FC1 launch
 *   qmoe_fp4_moe_layer_decode   the whole layer: routing, FC1, SwiGLU inside
 *                               FC2's staging, FC2 + finalize (h, y not written)
 *   qmoe_fp4_moe_layer_persistent  the whole layer in one kernel launch
 *   qmoe_fp4_moe_layer_decode_noalloc  the whole layer without a workspace
 *
 * and one host-only query: qmoe_fp4_resolve_path (the kernel path an FC call
 * takes).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Pointers named in a call are device pointers unless stated otherwise;
 *   qmoe_fp4_weights and qmoe_swiglu are host structs whose members point to
 *   device memory.  Every device pointer must be 16-byte aligned
 *   (QMOE_EALIGN otherwise).  The caller owns every buffer; the library
 *   allocates nothing, keeps no state between calls (the allocation-free
 *   layer call aside: its split-K sums live in a file-scope device array)
 *   and never synchronises.
 * - Work is enqueued on `stream` (a hipStream_t; 0 is the null stream) and is
 *   asynchronous.  All argument checks run on the host before any launch; a
 *   failed check returns its status and enqueues nothing.  QMOE_ELAUNCH
 *   reports a launch error; a call made of several launches (the layer
 *   calls, the fused FC2 + finalize, the concatenated-SwiGLU grouped FC1,
 *   any GEMV call with a split-K epilogue) may already have enqueued its
 *   earlier launches when a later one fails, and its outputs are then
 *   undefined.  Device faults surface at the caller's next synchronisation.
 * - bf16 values are passed as their 16-bit patterns (uint16_t).
 *
 * Data layouts
 * ------------
 * FP4 weights of one FC layer, E experts, reduction length K, N outputs:
 *   w      [E][K][N/2] uint8: byte (e,k,j) holds column 2j in its low nibble
 *          and column 2j+1 in its high nibble (the [K, N/2] "2 per byte
 *          along N" packing of the operator documentation, section 6.5).
 *          A nibble is an E2M1 code: bit 3 sign, bits 2..1 exponent (bias 1),
 *          bit 0 mantissa.
 *   scales [E][K/B][N] uint8: one block scale per B consecutive k of a
 *          column (the [e][k/group_size][n] order the decode GEMV reads,
 *          section 9b.2).  NVFP4: B = 16, E4M3FN bytes (section 9b).
 *          MXFP4: B = 32, E8M0 bytes (section 6.5).
 *   gscale [E] float32 per-expert global scale; required for NVFP4, optional
 *          for MXFP4 (NULL means 1.0).
 *   weight(e,k,n) = e2m1(code) * scale(e, k/B, n) * gscale(e).
 * FC1: K = hidden H, N = 2*I, columns interleaved (2j = gate, 2j+1 = linear),
 *      or concatenated (j = gate, I + j = linear) with qmoe_swiglu.fusion = 2.
 * FC2: K = I, N = H.
 */
#ifndef QMOE_H
#define QMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t *hipStream_t;

typedef enum {
  QMOE_OK = 0,
  QMOE_EINVAL = 1,        /* null pointer, non-positive size, k > E, missing NVFP4 global scale, bad enum */
  QMOE_EUNSUPPORTED = 2,  /* valid request outside what the kernels cover (see each call)                */
  QMOE_EALIGN = 3,        /* a device pointer is not 16-byte aligned                                       */
  QMOE_EWORKSPACE = 4,    /* the workspace passed is smaller than the size the call needs                 */
  QMOE_ELAUNCH = 5        /* the kernel launch failed                                                      */
} qmoe_status;

typedef enum {
  QMOE_FMT_NVFP4 = 0,     /* E4M3FN block-16 scales, float32 per-expert global scale required */
  QMOE_FMT_MXFP4 = 1      /* E8M0 block-32 scales, global scale optional (NULL = 1.0)         */
} qmoe_fmt;

typedef enum {
  QMOE_PATH_AUTO = 0,     /* GEMV for T*k <= 64 expanded rows, GROUPED above                   */
  QMOE_PATH_GEMV = 1,     /* FP4 decode GEMV; rejects T*k > 64 with QMOE_EUNSUPPORTED          */
  QMOE_PATH_GROUPED = 2   /* MFMA bf16 grouped GEMM over LDS-dequantised weight tiles          */
} qmoe_path;

typedef struct {
  const uint8_t *w;       /* [E][K][N/2] device */
  const uint8_t *scales;  /* [E][K/B][N] device */
  const float *gscale;    /* [E] device, or NULL (MXFP4 only) */
  int32_t E, K, N;
  int32_t fmt;            /* qmoe_fmt */
} qmoe_fp4_weights;

/* FC1 column layout of the SwiGLU pair (the swiglu_fusion attribute,
 * operator documentation section 8).  0 is read as interleaved, as the
 * section says the QMoE operator treats swiglu_fusion = 0. */
#define QMOE_SWIGLU_INTERLEAVED 1  /* gate = column 2j, linear = column 2j+1 */
#define QMOE_SWIGLU_CONCAT 2       /* gate = column j, linear = column I + j */

typedef struct {
  float alpha, beta, limit;  /* SwiGLU(G, L) = G*sigmoid(alpha*G)*(L+beta), G = min(gate, limit), L = clamp(lin, -limit, limit) */
  int32_t fusion;            /* 0 or QMOE_SWIGLU_INTERLEAVED, or QMOE_SWIGLU_CONCAT; other values: QMOE_EINVAL */
} qmoe_swiglu;

/* FP8 E4M3 weights of one FC layer (W8A16, operator documentation sections
 * 6.4 and 10): raw E4M3FN bytes, no block scales, no packing.
 *   w      [E][N][K] uint8 device: byte (e,n,k) is weight (k, n) of expert e
 *          (each output column's K weights contiguous).
 *   gscale [E] float32 device, required: weight(e,k,n) = e4m3(byte) * gscale(e),
 *          the per-expert scale the pages apply to the product in the epilogue. */
typedef struct {
  const uint8_t *w;
  const float *gscale;
  int32_t E, K, N;
} qmoe_fp8_weights;

#define QMOE_MAX_EXPERTS 256
#define QMOE_MAX_TOPK 8
/* the GEMV path: at most 64 expanded rows and N <= 8191 * 256 = 2,096,896
 * output columns (QMOE_EUNSUPPORTED otherwise) */
#define QMOE_GEMV_MAX_ROWS 64

/*
 * qmoe_route_topk -- softmax top-k routing and the per-expert permutation.
 *
 * Passages: operator documentation section 1 ("router (top-k softmax) ->
 * permute by expert"); PR 31156 "[CUDA] Cut the MoE routing prologue/epilogue
 * cost for small-batch decode" (register bitonic top-k per row with a stable
 * packed key; expert maps ranked by wave ballots).
 *
 * logits     [T][E] float32 router logits.
 * topk_idx   [T][k] int32 out: selected experts, largest logit first, equal
 *            logits ordered by lower expert index, -0 equal to +0.
 * topk_w     [T][k] float32 out: softmax over the k selected logits (sums to 1).
 * expert_offsets [E+1] int32 out: exclusive prefix sum of per-expert row counts;
 *            expert_offsets[E] = T*k.
 * perm_to_expanded [T*k] int32 out: permuted row p -> expanded row r = t*k + j.
 *            Rows are grouped by ascending expert, in ascending r inside an expert.
 * expanded_to_perm [T*k] int32 out: the inverse map.
 * Limits: 1 <= k <= min(E, 8), 1 <= E <= 256, T >= 1, T*k <= 2^24
 * (QMOE_EUNSUPPORTED beyond E or k limits).  NaN logits give unspecified
 * selections (but valid indices).
 */
qmoe_status qmoe_route_topk(const float *logits, int32_t T, int32_t E, int32_t k,
                            int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                            int32_t *perm_to_expanded, int32_t *expanded_to_perm,
                            hipStream_t stream);

/*
 * qmoe_route_topk_router_weights -- top-k routing with separate mixing weights.
 *
 * Passage: operator documentation section 2, input 14 (router_weights,
 * DeepSeek-style routing: router_probs only selects the experts, the mixing
 * weights are router_weights gathered at the selected indices).
 *
 * As qmoe_route_topk, with router_weights [T][E] float32 in; the selection
 * is made on logits alone, and topk_w[t][j] = router_weights[t][topk_idx[t][j]]
 * exactly (no softmax, no renormalisation).  router_weights NULL: QMOE_EINVAL
 * (call qmoe_route_topk for softmax weights).  Same limits.
 */
qmoe_status qmoe_route_topk_router_weights(const float *logits, const float *router_weights,
                                           int32_t T, int32_t E, int32_t k,
                                           int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                                           int32_t *perm_to_expanded, int32_t *expanded_to_perm,
                                           hipStream_t stream);

/*
 * qmoe_fp4_resolve_path -- the kernel path an FC call with these arguments takes.
 *
 * Passage: operator documentation section 4.3 (the decode GEMV for small
 * batches, the grouped GEMM otherwise); the AUTO rule is that of qmoe_path.
 *
 * T, k, w, path: as for qmoe_fp4_gemv_fc1_swiglu / qmoe_fp4_gemv_fc2 /
 * qmoe_fp4_gemv_fc2_finalize with the same weights.  *resolved (host) out:
 * QMOE_PATH_GEMV or QMOE_PATH_GROUPED.  Returns the status those calls'
 * shape checks return (QMOE_EUNSUPPORTED for a path the shape cannot take);
 * nothing is launched and no device memory is read.
 */
qmoe_status qmoe_fp4_resolve_path(int32_t T, int32_t k, const qmoe_fp4_weights *w, qmoe_path path,
                                  qmoe_path *resolved);

/*
 * qmoe_fp4_gemv_fc1_swiglu -- FC1 of every routed row with fused SwiGLU.
 *
 * Passages: PR 31159 "[CUDA] Speed up the NVFP4 QMoE decode GEMV and enable it
 * for MTP verify" (fused FP4 decode GEMV, expanded rows up to 64); operator
 * documentation sections 8 (SwiGLU, interleaved fusion) and 9b.2 (block-size
 * generic GEMV, scales[e][k/B][n]); section 12.1 (split-K SwiGLU: partials
 * first, SwiGLU on the reduced sum).
 *
 * x          [T][K] bf16 activations (K = H).
 * w1         FC1 weights, N = 2*I.
 * expert_offsets, perm_to_expanded  as written by qmoe_route_topk (same T, k).
 * act        SwiGLU parameters and column layout, or NULL for the standard
 *            SiLU(gate)*linear on interleaved columns.
 * h          [T*k][I] bf16 out, in permuted row order:
 *            h[p][j] = bf16_rne(SwiGLU(u[p][2j], u[p][2j+1])) (interleaved) or
 *            bf16_rne(SwiGLU(u[p][j], u[p][I+j])) (concatenated),
 *            u[p][n] = sum_k x[t(p)][k] * weight(e(p), k, n), accumulated in float32.
 * ws, ws_bytes  workspace.  With ws == NULL the call writes the size it
 *            needs to *ws_bytes and returns QMOE_OK without launching.
 *            Otherwise *ws_bytes is the size of ws (QMOE_EWORKSPACE if too
 *            small).  The workspace is scratch (split-K partial sums, or
 *            the concatenated layout's float32 u rows); its contents on
 *            entry do not matter.  Calls that share a workspace
 *            must be ordered (same stream).
 * path       AUTO, GEMV (T*k <= 64) or GROUPED.
 * Limits: K % B == 0, N % 32 == 0, E <= 256, k <= 8 (QMOE_EUNSUPPORTED).
 */
qmoe_status qmoe_fp4_gemv_fc1_swiglu(const uint16_t *x, int32_t T, int32_t k,
                                     const qmoe_fp4_weights *w1,
                                     const int32_t *expert_offsets, const int32_t *perm_to_expanded,
                                     const qmoe_swiglu *act, uint16_t *h,
                                     void *ws, size_t *ws_bytes, qmoe_path path,
                                     hipStream_t stream);

/*
 * qmoe_fp4_route_fc1_swiglu -- routing and FC1 + SwiGLU in one launch (decode).
 *
 * Passages: PR 29919 (fused routing and expert maps in one kernel for
 * single-token decode), extended here to E <= 256 and up to 64 expanded
 * rows and folded into the FC1 GEMV's prologue; operator documentation
 * section 2 (routing, input 14 router_weights) and the passages of
 * qmoe_fp4_gemv_fc1_swiglu.
 *
 * Equals qmoe_route_topk (router_weights NULL) or
 * qmoe_route_topk_router_weights, followed by qmoe_fp4_gemv_fc1_swiglu with
 * path GEMV, bit for bit: every workgroup of the GEMV selects the top-k
 * experts of all T tokens and ranks the rows by expert in LDS, so it finds
 * its expert without reading maps written by another launch.
 *
 * logits, router_weights (may be NULL), T, k, topk_idx, topk_w,
 * expert_offsets, perm_to_expanded, expanded_to_perm: as qmoe_route_topk /
 * qmoe_route_topk_router_weights (E = w1->E; the map and weight outputs are
 * written by the call).  x, w1, act, h, ws, ws_bytes: as
 * qmoe_fp4_gemv_fc1_swiglu (query the workspace size with ws == NULL).
 * Limits: T*k <= 64 (QMOE_EUNSUPPORTED beyond), and those of both calls.
 */
qmoe_status qmoe_fp4_route_fc1_swiglu(const float *logits, const float *router_weights, const uint16_t *x,
                                      int32_t T, int32_t k, const qmoe_fp4_weights *w1, const qmoe_swiglu *act,
                                      int32_t *topk_idx, float *topk_w, int32_t *expert_offsets,
                                      int32_t *perm_to_expanded, int32_t *expanded_to_perm, uint16_t *h, void *ws,
                                      size_t *ws_bytes, hipStream_t stream);

/*
 * qmoe_fp4_moe_layer_decode -- the whole decode MoE layer: routing, FC1,
 * SwiGLU, FC2 and the weighted un-permute, h never written.
 *
 * Passages: operator documentation section 1 (the chain), section 12.1
 * (split-K SwiGLU: partial sums first, SwiGLU on the reduced sum) and
 * section 9.8 (epilogue fusion); PR 31159 (the decode GEMV and its 64-row
 * window); PR 29919 (routing fused into the path) for route_in_fc1.
 *
 * FC1 writes only its split-K partial sums; every FC2 workgroup forms the
 * bf16 h values its k chunk needs from them (planes summed in order, SwiGLU,
 * round to nearest even, as qmoe_fp4_gemv_fc1_swiglu's epilogue does) while
 * staging its activations, and FC2's split-K planes go to the finalize.  out
 * equals qmoe_route_topk[_router_weights] + qmoe_fp4_gemv_fc1_swiglu (GEMV)
 * + qmoe_fp4_gemv_fc2_finalize (GEMV) bit for bit, as do the routing outputs.
 *
 * logits, router_weights (may be NULL: softmax weights), topk_idx, topk_w,
 * expert_offsets, perm_to_expanded, expanded_to_perm: as qmoe_route_topk /
 * qmoe_route_topk_router_weights (written by the call).  x, w1, act: as
 * qmoe_fp4_gemv_fc1_swiglu; w2: FC2 weights (w2->E == w1->E, w2->K == w1->N/2,
 * w2->N == w1->K).  out [T][H] bf16.
 * route_in_fc1  0: routing runs as its own launch first; 1: inside the FC1
 *            launch (as qmoe_fp4_route_fc1_swiglu).  Anything else: QMOE_EINVAL.
 * ws, ws_bytes  as for the FC calls (query with ws == NULL): both layers'
 *            float32 split-K partials.
 * Limits: T*k <= 64 (QMOE_EUNSUPPORTED beyond), H % 32 == 0, and those of
 * the separate calls; mismatched w1 / w2 shapes: QMOE_EINVAL.
 */
qmoe_status qmoe_fp4_moe_layer_decode(const float *logits, const float *router_weights, const uint16_t *x,
                                      int32_t T, int32_t k, const qmoe_fp4_weights *w1, const qmoe_fp4_weights *w2,
                                      const qmoe_swiglu *act, int32_t route_in_fc1, int32_t *topk_idx, float *topk_w,
                                      int32_t *expert_offsets, int32_t *perm_to_expanded, int32_t *expanded_to_perm,
                                      uint16_t *out, void *ws, size_t *ws_bytes, hipStream_t stream);

/*
 * qmoe_fp4_moe_layer_persistent -- the whole decode MoE layer in one kernel
 * launch: routing, FC1 + SwiGLU, FC2 and the weighted un-permute.
 *
 * Passages: operator documentation section 1 (the chain) and section 12.1
 * (split-K SwiGLU); PR 31159 (the decode GEMV, up to 64 rows); PR 31156 and
 * the fused single-token routing kernel it builds on (PR 29919), which this
 * call extends from the routing prologue to the whole layer.
 *
 * Every output equals qmoe_fp4_moe_layer_decode's (routing outputs and out)
 * bit for bit: the same partial sums, summation orders and roundings.  The
 * kernel's workgroups hand FC1 sums, h and FC2 sums to each other through the
 * workspace and counters in it; it launches no more workgroups than the GPU
 * holds at once (an occupancy query), and every wait in it is bounded.
 *
 * Arguments as qmoe_fp4_moe_layer_decode (without route_in_fc1; w1 and w2
 * share the format).  Workspace (query its size with ws == NULL): its first
 * QMOE_LAYER_SYNC_BYTES bytes are counters that MUST BE ZERO before the first
 * call on this workspace (hipMemset once after allocating it); every
 * completed call leaves them zero again, so calls on one stream need no
 * clearing in between.
 * Bytes 0..3 are an error word: a call that finds a wait run out (possible
 * only if other work keeps some of its workgroups off the GPU) ORs 1 into it,
 * its outputs are then invalid and the counters must be zeroed again; the
 * call never clears the word.  Calls that share a workspace must be ordered
 * (same stream).  Every wait polls at most 2^18 times; the environment
 * variable QMOE_LAYER_MAX_POLLS, read at each call, may lower that bound
 * (tests use a bound of 0 to take the error path on purpose).
 * Limits: T*k <= 64, H % 32 == 0, H <= 16384, I <= 4096, concatenated SwiGLU
 * only with I % 256 == 0 (QMOE_EUNSUPPORTED); w1 / w2 shapes or formats that
 * do not match: QMOE_EINVAL; and the limits of the separate calls.
 */
#define QMOE_LAYER_SYNC_BYTES 69888
qmoe_status qmoe_fp4_moe_layer_persistent(const float *logits, const float *router_weights, const uint16_t *x,
                                          int32_t T, int32_t k, const qmoe_fp4_weights *w1, const qmoe_fp4_weights *w2,
                                          const qmoe_swiglu *act, int32_t *topk_idx, float *topk_w,
                                          int32_t *expert_offsets, int32_t *perm_to_expanded,
                                          int32_t *expanded_to_perm, uint16_t *out, void *ws, size_t *ws_bytes,
                                          hipStream_t stream);

/*
 * qmoe_fp4_moe_layer_decode_noalloc -- qmoe_fp4_moe_layer_decode without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).
 *
 * Arguments and results as qmoe_fp4_moe_layer_decode; the split-K partial
 * sums go to a fixed device array inside the library instead: one copy per
 * GPU it runs on, QMOE_NOALLOC_SCRATCH_BYTES long, held until the process
 * ends (the copy of the current device is used; stream must belong to it).
 * The call allocates nothing and needs no zeroed memory.  A shape whose
 * partial sums exceed the array returns QMOE_EWORKSPACE before any launch
 * (e.g. 64 rows of a hidden 4096 / intermediate 2048 layer need 25.2 MB).
 * Every call on a GPU shares that GPU's array: calls that overlap on one GPU
 * (concurrent streams, other threads) race and must be ordered by the
 * caller.  QMOE_ELAUNCH also covers a failure to resolve the array's address.
 */
#define QMOE_NOALLOC_SCRATCH_BYTES (32u << 20)
qmoe_status qmoe_fp4_moe_layer_decode_noalloc(const float *logits, const float *router_weights, const uint16_t *x,
                                              int32_t T, int32_t k, const qmoe_fp4_weights *w1,
                                              const qmoe_fp4_weights *w2, const qmoe_swiglu *act,
                                              int32_t route_in_fc1, int32_t *topk_idx, float *topk_w,
                                              int32_t *expert_offsets, int32_t *perm_to_expanded,
                                              int32_t *expanded_to_perm, uint16_t *out, hipStream_t stream);

/*
 * qmoe_fp4_gemv_fc2 -- FC2 of every routed row.
 *
 * Passages: PR 31159 (the plain FP4 decode GEMV, "moe_gemv_kernel"); operator
 * documentation section 9b.2.
 *
 * h          [T*k][K] bf16 in permuted row order (K = I), as written by
 *            qmoe_fp4_gemv_fc1_swiglu.
 * w2         FC2 weights, N = H.
 * y_rows     [T*k][N] float32 out, permuted row order:
 *            y[p][n] = sum_i h[p][i] * weight(e(p), i, n), accumulated in float32.
 * T, k       token count and top-k of the routing (T*k rows; at most T rows
 *            per expert).  Workspace and path as for FC1.
 */
qmoe_status qmoe_fp4_gemv_fc2(const uint16_t *h, int32_t T, int32_t k,
                              const qmoe_fp4_weights *w2, const int32_t *expert_offsets,
                              float *y_rows, void *ws, size_t *ws_bytes, qmoe_path path,
                              hipStream_t stream);

/*
 * qmoe_fp4_gemv_fc2_finalize -- FC2 and the weighted un-permute in one call.
 *
 * Passages: operator documentation section 9.8 (epilogue fusion: the
 * finalize folded into the second GEMM's epilogue) and section 12.1;
 * PR 31156 (finalize reads each token's routing metadata once).
 *
 * out[t][n] = bf16_rne( sum_{j<k} topk_w[t][j] * y[expanded_to_perm[t*k+j]][n] )
 * with y = FC2(h) as qmoe_fp4_gemv_fc2 computes it, without writing y_rows:
 * the GEMV path keeps FC2's split-K partial sums in the workspace and the
 * finalize kernel adds them per routed row in the same order the split-K
 * epilogue would, so out equals qmoe_fp4_gemv_fc2 followed by qmoe_finalize
 * bit for bit.  The grouped path writes y's float32 rows to the workspace.
 *
 * h, T, k, w2, expert_offsets: as qmoe_fp4_gemv_fc2.  topk_w, expanded_to_perm:
 * as qmoe_finalize.  out [T][H] bf16 (H = w2->N).
 * ws, ws_bytes, path: as qmoe_fp4_gemv_fc2 (the size differs: query it).
 * Limits: those of qmoe_fp4_gemv_fc2 and qmoe_finalize.
 */
qmoe_status qmoe_fp4_gemv_fc2_finalize(const uint16_t *h, int32_t T, int32_t k,
                                       const qmoe_fp4_weights *w2, const int32_t *expert_offsets,
                                       const float *topk_w, const int32_t *expanded_to_perm,
                                       uint16_t *out, void *ws, size_t *ws_bytes, qmoe_path path,
                                       hipStream_t stream);

/*
 * qmoe_finalize -- weighted un-permute.
 *
 * Passages: operator documentation section 1 ("un-permute -> weighted sum");
 * PR 31156 (finalize stages the routing metadata once per block and splits
 * columns over blocks).
 *
 * out[t][n] = bf16_rne( sum_{j<k} topk_w[t][j] * y_rows[expanded_to_perm[t*k+j]][n] ),
 * summed in float32 in ascending j.  y_rows [T*k][H] float32, topk_w [T][k],
 * out [T][H] bf16.  Limits: H % 8 == 0, k <= 8.
 */
qmoe_status qmoe_finalize(const float *y_rows, const float *topk_w, const int32_t *expanded_to_perm,
                          int32_t T, int32_t k, int32_t H, uint16_t *out, hipStream_t stream);

/*
 * qmoe_dequant_fp4 -- FP4 weights to bf16, transposed to [E][N][K].
 *
 * Passages: PR 31349 "[CUDA] Coalesce QMoE MXFP4/NVFP4 weight dequantization"
 * (tiled, coalesced dequant; one kernel for both scale codecs; no integer
 * division); operator documentation sections 4.3 and 6.5.
 *
 * out[e][n][k] = bf16_rne( f32_rne( e2m1(code) * scale ) * gscale(e) ); the
 * product e2m1*scale is exact, so the output is bit-exact.  MXFP4 without a
 * global scale is exact in bf16.
 * Limits: K % 64 == 0, N % 256 == 0 (QMOE_EUNSUPPORTED otherwise).
 */
qmoe_status qmoe_dequant_fp4(const qmoe_fp4_weights *w, uint16_t *out, hipStream_t stream);

/*
 * qmoe_fp8_gemv_fc1_swiglu / qmoe_fp8_gemv_fc2 -- the FC calls for FP8 weights.
 *
 * Passages: operator documentation section 6.4 (FP8 e4m3: [E, N, K] bytes,
 * pack size 1, per-expert global scale only) and section 10 (W8A16: bf16
 * activations, GEMM output times the expert's global scale in the epilogue;
 * the activation between the GEMMs as for FP4).
 *
 * Arguments, outputs and row order as qmoe_fp4_gemv_fc1_swiglu and
 * qmoe_fp4_gemv_fc2, with w1 (K = H, N = 2*I) or w2 (K = I, N = H) in the FP8
 * layout.  u[p][n] = gscale(e) * sum_k x[k] * e4m3(w[e][n][k]), accumulated in
 * float32.  path: GEMV (any batch; rows in passes of up to 8 per expert),
 * GROUPED (bf16 MFMA grouped GEMM for prefill batches; K % 64 == 0 and
 * T*k*K*2 < 2^31, else QMOE_EUNSUPPORTED) or AUTO (GEMV up to 64 rows or
 * when K % 64 != 0, else GROUPED).  The workspace is needed only for the
 * concatenated SwiGLU layout (float32 u rows); the size query convention is
 * the FP4 calls'.
 * Limits: K % 16 == 0, N % 32 == 0, K*N < 2^31, E <= 256, k <= 8, T*k <= 2^24
 * (QMOE_EUNSUPPORTED); NULL w or gscale: QMOE_EINVAL.
 */
qmoe_status qmoe_fp8_gemv_fc1_swiglu(const uint16_t *x, int32_t T, int32_t k,
                                     const qmoe_fp8_weights *w1,
                                     const int32_t *expert_offsets, const int32_t *perm_to_expanded,
                                     const qmoe_swiglu *act, uint16_t *h,
                                     void *ws, size_t *ws_bytes, qmoe_path path, hipStream_t stream);
qmoe_status qmoe_fp8_gemv_fc2(const uint16_t *h, int32_t T, int32_t k,
                              const qmoe_fp8_weights *w2, const int32_t *expert_offsets,
                              float *y_rows, void *ws, size_t *ws_bytes, qmoe_path path, hipStream_t stream);

/*
 * qmoe_dequant_fp8 -- FP8 weights to bf16 (operator documentation section
 * 4.3, the dequant-to-A16 fallback's FP8 helper; section 10.3).
 *
 * out [E][N][K] bf16 (same layout as w): bf16_rne(float32(e4m3 * gscale(e)))
 * -- the product rounds to float32, then to bf16.  NaN bytes give NaN.
 * Limits: K*N % 16 == 0, E <= 65535 (QMOE_EUNSUPPORTED).
 */
qmoe_status qmoe_dequant_fp8(const qmoe_fp8_weights *w, uint16_t *out, hipStream_t stream);

/* Static string naming a status code. */
const char *qmoe_status_str(qmoe_status s);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_H */
