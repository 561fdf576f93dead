// Plain single-threaded C++17 CPU oracle of the FP4 weight-only MoE expert path.
//
// TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
// baseline of the benchmark load this library (oracle/cpp.py).  The HIP
// library never includes, links or calls it, and it shares no code, header
// or table with it.  Arithmetic is IEEE double; there is no threading, no
// SIMD intrinsic, no blocking or reordering beyond the definitions below.
//
// Sources (pages, by title and section):
//   [OpDoc]      "MoE and QMoE -- CUDA Operator Documentation": section 1
//                (the chain router top-k softmax -> permute -> GEMM1 ->
//                activation -> GEMM2 -> un-permute -> weighted sum), 6.4
//                (FP8 storage), 6.5 (FP4 packing and scale layouts), 8
//                (SwiGLU variants and fusion modes), 9b (NVFP4: E4M3
//                block-16 scales and the per-expert global scale), 13
//                (reference computation: dequantize, then multiply).
//   [GEMV PR]    "[CUDA] Speed up the NVFP4 QMoE decode GEMV and enable it
//                for MTP verify": expanded rows up to 64, nibble order.
//   [Dequant PR] "[CUDA] Coalesce QMoE MXFP4/NVFP4 weight dequantization":
//                E4M3FN / E8M0 scale codecs, output [E][N][K] bf16.
//   [Routing PR] "[CUDA] Cut the MoE routing prologue/epilogue cost for
//                small-batch decode": stable top-k key, expert maps,
//                finalize.
//
// Readings the pages leave open (the same ones the numpy oracle takes):
//   * low nibble of byte j = column 2j, high nibble = column 2j+1;
//   * block scales laid out [E][K/B][N]; FP8 weights [E][N][K];
//   * MXFP4 without a global scale uses g = 1;
//   * dequant to bf16: code*scale exact, *g rounds once to f32, f32 -> bf16 RNE;
//   * top-k chosen on the raw f32 logits, ties to the lower expert index,
//     -0 == +0, NaN ranks below -inf; weights = softmax over the k chosen;
//   * expanded row r = t*k + j; permuted order = expert ascending, then r;
//   * interleaved SwiGLU: column 2j gate, 2j+1 linear (fusion 2:
//     j gate, I+j linear); h = G*sigmoid(alpha*G)*(L+beta), G = min(gate,
//     limit), L = clamp(lin, -limit, limit);
//   * h is rounded to bf16 (RNE, one step from the exact value) between FC1
//     and FC2; y and the finalized output stay unrounded doubles.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <vector>

namespace {

enum Fmt { NVFP4 = 0, MXFP4 = 1, FP8 = 2 };

// E2M1 ([OpDoc] 9b.3): bit 3 sign, bits 2..1 exponent (bias 1), bit 0
// mantissa; exponent field 0 is the subnormal 0.5*m.  Code 8 is -0.
double e2m1(unsigned code) {
    unsigned e = (code >> 1) & 3u, m = code & 1u;
    double mag = (e == 0) ? 0.5 * m : std::ldexp(1.0 + 0.5 * m, (int)e - 1);
    return (code & 8u) ? -mag : mag;
}

// E4M3FN ([Dequant PR], the shared scale template): bias 7, exponent field
// 0 subnormal (m/8 * 2^-6), no infinity, S.1111.111 is NaN, max 448.
double e4m3fn(unsigned b) {
    unsigned e = (b >> 3) & 15u, m = b & 7u;
    double mag;
    if (e == 15 && m == 7) mag = NAN;
    else if (e == 0) mag = std::ldexp(m / 8.0, -6);
    else mag = std::ldexp(1.0 + m / 8.0, (int)e - 7);
    return (b & 0x80u) ? -mag : mag;
}

// E8M0 ([OpDoc] 6.5): 2^(b-127); 0xFF is NaN.
double e8m0(unsigned b) { return b == 255u ? NAN : std::ldexp(1.0, (int)b - 127); }

double block_scale(unsigned b, int fmt) { return fmt == NVFP4 ? e4m3fn(b) : e8m0(b); }

int block_size(int fmt) { return fmt == NVFP4 ? 16 : 32; }

// float32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
uint16_t bf16_from_f32(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    if (std::isnan(f)) return (uint16_t)((u >> 16) | 0x40u);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// double -> bf16 bits in ONE round-to-nearest-even step: 8 significant bits
// for normal magnitudes, a fixed quantum of 2^-133 below 2^-126, infinity
// once the rounded magnitude reaches 2^128.
uint16_t bf16_from_f64(double x) {
    if (std::isnan(x)) return 0x7FC0;
    uint16_t sign = std::signbit(x) ? 0x8000 : 0;
    double mag = std::fabs(x);
    if (std::isinf(mag)) return sign | 0x7F80;
    if (mag == 0.0) return sign;
    int e;
    std::frexp(mag, &e);                       // mag = f * 2^e, f in [0.5, 1)
    int qe = e - 8 > -133 ? e - 8 : -133;
    double q = std::ldexp(std::nearbyint(std::ldexp(mag, -qe)), qe);   // default mode: ties to even
    if (q >= std::ldexp(1.0, 128)) return sign | 0x7F80;
    float qf = (float)q;                       // exact: <= 8 significant bits, in float range
    uint32_t u;
    std::memcpy(&u, &qf, 4);
    return sign | (uint16_t)(u >> 16);
}

double bf16_value(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    std::memcpy(&f, &u, 4);
    return (double)f;
}

struct Weights {
    const uint8_t *w;        // FP4: [E][K][N/2]; FP8: [E][N][K]
    const uint8_t *s;        // FP4: [E][K/B][N]; FP8: unused
    const float *g;          // [E] or null (g = 1)
    int E, K, N, fmt;
};

// One dequantized weight W[e][k][n] as an exact double ([OpDoc] 13, 6.4, 6.5):
//   FP4: e2m1(code) * block scale * g;  FP8: e4m3(byte) * g.
double weight(const Weights &W, int e, int k, int n) {
    double g = W.g ? (double)W.g[e] : 1.0;
    if (W.fmt == FP8) {
        return e4m3fn(W.w[((size_t)e * W.N + n) * W.K + k]) * g;
    }
    uint8_t byte = W.w[((size_t)e * W.K + k) * (W.N / 2) + n / 2];
    unsigned code = (n & 1) ? (byte >> 4) : (byte & 15u);
    uint8_t sb = W.s[((size_t)e * (W.K / block_size(W.fmt)) + k / block_size(W.fmt)) * W.N + n];
    return e2m1(code) * block_scale(sb, W.fmt) * g;
}

// Ranks a before b in the top-k order: larger logit first, ties (including
// -0 vs +0) to the lower index, NaN below every number.
bool ranks_before(float la, int a, float lb, int b) {
    bool na = std::isnan(la), nb = std::isnan(lb);
    if (na != nb) return nb;
    if (!na && la != lb) return la > lb;
    return a < b;
}

double swiglu(double gate, double lin, double alpha, double beta, double limit) {
    double G = gate < limit ? gate : limit;
    double L = lin < -limit ? -limit : (lin > limit ? limit : lin);
    return G / (1.0 + std::exp(-alpha * G)) * (L + beta);
}

}  // namespace

extern "C" {

// ---- codecs (exported so the tests can pin them one value at a time) ----
double qo_e2m1(int code) { return e2m1((unsigned)code & 15u); }
double qo_e4m3fn(int byte) { return e4m3fn((unsigned)byte & 255u); }
double qo_e8m0(int byte) { return e8m0((unsigned)byte & 255u); }
uint16_t qo_bf16_from_f32(float f) { return bf16_from_f32(f); }
uint16_t qo_bf16_from_f64(double x) { return bf16_from_f64(x); }
void qo_bf16_from_f32_n(const float *a, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_from_f32(a[i]);
}
void qo_bf16_from_f64_n(const double *a, int64_t n, uint16_t *out) {
    for (int64_t i = 0; i < n; ++i) out[i] = bf16_from_f64(a[i]);
}

// ---- dequant ([OpDoc] 6.5, 13; [Dequant PR]) ----
// out[e][n][k] (bf16 bits) = RNE_bf16(RNE_f32(e2m1 * scale * g)); for FP8 the
// input is [E][N][K] bytes and the value e4m3 * g.  code*scale is exact in
// double, and so is its product with a float32 g (<= 30 significant bits).
void qo_dequant_bf16(const uint8_t *w, const uint8_t *s, const float *g, int E, int K, int N, int fmt,
                     uint16_t *out) {
    Weights W{w, s, g, E, K, N, fmt};
    for (int e = 0; e < E; ++e)
        for (int n = 0; n < N; ++n)
            for (int k = 0; k < K; ++k)
                out[((size_t)e * N + n) * K + k] = bf16_from_f32((float)weight(W, e, k, n));
}

// Dequantized weights of one expert as doubles, [K][N].
void qo_expert_weights_f64(const uint8_t *w, const uint8_t *s, const float *g, int E, int K, int N, int fmt,
                           int e, double *out) {
    Weights W{w, s, g, E, K, N, fmt};
    for (int k = 0; k < K; ++k)
        for (int n = 0; n < N; ++n) out[(size_t)k * N + n] = weight(W, e, k, n);
}

// ---- routing ([OpDoc] 1; [Routing PR]) ----
// For each token: the k experts of largest logit in rank order (repeated
// selection of the best remaining expert), then w_j = exp(l_j - l_max) /
// sum_i exp(l_i - l_max) over the k chosen.
void qo_route_topk(const float *logits, int T, int E, int k, int32_t *idx, double *wts) {
    std::vector<char> taken(E);
    std::vector<double> ex(k);
    for (int t = 0; t < T; ++t) {
        const float *row = logits + (size_t)t * E;
        std::fill(taken.begin(), taken.end(), 0);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e)
                if (!taken[e] && (best < 0 || ranks_before(row[e], e, row[best], best))) best = e;
            taken[best] = 1;
            idx[t * k + j] = best;
        }
        double lmax = row[idx[t * k]];
        double tot = 0.0;
        for (int j = 0; j < k; ++j) {
            ex[j] = std::exp((double)row[idx[t * k + j]] - lmax);
            tot += ex[j];
        }
        for (int j = 0; j < k; ++j) wts[t * k + j] = ex[j] / tot;
    }
}

// Selection as qo_route_topk; the mixing weights are router_weights[t][e] at
// the chosen experts, unchanged ([OpDoc] 2, input 14).
void qo_route_topk_router_weights(const float *logits, const float *router_weights, int T, int E, int k,
                                  int32_t *idx, double *wts) {
    qo_route_topk(logits, T, E, k, idx, wts);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) wts[t * k + j] = (double)router_weights[(size_t)t * E + idx[t * k + j]];
}

// Stable counting sort of the expanded rows r = t*k + j by expert:
// offsets[e] = rows of experts < e, offsets[E] = T*k; the row's permuted
// position p(r) = offsets[e_r] + #{r' < r : e_r' = e_r}.
void qo_expert_maps(const int32_t *idx, int T, int k, int E, int32_t *offsets, int32_t *p2e, int32_t *e2p) {
    int R = T * k;
    std::vector<int> count(E, 0), seen(E, 0);
    for (int r = 0; r < R; ++r) count[idx[r]]++;
    offsets[0] = 0;
    for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + count[e];
    for (int r = 0; r < R; ++r) {
        int e = idx[r];
        int p = offsets[e] + seen[e]++;
        p2e[p] = r;
        e2p[r] = p;
    }
}

// ---- FC1 + SwiGLU ([OpDoc] 1, 8, 13) ----
// For permuted row p of expert e (token t = p2e[p] / k):
//   u[p][n] = sum_k x[t][k] * W1[e][k][n]   (exact products, double sums)
//   h[p][j] = bf16(SwiGLU(gate, lin)) with (gate, lin) = (u[2j], u[2j+1]),
//   or (u[j], u[I+j]) for fusion 2.
// cols (ncols > 0): only these h columns (and their FC1 column pairs) are
// computed; the other h entries are written as 0 and u is left untouched.
// u may be null.  W1 has K = H, N = 2I.
void qo_fc1_swiglu(const uint16_t *x, int k, const uint8_t *w1, const uint8_t *s1, const float *g1, int E, int H,
                   int I, int fmt, const int32_t *offsets, const int32_t *p2e, double alpha, double beta,
                   double limit, int fusion, const int32_t *cols, int ncols, uint16_t *h, double *u) {
    Weights W{w1, s1, g1, E, H, 2 * I, fmt};
    int N = 2 * I;
    int R = offsets[E];
    std::vector<int> hcols;
    if (ncols > 0) hcols.assign(cols, cols + ncols);
    else for (int j = 0; j < I; ++j) hcols.push_back(j);
    for (size_t i = 0; i < (size_t)R * I; ++i) h[i] = 0;
    std::vector<double> wg(H), wl(H);
    for (int e = 0; e < E; ++e) {
        int lo = offsets[e], hi = offsets[e + 1];
        if (lo == hi) continue;
        for (int j : hcols) {
            int ng = fusion == 2 ? j : 2 * j;
            int nl = fusion == 2 ? I + j : 2 * j + 1;
            for (int kk = 0; kk < H; ++kk) {
                wg[kk] = weight(W, e, kk, ng);
                wl[kk] = weight(W, e, kk, nl);
            }
            for (int p = lo; p < hi; ++p) {
                const uint16_t *xr = x + (size_t)(p2e[p] / k) * H;
                double gate = 0.0, lin = 0.0;
                for (int kk = 0; kk < H; ++kk) {
                    double xv = bf16_value(xr[kk]);
                    gate += xv * wg[kk];
                    lin += xv * wl[kk];
                }
                if (u) {
                    u[(size_t)p * N + ng] = gate;
                    u[(size_t)p * N + nl] = lin;
                }
                h[(size_t)p * I + j] = bf16_from_f64(swiglu(gate, lin, alpha, beta, limit));
            }
        }
    }
}

// ---- FC2 ([OpDoc] 1, 13) ----
// y[p][m] = sum_i h[p][i] * W2[e][i][m] for the rows p of expert e (h read
// as bf16 values).  W2 has K = I, N = H.  cols (ncols > 0): only these
// output columns, y laid out [R][ncols]; otherwise y is [R][H].
void qo_fc2(const uint16_t *h, const uint8_t *w2, const uint8_t *s2, const float *g2, int E, int I, int H, int fmt,
            const int32_t *offsets, const int32_t *cols, int ncols, double *y) {
    Weights W{w2, s2, g2, E, I, H, fmt};
    int nc = ncols > 0 ? ncols : H;
    std::vector<double> wc(I);
    for (int e = 0; e < E; ++e) {
        int lo = offsets[e], hi = offsets[e + 1];
        if (lo == hi) continue;
        for (int c = 0; c < nc; ++c) {
            int m = ncols > 0 ? cols[c] : c;
            for (int i = 0; i < I; ++i) wc[i] = weight(W, e, i, m);
            for (int p = lo; p < hi; ++p) {
                double acc = 0.0;
                for (int i = 0; i < I; ++i) acc += bf16_value(h[(size_t)p * I + i]) * wc[i];
                y[(size_t)p * nc + c] = acc;
            }
        }
    }
}

// ---- finalize ([OpDoc] 1 un-permute and weighted sum; [Routing PR]) ----
// out[t][m] = sum_{j<k} w[t][j] * y[e2p[t*k + j]][m], j ascending; unrounded.
void qo_finalize(const double *y, const double *wts, const int32_t *e2p, int T, int k, int H, double *out) {
    for (int t = 0; t < T; ++t)
        for (int m = 0; m < H; ++m) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) acc += wts[t * k + j] * y[(size_t)e2p[t * k + j] * H + m];
            out[(size_t)t * H + m] = acc;
        }
}

// ---- the whole layer: route -> maps -> FC1+SwiGLU -> FC2 -> finalize ----
// router_weights may be null (softmax weights).  Outputs are caller-owned:
// idx/e2p/p2e [T*k], wts [T*k], offsets [E+1], h bf16 [T*k][I], y [T*k][H],
// out [T][H].
void qo_layer(const float *logits, const float *router_weights, const uint16_t *x, int T, int E, int k, int H,
              int I, int fmt, const uint8_t *w1, const uint8_t *s1, const float *g1, const uint8_t *w2,
              const uint8_t *s2, const float *g2, double alpha, double beta, double limit, int fusion,
              int32_t *idx, double *wts, int32_t *offsets, int32_t *p2e, int32_t *e2p, uint16_t *h, double *y,
              double *out) {
    if (router_weights) qo_route_topk_router_weights(logits, router_weights, T, E, k, idx, wts);
    else qo_route_topk(logits, T, E, k, idx, wts);
    qo_expert_maps(idx, T, k, E, offsets, p2e, e2p);
    qo_fc1_swiglu(x, k, w1, s1, g1, E, H, I, fmt, offsets, p2e, alpha, beta, limit, fusion, nullptr, 0, h, nullptr);
    qo_fc2(h, w2, s2, g2, E, I, H, fmt, offsets, nullptr, 0, y);
    qo_finalize(y, wts, e2p, T, k, H, out);
}

}  // extern "C"
