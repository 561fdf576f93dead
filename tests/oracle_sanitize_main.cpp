// Driver that runs every entry point of the C++ oracle (oracle/qmoe_oracle.cpp)
// on small inputs, for a build with AddressSanitizer and UndefinedBehavior-
// Sanitizer on the host (tests/test_oracle_sanitizers.py).  Test
// infrastructure: it exercises the oracle's loops and indexing at the shapes
// the tests use (both FP4 codecs, FP8, concatenated and GPT-OSS SwiGLU,
// router weights, column subsets, E = 256 / k = 8 routing) and checks a few
// invariants so that a silently wrong run also fails.  Exit status 0 = pass.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <vector>

extern "C" {
double qo_e2m1(int code);
double qo_e4m3fn(int byte);
double qo_e8m0(int byte);
uint16_t qo_bf16_from_f32(float f);
uint16_t qo_bf16_from_f64(double x);
void qo_bf16_from_f32_n(const float *a, int64_t n, uint16_t *out);
void qo_bf16_from_f64_n(const double *a, int64_t n, uint16_t *out);
void qo_dequant_bf16(const uint8_t *w, const uint8_t *s, const float *g, int E, int K, int N, int fmt, uint16_t *out);
void qo_expert_weights_f64(const uint8_t *w, const uint8_t *s, const float *g, int E, int K, int N, int fmt, int e,
                           double *out);
void qo_route_topk(const float *logits, int T, int E, int k, int32_t *idx, double *wts);
void qo_route_topk_router_weights(const float *logits, const float *router_weights, int T, int E, int k,
                                  int32_t *idx, double *wts);
void qo_expert_maps(const int32_t *idx, int T, int k, int E, int32_t *offsets, int32_t *p2e, int32_t *e2p);
void qo_fc1_swiglu(const uint16_t *x, int k, const uint8_t *w1, const uint8_t *s1, const float *g1, int E, int H,
                   int I, int fmt, const int32_t *offsets, const int32_t *p2e, double alpha, double beta,
                   double limit, int fusion, const int32_t *cols, int ncols, uint16_t *h, double *u);
void qo_fc2(const uint16_t *h, const uint8_t *w2, const uint8_t *s2, const float *g2, int E, int I, int H, int fmt,
            const int32_t *offsets, const int32_t *cols, int ncols, double *y);
void qo_finalize(const double *y, const double *wts, const int32_t *e2p, int T, int k, int H, double *out);
void qo_layer(const float *logits, const float *router_weights, const uint16_t *x, int T, int E, int k, int H,
              int I, int fmt, const uint8_t *w1, const uint8_t *s1, const float *g1, const uint8_t *w2,
              const uint8_t *s2, const float *g2, double alpha, double beta, double limit, int fusion,
              int32_t *idx, double *wts, int32_t *offsets, int32_t *p2e, int32_t *e2p, uint16_t *h, double *y,
              double *out);
}

namespace {

int g_fail = 0;

void expect(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "FAIL: %s\n", what);
        g_fail = 1;
    }
}

struct Rng {  // xorshift64*: input bytes only
    uint64_t s;
    uint64_t next() {
        s ^= s >> 12;
        s ^= s << 25;
        s ^= s >> 27;
        return s * 0x2545F4914F6CDD1DULL;
    }
    double uniform() { return (double)(next() >> 11) * 0x1p-53; }
};

// Scale bytes with finite values: E4M3 exponent field 3..8, E8M0 119..129.
uint8_t scale_byte(Rng &r, int fmt) {
    if (fmt == 0) return (uint8_t)(((r.next() & 1) << 7) | ((3 + r.next() % 6) << 3) | (r.next() & 7));
    return (uint8_t)(119 + r.next() % 11);
}

void run_layer(int fmt, int T, int E, int k, int H, int I, int fusion, bool rw, bool gmx, uint64_t seed) {
    Rng r{seed * 0x9E3779B97F4A7C15ULL + 1};
    const int R = T * k, N1 = 2 * I;
    const bool fp8 = fmt == 2;
    const int B = fmt == 0 ? 16 : 32;
    std::vector<float> logits((size_t)T * E), rwv((size_t)T * E);
    for (auto &v : logits) v = (float)(r.uniform() * 4.0 - 2.0);
    for (auto &v : rwv) v = (float)r.uniform();
    std::vector<uint16_t> x((size_t)T * H);
    for (auto &v : x) v = qo_bf16_from_f64(r.uniform() * 2.0 - 1.0);
    // FP4: w [E][K][N/2], s [E][K/B][N]; FP8: w [E][N][K]
    std::vector<uint8_t> w1(fp8 ? (size_t)E * N1 * H : (size_t)E * H * I), w2(fp8 ? (size_t)E * H * I : (size_t)E * I * (H / 2));
    for (auto &v : w1) v = fp8 ? (uint8_t)(((r.next() & 1) << 7) | ((4 + r.next() % 6) << 3) | (r.next() & 7))
                               : (uint8_t)r.next();
    for (auto &v : w2) v = fp8 ? (uint8_t)(((r.next() & 1) << 7) | ((4 + r.next() % 6) << 3) | (r.next() & 7))
                               : (uint8_t)r.next();
    std::vector<uint8_t> s1, s2;
    if (!fp8) {
        s1.resize((size_t)E * (H / B) * N1);
        s2.resize((size_t)E * (I / B) * H);
        for (auto &v : s1) v = scale_byte(r, fmt);
        for (auto &v : s2) v = scale_byte(r, fmt);
    }
    std::vector<float> g1(E), g2(E);
    for (auto &v : g1) v = (float)(0.5 + 1.5 * r.uniform());
    for (auto &v : g2) v = (float)(0.5 + 1.5 * r.uniform());
    const bool with_g = fmt != 1 || gmx;
    const float *pg1 = with_g ? g1.data() : nullptr, *pg2 = with_g ? g2.data() : nullptr;
    const uint8_t *ps1 = fp8 ? nullptr : s1.data(), *ps2 = fp8 ? nullptr : s2.data();
    const double alpha = fusion == 2 ? 1.702 : 1.0, beta = fusion == 2 ? 1.0 : 0.0;
    const double limit = fusion == 2 ? 7.0 : INFINITY;

    std::vector<int32_t> idx(R), off(E + 1), p2e(R), e2p(R);
    std::vector<double> wts(R), y((size_t)R * H), out((size_t)T * H);
    std::vector<uint16_t> h((size_t)R * I);
    qo_layer(logits.data(), rw ? rwv.data() : nullptr, x.data(), T, E, k, H, I, fmt, w1.data(), ps1, pg1, w2.data(),
             ps2, pg2, alpha, beta, limit, fusion, idx.data(), wts.data(), off.data(), p2e.data(), e2p.data(),
             h.data(), y.data(), out.data());
    // invariants: maps are inverse bijections, offsets cover every row
    expect(off[E] == R, "offsets[E] == T*k");
    for (int q = 0; q < R; ++q) expect(e2p[p2e[q]] == q, "e2p(p2e(p)) == p");
    if (!rw)
        for (int t = 0; t < T; ++t) {
            double s = 0.0;
            for (int j = 0; j < k; ++j) s += wts[t * k + j];
            expect(std::fabs(s - 1.0) < 1e-12, "softmax weights sum to 1");
        }
    // the step-wise entry points on the same data, with and without column subsets
    std::vector<uint16_t> h2((size_t)R * I);
    std::vector<double> u((size_t)R * N1);
    qo_fc1_swiglu(x.data(), k, w1.data(), ps1, pg1, E, H, I, fmt, off.data(), p2e.data(), alpha, beta, limit, fusion,
                  nullptr, 0, h2.data(), u.data());
    for (size_t i = 0; i < h.size(); ++i) expect(h[i] == h2[i], "fc1 equals the layer's h");
    const int32_t cols[3] = {0, I / 2, I - 1};
    qo_fc1_swiglu(x.data(), k, w1.data(), ps1, pg1, E, H, I, fmt, off.data(), p2e.data(), alpha, beta, limit, fusion,
                  cols, 3, h2.data(), nullptr);
    std::vector<double> y2((size_t)R * H), y3((size_t)R * 3);
    qo_fc2(h.data(), w2.data(), ps2, pg2, E, I, H, fmt, off.data(), nullptr, 0, y2.data());
    const int32_t hcols[3] = {0, H / 3, H - 1};
    qo_fc2(h.data(), w2.data(), ps2, pg2, E, I, H, fmt, off.data(), hcols, 3, y3.data());
    for (int q = 0; q < R; ++q)
        for (int c = 0; c < 3; ++c) expect(y3[(size_t)q * 3 + c] == y2[(size_t)q * H + hcols[c]], "fc2 column subset");
    std::vector<double> out2((size_t)T * H);
    qo_finalize(y2.data(), wts.data(), e2p.data(), T, k, H, out2.data());
    for (size_t i = 0; i < out.size(); ++i) expect(out[i] == out2[i], "finalize equals the layer's out");
    // dequant and one expert's dense weights
    std::vector<uint16_t> dq((size_t)E * N1 * H);
    qo_dequant_bf16(w1.data(), ps1, pg1, E, H, N1, fmt, dq.data());
    std::vector<double> dense((size_t)H * N1);
    qo_expert_weights_f64(w1.data(), ps1, pg1, E, H, N1, fmt, E - 1, dense.data());
    for (int kk = 0; kk < H; kk += 7)
        for (int n = 0; n < N1; n += 5)
            expect(dq[((size_t)(E - 1) * N1 + n) * H + kk] == qo_bf16_from_f32((float)dense[(size_t)kk * N1 + n]),
                   "dequant equals the dense weights rounded");
}

}  // namespace

int main() {
    // codecs over their whole input range
    for (int c = 0; c < 16; ++c) expect(std::fabs(qo_e2m1(c)) <= 6.0, "e2m1 range");
    for (int b = 0; b < 256; ++b) {
        const double v = qo_e4m3fn(b);
        expect(((b & 0x7F) == 0x7F) ? std::isnan(v) : std::fabs(v) <= 448.0, "e4m3 range");
        const double s = qo_e8m0(b);
        expect(b == 255 ? std::isnan(s) : s > 0.0, "e8m0 range");
    }
    const float fs[] = {0.f, -0.f, 1.f, -1.5f, 3.0e38f, -3.0e38f, 1e-40f, INFINITY, -INFINITY, NAN};
    std::vector<uint16_t> b16(10);
    qo_bf16_from_f32_n(fs, 10, b16.data());
    const double ds[] = {0.0, -0.0, 1.0, 1.0 + 0x1p-9, 1e300, -1e300, 1e-320, INFINITY, -INFINITY, NAN};
    qo_bf16_from_f64_n(ds, 10, b16.data());
    expect(qo_bf16_from_f64(1.0) == 0x3F80, "bf16(1) == 0x3F80");
    // routing at the largest E and k, with ties and infinities
    {
        const int T = 3, E = 256, k = 8;
        std::vector<float> lg((size_t)T * E, 0.5f);
        lg[5] = INFINITY;
        lg[E + 9] = -INFINITY;
        for (int e = 0; e < E; ++e) lg[2 * E + e] = (float)(e % 4);
        std::vector<int32_t> idx(T * k), off(E + 1), p2e(T * k), e2p(T * k);
        std::vector<double> wts(T * k);
        qo_route_topk(lg.data(), T, E, k, idx.data(), wts.data());
        qo_route_topk_router_weights(lg.data(), lg.data(), T, E, k, idx.data(), wts.data());
        qo_expert_maps(idx.data(), T, k, E, off.data(), p2e.data(), e2p.data());
        expect(idx[k] == 0 && idx[2 * k] == 3, "ties go to the lower expert");
    }
    run_layer(0, 3, 9, 4, 64, 32, 1, false, false, 1);   // NVFP4, interleaved
    run_layer(0, 5, 12, 3, 96, 48, 2, true, false, 2);   // NVFP4, GPT-OSS concatenated, router weights
    run_layer(1, 4, 8, 2, 64, 64, 1, false, false, 3);   // MXFP4
    run_layer(1, 2, 6, 6, 128, 32, 2, false, true, 4);   // MXFP4 + global scale, concatenated
    run_layer(2, 3, 10, 4, 48, 40, 1, false, false, 5);  // FP8
    run_layer(2, 2, 5, 5, 32, 16, 2, true, false, 6);    // FP8 concatenated, router weights, k = E
    if (g_fail) return 1;
    std::printf("oracle sanitizer run ok\n");
    return 0;
}
