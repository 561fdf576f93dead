"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments with exact status codes before
any launch (every call here returns during host-side validation)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qmoe.h")


@pytest.fixture(scope="module")
def q():
    import fp4_weight_only_amd
    return fp4_weight_only_amd


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qmoe_\w+)\s*\(", src)))


def test_header_declarations_are_exported(q):
    names = declared_functions()
    assert set(names) == set(q.EXPORTS), names
    for n in names:
        assert hasattr(q.lib, n), n


def test_exported_symbols_in_dynamic_table(q):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", q.LIB_PATH], capture_output=True, text=True).stdout
    for n in declared_functions():
        assert re.search(rf"\bT {n}$", out, flags=re.M), n


def test_status_strings(q):
    for s in range(6):
        assert q.lib.qmoe_status_str(s).startswith(b"QMOE_")


A = 4096          # an aligned placeholder address (never dereferenced: validation fails first)
MIS = 4096 + 4    # misaligned placeholder


def weights(q, E=8, K=256, N=256, fmt=0, w=A, s=A, g=A):
    return q.Fp4WeightsC(w, s, g, E, K, N, fmt)


def route(q, logits=A, T=1, E=8, k=2, idx=A, w=A, off=A, p2e=A, e2p=A):
    return q.lib.qmoe_route_topk(logits, T, E, k, idx, w, off, p2e, e2p, None)


def test_route_validation(q):
    assert route(q, logits=None) == q.QMOE_EINVAL
    assert route(q, T=0) == q.QMOE_EINVAL
    assert route(q, k=0) == q.QMOE_EINVAL
    assert route(q, k=9, E=8) == q.QMOE_EINVAL            # k > E
    assert route(q, idx=MIS) == q.QMOE_EALIGN
    assert route(q, E=257, k=2) == q.QMOE_EUNSUPPORTED
    assert route(q, E=64, k=9) == q.QMOE_EUNSUPPORTED


def fc1(q, wc, T=1, k=2, x=A, off=A, p2e=A, h=A, ws=None, nbytes=0, path=0):
    n = ctypes.c_size_t(nbytes)
    st = q.lib.qmoe_fp4_gemv_fc1_swiglu(x, T, k, ctypes.byref(wc), off, p2e, None, h, ws, ctypes.byref(n), path, None)
    return st, n.value


def fc2(q, wc, T=1, k=2, h=A, off=A, y=A, ws=None, nbytes=0, path=0):
    n = ctypes.c_size_t(nbytes)
    st = q.lib.qmoe_fp4_gemv_fc2(h, T, k, ctypes.byref(wc), off, y, ws, ctypes.byref(n), path, None)
    return st, n.value


def test_fc_validation(q):
    assert fc1(q, weights(q, g=0))[0] == q.QMOE_EINVAL                  # NVFP4 needs a global scale
    assert fc1(q, weights(q, fmt=1, g=0))[0] == q.QMOE_OK               # MXFP4 does not (size query)
    assert fc1(q, weights(q, fmt=7))[0] == q.QMOE_EINVAL
    assert fc1(q, weights(q), x=None)[0] == q.QMOE_EINVAL
    assert fc1(q, weights(q, w=MIS))[0] == q.QMOE_EALIGN
    assert fc1(q, weights(q), x=MIS)[0] == q.QMOE_EALIGN
    assert fc1(q, weights(q, K=200))[0] == q.QMOE_EUNSUPPORTED          # K % 16
    assert fc1(q, weights(q, fmt=1, K=272))[0] == q.QMOE_EUNSUPPORTED   # K % 32 for MXFP4
    assert fc1(q, weights(q, N=240))[0] == q.QMOE_EUNSUPPORTED          # N % 32
    assert fc1(q, weights(q, E=300), k=2)[0] == q.QMOE_EUNSUPPORTED
    assert fc1(q, weights(q), k=9)[0] == q.QMOE_EINVAL                  # k > E
    assert fc1(q, weights(q), path=5)[0] == q.QMOE_EINVAL
    assert fc2(q, weights(q), y=None)[0] == q.QMOE_EINVAL


def test_gemv_row_window(q):
    st, _ = fc1(q, weights(q, E=64), T=8, k=8, path=q.QMOE_PATH_GEMV)       # 64 rows
    assert st == q.QMOE_OK
    st, _ = fc1(q, weights(q, E=64), T=13, k=5, path=q.QMOE_PATH_GEMV)      # 65 rows
    assert st == q.QMOE_EUNSUPPORTED
    st, _ = fc2(q, weights(q, E=64), T=9, k=8, path=q.QMOE_PATH_GEMV)
    assert st == q.QMOE_EUNSUPPORTED


def test_workspace_query_and_too_small(q):
    st, need = fc1(q, weights(q, E=256, K=2048, N=1536), T=4, k=8)
    assert st == q.QMOE_OK and need > 0
    # K = 2048 spans at least two k chunks: float32 partials of 32 rows x 1536 columns each
    assert need >= 2 * 32 * 1536 * 4
    st, _ = fc1(q, weights(q, E=256, K=2048, N=1536), T=4, k=8, ws=A, nbytes=need - 1)
    assert st == q.QMOE_EWORKSPACE
    st, need2 = fc2(q, weights(q, E=256, K=768, N=2048), T=4, k=8)
    assert st == q.QMOE_OK and need2 > 0


def test_fc2_finalize_validation_and_workspace(q):
    L = q.lib
    wc = weights(q, E=256, K=768, N=2048)
    n = ctypes.c_size_t(0)
    call = lambda h=A, w=wc, off=A, tw=A, e2p=A, out=A, ws=None, T=4, k=8, path=0: L.qmoe_fp4_gemv_fc2_finalize(
        h, T, k, ctypes.byref(w), off, tw, e2p, out, ws, ctypes.byref(n), path, None)
    assert call() == q.QMOE_OK and n.value > 0
    # FC2 partials are kept even when they span several k chunks: at least one float32 plane of 32 x 2048
    assert n.value >= 32 * 2048 * 4
    need = n.value
    n.value = need - 1
    assert call(ws=A) == q.QMOE_EWORKSPACE
    assert call(tw=None) == q.QMOE_EINVAL
    assert call(e2p=None) == q.QMOE_EINVAL
    assert call(tw=MIS) == q.QMOE_EALIGN
    assert call(T=9, path=q.QMOE_PATH_GEMV) == q.QMOE_EUNSUPPORTED      # 72 rows on the GEMV
    n.value = 0
    assert call(T=9) == q.QMOE_OK and n.value >= 72 * 2048 * 4          # grouped: float32 rows in the workspace


def test_route_router_weights_validation(q):
    L = q.lib
    call = lambda lg=A, rw=A, T=1, E=8, k=2, idx=A: L.qmoe_route_topk_router_weights(
        lg, rw, T, E, k, idx, A, A, A, A, None)
    assert call(rw=None) == q.QMOE_EINVAL
    assert call(lg=None) == q.QMOE_EINVAL
    assert call(k=9) == q.QMOE_EINVAL
    assert call(rw=MIS) == q.QMOE_EALIGN
    assert call(E=257) == q.QMOE_EUNSUPPORTED


def test_auto_path_rule(q):
    """AUTO: the GEMV up to 64 expanded rows, the grouped kernel above (seen
    through qmoe_fp4_resolve_path and the workspace size each path asks for);
    the grouped kernel serves the decode window when asked for explicitly."""
    n = ctypes.c_size_t(0)

    def size(T, k, K, N, path):
        wc = weights(q, E=256, K=K, N=N)
        assert q.lib.qmoe_fp4_gemv_fc2(A, T, k, ctypes.byref(wc), A, A, None, ctypes.byref(n), path,
                                       None) == q.QMOE_OK
        return n.value

    G, V, AU = q.QMOE_PATH_GROUPED, q.QMOE_PATH_GEMV, q.QMOE_PATH_AUTO
    res = ctypes.c_int(-1)

    def resolved(T, k, K, N, path=AU):
        wc = weights(q, E=256, K=K, N=N)
        st = q.lib.qmoe_fp4_resolve_path(T, k, ctypes.byref(wc), path, ctypes.byref(res))
        return st, res.value

    assert resolved(8, 8, 768, 2048) == (q.QMOE_OK, V)              # 64 rows: the GEMV window
    assert resolved(1, 8, 2048, 1536) == (q.QMOE_OK, V)
    assert resolved(9, 8, 2048, 1536) == (q.QMOE_OK, G)             # 72 rows
    assert resolved(8, 8, 768, 2048, G) == (q.QMOE_OK, G)           # explicit grouped inside the window
    assert resolved(9, 8, 2048, 1536, V)[0] == q.QMOE_EUNSUPPORTED  # past the GEMV window
    assert resolved(8, 8, 784, 2048, G)[0] == q.QMOE_EUNSUPPORTED   # K % 64
    # the GEMV grid holds at most 8191 column tiles of 256 (N <= 2,096,896)
    assert resolved(8, 8, 32, 8191 * 256, V) == (q.QMOE_OK, V)
    assert resolved(8, 8, 32, 8191 * 256 + 32, V)[0] == q.QMOE_EUNSUPPORTED
    assert resolved(8, 8, 32, 8191 * 256 + 32)[0] == q.QMOE_EUNSUPPORTED  # AUTO in the GEMV window
    assert q.lib.qmoe_fp4_resolve_path(1, 1, ctypes.byref(weights(q)), AU, None) == q.QMOE_EINVAL
    assert size(8, 8, 768, 2048, G) != size(8, 8, 768, 2048, V)
    assert size(8, 8, 768, 2048, AU) == size(8, 8, 768, 2048, V)
    assert size(9, 8, 768, 2048, AU) == size(9, 8, 768, 2048, G)


def test_route_fc1_validation_and_workspace(q):
    L = q.lib
    wc = weights(q, E=16, K=256, N=512)
    n = ctypes.c_size_t(0)

    def call(lg=A, rw=None, x=A, T=4, k=2, w=wc, idx=A, tw=A, off=A, p2e=A, e2p=A, h=A):
        n.value = 0
        return L.qmoe_fp4_route_fc1_swiglu(lg, rw, x, T, k, ctypes.byref(w), None, idx, tw, off, p2e, e2p, h, None,
                                           ctypes.byref(n), None)

    assert call() == q.QMOE_OK
    fused = n.value
    n2 = ctypes.c_size_t(0)
    assert L.qmoe_fp4_gemv_fc1_swiglu(A, 4, 2, ctypes.byref(wc), A, A, None, A, None, ctypes.byref(n2),
                                      q.QMOE_PATH_GEMV, None) == q.QMOE_OK
    assert fused == n2.value                      # the same GEMV workspace
    assert call(rw=A) == q.QMOE_OK                # router_weights is optional
    for kw in ("lg", "x", "idx", "tw", "off", "p2e", "e2p", "h"):
        assert call(**{kw: None}) == q.QMOE_EINVAL, kw
    for kw in ("lg", "rw", "x", "idx", "tw", "off", "p2e", "e2p", "h"):
        assert call(**{kw: MIS}) == q.QMOE_EALIGN, kw
    assert call(T=8, k=8) == q.QMOE_OK            # 64 rows: the one-wave maps' limit
    assert call(T=33, k=2) == q.QMOE_EUNSUPPORTED  # 66 rows
    assert call(T=0) == q.QMOE_EINVAL
    assert call(k=17) == q.QMOE_EINVAL            # k > E
    assert call(w=weights(q, E=300, K=256, N=512), k=9) == q.QMOE_EUNSUPPORTED
    assert call(w=weights(q, E=16, K=250, N=512)) == q.QMOE_EUNSUPPORTED   # K % 16


def test_layer_decode_validation_and_workspace(q):
    L = q.lib
    w1 = weights(q, E=16, K=512, N=512)      # H = 512, 2I = 512
    w2 = weights(q, E=16, K=256, N=512)      # I = 256, H = 512
    n = ctypes.c_size_t(0)

    def call(lg=A, rw=None, x=A, T=4, k=2, a=w1, b=w2, rin=0, idx=A, tw=A, off=A, p2e=A, e2p=A, out=A):
        n.value = 0
        return L.qmoe_fp4_moe_layer_decode(lg, rw, x, T, k, ctypes.byref(a), ctypes.byref(b), None, rin, idx, tw,
                                           off, p2e, e2p, out, None, ctypes.byref(n), None)

    assert call() == q.QMOE_OK and n.value > 0
    both = n.value
    n1 = ctypes.c_size_t(0)
    assert L.qmoe_fp4_gemv_fc1_swiglu(A, 4, 2, ctypes.byref(w1), A, A, None, A, None, ctypes.byref(n1),
                                      q.QMOE_PATH_GEMV, None) == q.QMOE_OK
    assert both >= n1.value                       # both layers' partial sums
    assert call(rin=1) == q.QMOE_OK and n.value == both
    assert call(rin=2) == q.QMOE_EINVAL
    for kw in ("lg", "x", "idx", "tw", "off", "p2e", "e2p", "out"):
        assert call(**{kw: None}) == q.QMOE_EINVAL, kw
    for kw in ("lg", "rw", "x", "idx", "tw", "off", "p2e", "e2p", "out"):
        assert call(**{kw: MIS}) == q.QMOE_EALIGN, kw
    assert call(b=weights(q, E=16, K=128, N=512)) == q.QMOE_EINVAL   # FC2 K != FC1 N / 2
    assert call(b=weights(q, E=16, K=256, N=256)) == q.QMOE_EINVAL   # FC2 N != FC1 K
    assert call(b=weights(q, E=8, K=256, N=512)) == q.QMOE_EINVAL    # expert counts differ
    assert call(T=8, k=8) == q.QMOE_OK
    assert call(T=33, k=2) == q.QMOE_EUNSUPPORTED                     # 66 rows


def test_layer_decode_noalloc_validation(q):
    """The allocation-free layer call runs the same checks before touching the
    device, and refuses a shape whose partial sums exceed its fixed scratch."""
    L = q.lib
    w1 = weights(q, E=16, K=512, N=512)
    w2 = weights(q, E=16, K=256, N=512)

    def call(lg=A, x=A, T=4, k=2, a=w1, b=w2, rin=0, out=A):
        return L.qmoe_fp4_moe_layer_decode_noalloc(lg, None, x, T, k, ctypes.byref(a), ctypes.byref(b), None, rin,
                                                   A, A, A, A, A, out, None)

    assert call(rin=2) == q.QMOE_EINVAL
    assert call(lg=None) == q.QMOE_EINVAL
    assert call(out=MIS) == q.QMOE_EALIGN
    assert call(b=weights(q, E=16, K=128, N=512)) == q.QMOE_EINVAL
    assert call(T=33, k=2) == q.QMOE_EUNSUPPORTED
    big1 = weights(q, E=8, K=8192, N=8192)
    big2 = weights(q, E=8, K=4096, N=8192)
    assert call(T=8, k=8, a=big1, b=big2) == q.QMOE_EWORKSPACE      # 67 MB of partial sums
    assert q.NOALLOC_SCRATCH_BYTES == 32 << 20


def fc1_act(q, wc, act, T=1, k=2, path=0):
    n = ctypes.c_size_t(0)
    st = q.lib.qmoe_fp4_gemv_fc1_swiglu(A, T, k, ctypes.byref(wc), A, A, ctypes.byref(act), A, None,
                                        ctypes.byref(n), path, None)
    return st, n.value


def test_swiglu_fusion_modes_and_workspace(q):
    wc = weights(q, E=16, K=256, N=512)          # K = 256: one k chunk on the GEMV
    std = lambda f: q.SwigluC(1.0, 0.0, float("inf"), f)
    st0, n0 = fc1_act(q, wc, std(0))
    st1, n1 = fc1_act(q, wc, std(q.QMOE_SWIGLU_INTERLEAVED))
    st2, n2 = fc1_act(q, wc, std(q.QMOE_SWIGLU_CONCAT))
    assert st0 == st1 == st2 == q.QMOE_OK
    assert n0 == n1                                  # fusion 0 is the interleaved layout
    assert n2 >= 2 * 512 * 4                         # concatenated: float32 partials of 2 rows x 512
    assert fc1_act(q, wc, std(3))[0] == q.QMOE_EINVAL
    assert fc1_act(q, wc, std(-1))[0] == q.QMOE_EINVAL
    st, ng = fc1_act(q, wc, std(q.QMOE_SWIGLU_CONCAT), T=32, k=4, path=q.QMOE_PATH_GROUPED)
    assert st == q.QMOE_OK and ng >= 128 * 512 * 4   # grouped: float32 u rows
    st, ng1 = fc1_act(q, wc, std(q.QMOE_SWIGLU_INTERLEAVED), T=32, k=4, path=q.QMOE_PATH_GROUPED)
    assert st == q.QMOE_OK and ng1 < ng


def test_fp8_validation_and_workspace(q):
    L = q.lib
    W8 = lambda E=16, K=256, N=512, w=A, g=A: q.Fp8WeightsC(w, g, E, K, N)
    n = ctypes.c_size_t(0)
    fc1 = lambda wc, T=2, k=2, act=None, x=A, p2e=A, path=0: L.qmoe_fp8_gemv_fc1_swiglu(
        x, T, k, ctypes.byref(wc), A, p2e, None if act is None else ctypes.byref(act), A, None, ctypes.byref(n),
        path, None)
    fc2 = lambda wc, T=2, k=2, y=A, path=0: L.qmoe_fp8_gemv_fc2(A, T, k, ctypes.byref(wc), A, y, None,
                                                                  ctypes.byref(n), path, None)
    assert fc1(W8()) == q.QMOE_OK and n.value == 256             # interleaved: no workspace beyond the minimum
    assert fc1(W8(), act=q.SwigluC(1.0, 0.0, float("inf"), q.QMOE_SWIGLU_CONCAT)) == q.QMOE_OK
    assert n.value >= 4 * 512 * 4                                # concatenated: float32 u rows
    assert fc1(W8(), act=q.SwigluC(1.0, 0.0, float("inf"), 5)) == q.QMOE_EINVAL
    assert fc1(W8(g=0)) == q.QMOE_EINVAL                         # the global scale is required
    assert fc1(W8(w=0)) == q.QMOE_EINVAL
    assert fc1(W8(), p2e=None) == q.QMOE_EINVAL
    assert fc1(W8(w=MIS)) == q.QMOE_EALIGN
    assert fc1(W8(K=200)) == q.QMOE_EUNSUPPORTED                 # K % 16
    assert fc1(W8(N=528)) == q.QMOE_EUNSUPPORTED                 # N % 32
    assert fc1(W8(E=64), T=13, k=5) == q.QMOE_OK                 # 65 rows: row passes of 8
    assert fc1(W8(E=64), T=(1 << 22) + 1, k=4) == q.QMOE_EUNSUPPORTED   # T*k > 2^24
    assert fc1(W8(E=300)) == q.QMOE_EUNSUPPORTED
    assert fc1(W8(), k=17) == q.QMOE_EINVAL                      # k > E
    assert fc1(W8(K=65536, N=32768)) == q.QMOE_EUNSUPPORTED      # one expert beyond 32-bit offsets
    assert fc2(W8(), y=None) == q.QMOE_EINVAL
    assert fc2(W8()) == q.QMOE_OK
    assert fc1(W8(), path=7) == q.QMOE_EINVAL
    assert fc1(W8(K=272), T=32, k=4, path=q.QMOE_PATH_GROUPED) == q.QMOE_EUNSUPPORTED   # K % 64
    assert fc1(W8(K=272), T=32, k=4) == q.QMOE_OK                                      # AUTO falls back to the GEMV
    assert fc1(W8(), T=32, k=4, path=q.QMOE_PATH_GROUPED) == q.QMOE_OK
    dq = lambda wc, out=A: L.qmoe_dequant_fp8(ctypes.byref(wc), out, None)
    assert dq(W8(g=0)) == q.QMOE_EINVAL
    assert dq(W8(), out=MIS) == q.QMOE_EALIGN
    assert dq(W8(K=17, N=33)) == q.QMOE_EUNSUPPORTED


def test_finalize_and_dequant_validation(q):
    L = q.lib
    assert L.qmoe_finalize(None, A, A, 1, 2, 256, A, None) == q.QMOE_EINVAL
    assert L.qmoe_finalize(A, A, A, 1, 9, 256, A, None) == q.QMOE_EUNSUPPORTED
    assert L.qmoe_finalize(A, A, A, 1, 2, 250, A, None) == q.QMOE_EUNSUPPORTED
    assert L.qmoe_finalize(A, MIS, A, 1, 2, 256, A, None) == q.QMOE_EALIGN
    wc = weights(q, K=100)
    assert L.qmoe_dequant_fp4(ctypes.byref(wc), A, None) == q.QMOE_EUNSUPPORTED
    wc = weights(q, K=256, N=128)
    assert L.qmoe_dequant_fp4(ctypes.byref(wc), A, None) == q.QMOE_EUNSUPPORTED
    wc = weights(q, g=0)
    assert L.qmoe_dequant_fp4(ctypes.byref(wc), A, None) == q.QMOE_EINVAL
    wc = weights(q)
    assert L.qmoe_dequant_fp4(ctypes.byref(wc), MIS, None) == q.QMOE_EALIGN
