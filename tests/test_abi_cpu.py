"""C ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest

from bit_lifted_gemv_amd import lq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lq.h")


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lq_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    return lq.load_library()


def test_header_declares_the_binding_exports():
    assert _declared() == sorted(lq.EXPORTS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), name


def test_status_strings(L):
    for code, name in lq.STATUS.items():
        assert L.lq_status_string(code).decode() == name
    assert L.lq_status_string(99).decode() == "LQ_ERR_UNKNOWN"
    assert b"gfx950" in L.lq_version()


# Fake, never-dereferenced device addresses: every call below must fail in
# host-side validation, before any HIP call.
P = 0x10000000
MIS = 0x10000002


def _err(L):
    return L.lq_last_error().decode()


def test_gemv_validation(L):
    ws = 0
    assert L.lq_gemv(None, 8, 64, 4, P, P, 1, P, None, ws, None) == 1       # null weights
    assert L.lq_gemv(P, 8, 64, 4, P, P, 0, P, None, ws, None) == 2          # B = 0
    assert L.lq_gemv(P, 8, 64, 4, P, P, 17, P, None, ws, None) == 2         # B > 16
    assert "1..16" in _err(L)
    assert L.lq_gemv(P, 8, 64, 1, P, P, 1, P, None, ws, None) == 2          # ldw < K/32
    assert L.lq_gemv(P, 8, 96, 3, P, P, 1, P, None, ws, None) == 4          # ldw % 4
    assert L.lq_gemv(P, 8, 96, 6, P, P, 1, P, None, ws, None) == 4
    assert L.lq_gemv(P, 8, 66, 4, P, P, 1, P, None, ws, None) == 2          # K % 4
    assert L.lq_gemv(P + 8, 8, 64, 4, P, P, 1, P, None, ws, None) == 4      # w not 16B-aligned
    assert L.lq_gemv(MIS, 8, 64, 4, P, P, 1, P, None, ws, None) == 4        # misaligned w
    assert L.lq_gemv(P, 8, 64, 4, P, MIS, 1, P, None, ws, None) == 4       # misaligned a_lift
    assert L.lq_gemv(P, 0, 64, 4, P, P, 1, P, None, ws, None) == 2          # m = 0


def test_gemv_workspace_required(L):
    n = ctypes.c_size_t(0)
    m, K = 8192, 68096                 # 67 slices: too long for one workgroup's LDS
    assert L.lq_gemv_workspace_size(m, K, 1, ctypes.byref(n)) == 0
    assert n.value > 0, "this shape splits K and needs partial sums"
    assert L.lq_gemv(P, m, K, K // 32, P, P, 1, P, None, 0, None) == 7
    assert L.lq_gemv(P, m, K, K // 32, P, P, 1, P, P, n.value - 1, None) == 7
    assert L.lq_gemv_workspace_size(m, K, 0, ctypes.byref(n)) == 2
    assert L.lq_gemv_workspace_size(m, K, 1, None) == 1


def test_gemv_one_launch_needs_no_workspace(L):
    """Shapes whose every slice fits one workgroup's LDS take the one-launch
    kernel: no workspace, and a null workspace is accepted."""
    n = ctypes.c_size_t(1)
    for m, K, B in ((28672, 19456, 1), (4096, 10240, 1), (1280, 3072, 5), (4096, 10240, 2)):
        assert L.lq_gemv_workspace_size(m, K, B, ctypes.byref(n)) == 0
        assert n.value == 0, (m, K, B)


def test_gemv_noalloc_validation(L):
    """The no-allocation GEMV checks like lq_gemv, and rejects a shape whose
    workspace exceeds the library's scratch, all before any HIP call."""
    assert L.lq_gemv_noalloc(None, 8, 64, 4, P, P, 1, P, None) == 1
    assert L.lq_gemv_noalloc(P, 8, 64, 4, P, P, 17, P, None) == 2
    assert L.lq_gemv_noalloc(P, 8, 66, 4, P, P, 1, P, None) == 2
    assert L.lq_gemv_noalloc(MIS, 8, 64, 4, P, P, 1, P, None) == 4
    n = ctypes.c_size_t(0)
    m, K = 4096, 1 << 21               # 2048 slices: 32 MiB of partial sums
    assert L.lq_gemv_workspace_size(m, K, 1, ctypes.byref(n)) == 0
    assert n.value > (16 << 20)
    assert L.lq_gemv_noalloc(P, m, K, K // 32, P, P, 1, P, None) == 7
    assert "lq_gemv with a workspace" in _err(L)
    for m, K, B in ((28672, 19456, 16), (8192, 68096, 16), (8192, 68096, 5), (8192, 68096, 1)):
        assert L.lq_gemv_workspace_size(m, K, B, ctypes.byref(n)) == 0
        assert n.value <= (16 << 20), (m, K, B, n.value)


def test_lift_validation(L):
    F16, BF16 = lq.LQ_F16, lq.LQ_BF16
    ok = dict(B=1, n=1280, tb=128, d=10, D=24)

    def call(a=P, adt=F16, B=1, n=1280, t=P, tdt=F16, tb=128, M=P, d=10, D=24, out=P, odt=0):
        return L.lq_lift_activations(a, adt, B, n, t, tdt, tb, M, d, D, out, odt, None)

    assert call(a=None) == 1
    assert call(adt=7) == 3
    assert call(tb=64) == 5
    assert call(n=1300) == 2          # not a multiple of 128
    assert call(n=1280, d=12) == 2    # not a multiple of d
    assert call(d=0) == 2
    assert call(D=300) == 2
    assert call(n=1280, d=64, D=200) == 2   # d*D > 8192
    assert call(B=0) == 2
    assert call(t=MIS) == 4
    assert call(a=P + 8) == 4         # activations not 16-byte aligned
    assert ok  # the happy path needs a GPU and is covered by the GPU tests


def test_lift_parts_validation(L):
    F16, BF16, F32 = lq.LQ_F16, lq.LQ_BF16, lq.LQ_F32
    size = ctypes.c_size_t(0)
    assert L.lq_lift_parts_size(3072, ctypes.byref(size)) == 0
    # 3072 positions = 6 spans of 512, padded to whole groups of 8 spans
    assert size.value == 8 * (4 * 3 * 64 * 32 + 4 * 16 * 4)
    assert L.lq_lift_parts_size(0, ctypes.byref(size)) == 2
    big = size.value

    def call(a=P, adt=BF16, B=6, n=1280, t=P, tdt=BF16, tb=128, M=P, d=8, D=19, out=P, nb=big):
        return L.lq_lift_parts(a, adt, B, n, t, tdt, tb, M, d, D, out, nb, None)

    assert call(a=None) == 1
    assert call(out=None) == 1
    assert call(adt=F16) == 3          # a and t_inv of different types
    assert call(adt=F32, tdt=F32) == 3
    assert call(tb=64) == 5
    assert call(B=0) == 2
    assert call(B=17) == 2
    assert call(n=1300) == 2
    assert call(d=10, D=24) == 5       # d outside {4, 8, 16, 32}
    assert call(d=8, D=4) == 5         # D < d
    assert call(nb=big - 1) == 7       # image buffer too small
    assert call(t=MIS) == 4
    assert call(out=P + 8) == 4


def test_gemv_parts_validation(L):
    size = ctypes.c_size_t(0)
    assert L.lq_gemv_parts_workspace_size(256, 3072, 16, ctypes.byref(size)) == 0
    assert size.value >= 16 * 256 * 4
    assert L.lq_gemv_parts_workspace_size(256, 3072, 17, ctypes.byref(size)) == 2
    ws = size.value
    img = ctypes.c_size_t(0)
    assert L.lq_lift_parts_size(3072, ctypes.byref(img)) == 0

    def call(w=P, m=256, K=3072, ldw=96, s=P, parts=P, nb=img.value, B=16, out=P, wsp=P, nws=ws):
        return L.lq_gemv_parts(w, m, K, ldw, s, parts, nb, B, out, wsp, nws, None)

    assert call(parts=None) == 1
    assert call(wsp=None) == 1
    assert call(B=0) == 2
    assert call(B=17) == 2
    assert call(ldw=95) == 2
    assert call(nb=img.value - 16) == 7
    assert call(nws=ws - 4) == 7
    assert call(wsp=P + 16) == 4


def test_lift_kron_validation(L):
    F16 = lq.LQ_F16
    nb = ctypes.c_size_t(0)
    assert L.lq_lift_kron_workspace_size(4, 8192, ctypes.byref(nb)) == 0
    assert nb.value >= 4 * 8192 * 4 and nb.value % 256 == 0
    assert L.lq_lift_kron_workspace_size(0, 8192, ctypes.byref(nb)) == 2
    WS = 1 << 20

    def call(a=P, B=1, n=8192, n1=64, d=16, D=40, out=P, odt=0, ws=P, wsb=WS, s1=P):
        return L.lq_lift_kron(a, F16, B, n, n1, s1, P, P, P, P, d, D, out, odt, ws, wsb, None)

    assert call(a=None) == 1
    assert call(ws=None) == 1
    assert call(s1=None) == 1
    assert call(odt=9) == 3
    assert call(n1=60) == 2           # n not a multiple of n1
    assert call(n1=32) == 5           # n2 = 256 > 128
    assert call(n1=2048) == 5         # n1 > 256
    assert call(n=8190, n1=63) == 2   # n not a multiple of d
    assert call(n=8192, n1=128, d=48, D=48) == 2   # 8192 % 48 != 0
    assert call(B=0) == 2
    assert call(B=70000) == 2
    assert call(wsb=16) == 7
    assert call(ws=P + 16) == 4
    assert call(s1=MIS) == 4


def test_encode_validation(L):
    nb = ctypes.c_size_t(0)
    assert L.lq_encode_workspace_size(8, 16, ctypes.byref(nb)) == 0
    assert nb.value >= 16 * 16 * 4 and nb.value % 256 == 0
    assert L.lq_encode_workspace_size(8, 33, ctypes.byref(nb)) == 2
    WS = 1 << 12

    def call(w=P, G=10, M=P, A=P, d=8, D=16, codes=P, err=P, ws=P, wsb=WS):
        return L.lq_encode(w, G, M, A, d, D, codes, err, ws, wsb, None)

    assert call(G=0, w=None, M=None, codes=None) == 0      # empty: no-op
    assert call(w=None) == 1
    assert call(codes=None) == 1
    assert call(ws=None) == 1                              # the search needs the workspace
    assert call(d=0) == 2
    assert call(d=9, D=8) == 2                             # D < d
    assert call(D=33) == 2
    assert call(G=-1) == 2
    assert call(d=4, D=30) == 5                            # 2^26 search candidates
    assert call(A=None, d=8, D=25) == 5                    # 2^25 exhaustive candidates
    assert call(wsb=16) == 7
    assert call(ws=P + 16) == 4
    assert call(err=MIS) == 4


def test_softmin_and_adam_validation(L):
    nb = ctypes.c_size_t(0)
    assert L.lq_softmin_workspace_size(1000, 8, 16, ctypes.byref(nb)) == 0
    assert nb.value > 0 and nb.value % 256 == 0
    assert L.lq_softmin_workspace_size(0, 8, 16, ctypes.byref(nb)) == 2

    def call(w=P, N=100, M=P, d=8, D=16, T=10.0, loss=P, grad=P, ws=P, wsb=1 << 30):
        return L.lq_softmin_grad(w, N, M, d, D, T, loss, grad, ws, wsb, None)

    assert call(w=None) == 1
    assert call(ws=None) == 1
    assert call(N=0) == 2
    assert call(d=9, D=8) == 2
    assert call(D=26) == 5                     # valid shape, not built (2^26 codes)
    assert call(T=-1.0) == 2
    assert call(T=float("nan")) == 2
    assert call(wsb=16) == 7
    assert call(ws=P + 4) == 4
    assert call(grad=MIS) == 4

    def adam(M=P, g=P, m1=P, m2=P, n=10, step=1, b1=0.9, b2=0.999):
        return L.lq_adam_update(M, g, m1, m2, n, step, 0.01, b1, b2, 1e-8, None)

    assert adam(n=0, M=None) == 0              # empty: no-op
    assert adam(M=None) == 1
    assert adam(step=0) == 2
    assert adam(b1=1.0) == 2
    assert adam(m2=MIS) == 4


def test_gemm_decoded_validation(L):
    nb = ctypes.c_size_t(0)
    nb.value = 1
    assert L.lq_gemm_decoded_workspace_size(8192, 8192, ctypes.byref(nb)) == 0
    assert nb.value == 0, "the decoded weights stay on chip: no workspace"
    F16, BF16 = lq.LQ_F16, lq.LQ_BF16

    def call(w=P, m=64, n=512, ldw=40, M=P, d=16, D=40, s=P, u=P, udt=F16, B=8, out=P, ws=None,
             wsb=0):
        return L.lq_gemm_decoded(w, m, n, ldw, M, d, D, s, u, udt, B, out, ws, wsb, None)

    assert call(w=None) == 1
    assert call(u=None) == 1
    assert call(udt=BF16) == 3
    assert call(n=500) == 2                  # n % d
    assert call(ldw=39) == 2                 # K = 1280 needs 40 words
    assert call(d=65, n=520, ldw=64) == 2    # d > 64
    assert call(D=257) == 2                  # D > 256
    assert call(B=0) == 2
    assert call(n=(1 << 22) + 16, ldw=(1 << 22) * 5 // 64 + 8) == 2   # 32-bit offsets
    assert call(u=P + 1) == 4


def test_layer_b1_validation(L):
    nb = ctypes.c_size_t(0)
    assert L.lq_layer_b1_workspace_size(28672, 8192, 8, 19, ctypes.byref(nb)) == 0
    assert nb.value > 0
    assert L.lq_layer_b1_workspace_size(64, 256, 4, 4, ctypes.byref(nb)) == 0
    assert nb.value == 0                      # one slice: no partial sums
    BF16, F16 = lq.LQ_BF16, lq.LQ_F16

    def call(a=P, adt=BF16, n=8192, t=P, tdt=BF16, tb=128, M=P, d=8, D=19, w=P, m=64,
             ldw=608, s=P, out=P, ws=P, wsb=1 << 24):
        return L.lq_layer_b1(a, adt, n, t, tdt, tb, M, d, D, w, m, ldw, s, out, ws, wsb, None)

    assert call(a=None) == 1
    assert call(tdt=F16) == 3                 # a and t_inv differ
    assert call(tb=64) == 5
    assert call(n=8000) == 2                  # n % 128
    assert call(d=16, D=8, ldw=128) == 5      # below one bit per weight
    assert call(ldw=600) == 2                 # ldw < ceil(K/32) = 608
    assert call(ldw=610) == 4                 # ldw % 4
    assert call(a=P + 8) == 4
    assert call(wsb=16) == 7
    assert call(ws=P + 16) == 4


def test_gemm_and_pack_validation(L):
    assert L.lq_gemm(P, 8, 64, 2, P, P, lq.LQ_F32, 512, P, None) == 3       # f32 activations
    assert L.lq_gemm(P, 8, 60, 2, P, P, lq.LQ_F16, 512, P, None) == 2       # K % 8
    assert L.lq_gemm(P, 8, 64, 2, P, MIS, lq.LQ_F16, 512, P, None) == 4
    assert L.lq_gemm(P, 8, 64, 2, P, P, lq.LQ_BF16, 0, P, None) == 2
    assert L.lq_pack_signs(P, 4, 64, 64, P, 1, None) == 2                   # ldw too small
    assert L.lq_pack_signs(P, 4, 64, 32, P, 2, None) == 2                   # lds < K
    assert L.lq_pack_signs(None, 4, 64, 64, P, 2, None) == 1
    assert L.lq_pack_signs(P, 0, 64, 64, P, 2, None) == 0                   # empty: no-op
    assert L.lq_unpack_signs(P, 4, 64, 2, None, 64, None) == 1
    assert L.lq_unpack_signs(P, 4, 0, 0, P, 0, None) == 0                   # empty: no-op
    assert L.lq_workspace_clear(None, 16, None) == 1
    assert L.lq_workspace_clear(MIS, 16, None) == 4
    assert L.lq_workspace_clear(None, 0, None) == 0


def test_error_message_is_thread_local_and_cleared(L):
    import threading
    assert L.lq_gemv(None, 8, 64, 4, P, P, 1, P, None, 0, None) == 1
    seen = {}

    def other():
        seen["msg"] = L.lq_last_error().decode()

    th = threading.Thread(target=other)
    th.start()
    th.join()
    assert seen["msg"] == ""
    assert _err(L) != ""
    assert L.lq_pack_signs(P, 0, 64, 64, P, 2, None) == 0
    assert _err(L) == ""
