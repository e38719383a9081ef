"""Host-side tests of the C-ABI boundary (no GPU needed): the library loads,
exports every function the header declares, and rejects invalid arguments with
a clear status and message before making any HIP call."""
import ctypes
import os
import re

import pytest

from gemm_decode_q1_amd import q1 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include"))) if h.endswith(".h")]

pytestmark = pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="libq1.so not built")


def header_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q1_[a-z0-9_]+)\s*\(", text)))


def test_header_lists_the_four_calls():
    fns = header_functions()
    for f in ("q1_qmm", "q1_dequantize", "q1_embed_rows", "q1_ffn"):
        assert f in fns


def test_library_exports_every_header_symbol():
    L = B.load_library()
    for name in header_functions():
        assert hasattr(L, name), name
    assert set(header_functions()) == set(B.EXPORTS)


def test_version_and_empty_error():
    assert B.q1_version().startswith("q1-gfx950")


FAKE = 0x10000  # never dereferenced: validation fails first


def weight(**kw):
    d = dict(packed=FAKE, scales=FAKE, biases=None, meta_dtype=B.Q1_F16, symmetric=1, N=64, K=1024,
             group_size=128, reserved=0)
    d.update(kw)
    return B._Weight(d["packed"], d["scales"], d["biases"], d["meta_dtype"], d["symmetric"], d["N"], d["K"],
                     d["group_size"], d["reserved"])


def qmm(w, M=1, x=FAKE, xd=B.Q1_BF16, y=FAKE, yd=B.Q1_F32, ws=None, wsb=0):
    L = B.load_library()
    st = L.q1_qmm(ctypes.c_void_p(x), xd, M, ctypes.byref(w), ctypes.c_void_p(y), yd,
                  None if ws is None else ctypes.c_void_p(ws), wsb, None)
    return st, L.q1_last_error().decode()


@pytest.mark.parametrize("kw,code,msg", [
    (dict(K=1000), -1, "multiple of 128"),
    (dict(K=0), -1, "multiple of 128"),
    (dict(N=0), -1, "N must be positive"),
    (dict(group_size=64), -2, "group_size"),
    (dict(reserved=3), -1, "reserved"),
    (dict(meta_dtype=B.Q1_F32), -1, "metadata dtype"),
    (dict(symmetric=1, biases=FAKE), -1, "must not carry biases"),
    (dict(symmetric=0, biases=None), -1, "needs a biases pointer"),
    (dict(symmetric=2), -1, "symmetric must be 0 or 1"),
    (dict(packed=None), -1, "packed pointer is NULL"),
    (dict(scales=None), -1, "scales pointer is NULL"),
    (dict(packed=FAKE + 2), -1, "4-byte aligned"),
])
def test_weight_validation(kw, code, msg):
    st, err = qmm(weight(**kw))
    assert st == code and msg in err


def test_activation_validation():
    w = weight()
    assert qmm(w, xd=B.Q1_F32)[0] == -2
    assert qmm(w, M=-1)[0] == -1
    assert qmm(w, yd=7)[0] == -1
    st, err = qmm(w, x=FAKE + 8)
    assert st == -1 and "16-byte aligned" in err
    st, err = qmm(w, x=0)
    assert st == -1 and "NULL" in err


def test_empty_batch_is_a_no_op():
    assert qmm(weight(), M=0, x=0, y=0)[0] == 0


def test_workspace_validation():
    w = weight(K=17408, N=5120)
    L = B.load_library()
    need = L.q1_qmm_workspace_bytes(4, ctypes.byref(w))
    assert need > 0  # 4 rows, 17408 weights per row: a K split (partial sums + counters)
    st, err = qmm(w, M=4)
    assert st == -3 and "workspace too small" in err
    st, err = qmm(w, M=4, ws=FAKE, wsb=need - 1)
    assert st == -3
    wide = L.q1_qmm_workspace_bytes(9, ctypes.byref(w))
    # 9 rows: two blocks of 8 rows, each 2 KB of fp8 operand per 128-weight group
    assert wide >= 2 * (17408 // 128) * 2048


def test_dequant_and_gather_validation():
    L = B.load_library()
    w = weight()
    assert L.q1_dequantize(ctypes.byref(w), ctypes.c_void_p(FAKE), 9, None) == -1
    assert L.q1_dequantize(ctypes.byref(w), None, B.Q1_BF16, None) == -1
    assert L.q1_dequantize(ctypes.byref(weight(K=130)), ctypes.c_void_p(FAKE), B.Q1_BF16, None) == -1
    assert L.q1_embed_rows(ctypes.c_void_p(FAKE), 2, 4, ctypes.byref(w), ctypes.c_void_p(FAKE), B.Q1_BF16, None) == -1
    assert L.q1_embed_rows(ctypes.c_void_p(FAKE), 0, -1, ctypes.byref(w), ctypes.c_void_p(FAKE), B.Q1_BF16, None) == -1
    assert L.q1_embed_rows(None, 0, 0, ctypes.byref(w), None, B.Q1_BF16, None) == 0  # T = 0


def test_ffn_validation():
    L = B.load_library()
    g = weight(N=256, K=512)
    u = weight(N=256, K=512)
    d = weight(N=512, K=512)  # K must equal gate.N = 256
    st = L.q1_ffn(ctypes.c_void_p(FAKE), 1, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ctypes.c_void_p(FAKE),
                  None, 0, None)
    assert st == -1 and "FFN shapes" in L.q1_last_error().decode()
    d = weight(N=512, K=256)
    st = L.q1_ffn(ctypes.c_void_p(FAKE), 1, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d), ctypes.c_void_p(FAKE),
                  None, 0, None)
    assert st == -3
    assert L.q1_ffn_workspace_bytes(1, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d)) >= 256 * 2


def test_max_packed_rows_setter():
    L = B.load_library()
    prev = L.q1_set_max_packed_rows(4)
    try:
        assert prev == 8
        assert L.q1_set_max_packed_rows(0) == -1
        assert L.q1_set_max_packed_rows(9) == -1
        w = weight(K=1024, N=64)
        # M = 5 now goes to the wide path, whose workspace holds the fp8
        # operand image of one 8-row block (2 KB per 128-weight group)
        assert L.q1_qmm_workspace_bytes(5, ctypes.byref(w)) >= (1024 // 128) * 2048
    finally:
        L.q1_set_max_packed_rows(prev)


def test_noalloc_entry_validation():
    """q1_qmm_noalloc checks its arguments, and rejects a call whose scratch
    need exceeds the library's static array, before any HIP call."""
    L = B.load_library()
    w = weight(K=17408, N=5120)

    def call(M, x=FAKE, y=FAKE, yd=B.Q1_BF16):
        st = L.q1_qmm_noalloc(ctypes.c_void_p(x), B.Q1_BF16, M, ctypes.byref(w), ctypes.c_void_p(y), yd, None)
        return st, L.q1_last_error().decode()

    need = L.q1_qmm_workspace_bytes(512, ctypes.byref(w))
    assert need > (8 << 20)
    st, err = call(512)
    assert st == -3 and "static scratch" in err
    assert call(4, x=0)[0] == -1
    assert call(4, yd=9)[0] == -1
    assert call(0, x=0, y=0)[0] == 0
