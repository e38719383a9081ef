"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Dequantisation and gathering must match bit for bit; matmuls must satisfy
|y - y_ref| <= 1e-3 * sum_k |w_nk x_k| + 1e-6 per element on the stored
output.  Small variants keep K and shrink N so every output is checked; the
full-size workloads run in the launch configuration the benchmark times and
are checked on sampled rows."""
import contextlib
import functools
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
import q1_synth as S

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_decode_q1_amd as Q


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def wdict(w):
    return dict(packed=w.packed, scales=w.scales, biases=w.biases, meta=w.meta, symmetric=w.symmetric, K=w.K)


@functools.lru_cache(maxsize=None)
def wl(index, small=False):
    return S.workload(index, small=small)


@functools.lru_cache(maxsize=None)
def dev_weight(index, name, small=False):
    return Q.PackedQ1.from_host(wl(index, small).weights[name])


def x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def out_host(t):
    t = t.detach().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    return t.view(torch.int16).numpy().view(np.uint16)


TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.load_library()
    assert Q.q1_device_supported(0), Q.q1_last_error()
    yield
    torch.cuda.synchronize()


def check_qmm(y, out_dtype, w, x_bits, rows=None, label="", dense=False):
    """Packed and wide matrix-core paths (weights used exactly): against the
    exact-weight oracle.  Dense fallback (weights rounded to bf16, then a bf16
    GEMM): against the oracle of that definition, and against the
    exact-weight oracle within the tolerance plus the bf16 weight-rounding
    bound."""
    y_ref, A = O.qmm_ref(x_bits, **wdict(w), row_index=rows, weights_bf16=dense)
    got = out_host(y)
    if rows is not None:
        got = got[..., rows]
    ok, ratio, nbad = O.check_close(got, out_dtype, y_ref, A)
    _say(f"  {label}: worst err/bound = {ratio:.3e}, violations = {nbad}")
    assert ok, f"{label}: {nbad} elements outside tolerance (worst ratio {ratio})"
    if dense:
        y0, A0 = O.qmm_ref(x_bits, **wdict(w), row_index=rows)
        dev = np.abs(O.out_to_f64(got, out_dtype) - y0)
        lim = O.tolerance(A) + O.dense_rounding_bound(A0)
        _say(f"  {label}: vs exact weights, worst err/bound = {np.max(dev / lim):.3e}")
        assert (dev <= lim).all()
    return ratio


# ----------------------------------------------------------------- dequant / gather (bit-exact)

@pytest.mark.parametrize("index,small", [(1, False), (2, True), (3, True), (4, True)])
@pytest.mark.parametrize("out_dtype", ["bf16", "f16", "f32"])
def test_dequant_bitexact_small(index, small, out_dtype):
    _say(f"dequant cfg{index} small={small} out={out_dtype}")
    name = "w"
    w = wl(index, small).weights[name]
    got = out_host(Q.q1_dequantize(dev_weight(index, name, small), TORCH_DT[out_dtype]))
    ref = O.dequantize(w.packed, w.scales, w.biases, w.meta, w.symmetric, w.K, out_dtype)
    if out_dtype == "f32":
        got, ref = got.view(np.uint32), ref.view(np.uint32)
    assert np.array_equal(got, ref)


def test_dequant_bitexact_full_lm_head_sampled():
    _say("dequant cfg4 full, sampled rows")
    w = wl(4).weights["w"]
    got = Q.q1_dequantize(dev_weight(4, "w"), torch.bfloat16)
    rng = np.random.default_rng(0)
    rows = np.unique(np.concatenate([rng.integers(0, w.N, 300), [0, w.N - 1]]))
    ref = O.dequantize(w.packed[rows], w.scales[rows], None, w.meta, True, w.K, "bf16")
    assert np.array_equal(out_host(got[torch.from_numpy(rows).cuda()]), ref)


def test_dequant_signed_zero_and_negative_scales():
    _say("dequant signed zeros")
    rng = np.random.Generator(np.random.PCG64(21))
    N, K = 8, 256
    packed = rng.integers(0, 1 << 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    sc = np.array([[0.0, -0.0], [-1.5, 2.0], [1e-8, -3e-5], [0.0, 0.0]] * 2, dtype=np.float32)
    bi = np.array([[-0.0, 0.0], [0.0, -0.0], [-0.0, -0.0], [1.0, -1.0]] * 2, dtype=np.float32)
    for meta in ("f16", "bf16"):
        for sym in (True, False):
            w = S.Q1Weight(packed, S.meta_bits(sc, meta), None if sym else S.meta_bits(bi, meta), meta, N, K)
            for od in ("bf16", "f16", "f32"):
                got = out_host(Q.q1_dequantize(Q.PackedQ1.from_host(w), TORCH_DT[od]))
                ref = O.dequantize(w.packed, w.scales, w.biases, meta, sym, K, od)
                if od == "f32":
                    got, ref = got.view(np.uint32), ref.view(np.uint32)
                assert np.array_equal(got, ref), (meta, sym, od)


def test_embed_rows_full_table_bitexact():
    _say("embed cfg4 full: 4096 ids")
    wk = wl(4)
    w = wk.weights["w"]
    ids = torch.from_numpy(wk.ids).cuda()
    got = out_host(Q.q1_embed_rows(ids, dev_weight(4, "w"), torch.bfloat16))
    ref = O.embed_rows(wk.ids, w.packed, w.scales, None, w.meta, True, w.K, "bf16")
    assert got.shape == (4096, 5120)
    assert np.array_equal(got, ref)
    # rows equal the full dequantisation's rows byte for byte
    sub = wk.ids[:64]
    deq = Q.q1_dequantize(dev_weight(4, "w"), torch.bfloat16)
    assert np.array_equal(out_host(deq[torch.from_numpy(sub.astype(np.int64)).cuda()]), got[:64])


def test_embed_rows_bad_ids_and_int64():
    _say("embed bad ids")
    w = wl(4, True).weights["w"]
    bad = np.array([-1, w.N, 2 ** 31 - 1, 5, 0, w.N - 1], dtype=np.int64)
    for dt in (np.int32, np.int64):
        ids = torch.from_numpy(bad.astype(dt)).cuda()
        for od in ("bf16", "f32"):
            got = out_host(Q.q1_embed_rows(ids, dev_weight(4, "w", True), TORCH_DT[od]))
            ref = O.embed_rows(bad, w.packed, w.scales, None, w.meta, True, w.K, od)
            if od == "f32":
                got, ref = got.view(np.uint32), ref.view(np.uint32)
            assert np.array_equal(got, ref)
    empty = torch.empty(0, dtype=torch.int32, device="cuda")
    assert Q.q1_embed_rows(empty, dev_weight(4, "w", True)).shape == (0, w.K)


# ----------------------------------------------------------------- packed GEMV, every output

@pytest.mark.parametrize("index,small,M", [(1, False, 1), (1, False, 2)] + [(2, True, m) for m in range(1, 9)] +
                         [(3, True, m) for m in range(1, 9)] + [(4, True, 1)])
def test_qmm_small_all_outputs(index, small, M):
    w_l = wl(index, small)
    w = w_l.weights["w"]
    x = w_l.x["x"][:M]
    _say(f"qmm cfg{index} small={small} M={M} N={w.N} K={w.K}")
    y = Q.q1_qmm(x_dev(x), dev_weight(index, "w", small), TORCH_DT[w_l.out_dtype])
    check_qmm(y, w_l.out_dtype, w, x, label=f"cfg{index} M={M}")


@pytest.mark.parametrize("out_dtype", ["f32", "bf16", "f16"])
def test_qmm_output_dtypes(out_dtype):
    w_l = wl(3, True)
    w = w_l.weights["w"]
    x = w_l.x["x"][:3]
    _say(f"qmm out dtype {out_dtype}")
    y = Q.q1_qmm(x_dev(x), dev_weight(3, "w", True), TORCH_DT[out_dtype])
    check_qmm(y, out_dtype, w, x, label=out_dtype)


@pytest.mark.parametrize("N,K,meta,sym", [(1, 128, "f16", True), (3, 1152, "bf16", False), (33, 2176, "f16", True),
                                          (17, 4224, "bf16", True), (130, 9216, "f16", False)])
@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_qmm_ragged_shapes(N, K, meta, sym, M):
    _say(f"qmm ragged N={N} K={K} {meta} sym={sym} M={M}")
    rng = np.random.Generator(np.random.PCG64(N * 7 + K + M))
    w = S.draw_weight(rng, N, K, meta, sym)
    x = S.draw_x(rng, M, K)
    y = Q.q1_qmm(x_dev(x), Q.PackedQ1.from_host(w), torch.float32)
    check_qmm(y, "f32", w, x, label=f"N={N} K={K} M={M}")


def test_qmm_one_hot_columns_exact():
    # x = one-hot at k (bf16 1.0): y[:, n] is exactly the fp32 dequantised
    # column -- independent of summation order.
    _say("qmm one-hot columns")
    w = wl(2, True).weights["w"]
    K = w.K
    ks = [0, 1, 31, 32, 127, 128, 1023, 1024, 4095, K - 1]
    x = np.zeros((len(ks[:8]), K), dtype=np.float32)
    for r, k in enumerate(ks[:8]):
        x[r, k] = 1.0
    xb = O.f32_to_bf16_rne(x)
    y = out_host(Q.q1_qmm(x_dev(xb), dev_weight(2, "w", True), torch.float32))
    deq = O.dequant_f32(w.packed, w.scales, None, w.meta, True, K)
    for r, k in enumerate(ks[:8]):
        assert np.array_equal(y[r], deq[:, k]), k  # values: a zero scale may give either signed zero


def test_qmm_leading_dims_identical_bytes():
    _say("qmm [2,4,K] vs [8,K]")
    w_l = wl(3, True)
    x = w_l.x["x"][:8]
    W = dev_weight(3, "w", True)
    y8 = Q.q1_qmm(x_dev(x), W, torch.bfloat16)
    y24 = Q.q1_qmm(x_dev(x).view(2, 4, -1), W, torch.bfloat16)
    assert y24.shape == (2, 4, W.N)
    assert torch.equal(y24.view(8, -1).view(torch.int16), y8.view(torch.int16))


def test_qmm_deterministic():
    _say("qmm determinism")
    w_l = wl(3)
    x = x_dev(w_l.x["x"][:2])
    W = dev_weight(3, "w")
    a = Q.q1_qmm(x, W, torch.float32)
    b = Q.q1_qmm(x, W, torch.float32)
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_qmm_empty_batch():
    W = dev_weight(1, "w")
    y = Q.q1_qmm(torch.empty(0, 1024, dtype=torch.bfloat16, device="cuda"), W, torch.float32)
    assert y.shape == (0, 1024)


# ----------------------------------------------------------------- full sizes, sampled rows

def _sample_rows(N, n=384, seed=0):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.integers(0, N, n), [0, 1, N - 2, N - 1]]))


@pytest.mark.parametrize("M", list(range(1, 9)))
def test_qmm_full_ffn_up_sampled(M):
    w_l = wl(2)
    w = w_l.weights["w"]
    x = w_l.x["x"][:M]
    _say(f"qmm cfg2 full M={M}")
    y = Q.q1_qmm(x_dev(x), dev_weight(2, "w"), torch.bfloat16)
    check_qmm(y, "bf16", w, x, rows=_sample_rows(w.N, seed=M), label=f"cfg2 M={M}")


@pytest.mark.parametrize("M", list(range(1, 10)))
def test_qmm_full_ffn_down_sampled(M):
    w_l = wl(3)
    w = w_l.weights["w"]
    x = w_l.x["x"][:M]
    _say(f"qmm cfg3 full M={M} ({'wide' if M > 8 else 'packed'})")
    y = Q.q1_qmm(x_dev(x), dev_weight(3, "w"), torch.bfloat16)
    check_qmm(y, "bf16", w, x, rows=_sample_rows(w.N, seed=100 + M), label=f"cfg3 M={M}")


def test_qmm_full_lm_head_sampled():
    w_l = wl(4)
    w = w_l.weights["w"]
    x = w_l.x["x"][:1]
    _say("qmm cfg4 full M=1 (tied head)")
    y = Q.q1_qmm(x_dev(x), dev_weight(4, "w"), torch.float32)
    check_qmm(y, "f32", w, x, rows=_sample_rows(w.N, 1024), label="cfg4 M=1")


def test_dispatch_threshold_override():
    _say("threshold override")
    w_l = wl(2, True)
    w = w_l.weights["w"]
    x = w_l.x["x"][:5]
    prev = Q.q1_set_max_packed_rows(4)
    try:
        y = Q.q1_qmm(x_dev(x), dev_weight(2, "w", True), torch.float32)  # M=5 -> wide path
        check_qmm(y, "f32", w, x, label="M=5 wide")
    finally:
        Q.q1_set_max_packed_rows(prev)


# ----------------------------------------------------------------- wide path (M > 8)

@contextlib.contextmanager
def dense_fallback():
    """Routes M > max rows to the dense fallback (dequantise to bf16 + bf16
    GEMM) instead of the wide matrix-core kernel, for the calls inside."""
    prev = os.environ.get("Q1_WIDE_KERNEL")
    os.environ["Q1_WIDE_KERNEL"] = "dequant"
    try:
        yield
    finally:
        if prev is None:
            del os.environ["Q1_WIDE_KERNEL"]
        else:
            os.environ["Q1_WIDE_KERNEL"] = prev


def test_wide_m512_against_oracle_and_packed():
    w_l = wl(5)
    w = w_l.weights["gate"]
    x = w_l.x["x"]
    _say("wide M=512 K=5120 N=17408")
    W = dev_weight(5, "gate")
    y = Q.q1_qmm(x_dev(x), W, torch.bfloat16)
    rows = _sample_rows(w.N, 256, seed=5)
    msel = np.array([0, 1, 15, 16, 100, 255, 300, 511])
    check_qmm(y[torch.from_numpy(msel).cuda()], "bf16", w, x[msel], rows=rows, label="wide M=512")
    # against the packed path, 8 rows at a time: both within their bounds of
    # the exact-weight product, so within the sum of the bounds of each other
    yw = O.out_to_f64(out_host(y), "bf16")
    for m0 in (0, 248, 504):
        yp = O.out_to_f64(out_host(Q.q1_qmm(x_dev(x[m0:m0 + 8]), W, torch.bfloat16)), "bf16")
        _, A0 = O.qmm_ref(x[m0:m0 + 8], **wdict(w), row_index=rows)
        diff = np.abs(yp[:, rows] - yw[m0:m0 + 8][:, rows])
        lim = 2 * O.tolerance(A0)
        _say(f"  packed vs wide rows {m0}..{m0 + 7}: worst diff/bound = {np.max(diff / lim):.3e}")
        assert (diff <= lim).all()


@pytest.mark.parametrize("M", [9, 40])
def test_wide_small_all_outputs(M):
    w_l = wl(5, True)
    w = w_l.weights["gate"]
    x = w_l.x["x"][:M]
    _say(f"wide small M={M}")
    y = Q.q1_qmm(x_dev(x), dev_weight(5, "gate", True), torch.float32)
    check_qmm(y, "f32", w, x, label=f"wide M={M}")


@pytest.mark.parametrize("meta,sym", [("f16", True), ("bf16", False)])
@pytest.mark.parametrize("M,N,K", [(23, 1000, 640), (17, 37, 128), (130, 300, 1152)])
def test_wide_ragged_shapes(M, N, K, meta, sym):
    """Ragged edges of the wide kernel: groups that do not fill the last span
    (K/128 = 5, 1, 9), weight rows that do not fill a column block or a
    workgroup tile, activation rows that do not fill a 16-row block or the
    8-block tile, all outputs checked."""
    rng = np.random.Generator(np.random.PCG64(7000 + M + N + K + sym))
    w = S.draw_weight(rng, N, K, meta, sym)
    x = S.draw_x(rng, M, K)
    _say(f"wide ragged M={M} N={N} K={K} {meta} sym={sym}")
    y = Q.q1_qmm(x_dev(x), Q.PackedQ1.from_host(w), torch.float32)
    check_qmm(y, "f32", w, x, label=f"wide ragged M={M} N={N} K={K}")


def test_wide_dense_fallback_small():
    w_l = wl(5, True)
    w = w_l.weights["gate"]
    x = w_l.x["x"][:40]
    _say("dense fallback small M=40")
    with dense_fallback():
        y = Q.q1_qmm(x_dev(x), dev_weight(5, "gate", True), torch.float32)
    check_qmm(y, "f32", w, x, label="dense M=40", dense=True)


# ----------------------------------------------------------------- fused FFN

def _ffn_check(index, small, M, label, dense=False):
    w_l = wl(index, small)
    g, u, d = (w_l.weights[k] for k in ("gate", "up", "down"))
    x = w_l.x["x"][:M]
    _say(f"ffn {label} M={M}")
    with (dense_fallback() if dense else contextlib.nullcontext()):
        y, h = Q.q1_ffn(x_dev(x), *(dev_weight(index, k, small) for k in ("gate", "up", "down")),
                        return_hidden=True)
    ref = O.ffn_ref(x, wdict(g), wdict(u), wdict(d), weights_bf16=dense)
    hg = out_host(h)
    dh = np.abs(O.bf16_to_f32(hg).astype(np.float64) - ref["h64"])
    hb = O.ffn_h_bound(ref)
    _say(f"  h: worst ratio {np.max(dh / hb):.3e}")
    assert (dh <= hb).all()
    # down stage on the GPU's own h
    y_h, A_h = O.qmm_ref(hg, **wdict(d), weights_bf16=dense)
    ok, ratio, _ = O.check_close(out_host(y), "bf16", y_h, A_h)
    _say(f"  y (on gpu h): worst ratio {ratio:.3e}")
    assert ok
    yb = O.ffn_y_bound(ref, wdict(d), weights_bf16=dense)
    assert O.check_within(out_host(y), "bf16", ref["y"], yb)[0]


@pytest.mark.parametrize("M", list(range(1, 9)))
def test_ffn_small(M):
    _ffn_check(5, True, M, "small")


@pytest.mark.parametrize("M", [1, 5, 7, 8])
def test_ffn_full(M):
    _ffn_check(5, False, M, "full")


def test_ffn_wide_small():
    _ffn_check(5, True, 24, "wide")


def test_ffn_dense_fallback_small():
    _ffn_check(5, True, 24, "dense", dense=True)


@pytest.mark.parametrize("M,up_sym", [(3, False), (20, False), (20, True), (33, None)])
def test_ffn_mixed_formats(M, up_sym):
    """Gate f16 symmetric with up bf16 affine (the narrow path cannot pair
    them; the wide path converts x once per kind), up of the gate's kind (one
    activation image for both), and all three affine (up_sym None)."""
    _say(f"ffn mixed formats M={M} up_sym={up_sym}")
    rng = np.random.Generator(np.random.PCG64(55 + M))
    H, I, Ho = 1024, 640, 384
    gsym = up_sym is not None
    g = S.draw_weight(rng, I, H, "f16" if gsym else "bf16", gsym)
    u = S.draw_weight(rng, I, H, "f16" if up_sym else "bf16", bool(up_sym))
    d = S.draw_weight(rng, Ho, I, "bf16", False)
    x = S.draw_x(rng, M, H)
    y, h = Q.q1_ffn(x_dev(x), *(Q.PackedQ1.from_host(t) for t in (g, u, d)), return_hidden=True)
    ref = O.ffn_ref(x, wdict(g), wdict(u), wdict(d))
    dh = np.abs(O.bf16_to_f32(out_host(h)).astype(np.float64) - ref["h64"])
    assert (dh <= O.ffn_h_bound(ref)).all()
    assert O.check_within(out_host(y), "bf16", ref["y"], O.ffn_y_bound(ref, wdict(d)))[0]
