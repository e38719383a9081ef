"""GPU parity of the kernel choices that only an override selects, and of
the wide path's tile variants, through the C ABI.

* The dense fallback (Higgs PR #212, "Limitations": wider forwards dequantise
  to bf16 and run a dense GEMM) at the wide workload's full size, M = 512,
  K = 5120, N = 17408, on sampled outputs: against the oracle of that
  definition (weights rounded to bf16) and against the packed path.
* The wide kernel with 16-row column blocks (chosen at M = 512, N = 16384).
* Q1_PACKED_KERNEL=table for 2..8 rows (the packed fallback for shapes the
  matrix-core plan rejects) and =mma for one row, every output checked."""
import contextlib
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


def _x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _host(t):
    t = t.detach().cpu()
    return t.numpy() if t.dtype == torch.float32 else t.view(torch.int16).numpy().view(np.uint16)


def _wd(w):
    return dict(packed=w.packed, scales=w.scales, biases=w.biases, meta=w.meta, symmetric=w.symmetric, K=w.K)


@contextlib.contextmanager
def _env(name, value):
    prev = os.environ.get(name)
    os.environ[name] = value
    try:
        yield
    finally:
        if prev is None:
            del os.environ[name]
        else:
            os.environ[name] = prev


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.load_library()
    assert Q.q1_device_supported(0), Q.q1_last_error()
    yield
    torch.cuda.synchronize()


def _rows(N, n, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.integers(0, N, n), [0, N - 1]]))


def test_dense_fallback_full_m512():
    wl = S.workload(5)
    w = wl.weights["gate"]
    x = wl.x["x"]
    W = Q.PackedQ1.from_host(w)
    _say("dense fallback M=512 K=5120 N=17408")
    with _env("Q1_WIDE_KERNEL", "dequant"):
        y = Q.q1_qmm(_x_dev(x), W, torch.bfloat16)
    torch.cuda.synchronize()
    rows = _rows(w.N, 192, 55)
    msel = np.array([0, 7, 64, 200, 383, 511])
    got = O.out_to_f64(_host(y[torch.from_numpy(msel).cuda()]), "bf16")[:, rows]
    ref, A = O.qmm_ref(x[msel], **_wd(w), row_index=rows, weights_bf16=True)
    err = np.abs(got - ref)
    _say(f"  vs bf16-weight oracle: worst err/bound {np.max(err / O.tolerance(A)):.3e}")
    assert (err <= O.tolerance(A)).all()
    ref0, A0 = O.qmm_ref(x[msel], **_wd(w), row_index=rows)
    lim = O.tolerance(A) + O.dense_rounding_bound(A0)
    assert (np.abs(got - ref0) <= lim).all()
    # against the packed path (exact weights), 8 rows at a time
    yd = O.out_to_f64(_host(y), "bf16")
    for m0 in (0, 504):
        yp = O.out_to_f64(_host(Q.q1_qmm(_x_dev(x[m0:m0 + 8]), W, torch.bfloat16)), "bf16")
        _, Ap = O.qmm_ref(x[m0:m0 + 8], **_wd(w), row_index=rows)
        diff = np.abs(yp[:, rows] - yd[m0:m0 + 8][:, rows])
        assert (diff <= 2 * O.tolerance(Ap) + O.dense_rounding_bound(Ap)).all()


@pytest.mark.parametrize("meta,sym", [("f16", True), ("bf16", False)])
def test_wide_tnb16(meta, sym):
    rng = np.random.Generator(np.random.PCG64(16 + sym))
    M, N, K = 512, 16384, 1024
    w = S.draw_weight(rng, N, K, meta, sym)
    x = S.draw_x(rng, M, K)
    _say(f"wide M={M} N={N} K={K} (16 column blocks per workgroup) {meta} sym={sym}")
    y = Q.q1_qmm(_x_dev(x), Q.PackedQ1.from_host(w), torch.float32)
    rows = _rows(N, 256, 3)
    msel = np.array([0, 1, 127, 128, 300, 511])
    got = _host(y[torch.from_numpy(msel).cuda()])[:, rows]
    ref, A = O.qmm_ref(x[msel], **_wd(w), row_index=rows)
    ok, ratio, nbad = O.check_close(got, "f32", ref, A)
    _say(f"  worst err/bound {ratio:.3e}")
    assert ok, nbad


@pytest.mark.parametrize("M", list(range(2, 9)))
@pytest.mark.parametrize("meta,sym,N,K", [("f16", True, 70, 5120), ("bf16", False, 45, 3200)])
def test_forced_table_kernel(M, meta, sym, N, K):
    rng = np.random.Generator(np.random.PCG64(300 + M + N))
    w = S.draw_weight(rng, N, K, meta, sym)
    x = S.draw_x(rng, M, K)
    _say(f"table kernel M={M} N={N} K={K} {meta} sym={sym}")
    with _env("Q1_PACKED_KERNEL", "table"):
        y = Q.q1_qmm(_x_dev(x), Q.PackedQ1.from_host(w), torch.float32)
    ref, A = O.qmm_ref(x, **_wd(w))
    ok, ratio, nbad = O.check_close(_host(y), "f32", ref, A)
    _say(f"  worst err/bound {ratio:.3e}")
    assert ok, nbad


@pytest.mark.parametrize("meta,sym,N,K", [("f16", True, 70, 5120), ("bf16", False, 45, 17408)])
def test_forced_mma_kernel_one_row(meta, sym, N, K):
    rng = np.random.Generator(np.random.PCG64(400 + N))
    w = S.draw_weight(rng, N, K, meta, sym)
    x = S.draw_x(rng, 1, K)
    _say(f"matrix-core kernel M=1 N={N} K={K} {meta} sym={sym}")
    with _env("Q1_PACKED_KERNEL", "mma"):
        y = Q.q1_qmm(_x_dev(x), Q.PackedQ1.from_host(w), torch.float32)
    ref, A = O.qmm_ref(x, **_wd(w))
    ok, ratio, nbad = O.check_close(_host(y), "f32", ref, A)
    _say(f"  worst err/bound {ratio:.3e}")
    assert ok, nbad


@pytest.mark.parametrize("M", [2, 5])
def test_forced_table_ffn_pair(M):
    """The table kernel's gate/up pair mode with the SiLU*mul epilogue."""
    wl = S.workload(5, small=True)
    g, u, d = (wl.weights[k] for k in ("gate", "up", "down"))
    x = wl.x["x"][:M]
    _say(f"ffn with the table kernel M={M}")
    with _env("Q1_PACKED_KERNEL", "table"):
        y, h = Q.q1_ffn(_x_dev(x), *(Q.PackedQ1.from_host(t) for t in (g, u, d)), return_hidden=True)
    ref = O.ffn_ref(x, _wd(g), _wd(u), _wd(d))
    dh = np.abs(O.bf16_to_f32(_host(h)).astype(np.float64) - ref["h64"])
    assert (dh <= O.ffn_h_bound(ref)).all()
    assert O.check_within(_host(y), "bf16", ref["y"], O.ffn_y_bound(ref, _wd(d)))[0]


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
@pytest.mark.parametrize("meta,sym", [("f16", True), ("bf16", False)])
def test_ffn_pair_split_k(M, meta, sym):
    """Gate/up pairs whose K (H = 9216) does not fit one workgroup's LDS image:
    the pair is split along K and the reduce launch adds the segments and
    applies SiLU * mul (the table kernel's own split reduction at M = 1).  h
    and y checked against the oracle on every element."""
    H, I, Ho = 9216, 640, 384
    rng = np.random.Generator(np.random.PCG64(500 + M))
    g = S.draw_weight(rng, I, H, meta, sym)
    u = S.draw_weight(rng, I, H, meta, sym)
    d = S.draw_weight(rng, Ho, I, meta, sym)
    x = S.draw_x(rng, M, H)
    W = [Q.PackedQ1.from_host(t) for t in (g, u, d)]
    # the partial sums need workspace beyond the counter block and h
    assert Q.q1_ffn_workspace_bytes(M, *W) > 16384 + M * I * 2 + 256
    _say(f"ffn pair split K M={M} H={H} {meta} sym={sym}")
    y, h = Q.q1_ffn(_x_dev(x), *W, return_hidden=True)
    ref = O.ffn_ref(x, _wd(g), _wd(u), _wd(d))
    dh = np.abs(O.bf16_to_f32(_host(h)).astype(np.float64) - ref["h64"])
    hb = O.ffn_h_bound(ref)
    _say(f"  h worst ratio {np.max(dh / hb):.3e}")
    assert (dh <= hb).all()
    y_h, A_h = O.qmm_ref(_host(h), **_wd(d))
    ok, ratio, nbad = O.check_close(_host(y), "bf16", y_h, A_h)
    _say(f"  y (on gpu h) worst ratio {ratio:.3e}")
    assert ok, nbad
    assert O.check_within(_host(y), "bf16", ref["y"], O.ffn_y_bound(ref, _wd(d)))[0]


GRAPH_CASES = [  # (label, M, N, K, meta, symmetric, Q1_PACKED_KERNEL)
    ("mma", 4, 1040, 5120, "f16", True, None),
    ("mma_split", 3, 520, 17408, "bf16", False, None),
    ("mma_one_row_split", 1, 1000, 9216, "f16", True, None),
    ("table_split", 1, 1000, 9216, "f16", True, "table"),
    ("mma_two_rows", 2, 700, 3072, "bf16", True, None),
    ("wide", 40, 600, 2048, "f16", True, None),
]


@pytest.mark.parametrize("case", GRAPH_CASES, ids=lambda c: c[0])
def test_qmm_replays_in_a_graph(case):
    """q1_qmm captured once in a HIP graph (with its reduce or image launch)
    and replayed four times, with eager changes to x and an eager call on a
    second workspace between the replays: every replay equals the eager call
    on the same x bit for bit, and the first is within the oracle's bound."""
    label, M, N, K, meta, sym, kernel = case
    if kernel is None:
        _qmm_graph_case(label, M, N, K, meta, sym)
    else:
        with _env("Q1_PACKED_KERNEL", kernel):
            _qmm_graph_case(label, M, N, K, meta, sym)


def _qmm_graph_case(label, M, N, K, meta, sym):
    rng = np.random.Generator(np.random.PCG64(600 + M))
    w = S.draw_weight(rng, N, K, meta, sym)
    W = Q.PackedQ1.from_host(w)
    xd = _x_dev(S.draw_x(rng, M, K))
    need = Q.q1_qmm_workspace_bytes(M, W)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    y = torch.empty(M, N, dtype=torch.float32, device="cuda")
    _say(f"graph replay {label}: M={M} N={N} K={K} {meta} sym={sym} workspace {need}")
    Q.q1_qmm(xd, W, torch.float32, y=y, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Q.q1_qmm(xd, W, torch.float32, y=y, workspace=ws)
    for step in range(4):
        if step > 0:
            xd.copy_(_x_dev(S.draw_x(rng, M, K)))
        graph.replay()
        torch.cuda.synchronize()
        y_eager = Q.q1_qmm(xd, W, torch.float32, workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_eager.view(torch.int32)), step
        if step == 0:
            ref, A = O.qmm_ref(_host(xd), **_wd(w))
            ok, ratio, nbad = O.check_close(_host(y), "f32", ref, A)
            _say(f"  worst err/bound {ratio:.3e}")
            assert ok, nbad


@pytest.mark.parametrize("M", [1, 4])
def test_ffn_replays_in_a_graph(M):
    """The two-launch q1_ffn (gate/up pair, then a down projection split
    along K = 9216 with its reduce launch) captured in a HIP graph and
    replayed four times with eager changes to x between replays: every replay
    equals an eager call bit for bit."""
    H, I, Ho = 1024, 9216, 500
    rng = np.random.Generator(np.random.PCG64(700 + M))
    W = [Q.PackedQ1.from_host(S.draw_weight(rng, n, k, "f16", True)) for n, k in ((I, H), (I, H), (Ho, I))]
    xd = _x_dev(S.draw_x(rng, M, H))
    need = Q.q1_ffn_workspace_bytes(M, *W)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y = torch.empty(M, Ho, dtype=torch.bfloat16, device="cuda")
    _say(f"ffn graph replay M={M}")
    Q.q1_ffn(xd, *W, y=y, workspace=ws)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Q.q1_ffn(xd, *W, y=y, workspace=ws)
    for step in range(4):
        if step > 0:
            xd.copy_(_x_dev(S.draw_x(rng, M, H)))
        graph.replay()
        torch.cuda.synchronize()
        y_eager = Q.q1_ffn(xd, *W, workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), step
