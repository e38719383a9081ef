"""GPU parity of the single-launch packed FFN (gate/up, SiLU*mul and down in
one persistent launch; Higgs PR #212, "What": fused dense-FFN operations),
through the C ABI.

Every output is checked against the oracle: h (bf16) within ffn_h_bound, y
within the standard matmul tolerance on the GPU's own h and within
ffn_y_bound end to end.  Q1_FFN_KERNEL=single selects the launch for the
whole module.  The shapes take the single launch (hidden and
intermediate sizes multiples of 1024, the three matrices of one kind) and
cover one and several K segments of the down projection (I = 2048 .. 17408),
ragged output widths, both metadata dtypes and affine tensors.  The launch
must leave the workspace's counter block zero (status word included), stay
correct when calls of different M reuse one workspace, and replay from a HIP
graph with the same bits as the eager call."""
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

RESERVED = 16384


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
    with _env("Q1_FFN_KERNEL", "single"):
        yield
        torch.cuda.synchronize()


def _weights(seed, H, I, Ho, meta, sym):
    rng = np.random.Generator(np.random.PCG64(seed))
    g = S.draw_weight(rng, I, H, meta, sym)
    u = S.draw_weight(rng, I, H, meta, sym)
    d = S.draw_weight(rng, Ho, I, meta, sym)
    x = S.draw_x(rng, 8, H)
    return g, u, d, x


def _check(g, u, d, x, y, h, label):
    ref = O.ffn_ref(x, _wd(g), _wd(u), _wd(d))
    hg = _host(h)
    dh = np.abs(O.bf16_to_f32(hg).astype(np.float64) - ref["h64"])
    hb = O.ffn_h_bound(ref)
    _say(f"  {label} h: worst ratio {np.max(dh / hb):.3e}")
    assert (dh <= hb).all()
    y_h, A_h = O.qmm_ref(hg, **_wd(d))
    ok, ratio, nbad = O.check_close(_host(y), "bf16", y_h, A_h)
    _say(f"  {label} y (on gpu h): worst ratio {ratio:.3e}")
    assert ok, nbad
    assert O.check_within(_host(y), "bf16", ref["y"], O.ffn_y_bound(ref, _wd(d)))[0]


def _counters_clear(ws):
    torch.cuda.synchronize()
    block = ws[:RESERVED].cpu().numpy()
    assert not block.any(), np.nonzero(block)[0][:16]


CASES = [  # (seed, H, I, Ho, meta, symmetric)
    (11, 1024, 2048, 640, "f16", True),
    (12, 2048, 3072, 1000, "bf16", True),
    (13, 1024, 2048, 513, "bf16", False),
    (14, 1024, 17408, 320, "f16", True),
    (15, 3072, 5120, 17, "f16", False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"H{c[1]}_I{c[2]}_Ho{c[3]}_{c[4]}_{'sym' if c[5] else 'aff'}")
@pytest.mark.parametrize("M", [1, 2, 3, 4, 5, 6, 7, 8])
def test_single_launch_ffn(case, M):
    seed, H, I, Ho, meta, sym = case
    g, u, d, x = _weights(seed, H, I, Ho, meta, sym)
    x = x[:M]
    _say(f"single-launch ffn M={M} H={H} I={I} Ho={Ho} {meta} sym={sym}")
    W = [Q.PackedQ1.from_host(t) for t in (g, u, d)]
    need = Q.q1_ffn_workspace_bytes(M, *W)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    y, h = Q.q1_ffn(_x_dev(x), *W, workspace=ws, return_hidden=True)
    _counters_clear(ws)
    _check(g, u, d, x, y, h, "single")


def test_single_launch_reuses_its_workspace():
    """Calls of M = 8, 3, 8, 1 in a row on one workspace (the counters each
    call leaves behind are the next call's start), no synchronisation in
    between; every result checked."""
    g, u, d, x = _weights(21, 1024, 17408, 320, "f16", True)
    W = [Q.PackedQ1.from_host(t) for t in (g, u, d)]
    need = max(Q.q1_ffn_workspace_bytes(M, *W) for M in (1, 3, 8))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    outs = []
    for M in (8, 3, 8, 1):
        xm = x[:M] if M != 3 else x[5:8]
        outs.append((xm,) + Q.q1_ffn(_x_dev(xm), *W, workspace=ws, return_hidden=True))
    _counters_clear(ws)
    for i, (xm, y, h) in enumerate(outs):
        _check(g, u, d, xm, y, h, f"call {i} M={xm.shape[0]}")


def test_single_launch_matches_split_path():
    """The single launch and the two-launch form (Q1_FFN_KERNEL=split, the
    default) on the
    same inputs: both within the oracle's bounds; h agrees to the bf16
    rounding of nearly equal fp32 sums (at most one ulp)."""
    g, u, d, x = _weights(31, 2048, 3072, 1000, "f16", True)
    W = [Q.PackedQ1.from_host(t) for t in (g, u, d)]
    y1, h1 = Q.q1_ffn(_x_dev(x[:4]), *W, return_hidden=True)
    with _env("Q1_FFN_KERNEL", "split"):
        y2, h2 = Q.q1_ffn(_x_dev(x[:4]), *W, return_hidden=True)
    _check(g, u, d, x[:4], y1, h1, "single")
    _check(g, u, d, x[:4], y2, h2, "split")
    a = _host(h1).astype(np.int32)
    b = _host(h2).astype(np.int32)
    assert np.max(np.abs(a - b)) <= 1


def test_single_launch_replays_in_a_graph():
    """One call captured in a HIP graph and replayed four times, with eager
    changes to x between replays: every replay equals, bit for bit, an eager
    call on the same x (the launch's sums run in a fixed order), and the
    counter block is zero after each."""
    g, u, d, x = _weights(41, 1024, 17408, 320, "bf16", True)
    W = [Q.PackedQ1.from_host(t) for t in (g, u, d)]
    M = 4
    need = Q.q1_ffn_workspace_bytes(M, *W)
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    ws_eager = torch.zeros(need, dtype=torch.uint8, device="cuda")
    xd = _x_dev(x[:M])
    y = torch.empty(M, 320, dtype=torch.bfloat16, device="cuda")
    Q.q1_ffn(xd, *W, y=y, workspace=ws)  # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        Q.q1_ffn(xd, *W, y=y, workspace=ws)
    rng = np.random.Generator(np.random.PCG64(42))
    for step in range(4):
        if step > 0:
            xd.copy_(_x_dev(S.draw_x(rng, M, 1024)))
        graph.replay()
        torch.cuda.synchronize()
        y_eager = Q.q1_ffn(xd, *W, workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_eager.view(torch.int16)), step
        _counters_clear(ws)
    _check(g, u, d, _host(xd), y, ws[RESERVED:RESERVED + M * 17408 * 2].view(torch.bfloat16).view(M, 17408), "graph")
