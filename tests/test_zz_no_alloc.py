"""q1_qmm_noalloc (the entry point for callers that cannot allocate) against
q1_qmm, through the C ABI: identical bytes on two calls in a row, the second
with a smaller input, for shapes whose kernels use scratch (split-K partial
sums and arrival counters; the wide path's activation image), and within the
oracle's tolerance."""
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


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.load_library()
    assert Q.q1_device_supported(0), Q.q1_last_error()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("N,K,meta,sym,Ms", [
    (5120, 17408, "bf16", False, (8, 3)),   # packed, split K: partial sums + counters
    (1000, 9216, "f16", True, (5, 2)),      # packed, split K
    (300, 1024, "f16", True, (40, 17)),     # wide: activation image
    (200, 1152, "bf16", False, (24, 9)),    # wide, affine
])
def test_noalloc_matches_qmm(N, K, meta, sym, Ms):
    rng = np.random.Generator(np.random.PCG64(N + K + Ms[0]))
    w = S.draw_weight(rng, N, K, meta, sym)
    W = Q.PackedQ1.from_host(w)
    assert Q.q1_qmm_workspace_bytes(Ms[0], W) > 0  # the kernels of this shape use scratch
    for M in Ms:
        x = S.draw_x(rng, M, K)
        _say(f"noalloc N={N} K={K} {meta} sym={sym} M={M}")
        xd = _x_dev(x)
        y_ref = Q.q1_qmm(xd, W, torch.float32)
        y = Q.q1_qmm_noalloc(xd, W, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int32), y_ref.view(torch.int32)), f"M={M}: differs from q1_qmm"
        ref, A = O.qmm_ref(x, w.packed, w.scales, w.biases, meta, sym, K)
        ok, ratio, nbad = O.check_close(y.cpu().numpy(), "f32", ref, A)
        _say(f"  identical to q1_qmm; worst err/bound {ratio:.3e}")
        assert ok, nbad


def test_noalloc_rejects_oversize():
    rng = np.random.Generator(np.random.PCG64(9))
    w = S.draw_weight(rng, 64, 17408, "f16", True)
    W = Q.PackedQ1.from_host(w)
    x = _x_dev(S.draw_x(rng, 512, 17408))
    with pytest.raises(Q.Q1Error) as e:
        Q.q1_qmm_noalloc(x, W, torch.float32)
    assert e.value.status == -3 and "static scratch" in str(e.value)
