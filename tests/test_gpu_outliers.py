"""Matmul tolerance with outlier activations and unequal code weights.

|y - y_ref| <= 1e-3 sum_k |w_nk x_k| + 1e-6 must hold for any bf16
activations, including blocks where one value is 2^12..2^16 times its
neighbours, and for affine groups where one code weighs (exactly) zero, so
that the tolerance does not contain the outlier's term (Higgs PR #212,
"Measured impact": affine tensors keep a stored bias).  Every output is
checked, through the C ABI, for the one-row table kernel (M = 1), the
matrix-core kernel (M = 2, 8) and the wide kernel (M = 40)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import q1_synth as S
from tests.outlier_inputs import outlier_positions, outlier_x, worked_case, zero_weight_codes

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_decode_q1_amd as Q


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _check(w, x, label):
    y = Q.q1_qmm(_x_dev(x), Q.PackedQ1.from_host(w), torch.float32).cpu().numpy()
    ref, A = O.qmm_ref(x, w.packed, w.scales, w.biases, w.meta, w.symmetric, w.K)
    ok, ratio, nbad = O.check_close(y, "f32", ref, A)
    _say(f"  {label}: worst err/bound {ratio:.3e}, violations {nbad}")
    assert ok, f"{label}: {nbad} outputs outside the tolerance (worst ratio {ratio:.3g})"


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.load_library()
    assert Q.q1_device_supported(0), Q.q1_last_error()
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("M", [1, 2, 8, 40])
@pytest.mark.parametrize("clear_small", [False, True])
def test_worked_case_zero_weight_outlier(M, clear_small):
    """Set bits weigh 0 and carry a 1024 outlier per 32 weights; the result
    is the clear bits' sum times -0.25 (K = 1024: 32 blocks)."""
    w, x1 = worked_case(1024, 48, clear_small)
    x = np.repeat(x1, M, axis=0)
    _say(f"worked case M={M} clear_small={clear_small}")
    _check(w, x, f"worked M={M}")


@pytest.mark.parametrize("M", [1, 2, 8, 40])
@pytest.mark.parametrize("ratio", [12, 14, 16])
@pytest.mark.parametrize("sym", [False, True])
def test_outlier_blocks(M, ratio, sym):
    """Affine: every outlier sits on the code that weighs 0 in its group, so
    the tolerance holds only the small terms; symmetric: all codes weigh
    s/2."""
    rng = np.random.Generator(np.random.PCG64(900 + 7 * M + ratio + 100 * sym))
    N, K = 96, 2048
    pos = outlier_positions(rng, K)
    w = S.draw_weight(rng, N, K, "f16", True) if sym else zero_weight_codes(rng, N, K, "bf16", pos)
    x = outlier_x(rng, M, K, ratio, pos)
    _say(f"outliers 2^{ratio} M={M} {'sym' if sym else 'affine, outliers on zero-weight codes'}")
    _check(w, x, f"2^{ratio} M={M} sym={sym}")


@pytest.mark.parametrize("M", [1, 3, 6])
def test_outliers_affine_f16_long_rows(M):
    """K = 17408 (split K in the matrix-core kernel, several segments)."""
    rng = np.random.Generator(np.random.PCG64(77 + M))
    pos = outlier_positions(rng, 17408)
    w = zero_weight_codes(rng, 40, 17408, "f16", pos)
    x = outlier_x(rng, M, 17408, 14, pos)
    _say(f"outliers affine f16 K=17408 M={M}")
    _check(w, x, f"K=17408 M={M}")
