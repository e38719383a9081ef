"""GPU parity at the size limits of the boundary: the largest packed matrix the
narrow-M kernels accept (packed words just under 2 GiB, the reach of their
32-bit buffer offsets), a matrix one row over it (rejected before any launch),
and a gather whose output exceeds 2^31 pieces of 8 values (split into several
launches).  Checked on sampled rows against the CPU oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import q1_synth as S

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_decode_q1_amd as Q

K = 5120
ROW_BYTES = K // 8
N_MAX = (2 ** 31 - 1) // ROW_BYTES  # largest N with N * K / 8 < 2^31


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def x_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.load_library()
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_qmm_largest_packed_matrix():
    """N * K / 8 = 2^31 - 128 bytes of packed words: the one-row table kernel
    and the matrix-core kernel (M = 4) on rows sampled up to the last one."""
    _say(f"largest packed matrix N={N_MAX} K={K}")
    rng = np.random.Generator(np.random.PCG64(4242))
    w = S.draw_weight(rng, N_MAX, K, "f16", True)
    x = S.draw_x(rng, 4, K)
    W = Q.PackedQ1.from_host(w)
    rows = np.unique(np.concatenate([[0, 1, N_MAX // 2, N_MAX - 2, N_MAX - 1],
                                     rng.integers(0, N_MAX, 60)]))
    for M in (1, 4):
        y = Q.q1_qmm(x_dev(x[:M]), W, torch.float32)
        got = y[:, torch.from_numpy(rows).cuda()].cpu().numpy()
        ref, A = O.qmm_ref(x[:M], w.packed, w.scales, None, "f16", True, K, row_index=rows)
        ok, ratio, nbad = O.check_close(got, "f32", ref, A)
        _say(f"  M={M}: worst err/bound {ratio:.3e}")
        assert ok, (M, ratio, nbad)
        del y
    del W, w


def test_qmm_one_row_over_the_limit_is_rejected():
    """One more row reaches 2^31 bytes of packed words: the call fails with
    Q1_ERR_UNSUPPORTED before any launch (all memory is allocated, so nothing
    could be read out of bounds even if it did not)."""
    N = N_MAX + 1
    _say(f"over the limit N={N}")
    packed = torch.zeros(N, K // 32, dtype=torch.int32, device="cuda")
    scales = torch.zeros(N, K // 128, dtype=torch.float16, device="cuda")
    W = Q.PackedQ1(packed, scales, None, N, K)
    x = torch.zeros(1, K, dtype=torch.bfloat16, device="cuda")
    for M in (1, 4):
        with pytest.raises(Q.Q1Error) as e:
            Q.q1_qmm(x.expand(M, K).contiguous(), W, torch.float32)
        assert e.value.status == -2, str(e.value)
        assert "too large" in str(e.value)
    del packed, scales, W
    torch.cuda.empty_cache()


def test_gather_beyond_2g_pieces_is_chunked():
    """T * K / 8 > 2^31: the gather runs as several launches; rows on both
    sides of the launch boundary and at the end match the oracle bit for bit."""
    rows_per_launch = (2 ** 31) // ROW_BYTES
    T = rows_per_launch + 4096
    _say(f"gather T={T} rows of K={K} ({T * K * 2 / 2 ** 30:.1f} GiB of bf16)")
    rng = np.random.Generator(np.random.PCG64(4343))
    w = S.draw_weight(rng, 1024, K, "bf16", False)
    ids = rng.integers(0, 1024, size=T).astype(np.int32)
    ids[-3:] = [-1, 1024, 7]  # out-of-range ids give zero rows
    W = Q.PackedQ1.from_host(w)
    out = Q.q1_embed_rows(torch.from_numpy(ids).cuda(), W, torch.bfloat16)
    sample = np.array([0, 1, rows_per_launch - 2, rows_per_launch - 1, rows_per_launch, rows_per_launch + 1,
                       T // 2, T - 4, T - 3, T - 2, T - 1])
    got = out[torch.from_numpy(sample).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
    ref = O.embed_rows(ids[sample], w.packed, w.scales, w.biases, "bf16", False, K, "bf16")
    assert np.array_equal(got, ref)
    del out
    torch.cuda.empty_cache()
