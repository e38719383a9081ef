"""GPU parity of the metadata calls (through the C ABI) against the CPU oracle:
q1_pack_signs (packed words, scales and the inexact-group count, all bit for
bit) and q1_check_symmetric (the mismatch count, exactly)."""
import sys

import numpy as np
import pytest
import torch

import oracle as O
import q1_synth as S

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import gemm_decode_q1_amd as Q

TORCH_DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev16(bits, dt):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(TORCH_DT[dt]).cuda()


def host16(t):
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def host32(t):
    return t.detach().cpu().numpy().view(np.uint32)


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    Q.load_library()
    assert Q.q1_device_supported(0), Q.q1_last_error()
    yield
    torch.cuda.synchronize()


def mixed_dense(rng, N, K, dense, meta):
    """Dense weights with a mix of exact and inexact groups: most groups are
    +-v (exact), some have one weight perturbed, one is all zeros, one holds a
    -0.0, one a NaN."""
    w = S.draw_weight(rng, N, K, meta, True)
    sc = O.round_to(np.maximum(O.meta_to_f32(w.scales, meta), np.float32(2.0 ** -10)), meta)
    d = O.dequantize(w.packed, sc, None, meta, True, K, dense).copy()
    G = K // 128
    for n in range(N):
        if n % 3 == 1:
            d[n, (n % G) * 128 + (n * 7) % 128] ^= np.uint16(1)
    d[0, 0:128] = 0
    if G > 1:
        d[0, 128:256] = 0
        d[0, 200] = 0x8000
    if N > 2:
        d[2, 5] = 0x7FC0 if dense == "bf16" else 0x7E00
    return d


@pytest.mark.parametrize("dense,meta", [("bf16", "bf16"), ("bf16", "f16"), ("f16", "f16"), ("f16", "bf16")])
@pytest.mark.parametrize("N,K", [(1, 128), (5, 1024), (37, 2176), (130, 5120)])
def test_pack_matches_oracle(dense, meta, N, K):
    _say(f"pack dense={dense} meta={meta} N={N} K={K}")
    rng = np.random.Generator(np.random.PCG64(100 + N + K))
    d = mixed_dense(rng, N, K, dense, meta)
    p_ref, s_ref, bad_ref = O.pack_signs(d, dense, meta)
    W, bad = Q.q1_pack_signs(dev16(d, dense), TORCH_DT[meta])
    assert np.array_equal(host32(W.packed), p_ref)
    assert np.array_equal(host16(W.scales), s_ref)
    assert int(bad.item()) == bad_ref
    _say(f"  inexact groups {bad_ref} of {N * K // 128}")


def test_pack_round_trip_full_size():
    """FFN up/gate shape (K=5120, N=17408): a symmetric bf16-metadata tensor
    dequantised on the GPU packs back to the same words and scales, with no
    inexact group, and dequantises again to the same bytes."""
    _say("pack round trip K=5120 N=17408")
    w = S.workload(2).weights["w"]
    sc = O.round_to(np.maximum(O.meta_to_f32(w.scales, "f16"), np.float32(2.0 ** -10)), "bf16")
    W0 = Q.PackedQ1(torch.from_numpy(w.packed.view(np.int32)).cuda(), dev16(sc, "bf16"), None, w.N, w.K)
    dense = Q.q1_dequantize(W0, torch.bfloat16)
    W1, bad = Q.q1_pack_signs(dense, torch.bfloat16)
    assert int(bad.item()) == 0
    assert torch.equal(W1.packed, W0.packed) and torch.equal(W1.scales.view(torch.int16), W0.scales.view(torch.int16))
    again = Q.q1_dequantize(W1, torch.bfloat16)
    assert torch.equal(again.view(torch.int16), dense.view(torch.int16))
    # sampled rows against the oracle's dequantisation
    rows = np.array([0, 1, 4095, 9000, 17407])
    ref = O.dequantize(w.packed[rows], sc[rows], None, "bf16", True, w.K, "bf16")
    assert np.array_equal(host16(dense)[rows], ref)


@pytest.mark.parametrize("meta", ["bf16", "f16"])
@pytest.mark.parametrize("N,K", [(1, 128), (33, 1024), (517, 17408)])
def test_symmetric_check_matches_oracle(meta, N, K):
    _say(f"symmetric check meta={meta} N={N} K={K}")
    rng = np.random.Generator(np.random.PCG64(200 + N))
    w = S.draw_weight(rng, N, K, meta, True)
    half = O.round_to((np.float32(-0.5) * O.meta_to_f32(w.scales, meta)).astype(np.float32), meta)
    for variant in ("derived", "perturbed", "random"):
        if variant == "derived":
            b = half.copy()
        elif variant == "perturbed":
            b = half.copy()
            b.reshape(-1)[::7] ^= np.uint16(1)
            b.reshape(-1)[::11] = 0x7FC0 if meta == "bf16" else 0x7E00
        else:
            b = S.draw_weight(rng, N, K, meta, False).biases
        ref = O.symmetric_mismatches(w.scales, b, meta)
        Wd = Q.PackedQ1(torch.from_numpy(w.packed.view(np.int32)).cuda(), dev16(w.scales, meta), dev16(b, meta), N, K)
        got = int(Q.q1_check_symmetric(Wd).item())
        _say(f"  {variant}: {got} of {N * K // 128} groups (oracle {ref})")
        assert got == ref


def test_symmetric_check_edge_groups():
    # zero scales with either zero bias match; a subnormal scale whose half is
    # not an fp16 value, an infinite scale and a NaN bias do not
    scales = np.array([[0x0000, 0x0000, 0x0001, 0x7C00, 0x3800, 0x3800]], dtype=np.uint16)
    biases = np.array([[0x0000, 0x8000, 0x8000, 0xFC00, 0x7E00, 0xB400]], dtype=np.uint16)
    packed = np.zeros((1, 768 // 32), dtype=np.uint32)
    W = Q.PackedQ1(torch.from_numpy(packed.view(np.int32)).cuda(), dev16(scales, "f16"), dev16(biases, "f16"), 1, 768)
    assert O.symmetric_mismatches(scales, biases, "f16") == 3  # the last group (0.5, -0.25) matches
    assert int(Q.q1_check_symmetric(W).item()) == O.symmetric_mismatches(scales, biases, "f16")


def test_compacted_tensor_gives_the_same_weights():
    """A tensor whose check returns 0 dequantises to the same bytes with the
    biases dropped, and its products stay within the tolerance of the same
    oracle value either way (down-projection shape, K=17408)."""
    w = S.workload(3, small=True).weights["w"]
    half = O.round_to((np.float32(-0.5) * O.meta_to_f32(w.scales, "bf16")).astype(np.float32), "bf16")
    P = torch.from_numpy(w.packed.view(np.int32)).cuda()
    Wa = Q.PackedQ1(P, dev16(w.scales, "bf16"), dev16(half, "bf16"), w.N, w.K)
    assert int(Q.q1_check_symmetric(Wa).item()) == 0
    Ws = Q.PackedQ1(P, dev16(w.scales, "bf16"), None, w.N, w.K)
    assert torch.equal(Q.q1_dequantize(Wa, torch.float32), Q.q1_dequantize(Ws, torch.float32))
    x = S.workload(3, small=True).x["x"][:3]
    xd = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    y_ref, A = O.qmm_ref(x, w.packed, w.scales, None, "bf16", True, w.K)
    for W in (Wa, Ws):
        y = Q.q1_qmm(xd, W, torch.float32).cpu().numpy()
        ok, ratio, nbad = O.check_close(y, "f32", y_ref, A)
        assert ok, (ratio, nbad)


def test_errors_are_reported():
    w = S.workload(1).weights["w"]
    Ws = Q.PackedQ1.from_host(w)
    with pytest.raises(ValueError):
        Q.q1_check_symmetric(Ws)  # already symmetric
    bad = torch.zeros(4, 100, dtype=torch.bfloat16, device="cuda")  # K not a multiple of 128
    with pytest.raises(Q.Q1Error):
        Q.q1_pack_signs(bad)
    assert "multiple of 128" in Q.q1_last_error()


def test_meta_calls_replay_in_a_graph():
    """Both calls captured once in a HIP graph and replayed several times, with
    eager changes to their inputs between replays: every replay clears its
    counter and counts afresh (the counters are cleared by a kernel, not a
    memset node)."""
    rng = np.random.Generator(np.random.PCG64(300))
    N, K = 64, 1024
    w = S.draw_weight(rng, N, K, "bf16", True)
    half = O.round_to((np.float32(-0.5) * O.meta_to_f32(w.scales, "bf16")).astype(np.float32), "bf16")
    P = torch.from_numpy(w.packed.view(np.int32)).cuda()
    sc, bi = dev16(w.scales, "bf16"), dev16(half, "bf16")
    W = Q.PackedQ1(P, sc, bi, N, K)
    dense = Q.q1_dequantize(Q.PackedQ1(P, sc, None, N, K), torch.bfloat16)
    count = torch.empty(1, dtype=torch.int32, device="cuda")
    Q.q1_check_symmetric(W, count)
    Wp, bad = Q.q1_pack_signs(dense, torch.bfloat16)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        Q.q1_check_symmetric(W, count)
        Wp, bad = Q.q1_pack_signs(dense, torch.bfloat16)
    bias_bits, dense_bits = bi.view(torch.int16), dense.view(torch.int16)
    for step in range(4):
        if step > 0:  # eager changes between replays: one more bad bias, one more inexact group
            bias_bits[step, 0] ^= 1
            dense_bits[step, 3] ^= 1
        g.replay()
        torch.cuda.synchronize()
        exp_check = O.symmetric_mismatches(w.scales, host16(bi), "bf16")
        _, _, exp_bad = O.pack_signs(host16(dense), "bf16", "bf16")
        assert exp_check == step and exp_bad == step
        assert int(count.item()) == exp_check and int(bad.item()) == exp_bad


def test_stream_read_reads_its_input():
    """The read-ceiling aid really reads the data: one 16-byte vector whose
    words XOR to the sentinel makes the kernel store it; any other data leaves
    the sink alone.  Bad sizes and alignment are rejected."""
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    data = torch.tensor([0x9E3779B9 - (1 << 32), 0, 0, 0], dtype=torch.int64).to(torch.int32).cuda()
    Q.q1_stream_read(torch.tensor([1, 0, 0, 0], dtype=torch.int32, device="cuda"), sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0
    Q.q1_stream_read(data, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) & 0xFFFFFFFF == 0x9E3779B9
    with pytest.raises(Q.Q1Error):
        Q.q1_stream_read(torch.zeros(3, dtype=torch.int32, device="cuda"), sink)  # 12 bytes
    with pytest.raises(Q.Q1Error):
        Q.q1_stream_read(torch.zeros(8, dtype=torch.int32, device="cuda")[1:5], sink)  # misaligned
