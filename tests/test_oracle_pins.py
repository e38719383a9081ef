"""Pins for the CPU oracle: each check ties an oracle function to something
other than itself -- hand-worked fixtures from the format description, library
routines, closed forms, exact rational arithmetic, or invariants the format
implies.  A final group plants plausible mistakes in the oracle and checks
that at least one pin catches each."""
import math
import struct
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

import oracle as O
import q1_synth as S
from tests.golden.fixtures import load_cases

CASES = load_cases()


def _w(case):
    return dict(packed=case["packed"], scales=case["scales"], biases=case["biases"], meta=case["meta"],
                symmetric=case["biases"] is None, K=case["K"])


# ---------------------------------------------------------------- scalar formats

def _special_f32():
    vals = [0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38, 1e-40, -1e-40, 1.17549435e-38, 65504.0, 1 / 3,
            float("inf"), float("-inf")]
    base = np.array(vals, dtype=np.float32)
    # exact ties: low 16 bits == 0x8000, with both parities of bit 16
    rng = np.random.default_rng(1)
    hi = rng.integers(0, 0x7F7F, size=2000, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).astype(np.uint32).view(np.float32)
    near = ((hi << 16) | rng.choice([0x7FFF, 0x8001, 0x0001, 0xFFFF], size=2000)).astype(np.uint32).view(np.float32)
    neg = -ties
    randf = rng.standard_normal(20000).astype(np.float32) * np.float32(10.0) ** rng.integers(-30, 30, 20000)
    return np.concatenate([base, ties, near, neg, randf.astype(np.float32)])


def test_bf16_rne_matches_torch():
    v = _special_f32()
    mine = O.f32_to_bf16_rne(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)


def test_bf16_ties_go_to_even_by_hand():
    # 1 + 2^-8 lies exactly between bf16 1.0 (0x3F80) and 1.0078125 (0x3F81): even -> 0x3F80
    # 1 + 3*2^-8 lies between 0x3F81 and 0x3F82: even -> 0x3F82
    v = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8)], dtype=np.float32)
    assert list(O.f32_to_bf16_rne(v)) == [0x3F80, 0x3F82, 0xBF80]


def test_bf16_decode_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = O.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float32).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].view(np.uint32), ref[~nan].view(np.uint32))


def test_f16_decode_all_patterns():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    mine = O.f16_to_f32(bits)
    ref = np.array([struct.unpack("<e", int(b).to_bytes(2, "little"))[0] for b in bits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert np.array_equal(mine[~nan].astype(np.float64), ref[~nan])


def test_f16_rne_by_hand():
    # 1 + 2^-11 is a tie between 1.0 (0x3C00) and 1+2^-10 (0x3C01): even -> 0x3C00
    v = np.array([1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, 65520.0], dtype=np.float32)
    assert list(O.f32_to_f16_rne(v)) == [0x3C00, 0x3C02, 0x7C00]


# ---------------------------------------------------------------- unpacking

def test_unpack_one_hot():
    rng = np.random.default_rng(2)
    K = 384
    for _ in range(50):
        k = int(rng.integers(0, K))
        packed = np.zeros((1, K // 32), dtype=np.uint32)
        packed[0, k // 32] = np.uint32(1) << np.uint32(k % 32)
        bits = O.unpack_bits(packed, K)
        assert bits.sum() == 1 and bits[0, k] == 1


def test_unpack_matches_numpy_unpackbits_little():
    rng = np.random.default_rng(3)
    packed = rng.integers(0, 1 << 32, size=(7, 40), dtype=np.uint64).astype(np.uint32)
    ref = np.unpackbits(packed.view(np.uint8), axis=1, bitorder="little")
    assert np.array_equal(O.unpack_bits(packed, 40 * 32), ref)


# ---------------------------------------------------------------- hand-worked fixtures

@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_dequant(case):
    w = O.dequant_f32(**_w(case))
    assert w.shape == (1, case["K"])
    assert np.array_equal(w[0].astype(np.float64), case["dequant"])


@pytest.mark.parametrize("case", [c for c in CASES if "y" in c], ids=[c["name"] for c in CASES if "y" in c])
def test_golden_gemv(case):
    x_bits = O.f32_to_bf16_rne(case["x"].astype(np.float32))[None, :]
    assert np.array_equal(O.bf16_to_f32(x_bits)[0].astype(np.float64), case["x"])  # x exact in bf16
    y, A = O.qmm_ref(x_bits, **_w(case))
    assert y.shape == (1, 1)
    assert y[0, 0] == case["y"]
    assert A[0, 0] == np.sum(np.abs(case["dequant"] * case["x"]))


# ---------------------------------------------------------------- invariants of the format

def test_symmetric_groups_hold_exactly_two_values():
    wl = S.workload(1)
    w = wl.weights["w"]
    deq = O.dequant_f32(w.packed, w.scales, None, w.meta, True, w.K)
    bits = O.unpack_bits(w.packed, w.K)
    s = O.f16_to_f32(w.scales).astype(np.float64)
    for n in range(0, w.N, 97):
        for g in range(w.K // 128):
            half = Fraction(float(s[n, g])) / 2
            vals = deq[n, 128 * g:128 * g + 128]
            b = bits[n, 128 * g:128 * g + 128]
            assert all(Fraction(float(v)) == (half if bb else -half) for v, bb in zip(vals, b))


def test_symmetric_equals_explicit_bias_when_representable():
    # Scales drawn as 2 * (an fp16 value) so that -scale/2 is itself an fp16
    # value; the explicit-bias tensor must then dequantise bit-identically.
    rng = np.random.Generator(np.random.PCG64(77))
    N, K = 64, 512
    half = np.abs(rng.normal(0, 0.01, size=(N, K // 128))).astype(np.float16)
    scales = (half.astype(np.float32) * 2).astype(np.float16)
    assert np.array_equal(scales.astype(np.float32), half.astype(np.float32) * 2)
    biases = (-half).view(np.uint16)
    packed = rng.integers(0, 1 << 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    a = O.dequant_f32(packed, scales.view(np.uint16), None, "f16", True, K)
    b = O.dequant_f32(packed, scales.view(np.uint16), biases, "f16", False, K)
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


def test_symmetric_equals_explicit_bias_on_random_groups():
    # On the config-1 tensor: wherever fp16(-scale/2) is exact, the derived and
    # the explicit bias agree bit for bit.
    wl = S.workload(1)
    w = wl.weights["w"]
    s = O.f16_to_f32(w.scales)
    b16 = (np.float32(-0.5) * s).astype(np.float16)
    exact = b16.astype(np.float32) == np.float32(-0.5) * s
    assert exact.mean() > 0.99
    a = O.dequant_f32(w.packed, w.scales, None, "f16", True, w.K)
    b = O.dequant_f32(w.packed, w.scales, b16.view(np.uint16), "f16", False, w.K)
    g = np.arange(w.K) // 128
    mask = exact[:, g]
    assert np.array_equal(a[mask].view(np.uint32), b[mask].view(np.uint32))


def test_zero_scale_gives_positive_zero():
    packed = np.array([[0xFFFF0000, 0, 0, 0]], dtype=np.uint32)
    w = O.dequant_f32(packed, np.array([[0x0000]], np.uint16), None, "f16", True, 128)
    assert np.all(w.view(np.uint32) == 0)  # both codes give +0.0 (not -0.0)


# ---------------------------------------------------------------- closed forms and brute force

def _closed_form_ones(packed, scales, biases, meta, K):
    s = O.meta_to_f32(scales, meta)
    bits = O.unpack_bits(packed, K)
    N, G = s.shape
    out = []
    for n in range(N):
        tot = Fraction(0)
        for g in range(G):
            pc = int(bits[n, 128 * g:128 * g + 128].sum())
            if biases is None:
                tot += Fraction(float(s[n, g])) / 2 * (2 * pc - 128)
            else:
                b = float(O.meta_to_f32(biases[n:n + 1, g:g + 1], meta)[0, 0])
                w1 = float(np.float32(np.float32(s[n, g]) + np.float32(b)))   # fl32(s + b)
                tot += pc * Fraction(w1) + (128 - pc) * Fraction(b)
        out.append(tot)
    return out


@pytest.mark.parametrize("symmetric,meta", [(True, "f16"), (False, "bf16"), (False, "f16")])
def test_closed_form_constant_x(symmetric, meta):
    rng = np.random.Generator(np.random.PCG64(5))
    w = S.draw_weight(rng, 23, 1024, meta, symmetric)
    x = O.f32_to_bf16_rne(np.ones((1, 1024), np.float32))
    y, _ = O.qmm_ref(x, w.packed, w.scales, w.biases, meta, symmetric, 1024)
    cf = _closed_form_ones(w.packed, w.scales, w.biases, meta, 1024)
    for n in range(23):
        assert abs(Fraction(float(y[0, n])) - cf[n]) <= abs(cf[n]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 80)


@pytest.mark.parametrize("symmetric,meta,K,N,M", [(True, "f16", 128, 3, 2), (False, "bf16", 256, 4, 3),
                                                  (True, "bf16", 256, 2, 1), (False, "f16", 128, 4, 2)])
def test_bruteforce_exact_rational(symmetric, meta, K, N, M):
    rng = np.random.Generator(np.random.PCG64(K + N + M))
    w = S.draw_weight(rng, N, K, meta, symmetric)
    x = S.draw_x(rng, M, K)
    y, A = O.qmm_ref(x, w.packed, w.scales, w.biases, meta, symmetric, K)
    ex = O.qmm_exact(x, w.packed, w.scales, w.biases, meta, symmetric, K)
    assert y.shape == (M, N)
    for m in range(M):
        for n in range(N):
            err = abs(Fraction(float(y[m, n])) - ex[m][n])
            assert err <= Fraction(float(A[m, n])) * Fraction(1, 2 ** 45)


def test_leading_dims_flatten():
    rng = np.random.Generator(np.random.PCG64(9))
    w = S.draw_weight(rng, 50, 1024, "bf16", False)
    x = S.draw_x(rng, 8, 1024)
    y8, A8 = O.qmm_ref(x, w.packed, w.scales, w.biases, "bf16", False, 1024)
    y24, A24 = O.qmm_ref(x.reshape(2, 4, 1024), w.packed, w.scales, w.biases, "bf16", False, 1024)
    assert y24.shape == (2, 4, 50)
    assert np.array_equal(y24.reshape(8, 50), y8) and np.array_equal(A24.reshape(8, 50), A8)


def test_row_index_sampling_matches_full():
    rng = np.random.Generator(np.random.PCG64(10))
    w = S.draw_weight(rng, 300, 512, "f16", True)
    x = S.draw_x(rng, 2, 512)
    yf, Af = O.qmm_ref(x, w.packed, w.scales, None, "f16", True, 512, block_rows=64)
    idx = np.array([0, 5, 299, 128, 64])
    ys, As = O.qmm_ref(x, w.packed, w.scales, None, "f16", True, 512, row_index=idx)
    assert np.array_equal(ys, yf[:, idx]) and np.array_equal(As, Af[:, idx])


def test_check_close_detects_violation():
    y = np.array([[1.0, 2.0]])
    A = np.array([[10.0, 10.0]])
    ok, _, _ = O.check_close(np.float32(y), "f32", y, A)
    assert ok
    bad = y.copy()
    bad[0, 1] += 2e-2  # bound is 1e-2 + 1e-6
    ok, ratio, nbad = O.check_close(np.float32(bad), "f32", y, A)
    assert not ok and nbad == 1 and ratio > 1.9


# ---------------------------------------------------------------- embedding rows

def test_embed_rows_are_dequant_rows():
    rng = np.random.Generator(np.random.PCG64(11))
    w = S.draw_weight(rng, 300, 256, "f16", True)
    ids = np.array([0, 299, 17, 17, 150], dtype=np.int32)
    full = O.dequantize(w.packed, w.scales, None, "f16", True, 256, "bf16")
    got = O.embed_rows(ids, w.packed, w.scales, None, "f16", True, 256, "bf16")
    assert np.array_equal(got, full[ids])


def test_embed_rows_out_of_range_is_zero():
    rng = np.random.Generator(np.random.PCG64(12))
    w = S.draw_weight(rng, 10, 128, "bf16", False)
    got = O.embed_rows(np.array([-1, 10, 3]), w.packed, w.scales, w.biases, "bf16", False, 128, "bf16")
    assert np.all(got[0] == 0) and np.all(got[1] == 0)
    assert np.array_equal(got[2], O.dequantize(w.packed[3:4], w.scales[3:4], w.biases[3:4], "bf16", False, 128,
                                               "bf16")[0])


# ---------------------------------------------------------------- FFN pieces

def test_silu_against_mpmath():
    zs = [-40.0, -10.0, -1.5, -1e-3, 0.0, 1e-3, 0.5, 2.0, 9.0, 30.0]
    got = O.silu(np.array(zs))
    mpmath.mp.dps = 40
    for z, g in zip(zs, got):
        ref = float(mpmath.mpf(z) / (1 + mpmath.e ** (-mpmath.mpf(z))))
        assert g == pytest.approx(ref, rel=1e-14, abs=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0


def test_silu_grad_against_finite_difference():
    z = np.linspace(-6, 6, 25)
    h = 1e-6
    fd = (O.silu(z + h) - O.silu(z - h)) / (2 * h)
    assert np.allclose(O.silu_grad(z), fd, rtol=1e-7, atol=1e-9)


def test_ffn_ref_stages():
    rng = np.random.Generator(np.random.PCG64(13))
    H, I, Hout = 256, 384, 128
    wg = S.draw_weight(rng, I, H, "f16", True)
    wu = S.draw_weight(rng, I, H, "f16", True)
    wd = S.draw_weight(rng, Hout, I, "bf16", False)
    x = S.draw_x(rng, 3, H)
    d = lambda w: dict(packed=w.packed, scales=w.scales, biases=w.biases, meta=w.meta, symmetric=w.symmetric, K=w.K)
    ref = O.ffn_ref(x, d(wg), d(wu), d(wd))
    # gate/up: x times the dense dequantised matrices, checked one element exactly
    ex_g = O.qmm_exact(x[:1], wg.packed[:2], wg.scales[:2], None, "f16", True, H)
    assert abs(Fraction(float(ref["g"][0, 1])) - ex_g[0][1]) <= Fraction(float(ref["Ag"][0, 1])) / 2 ** 45
    # h = silu(g) * u element-wise, with silu(z) = z / (1 + e^-z) computed independently
    i, m = 7, 2
    g, u = ref["g"][m, i], ref["u"][m, i]
    assert ref["h64"][m, i] == pytest.approx(g / (1 + math.exp(-g)) * u, rel=1e-14)
    # h rounded once to bf16, then the down projection on that rounded h
    assert np.array_equal(ref["hb"], torch.from_numpy(ref["h64"].astype(np.float32)).to(torch.bfloat16)
                          .view(torch.int16).numpy().view(np.uint16))
    ex_y = O.qmm_exact(ref["hb"][1:2], wd.packed[3:4], wd.scales[3:4], wd.biases[3:4], "bf16", False, I)
    assert abs(Fraction(float(ref["y"][1, 3])) - ex_y[0][0]) <= Fraction(float(ref["Ad"][1, 3])) / 2 ** 45
    assert np.all(O.ffn_h_bound(ref) > 0) and O.ffn_y_bound(ref, d(wd)).shape == ref["y"].shape


# ---------------------------------------------------------------- planted mistakes must be caught

def _pins_pass():
    """Run the fixture and invariant pins against the (possibly patched) oracle."""
    try:
        for case in CASES:
            test_golden_dequant(case)
            if "y" in case:
                test_golden_gemv(case)
        test_unpack_one_hot()
        test_closed_form_constant_x(False, "bf16")
        test_bruteforce_exact_rational(False, "bf16", 256, 4, 3)
        test_symmetric_groups_hold_exactly_two_values()
    except AssertionError:
        return False
    return True


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(O.q1_oracle, name, fn)
    monkeypatch.setattr(O, name, fn)


def test_unpatched_oracle_passes_pins():
    assert _pins_pass()


def test_planted_msb_first_is_caught(monkeypatch):
    def msb_first(packed, K):
        k = np.arange(K)
        words = np.asarray(packed, np.uint32)[:, k >> 5]
        return ((words >> (31 - (k & 31)).astype(np.uint32)) & np.uint32(1)).astype(np.uint8)
    _patch(monkeypatch, "unpack_bits", msb_first)
    assert not _pins_pass()


def test_planted_bias_sign_is_caught(monkeypatch):
    orig = O.q1_oracle.group_scale_bias

    def flipped(scales, biases, meta, symmetric):
        s, b = orig(scales, biases, meta, symmetric)
        return s, (-b).astype(np.float32)
    _patch(monkeypatch, "group_scale_bias", flipped)
    assert not _pins_pass()


def test_planted_unhalved_scale_is_caught(monkeypatch):
    orig = O.q1_oracle.group_scale_bias

    def unhalved(scales, biases, meta, symmetric):
        s, b = orig(scales, biases, meta, symmetric)
        return s, (b * 2 if symmetric else b).astype(np.float32)
    _patch(monkeypatch, "group_scale_bias", unhalved)
    assert not _pins_pass()


def test_planted_dropped_bias_is_caught(monkeypatch):
    orig = O.q1_oracle.group_scale_bias

    def nobias(scales, biases, meta, symmetric):
        s, b = orig(scales, biases, meta, symmetric)
        return s, np.zeros_like(b)
    _patch(monkeypatch, "group_scale_bias", nobias)
    assert not _pins_pass()


def test_planted_group_index_is_caught(monkeypatch):
    orig = O.q1_oracle.dequant_f32

    def wrong_group(packed, scales, biases, meta, symmetric, K):
        bits = O.unpack_bits(packed, K).astype(np.float32)
        s, b = O.q1_oracle.group_scale_bias(scales, biases, meta, symmetric)
        g = (np.arange(K) // 128)[::-1].copy()  # groups reversed
        return ((s[:, g] * bits).astype(np.float32) + b[:, g]).astype(np.float32)
    _patch(monkeypatch, "dequant_f32", wrong_group)
    assert not _pins_pass()
    assert orig is not wrong_group


def test_planted_transposed_operand_is_caught(monkeypatch):
    orig = O.q1_oracle.qmm_ref

    def transposed(x_bits, packed, scales, biases, meta, symmetric, K, block_rows=4096, row_index=None):
        y, A = orig(x_bits, packed, scales, biases, meta, symmetric, K, block_rows, row_index)
        return y[..., ::-1].copy(), A[..., ::-1].copy()   # columns mixed up
    _patch(monkeypatch, "qmm_ref", transposed)
    assert not _pins_pass()


# ---------------------------------------------------------------- dense fallback (bf16 weights)

def test_dense_bf16_equals_exact_when_weights_are_bf16():
    # bf16 symmetric metadata: +-scale/2 is itself a bf16 value, so rounding the
    # dequantised matrix to bf16 changes nothing.
    rng = np.random.Generator(np.random.PCG64(31))
    w = S.draw_weight(rng, 40, 1024, "bf16", True)
    x = S.draw_x(rng, 3, 1024)
    a = O.qmm_ref(x, w.packed, w.scales, None, "bf16", True, 1024)
    b = O.qmm_ref(x, w.packed, w.scales, None, "bf16", True, 1024, weights_bf16=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.mark.parametrize("symmetric,meta", [(True, "f16"), (False, "bf16")])
def test_dense_bf16_bruteforce_and_bound(symmetric, meta):
    rng = np.random.Generator(np.random.PCG64(32))
    w = S.draw_weight(rng, 3, 256, meta, symmetric)
    x = S.draw_x(rng, 2, 256)
    y, A = O.qmm_ref(x, w.packed, w.scales, w.biases, meta, symmetric, 256, weights_bf16=True)
    ex = O.qmm_exact(x, w.packed, w.scales, w.biases, meta, symmetric, 256, weights_bf16=True)
    for m in range(2):
        for n in range(3):
            assert abs(Fraction(float(y[m, n])) - ex[m][n]) <= Fraction(float(A[m, n])) / 2 ** 45
    y0, A0 = O.qmm_ref(x, w.packed, w.scales, w.biases, meta, symmetric, 256)
    assert (np.abs(y - y0) <= O.dense_rounding_bound(A0)).all()
    if meta == "f16":
        assert not np.array_equal(y, y0)  # fp16-derived weights do move under bf16 rounding


def test_planted_missing_bf16_rounding_is_caught(monkeypatch):
    orig = O.q1_oracle.qmm_ref

    def no_rounding(*args, weights_bf16=False, **kw):
        return orig(*args, **kw)
    _patch(monkeypatch, "qmm_ref", no_rounding)
    with pytest.raises(AssertionError):
        test_dense_bf16_bruteforce_and_bound(True, "f16")


# ---------------------------------------------------------------- outlier inputs (GPU tolerance tests)

def test_worked_outlier_case_has_the_hand_computed_result():
    """Scale 0.25, bias -0.25: set bits weigh 0, clear bits -0.25; each
    32-block contributes -0.25 * 16 * 2^-6 = -1/16, so K = 1024 gives -2
    exactly, with sum |w x| = 2 (hand-worked)."""
    from tests.outlier_inputs import worked_case
    w, x = worked_case(1024, 3, False)
    y, A = O.qmm_ref(x, w.packed, w.scales, w.biases, w.meta, False, w.K)
    assert np.all(y == -2.0) and np.all(A == 2.0)
    deq = O.dequant_f32(w.packed, w.scales, w.biases, w.meta, False, w.K)
    assert set(np.unique(deq).tolist()) == {0.0, -0.25}


def test_adversarial_outlier_inputs_put_outliers_on_zero_weights():
    """Every outlier of the GPU outlier tests meets a dequantised weight of
    exactly 0, so the tolerance holds none of the outlier terms."""
    from tests.outlier_inputs import outlier_positions, outlier_x, zero_weight_codes
    rng = np.random.Generator(np.random.PCG64(1))
    pos = outlier_positions(rng, 1024)
    w = zero_weight_codes(rng, 6, 1024, "bf16", pos)
    deq = O.dequant_f32(w.packed, w.scales, w.biases, "bf16", False, 1024)
    assert np.all(deq[:, pos] == 0.0) and np.count_nonzero(deq) > deq.size // 3
    x = O.bf16_to_f32(outlier_x(rng, 2, 1024, 12, pos))
    assert np.all(np.abs(x[:, pos]) >= 2.0 ** 12)


# ---------------------------------------------------------------- output rounding in the tolerance

def test_output_half_ulp_hand_values():
    """Half the spacing of the output grid at the stored value.  bf16 keeps 8
    significant bits: 1.0 and 1.9921875 sit in [1, 2) with spacing 2^-7, 2.0
    and -3.0 in [2, 4) with 2^-6; below 2^-126 the spacing is the subnormal
    one, 2^-133 (so zero and every subnormal get 2^-134).  f32 outputs get
    nothing: the fp32 accumulator is stored as it is."""
    bf = O.f32_to_bf16_rne(np.array([1.0, 1.9921875, 2.0, -3.0, 0.0, 2.0 ** -126, 2.0 ** -130], np.float32))
    assert O.output_half_ulp(bf, "bf16").tolist() == [2.0 ** -8, 2.0 ** -8, 2.0 ** -7, 2.0 ** -7, 2.0 ** -134,
                                                      2.0 ** -134, 2.0 ** -134]
    assert O.output_half_ulp(np.array([1.0, -7.5], np.float32), "f32").tolist() == [0.0, 0.0]


def test_output_half_ulp_f16_matches_numpy_spacing():
    """For binary16 the same quantity is half of NumPy's own float16 spacing
    (a library routine) at every finite value below the largest."""
    bits = np.arange(0, 0x7BFF, dtype=np.uint16)  # +0 .. the value below 65504
    bits = np.concatenate([bits, bits | np.uint16(0x8000)])
    want = np.spacing(np.abs(bits.view(np.float16))).astype(np.float64) / 2.0
    assert np.array_equal(O.output_half_ulp(bits, "f16"), want)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_output_half_ulp_bounds_round_to_nearest(dtype):
    """Brute force: every float32 value v, rounded to nearest even to the
    output grid, lands within output_half_ulp(stored) of v -- and exact ties
    (v halfway between two grid points) reach the bound, so it is tight."""
    rng = np.random.Generator(np.random.PCG64(17))
    mant = rng.integers(0, 1 << 23, size=200_000, dtype=np.uint32)
    expo = rng.integers(127 - 30, 127 + 14, size=mant.size, dtype=np.uint32)
    sign = rng.integers(0, 2, size=mant.size, dtype=np.uint32) << np.uint32(31)
    v = (sign | (expo << np.uint32(23)) | mant).view(np.float32)
    stored = O.round_to(v, dtype)
    gap = np.abs(O.out_to_f64(stored, dtype) - v.astype(np.float64))
    half = O.output_half_ulp(stored, dtype)
    assert np.all(gap <= half)
    assert np.any(gap == half)


def test_check_close_allows_exactly_the_output_rounding():
    """Hand case, bf16 output, sum |w x| = 1e-9 (tolerance about 1e-6): an
    exact result of 1 + 2^-8 (a tie) stored as 1.0 passes (error = half an
    ulp); 1 + 2^-8 + 1e-5 stored as 1.0 fails (it rounds to 1 + 2^-7); the
    next grid value up also fails; a float32 output gets no rounding term."""
    one = O.f32_to_bf16_rne(np.array([1.0], np.float32))
    up = O.f32_to_bf16_rne(np.array([1.0 + 2.0 ** -7], np.float32))
    A = np.array([1e-9])
    assert O.check_close(one, "bf16", np.array([1.0 + 2.0 ** -8]), A)[0]
    assert not O.check_close(one, "bf16", np.array([1.0 + 2.0 ** -8 + 1e-5]), A)[0]
    assert not O.check_close(up, "bf16", np.array([1.0 + 2.0 ** -9]), A)[0]
    assert not O.check_close(np.array([1.0], np.float32), "f32", np.array([1.0 + 2.0 ** -19]), A)[0]
    assert O.check_close(np.array([1.0], np.float32), "f32", np.array([1.0 + 5e-7]), A)[0]
