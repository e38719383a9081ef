"""Pins for the oracle's metadata functions: the symmetric-bias check and the
sign packer.  Each is tied to something other than itself: values worked out by
hand from the format (rMLX issue #207: bit 0 -> -s_g, bit 1 -> +s_g, stored
scale 2 s_g, weight k = bit k & 31 of word k >> 5), the round trip through the
oracle's dequantisation (itself pinned by hand fixtures), and the definition of
"a bias that can be dropped" evaluated element by element.  Planted mistakes
must be caught."""
import numpy as np
import pytest

import oracle as O
import q1_synth as S

# bf16 / fp16 bit patterns used below
BF16_QUARTER, BF16_EIGHTH, BF16_HALF = 0x3E80, 0x3E00, 0x3F00
F16_HALF, F16_QUARTER = 0x3800, 0x3400


def _row(values_bits):
    return np.array([values_bits], dtype=np.uint16)


# ---------------------------------------------------------------- sign packer by hand

def test_pack_all_positive_group():
    # 128 weights of +0.25: every bit set, stored scale 2 * 0.25 = 0.5
    packed, scales, bad = O.pack_signs(_row([BF16_QUARTER] * 128), "bf16", "bf16")
    assert packed.tolist() == [[0xFFFFFFFF] * 4]
    assert scales.tolist() == [[BF16_HALF]]
    assert bad == 0


def test_pack_alternating_signs_lsb_first():
    # weight k = -0.25 for even k, +0.25 for odd k: bits 1, 3, 5, .. of every word
    vals = [BF16_QUARTER | (0x8000 if k % 2 == 0 else 0) for k in range(128)]
    packed, scales, bad = O.pack_signs(_row(vals), "bf16", "bf16")
    assert packed.tolist() == [[0xAAAAAAAA] * 4]
    assert scales.tolist() == [[BF16_HALF]] and bad == 0


def test_pack_one_odd_weight_is_inexact():
    # as above, but weight 4 (even, negative) replaced by +0.125: bit 4 becomes
    # 1, the scale stays 2 * max|w| = 0.5, and the group no longer round-trips
    vals = [BF16_QUARTER | (0x8000 if k % 2 == 0 else 0) for k in range(128)]
    vals[4] = BF16_EIGHTH
    packed, scales, bad = O.pack_signs(_row(vals), "bf16", "bf16")
    assert packed.tolist() == [[0xAAAAAABA, 0xAAAAAAAA, 0xAAAAAAAA, 0xAAAAAAAA]]
    assert scales.tolist() == [[BF16_HALF]] and bad == 1


def test_pack_zero_groups():
    # all +0.0: bits 0, scale 0, exact (a zero scale dequantises both codes to
    # +0.0); one -0.0 in the group cannot come back
    packed, scales, bad = O.pack_signs(_row([0] * 256), "bf16", "f16")
    assert packed.tolist() == [[0] * 8] and scales.tolist() == [[0, 0]] and bad == 0
    vals = [0] * 256
    vals[130] = 0x8000
    assert O.pack_signs(_row(vals), "bf16", "f16")[2] == 1


def test_pack_nan_and_overflow_are_inexact():
    vals = [BF16_QUARTER] * 128
    vals[7] = 0x7FC0  # NaN
    assert O.pack_signs(_row(vals), "bf16", "bf16")[2] == 1
    # 2 * 40000 does not fit fp16 metadata (max 65504): scale inf, inexact
    big = 0x471C  # bf16 39936
    assert O.pack_signs(_row([big] * 128), "bf16", "f16")[2] == 1
    assert O.pack_signs(_row([big] * 128), "bf16", "bf16")[2] == 0


def test_pack_fp16_dense_fp16_meta():
    # fp16 weights +-0.25, fp16 scale 0.5; the second group mixes in -0.25 only
    vals = [F16_QUARTER] * 128 + [F16_QUARTER | 0x8000] * 128
    packed, scales, bad = O.pack_signs(_row(vals), "f16", "f16")
    assert packed.tolist() == [[0xFFFFFFFF] * 4 + [0] * 4]
    assert scales.tolist() == [[F16_HALF, F16_HALF]] and bad == 0


# ---------------------------------------------------------------- sign packer round trip

@pytest.mark.parametrize("meta", ["bf16", "f16"])
def test_pack_inverts_dequantize(meta):
    # any symmetric tensor whose half-scales are exact in the dense dtype comes
    # back bit for bit: pack(dequantize(P, S)) == (P, S)
    rng = np.random.Generator(np.random.PCG64(11))
    w = S.draw_weight(rng, 24, 512, meta, True)
    s = O.meta_to_f32(w.scales, meta)
    floor = np.float32(2.0 ** -10)  # keeps s/2 a normal fp16 number
    scales = O.round_to(np.maximum(s, floor).astype(np.float32), meta)
    dense = O.dequantize(w.packed, scales, None, meta, True, 512, meta)
    packed, back_scales, bad = O.pack_signs(dense, meta, meta)
    assert bad == 0
    assert np.array_equal(packed, w.packed) and np.array_equal(back_scales, scales)


def test_pack_counts_inexact_groups_exactly():
    # perturb one weight in a known set of groups: exactly those are inexact
    rng = np.random.Generator(np.random.PCG64(12))
    w = S.draw_weight(rng, 8, 1024, "bf16", True)
    scales = O.round_to(np.maximum(O.meta_to_f32(w.scales, "bf16"), np.float32(1e-3)), "bf16")
    dense = O.dequantize(w.packed, scales, None, "bf16", True, 1024, "bf16").copy()
    hit = [(0, 0), (3, 5), (7, 7), (7, 6)]
    for n, g in hit:
        dense[n, g * 128 + 17] ^= 0x0001  # one ulp off
    assert O.pack_signs(dense, "bf16", "bf16")[2] == len(hit)


# ---------------------------------------------------------------- symmetric check

def test_symmetric_check_by_hand():
    # fp16 metadata; groups and the expected verdict (True = bias can go):
    cases = [
        (F16_HALF, F16_QUARTER | 0x8000, True),    # bias -0.25 == -0.5/2
        (F16_HALF, 0xB401, False),                 # one ulp below -0.25
        (0x0000, 0x0000, True),                    # zero scale, +0 bias: both codes +0.0 either way
        (0x0000, 0x8000, True),                    # zero scale, -0 bias
        (0x0001, 0x8000, False),                   # 2^-24 scale: -2^-25 is not an fp16 value
        (0x7C00, 0xFC00, False),                   # infinite scale
        (F16_HALF, 0x7E00, False),                 # NaN bias
    ]
    scales = np.array([[c[0] for c in cases]], dtype=np.uint16)
    biases = np.array([[c[1] for c in cases]], dtype=np.uint16)
    assert O.symmetric_mismatches(scales, biases, "f16") == sum(not c[2] for c in cases)
    for s, b, ok in cases:
        assert O.symmetric_mismatches(np.array([[s]], np.uint16), np.array([[b]], np.uint16), "f16") == (0 if ok else 1)


@pytest.mark.parametrize("meta", ["bf16", "f16"])
def test_symmetric_check_is_dequant_equality(meta):
    # the count equals the number of groups whose dequantised weights change
    # when the stored bias is replaced by -scale/2 (finite metadata)
    rng = np.random.Generator(np.random.PCG64(13))
    w = S.draw_weight(rng, 32, 1024, meta, True)
    half = O.round_to((np.float32(-0.5) * O.meta_to_f32(w.scales, meta)).astype(np.float32), meta)
    biases = half.copy()
    biases[::3, ::4] ^= np.uint16(1)  # some groups off by one ulp
    K = 1024
    a = O.dequant_f32(w.packed, w.scales, biases, meta, False, K).view(np.uint32)
    b = O.dequant_f32(w.packed, w.scales, None, meta, True, K).view(np.uint32)
    changed = (a != b).reshape(32, K // 128, 128).any(axis=2)
    # a group whose packed bits are all 0 or all 1 only tests one code; the
    # check looks at both codes, so compare on groups that use both
    bits = O.unpack_bits(w.packed, K).reshape(32, K // 128, 128)
    both = bits.any(axis=2) & (~bits.astype(bool)).any(axis=2)
    assert both.all()
    assert O.symmetric_mismatches(w.scales, biases, meta) == int(changed.sum())


# ---------------------------------------------------------------- planted mistakes

def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(O.q1_oracle, name, fn)
    monkeypatch.setattr(O, name, fn)


def _pack_pins_pass():
    try:
        test_pack_all_positive_group()
        test_pack_alternating_signs_lsb_first()
        test_pack_one_odd_weight_is_inexact()
        test_pack_zero_groups()
        test_pack_inverts_dequantize("bf16")
    except AssertionError:
        return False
    return True


def test_unpatched_packer_passes():
    assert _pack_pins_pass()


def test_planted_msb_first_packer_is_caught(monkeypatch):
    real = O.pack_signs

    def msb(dense_bits, dense, meta):
        p, s, n = real(dense_bits, dense, meta)
        rev = np.zeros_like(p)
        for i in range(32):
            rev |= ((p >> np.uint32(i)) & np.uint32(1)) << np.uint32(31 - i)
        return rev, s, n
    _patch(monkeypatch, "pack_signs", msb)
    assert not _pack_pins_pass()


def test_planted_undoubled_scale_is_caught(monkeypatch):
    real = O.pack_signs

    def half_scale(dense_bits, dense, meta):
        p, s, n = real(dense_bits, dense, meta)
        return p, O.round_to(O.meta_to_f32(s, meta) * np.float32(0.5), meta), n
    _patch(monkeypatch, "pack_signs", half_scale)
    assert not _pack_pins_pass()


def test_planted_nonnegative_sign_is_caught(monkeypatch):
    real = O.pack_signs

    def ge_zero(dense_bits, dense, meta):
        p, s, n = real(dense_bits, dense, meta)
        w = O.meta_to_f32(dense_bits, dense)
        zero = (w == 0).reshape(w.shape[0], -1, 32)
        for i in range(32):
            p |= zero[:, :, i].astype(np.uint32) << np.uint32(i)
        return p, s, n
    _patch(monkeypatch, "pack_signs", ge_zero)
    assert not _pack_pins_pass()


def test_planted_meta_compare_check_is_caught(monkeypatch):
    # comparing the stored bias with round_meta(-s/2) instead of the dequantised
    # values rejects a zero scale with a +0 bias
    def meta_compare(scales, biases, meta):
        half = O.round_to((np.float32(-0.5) * O.meta_to_f32(scales, meta)).astype(np.float32), meta)
        return int((np.asarray(half) != np.asarray(biases)).sum())
    _patch(monkeypatch, "symmetric_mismatches", meta_compare)
    with pytest.raises(AssertionError):
        test_symmetric_check_by_hand()
