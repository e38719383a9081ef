"""Seeded activations with in-block outliers, and weights whose codes carry
very unequal weights, for the matmul tolerance tests.

Large activations next to small ones are usual in LLM decode, and affine Q1
tensors (Higgs PR #212, "Measured impact": a few tensors keep a stored bias)
can give one code of a group a weight near zero.  These generators build such
inputs; they do none of the method's arithmetic (no unpacking, dequantisation
or products).
"""
import numpy as np

import q1_synth as S


def worked_case(K: int, N: int, clear_bits_small: bool):
    """Affine bf16 tensor with scale 0.25 and bias -0.25 in every group, so a
    set bit has weight 0 and a clear bit weight -0.25.  Every 32-weight word
    of every row is 0x0000FFFF: weights 0..15 of the word set, 16..31 clear.
    Activations (one row) per 32-block: 1024 on weight 0, about 0.012 on
    weights 1..15, and on weights 16..31 either 2^-6 (on the fp8 grid of the
    block) or, with ``clear_bits_small``, values near 0.012 as well.

    Returns (weight, x bits [1, K])."""
    rng = np.random.Generator(np.random.PCG64(4242 + K + int(clear_bits_small)))
    G = K // 128
    packed = np.full((N, K // 32), 0x0000FFFF, dtype=np.uint32)
    scales = S.meta_bits(np.full((N, G), 0.25, dtype=np.float32), "bf16")
    biases = S.meta_bits(np.full((N, G), -0.25, dtype=np.float32), "bf16")
    x = np.empty((1, K), dtype=np.float32)
    for w in range(K // 32):
        blk = np.empty(32, dtype=np.float32)
        blk[0] = 1024.0
        blk[1:16] = 0.012 * (1.0 + 0.1 * rng.standard_normal(15))
        if clear_bits_small:
            blk[16:] = 0.012 * (1.0 + 0.1 * rng.standard_normal(16))
        else:
            blk[16:] = 2.0 ** -6
        x[0, 32 * w:32 * w + 32] = blk
    return S.Q1Weight(packed, scales, biases, "bf16", N, K), S.bf16_bits(x)


def outlier_positions(rng, K: int) -> np.ndarray:
    """One position per 32-weight block (shared by every activation row)."""
    return np.arange(0, K, 32) + rng.integers(0, 32, size=K // 32)


def zero_weight_codes(rng, N: int, K: int, meta: str, pos=None):
    """Affine tensor whose groups alternate between bias = -scale (set bits
    weigh 0) and bias = 0 (clear bits weigh 0); scales |N(0, 0.02)|, bits
    uniform.  With ``pos`` (outlier positions), the bit at each position is
    set to the code that weighs 0 in its group, so no outlier contributes to
    sum |w x| and the tolerance holds only the other terms."""
    G = K // 128
    packed = rng.integers(0, 1 << 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    sb = S.meta_bits(np.abs(rng.normal(0.0, 0.02, size=(N, G))).astype(np.float32), meta)
    kind = (np.arange(N)[:, None] + np.arange(G)[None, :]) % 2
    # -scale exactly: the same bit pattern with the sign bit set
    bb = np.where(kind == 0, sb ^ np.uint16(0x8000), np.uint16(0)).astype(np.uint16)
    if pos is not None:
        for k in pos:
            bit = np.uint32(1) << np.uint32(k & 31)
            set_ = kind[:, k // 128] == 0
            packed[set_, k >> 5] |= bit
            packed[~set_, k >> 5] &= ~bit
    return S.Q1Weight(packed, sb, bb, meta, N, K)


def outlier_x(rng, M: int, K: int, ratio_log2: int, pos=None):
    """Activations N(0, 1) with, in every 32-block, one outlier of magnitude
    2^ratio_log2 (times 1..2) -- at ``pos`` when given, else at a random
    position per row -- and four elements scaled down by up to 2^-ratio_log2,
    so blocks span about 2^(2 ratio_log2)."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    for m in range(M):
        for w in range(K // 32):
            j = int(pos[w]) if pos is not None else 32 * w + int(rng.integers(32))
            x[m, j] = np.float32((1.0 + rng.random()) * 2.0 ** ratio_log2 * rng.choice([-1.0, 1.0]))
            small = 32 * w + rng.integers(32, size=4)
            small = small[small != j]
            x[m, small] *= np.float32(2.0) ** -rng.integers(0, ratio_log2 + 1, size=small.size).astype(np.float32)
    return S.bf16_bits(x)
