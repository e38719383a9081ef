"""CPU oracle for the packed Q1 (1-bit affine, group 128) decode path.

TEST INFRASTRUCTURE ONLY.  Nothing in the library imports, links or calls this
module; only the tests, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP path: every step below is written from the
pages' description of the format and from the plain definition of the
operation, in NumPy, slowly and visibly.

What it computes and where that is defined
------------------------------------------
* Packing (rMLX issue #207, "The good news -- packing is standard"): weights
  are stored 32 per uint32 word; the Cactus PR #775 commit notes call it the
  "linear LSB layout".  Weight ``k`` of a row is bit ``k & 31`` of word
  ``k >> 5`` (least significant bit first).
* Groups (same passage; mlx-gen backlog 0004, "Context"): one scale (and, for
  affine tensors, one bias) per 128 consecutive weights along K, stored as
  fp16 or bf16.
* Affine dequantisation (Higgs PR #212, "What" and "Why"):
  ``w = scale * bit + bias``.
* Symmetric tensors (Higgs PR #212, "What": bias derived as ``-scale / 2``;
  rMLX #207: bit 0 -> ``-s_g``, bit 1 -> ``+s_g``): the bias is not stored and
  ``bias = -scale / 2``, so the two codes map to ``-scale/2`` and ``+scale/2``
  (the pages' ``s_g`` is half the stored scale).  The halving is done in fp32,
  where it is exact.
* Narrow/wide matmul (Higgs PR #212, "What", "Validation"): ``y = x W^T`` over
  the flattened leading dimensions of ``x``; the validation compares the packed
  result with a matmul against the densely dequantised matrix -- which is what
  :func:`qmm_ref` does, in fp64.
* Fused dense FFN (Higgs PR #212, "What"): gate and up projections, then
  ``SiLU(gate) * up``, then the down projection.

Readings of the pages taken here (each also listed in the design notes):
the dequantised weight is ``fl32(fl32(s * bit) + b)`` (one rounding, the add);
outputs of dequantisation and gathering are rounded to the output dtype with
round-to-nearest-even; the FFN keeps gate/up in full precision and rounds the
hidden activation ``h`` once to bf16 before the down projection; token ids
outside ``[0, V)`` give an all-zero row; the matmul tolerance
``1e-3 sum|w x| + 1e-6`` bounds the fp32 accumulation, which is then rounded
to the output dtype, so a stored f16/bf16 output may differ from it by a
further half ulp (:func:`check_close`).

Every function here is pinned by ``tests/test_oracle_pins.py`` (the FFN error
bounds by ``tests/test_oracle_ffn_bound_pins.py``) against values
fixed by the format or by mathematics (hand-worked fixtures, closed forms,
exact rational brute force, library routines).  No function is left unpinned.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Optional

import numpy as np

GROUP = 128

# --------------------------------------------------------------------------
# Scalar formats (bit patterns in, float32 out; float32 in, bit patterns out)
# --------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float32, exact: the bf16 pattern is the
    upper half of the float32 pattern."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def f16_to_f32(bits: np.ndarray) -> np.ndarray:
    """IEEE binary16 bit patterns -> float32 (exact widening)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float32)


def meta_to_f32(bits: np.ndarray, meta: str) -> np.ndarray:
    if meta == "f16":
        return f16_to_f32(bits)
    if meta == "bf16":
        return bf16_to_f32(bits)
    raise ValueError(meta)


def f32_to_bf16_rne(values: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even.

    Keep the upper 16 bits after adding ``0x7FFF`` plus the lowest kept bit:
    below half an ulp rounds down, above rounds up, an exact tie rounds to the
    even neighbour.  NaN inputs are quieted instead (never produced here).
    """
    v = np.ascontiguousarray(values, dtype=np.float32)
    u = v.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32) & np.uint32(0xFFFF)
    nan = np.isnan(v)
    if nan.any():
        r = np.where(nan, ((u >> np.uint64(16)).astype(np.uint32) | np.uint32(0x40)) & np.uint32(0xFFFF), r)
    return r.astype(np.uint16)


def f32_to_f16_rne(values: np.ndarray) -> np.ndarray:
    """float32 -> IEEE binary16 bit patterns; NumPy's conversion is the IEEE
    round-to-nearest-even one."""
    with np.errstate(over="ignore"):   # overflow to +-inf is the IEEE result
        return np.ascontiguousarray(values, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_to(values_f32: np.ndarray, out_dtype: str) -> np.ndarray:
    """Round float32 values to ``out_dtype``; returns uint16 bit patterns for
    bf16/f16 and float32 values for f32."""
    if out_dtype == "bf16":
        return f32_to_bf16_rne(values_f32)
    if out_dtype == "f16":
        return f32_to_f16_rne(values_f32)
    if out_dtype == "f32":
        return np.ascontiguousarray(values_f32, dtype=np.float32)
    raise ValueError(out_dtype)


def out_to_f64(values: np.ndarray, out_dtype: str) -> np.ndarray:
    """Stored output (bit patterns or float32) -> float64."""
    if out_dtype == "bf16":
        return bf16_to_f32(values).astype(np.float64)
    if out_dtype == "f16":
        return f16_to_f32(values).astype(np.float64)
    return np.asarray(values, dtype=np.float32).astype(np.float64)


# --------------------------------------------------------------------------
# Unpacking and dequantisation
# --------------------------------------------------------------------------


def unpack_bits(packed: np.ndarray, K: int) -> np.ndarray:
    """``[N, K/32]`` uint32 -> ``[N, K]`` uint8 codes; weight ``k`` is bit
    ``k & 31`` of word ``k >> 5`` (LSB first)."""
    packed = np.asarray(packed, dtype=np.uint32)
    k = np.arange(K)
    words = packed[:, k >> 5]
    return ((words >> (k & 31).astype(np.uint32)) & np.uint32(1)).astype(np.uint8)


def group_scale_bias(scales: np.ndarray, biases: Optional[np.ndarray], meta: str,
                     symmetric: bool) -> tuple[np.ndarray, np.ndarray]:
    """Per-group fp32 scale and bias ``[N, G]``.  Symmetric: ``b = -0.5 * s``
    computed in fp32 (exact)."""
    s = meta_to_f32(scales, meta)
    if symmetric:
        if biases is not None:
            raise ValueError("symmetric tensors carry no stored bias")
        b = (np.float32(-0.5) * s).astype(np.float32)
    else:
        if biases is None:
            raise ValueError("affine tensors need a stored bias")
        b = meta_to_f32(biases, meta)
    return s, b


def dequant_f32(packed: np.ndarray, scales: np.ndarray, biases: Optional[np.ndarray], meta: str,
                symmetric: bool, K: int) -> np.ndarray:
    """Dense float32 weights ``[N, K]``: ``w = fl32(fl32(s * bit) + b)``."""
    bits = unpack_bits(packed, K).astype(np.float32)
    s, b = group_scale_bias(scales, biases, meta, symmetric)
    g = np.arange(K) // GROUP
    sk = s[:, g]
    bk = b[:, g]
    prod = (sk * bits).astype(np.float32)       # exact: bit is 0 or 1
    return (prod + bk).astype(np.float32)       # the one rounding


def dequantize(packed, scales, biases, meta, symmetric, K, out_dtype):
    """Dequantised matrix rounded to ``out_dtype`` (bit patterns for 16-bit
    types, float32 values for f32)."""
    return round_to(dequant_f32(packed, scales, biases, meta, symmetric, K), out_dtype)


def embed_rows(ids: np.ndarray, packed, scales, biases, meta, symmetric, K, out_dtype):
    """Rows ``ids`` of the dequantised table, rounded to ``out_dtype``; an id
    outside ``[0, V)`` yields a row of zeros."""
    ids = np.asarray(ids).astype(np.int64)
    V = packed.shape[0]
    ok = (ids >= 0) & (ids < V)
    safe = np.where(ok, ids, 0)
    rows = dequant_f32(packed[safe], scales[safe], None if biases is None else biases[safe], meta, symmetric, K)
    rows[~ok] = 0.0
    return round_to(rows, out_dtype)


# --------------------------------------------------------------------------
# Matmul reference and tolerance
# --------------------------------------------------------------------------


def qmm_ref(x_bits: np.ndarray, packed, scales, biases, meta, symmetric, K, block_rows: int = 4096,
            row_index: Optional[np.ndarray] = None, weights_bf16: bool = False):
    """``y = x W^T`` in fp64 plus ``A = |x| |W|^T`` (for the tolerance).

    ``x_bits``: bf16 bit patterns ``[..., K]``; leading dims are flattened to M
    rows and restored on the output.  ``row_index`` restricts the output
    columns to the given weight rows (for sampled checks of large matrices).
    ``weights_bf16``: the dense fallback for wide M (Higgs PR #212,
    "Limitations": wider forwards dequantise to the input dtype, bf16 here,
    before the dense matmul) -- W is rounded to bf16 before the product.
    Returns ``(y, A)`` of shape ``[..., n_out]``.
    """
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    lead = x_bits.shape[:-1]
    x = bf16_to_f32(x_bits.reshape(-1, K)).astype(np.float64)
    rows = np.arange(packed.shape[0]) if row_index is None else np.asarray(row_index, dtype=np.int64)
    M = x.shape[0]
    y = np.empty((M, rows.size), dtype=np.float64)
    A = np.empty((M, rows.size), dtype=np.float64)
    ax = np.abs(x)
    for r0 in range(0, rows.size, block_rows):
        sel = rows[r0:r0 + block_rows]
        w = dequant_f32(packed[sel], scales[sel], None if biases is None else biases[sel], meta, symmetric, K)
        if weights_bf16:
            w = bf16_to_f32(f32_to_bf16_rne(w))
        w = w.astype(np.float64)
        y[:, r0:r0 + sel.size] = x @ w.T
        A[:, r0:r0 + sel.size] = ax @ np.abs(w).T
    return y.reshape(*lead, rows.size), A.reshape(*lead, rows.size)


def dense_rounding_bound(A: np.ndarray) -> np.ndarray:
    """Bound on ``|x W_bf16^T - x W^T|``: each weight moves by at most half a
    bf16 ulp, i.e. ``2^-8 |w|``, so the product moves by at most ``2^-8 A``."""
    return np.asarray(A, dtype=np.float64) * 2.0 ** -8


def tolerance(A: np.ndarray) -> np.ndarray:
    """Per-element bound on ``|y - y_ref|``: ``1e-3 * sum_k |w_nk x_k| + 1e-6``."""
    return 1e-3 * np.asarray(A, dtype=np.float64) + 1e-6


def output_half_ulp(y_stored: np.ndarray, out_dtype: str) -> np.ndarray:
    """Half a unit in the last place of each stored output value: 0 for f32
    outputs (the fp32 accumulator is stored as it is), else half the spacing
    of the f16 / bf16 grid in the binade of the stored value (8 significant
    bits for bf16, 11 for f16; subnormal spacing below the smallest normal).

    A value ``v`` that rounds to nearest to the stored ``y`` lies within this
    of ``y``: inside y's binade by definition, and a ``v`` just below a power
    of two that rounds up to it is within half the lower binade's spacing,
    which is smaller."""
    if out_dtype == "f32":
        return np.zeros(np.shape(y_stored), dtype=np.float64)
    v = np.abs(out_to_f64(y_stored, out_dtype))
    p, emin = (8, -126) if out_dtype == "bf16" else (11, -14)
    _, e = np.frexp(v)  # v = m 2^e, 0.5 <= m < 1: binade [2^(e-1), 2^e)
    e = np.where(v == 0.0, emin + 1, e)
    return np.ldexp(1.0, np.maximum(e - 1, emin) - (p - 1)) / 2.0


def check_within(y_stored: np.ndarray, out_dtype: str, y_ref: np.ndarray, bound: np.ndarray):
    """Stored outputs against ``y_ref`` for a bound on the value *before* its
    rounding to the output dtype: passes where
    ``|y - y_ref| <= bound + output_half_ulp(y)``.  Returns ``(ok, worst
    err/allowed ratio, number of violations)``."""
    y = out_to_f64(y_stored, out_dtype)
    err = np.abs(y - y_ref)
    allowed = np.asarray(bound, dtype=np.float64) + output_half_ulp(y_stored, out_dtype)
    ratio = err / allowed
    return bool((err <= allowed).all()), float(ratio.max(initial=0.0)), int((err > allowed).sum())


def check_close(y_stored: np.ndarray, out_dtype: str, y_ref: np.ndarray, A: np.ndarray):
    """The matmul tolerance: the fp32 accumulation is within
    ``1e-3 * sum_k |w_nk x_k| + 1e-6`` of ``y_ref``, then rounded to the
    output dtype (so a stored f16 / bf16 value may also differ from it by half
    its ulp).  Returns ``(ok, worst err/allowed ratio, number of violations)``."""
    return check_within(y_stored, out_dtype, y_ref, tolerance(A))


def qmm_exact(x_bits: np.ndarray, packed, scales, biases, meta, symmetric, K, weights_bf16: bool = False) -> list:
    """Exact rational ``x W^T`` for tiny inputs (pure-Python ``Fraction``s of
    the bf16 activations and the fp32 dequantised weights, or of their bf16
    roundings with ``weights_bf16``)."""
    x = bf16_to_f32(np.asarray(x_bits, dtype=np.uint16).reshape(-1, K))
    w = dequant_f32(packed, scales, biases, meta, symmetric, K)
    if weights_bf16:
        w = bf16_to_f32(f32_to_bf16_rne(w))
    out = []
    for m in range(x.shape[0]):
        row = []
        for n in range(w.shape[0]):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(float(x[m, k])) * Fraction(float(w[n, k]))
            row.append(acc)
        out.append(row)
    return out


# --------------------------------------------------------------------------
# Fused dense FFN
# --------------------------------------------------------------------------


def silu(z: np.ndarray) -> np.ndarray:
    """``z * sigmoid(z) = z / (1 + exp(-z))`` in fp64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def silu_grad(z: np.ndarray) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        sg = 1.0 / (1.0 + np.exp(-z))
    return sg * (1.0 + z * (1.0 - sg))


def ffn_ref(x_bits: np.ndarray, gate: dict, up: dict, down: dict, weights_bf16: bool = False):
    """Reference for ``y = (SiLU(x Wg^T) * (x Wu^T)) Wd^T``.

    Each weight is a dict with keys packed, scales, biases, meta, symmetric, K.
    ``weights_bf16`` selects the wide-M (dense fallback) definition for all
    three projections.  Returns a dict with the fp64 gate/up products, their tolerance sums, the
    fp64 hidden activation ``h64``, its bf16 rounding ``hb`` (bit patterns),
    and ``y_ref = hb Wd^T`` with ``A_d = |hb| |Wd|^T``.
    """
    g, Ag = qmm_ref(x_bits, **gate, weights_bf16=weights_bf16)
    u, Au = qmm_ref(x_bits, **up, weights_bf16=weights_bf16)
    h64 = silu(g) * u
    hb = f32_to_bf16_rne(h64.astype(np.float32))
    y, Ad = qmm_ref(hb, **down, weights_bf16=weights_bf16)
    return {"g": g, "Ag": Ag, "u": u, "Au": Au, "h64": h64, "hb": hb, "y": y, "Ad": Ad}


# Largest |SiLU''(z)| over the reals (reached at z = 0: SiLU'' = sigma'(z)
# (2 + z (1 - 2 sigma(z))), which is 1/4 * 2 there).  Used by the mean-value
# bound below.
SILU_CURVATURE = 0.5
# Relative error allowed for the kernel's own fp32 evaluation of
# SiLU(g) * u (exp, add, divide and multiply, each a few ulp of 2^-24).
F32_EVAL_REL = 2.0 ** -20
# Half an ulp of bf16, relative: |RNE_bf16(v) - v| <= 2^-8 |v| for normal v.
BF16_HALF_ULP_REL = 2.0 ** -8


def h_perturbation_bound(g, u, dg, du) -> np.ndarray:
    """Bound on ``|SiLU(g') u' - SiLU(g) u|`` for every ``|g' - g| <= dg`` and
    ``|u' - u| <= du`` (element-wise).

    Write ``SiLU(g') u' - SiLU(g) u = (SiLU(g') - SiLU(g)) u' + SiLU(g) (u' - u)``.
    By the mean-value theorem ``|SiLU(g') - SiLU(g)| <= dg * max |SiLU'|`` over
    ``[g - dg, g + dg]``, and ``max |SiLU'| <= |SiLU'(g)| + SILU_CURVATURE * dg``
    there; ``|u'| <= |u| + du``."""
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    dg = np.asarray(dg, dtype=np.float64)
    du = np.asarray(du, dtype=np.float64)
    slope = np.abs(silu_grad(g)) + SILU_CURVATURE * dg
    return slope * dg * (np.abs(u) + du) + np.abs(silu(g)) * du


def ffn_h_bound(ref: dict) -> np.ndarray:
    """Allowed ``|h_gpu - h64|`` for the kernel's bf16 hidden activation.

    The kernel's gate and up sums are each within the matmul tolerance of the
    exact ``g`` and ``u`` (``dg = 1e-3 A_g + 1e-6``, ``du`` likewise); it
    evaluates ``SiLU(g) u`` in fp32 (relative error ``F32_EVAL_REL``) and
    rounds once to bf16 (half an ulp, ``BF16_HALF_ULP_REL``).  With ``P`` the
    perturbation bound of :func:`h_perturbation_bound`, the fp32 value lies
    within ``P`` of ``h64`` and the stored one within
    ``P + (F32_EVAL_REL + BF16_HALF_ULP_REL) (|h64| + P) + 1e-6``."""
    g, u = ref["g"], ref["u"]
    dg = tolerance(ref["Ag"])
    du = tolerance(ref["Au"])
    prop = h_perturbation_bound(g, u, dg, du)
    return prop + (F32_EVAL_REL + BF16_HALF_ULP_REL) * (np.abs(ref["h64"]) + prop) + 1e-6


def ffn_y_bound(ref: dict, down: dict, weights_bf16: bool = False) -> np.ndarray:
    """Allowed ``|y_gpu - y_ref|`` end to end, with ``y_ref = hb Wd^T``.

    The kernel's down projection is within the matmul tolerance of
    ``h_gpu Wd^T`` *for its own input*: ``1e-3 |h_gpu| |Wd|^T + 1e-6``.  With
    ``dh = ffn_h_bound + |h64 - hb|`` bounding ``|h_gpu - hb|`` element-wise:
    ``|h_gpu Wd^T - hb Wd^T| <= dh |Wd|^T`` and ``|h_gpu| <= |hb| + dh``, so
    ``|y_gpu - y_ref| <= 1e-3 A_d + 1e-6 + (1 + 1e-3) dh |Wd|^T``."""
    hb = bf16_to_f32(ref["hb"]).astype(np.float64)
    dh = ffn_h_bound(ref) + np.abs(ref["h64"] - hb)
    wd = dequant_f32(down["packed"], down["scales"], down["biases"], down["meta"], down["symmetric"], down["K"])
    if weights_bf16:
        wd = bf16_to_f32(f32_to_bf16_rne(wd))
    wd = np.abs(wd.astype(np.float64))
    lead = dh.shape[:-1]
    prop = dh.reshape(-1, dh.shape[-1]) @ wd.T
    return tolerance(ref["Ad"]) + (1.0 + 1e-3) * prop.reshape(*lead, wd.shape[0])


# --------------------------------------------------------------------------
# Metadata: symmetric-bias check and sign packer
# --------------------------------------------------------------------------


def symmetric_mismatches(scales: np.ndarray, biases: np.ndarray, meta: str) -> int:
    """Groups of an affine tensor whose stored bias cannot be replaced by the
    derived ``-scale/2`` (Higgs PR #212, "What": validate symmetric Q1
    metadata; "Walkthrough": loaders compact exact symmetric biases).

    A group matches when scale and bias are finite and each code dequantises to
    the same float32 value (bit for bit) with the stored bias as with
    ``-0.5 * scale`` -- the literal formula of :func:`dequant_f32` taken both
    ways.  Returns the number of groups that do not match."""
    s = meta_to_f32(scales, meta)
    b = meta_to_f32(biases, meta)
    d = (np.float32(-0.5) * s).astype(np.float32)
    same = np.isfinite(s) & np.isfinite(b)
    with np.errstate(over="ignore", invalid="ignore"):
        for code in (0.0, 1.0):
            prod = (s * np.float32(code)).astype(np.float32)
            with_bias = (prod + b).astype(np.float32)
            derived = (prod + d).astype(np.float32)
            same &= with_bias.view(np.uint32) == derived.view(np.uint32)
    return int((~same).sum())


def pack_signs(dense_bits: np.ndarray, dense: str, meta: str):
    """Dense ``[N, K]`` bf16/f16 weights -> a symmetric packed tensor (Cactus
    PR #775, commit notes: groups holding exactly {-s, +s} repack to sign bits
    with zero error; rMLX issue #207: bit 0 -> -s_g, bit 1 -> +s_g, 32 weights
    per word LSB first).

    Per group of 128 weights: ``scale = round_meta(2 * max|w|)`` (NaNs left
    out of the maximum), ``bit = (w > 0)``.  The group is exact when
    dequantising the result to the dense dtype gives back every weight's bit
    pattern and the group holds no NaN.  Returns ``(packed uint32 [N, K/32],
    scales uint16 bits [N, K/128], number of inexact groups)``."""
    dense_bits = np.asarray(dense_bits, dtype=np.uint16)
    N, K = dense_bits.shape
    G = K // GROUP
    w = meta_to_f32(dense_bits, dense)              # the same decoders serve both 16-bit types
    mag = np.abs(w).reshape(N, G, GROUP)
    has_nan = np.isnan(mag).any(axis=2)
    amax = np.fmax.reduce(mag, axis=2, initial=np.float32(0.0)).astype(np.float32)
    with np.errstate(over="ignore"):
        scale_bits = round_to((np.float32(2.0) * amax).astype(np.float32), meta)
    bits = (w > 0).astype(np.uint32)                # NaN > 0 is False
    packed = np.zeros((N, K // 32), dtype=np.uint32)
    for i in range(32):                             # weight 32j + i -> bit i of word j
        packed |= bits[:, i::32] << np.uint32(i)
    with np.errstate(invalid="ignore"):
        back = dequantize(packed, scale_bits, None, meta, True, K, dense)
    exact = (back.reshape(N, G, GROUP) == dense_bits.reshape(N, G, GROUP)).all(axis=2) & ~has_nan
    return packed, scale_bits, int((~exact).sum())
