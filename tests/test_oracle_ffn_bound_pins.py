"""Pins for the oracle's FFN error bounds (``h_perturbation_bound``,
``ffn_h_bound``, ``ffn_y_bound``).

The bounds decide pass/fail of the fused FFN (Higgs PR #212, "What": fused
dense-FFN operations; gate and up, ``SiLU(gate) * up``, down).  Each pin ties
them to something other than their own formula:

* soundness by brute force -- the largest deviation reachable inside the
  allowed input box, evaluated at 40 significant digits with mpmath (which
  shares nothing with the oracle's NumPy SiLU), never exceeds the bound;
* tightness -- for small perturbations the bound is within 0.1 % of that
  largest deviation, so no term is doubled or superfluous;
* hand-worked cases whose bound and worst case were worked out by hand;
* planted mistakes (a dropped gate, up, curvature or rounding term, a doubled
  ulp, a signed or transposed down matrix), each caught by at least one pin.
"""
import itertools
from fractions import Fraction

import mpmath
import numpy as np
import pytest

import oracle as O
import q1_synth as S

mpmath.mp.dps = 40


def _silu_mp(z):
    z = mpmath.mpf(z)
    return z / (1 + mpmath.exp(-z))


def _worst_h_deviation(g, u, dg, du, n=81):
    """max |SiLU(g') u' - SiLU(g) u| over g' in [g-dg, g+dg] (n grid points
    plus the endpoints; SiLU is smooth, the grid plus endpoints finds the
    maximum of the sampled problems below to well within the tolerances
    used) and u' in {u-du, u+du} (the expression is linear in u')."""
    base = _silu_mp(g) * mpmath.mpf(u)
    best = mpmath.mpf(0)
    for i in range(n + 1):
        gp = mpmath.mpf(g) - mpmath.mpf(dg) + 2 * mpmath.mpf(dg) * i / n
        sg = _silu_mp(gp)
        for up in (mpmath.mpf(u) - mpmath.mpf(du), mpmath.mpf(u) + mpmath.mpf(du)):
            best = max(best, abs(sg * up - base))
    return float(best)


def _cases():
    rng = np.random.default_rng(31)
    z0 = -1.2784645427610738  # SiLU'(z0) = 0: only the curvature term bounds the gate part there
    out = [(0.0, 8.0, 1.0, 1e-6), (z0, 10.0, 0.5, 1e-6), (z0, -3.0, 2.0, 0.3), (20.0, 0.05, 1e-6, 1e-6),
           (-30.0, 5.0, 3.0, 0.1), (2.4, 1.0, 1e-3, 2.0), (0.0, 0.0, 0.1, 0.1), (-5.0, 1e4, 1e-4, 1e-4)]
    for _ in range(40):
        out.append((float(rng.uniform(-12, 12)), float(rng.uniform(-20, 20)),
                    float(10.0 ** rng.uniform(-6, 0.5)), float(10.0 ** rng.uniform(-6, 0.5))))
    return out


# ---------------------------------------------------------------- SiLU facts the bound relies on

def test_silu_curvature_constant():
    """max |SiLU''| = 1/2, reached at z = 0 (second derivative by mpmath's
    numerical differentiation on a dense grid, plus the tails)."""
    zs = list(np.linspace(-12, 12, 481)) + [-40.0, -25.0, 25.0, 40.0]
    vals = [abs(float(mpmath.diff(_silu_mp, z, 2))) for z in zs]
    assert max(vals) <= O.SILU_CURVATURE * (1 + 1e-12)
    assert abs(float(mpmath.diff(_silu_mp, 0, 2)) - 0.5) < 1e-30


def test_h_bound_constants_by_hand():
    # half an ulp of bf16: the spacing just above 1.0 is 2^-7
    assert O.BF16_HALF_ULP_REL == 2.0 ** -8
    assert O.F32_EVAL_REL <= 2.0 ** -18 and O.F32_EVAL_REL >= 8 * 2.0 ** -24


# ---------------------------------------------------------------- h: soundness and tightness

@pytest.mark.parametrize("case", range(48))
def test_h_perturbation_bound_is_sound(case):
    g, u, dg, du = _cases()[case]
    bound = float(O.h_perturbation_bound(np.array(g), np.array(u), np.array(dg), np.array(du)))
    worst = _worst_h_deviation(g, u, dg, du)
    assert worst <= bound * (1 + 1e-9) + 1e-300, (g, u, dg, du, worst, bound)


@pytest.mark.parametrize("g,u", [(0.7, 3.0), (-2.0, -5.0), (5.0, 0.25), (-0.3, 12.0), (1.5, -0.8)])
def test_h_perturbation_bound_is_tight_for_small_perturbations(g, u):
    dg = du = 1e-7 * max(1.0, abs(u))
    bound = float(O.h_perturbation_bound(np.array(g), np.array(u), np.array(dg), np.array(du)))
    worst = _worst_h_deviation(g, u, dg, du)
    assert bound <= worst * (1 + 1e-3), (bound, worst)


def test_h_perturbation_bound_hand_case_gate_only():
    """g = 0, u = 8, dg = 1, du = 0: SiLU(0) = 0 and SiLU'(0) = 1/2, so the
    bound is (1/2 + 1/2 * 1) * 1 * 8 = 8; the largest reachable value is
    SiLU(1) * 8 = 8 / (1 + e^-1) = 5.8484686...  (by hand)."""
    b = float(O.h_perturbation_bound(np.array(0.0), np.array(8.0), np.array(1.0), np.array(0.0)))
    assert b == 8.0
    assert abs(_worst_h_deviation(0.0, 8.0, 1.0, 0.0) - 5.848468629040039) < 1e-12


def test_h_perturbation_bound_hand_case_up_only():
    """dg = 0: the bound is |SiLU(g)| du; at g = 2, du = 0.5 that is
    2 / (1 + e^-2) * 0.5 = 0.880797077977882... (by hand), reached at u' = u +- du."""
    b = float(O.h_perturbation_bound(np.array(2.0), np.array(-3.0), np.array(0.0), np.array(0.5)))
    assert abs(b - 0.8807970779778823) < 1e-15


def test_ffn_h_bound_rounding_tie():
    """h64 = 1 + 2^-8 exactly (a bf16 tie between 1 and 1 + 2^-7), perturbations
    of 1e-6: a kernel value within them of the tie may round either way, so an
    error of 2^-8 is reachable and the bound must cover it -- and with a
    doubled ulp it would be about twice that (hand-worked)."""
    g = 20.0
    u = (1 + 2.0 ** -8) / float(_silu_mp(g))
    ref = {"g": np.array([g]), "u": np.array([u]), "Ag": np.array([0.0]), "Au": np.array([0.0]),
           "h64": np.array([float(_silu_mp(g) * mpmath.mpf(u))])}
    b = float(O.ffn_h_bound(ref)[0])
    reachable = 2.0 ** -8
    assert b >= reachable
    # P ~ 20 * 1e-6 + SiLU'(20) * 1e-6 * u, then (2^-8 + 2^-20) (1 + 2^-8 + P) + 1e-6
    assert b <= reachable * (1 + 2.0 ** -8) + 2.0 ** -20 * 1.01 + 2.2e-5 + 1e-6, b


def test_ffn_h_bound_covers_rounded_corners():
    """Brute force of the whole h pipeline on random cases: every corner value
    of (g', u') rounded to bf16, and the rounding of the kernel's fp32
    evaluation error in both directions, stays within ffn_h_bound."""
    rng = np.random.default_rng(5)
    for _ in range(60):
        g = float(rng.uniform(-8, 8))
        u = float(rng.uniform(-6, 6))
        Ag, Au = float(10 ** rng.uniform(-3, 2)), float(10 ** rng.uniform(-3, 2))
        ref = {"g": np.array([g]), "u": np.array([u]), "Ag": np.array([Ag]), "Au": np.array([Au]),
               "h64": np.array([float(_silu_mp(g) * mpmath.mpf(u))])}
        b = float(O.ffn_h_bound(ref)[0])
        dg, du = 1e-3 * Ag + 1e-6, 1e-3 * Au + 1e-6
        for sg, su, se in itertools.product((-1, 1), (-1, 1), (-1, 1)):
            v = float(_silu_mp(g + sg * dg) * (u + su * du)) * (1 + se * 2.0 ** -21)
            vb = float(O.bf16_to_f32(O.f32_to_bf16_rne(np.array([v], dtype=np.float32)))[0])
            assert abs(vb - ref["h64"][0]) <= b, (g, u, Ag, Au)


# ---------------------------------------------------------------- y: soundness and exactness at the corner

def _tiny_ffn(seed, aligned):
    rng = np.random.Generator(np.random.PCG64(seed))
    I, Hout = 128, 3
    wd = S.draw_weight(rng, Hout, I, "bf16", False)
    g = rng.normal(0, 2, size=(1, I))
    u = rng.normal(0, 2, size=(1, I))
    h64 = np.array([[float(_silu_mp(a) * mpmath.mpf(b)) for a, b in zip(g[0], u[0])]])
    if aligned:
        # make sign(h) equal sign(Wd[0, j]) so that one corner reaches the bound
        wdf = O.dequant_f32(wd.packed, wd.scales, wd.biases, "bf16", False, I)[0].astype(np.float64)
        flip = np.sign(h64[0]) != np.sign(wdf)
        u[0, flip] = -u[0, flip]
        h64[0, flip] = -h64[0, flip]
    hb = O.f32_to_bf16_rne(h64.astype(np.float32))
    Ag = np.abs(rng.normal(0, 20, size=(1, I)))
    Au = np.abs(rng.normal(0, 20, size=(1, I)))
    wdd = dict(packed=wd.packed, scales=wd.scales, biases=wd.biases, meta="bf16", symmetric=False, K=I)
    y, Ad = O.qmm_ref(hb, **wdd)
    ref = {"g": g, "u": u, "Ag": Ag, "Au": Au, "h64": h64, "hb": hb, "y": y, "Ad": Ad}
    return ref, wdd


def _corner_deviation(ref, wdd, signs, n):
    """|y_gpu - y_ref| for the kernel input h' = hb + signs * dh (dh the
    element-wise allowance) and a down product that errs by its full
    tolerance 1e-3 |h'| |Wd| + 1e-6 in the same direction -- in exact
    rational arithmetic."""
    hb = O.bf16_to_f32(ref["hb"]).astype(np.float64)[0]
    dh = O.ffn_h_bound(ref)[0] + np.abs(ref["h64"][0] - hb)
    wd = O.dequant_f32(wdd["packed"], wdd["scales"], wdd["biases"], wdd["meta"], wdd["symmetric"], wdd["K"])[n]
    hp = [Fraction(float(a)) + s * Fraction(float(d)) for a, s, d in zip(hb, signs, dh)]
    shift = sum((p - Fraction(float(a))) * Fraction(float(w)) for p, a, w in zip(hp, hb, wd))
    own = Fraction(1, 1000) * sum(abs(p) * abs(Fraction(float(w))) for p, w in zip(hp, wd)) + Fraction(1, 10 ** 6)
    return float(abs(shift) + own)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_ffn_y_bound_reached_at_the_aligned_corner(seed):
    ref, wdd = _tiny_ffn(seed, aligned=True)
    yb = O.ffn_y_bound(ref, wdd)[0]
    wd = O.dequant_f32(wdd["packed"], wdd["scales"], wdd["biases"], "bf16", False, wdd["K"])[0]
    signs = np.where(wd >= 0, 1, -1)
    dev = _corner_deviation(ref, wdd, signs, 0)
    # the bound's only slack is the factor (1 + 1e-3) on the propagated part
    prop = yb[0] - O.tolerance(ref["Ad"])[0, 0]
    assert dev <= yb[0] * (1 + 1e-12)
    assert dev >= yb[0] - 1.1e-3 * prop - 1e-12 * yb[0], (dev, yb[0])


@pytest.mark.parametrize("seed", [4, 5])
def test_ffn_y_bound_covers_random_corners(seed):
    ref, wdd = _tiny_ffn(seed, aligned=False)
    yb = O.ffn_y_bound(ref, wdd)[0]
    rng = np.random.default_rng(seed)
    for n in range(3):
        wd = O.dequant_f32(wdd["packed"], wdd["scales"], wdd["biases"], "bf16", False, wdd["K"])[n]
        worst = np.where(wd >= 0, 1, -1)
        for signs in [worst, -worst] + [rng.choice([-1, 1], size=wdd["K"]) for _ in range(6)]:
            assert _corner_deviation(ref, wdd, signs, n) <= yb[n] * (1 + 1e-12)


# ---------------------------------------------------------------- planted mistakes

def _bound_pins_pass():
    try:
        for c in range(48):
            test_h_perturbation_bound_is_sound(c)
        for g, u in [(0.7, 3.0), (-2.0, -5.0), (5.0, 0.25), (-0.3, 12.0), (1.5, -0.8)]:
            test_h_perturbation_bound_is_tight_for_small_perturbations(g, u)
        test_ffn_h_bound_rounding_tie()
        test_ffn_h_bound_covers_rounded_corners()
        for seed in (1, 2, 3):
            test_ffn_y_bound_reached_at_the_aligned_corner(seed)
        for seed in (4, 5):
            test_ffn_y_bound_covers_random_corners(seed)
    except AssertionError:
        return False
    return True


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(O.q1_oracle, name, fn)
    monkeypatch.setattr(O, name, fn)


_orig_hpb = O.h_perturbation_bound
_orig_hb = O.ffn_h_bound
_orig_yb = O.ffn_y_bound


def test_unpatched_bounds_pass_pins():
    assert _bound_pins_pass()


def _hpb(gate=True, up=True, curv=True):
    def f(g, u, dg, du):
        g, u, dg, du = (np.asarray(a, dtype=np.float64) for a in (g, u, dg, du))
        slope = np.abs(O.silu_grad(g)) + (O.SILU_CURVATURE * dg if curv else 0.0)
        return (slope * dg * (np.abs(u) + du) if gate else 0.0) + (np.abs(O.silu(g)) * du if up else 0.0)
    return f


@pytest.mark.parametrize("kw", [dict(gate=False), dict(up=False), dict(curv=False)])
def test_planted_dropped_propagation_term_is_caught(monkeypatch, kw):
    _patch(monkeypatch, "h_perturbation_bound", _hpb(**kw))
    assert not _bound_pins_pass()


def test_planted_dropped_rounding_term_is_caught(monkeypatch):
    def hb(ref):
        p = _orig_hpb(ref["g"], ref["u"], O.tolerance(ref["Ag"]), O.tolerance(ref["Au"]))
        return p + O.F32_EVAL_REL * (np.abs(ref["h64"]) + p) + 1e-6
    _patch(monkeypatch, "ffn_h_bound", hb)
    assert not _bound_pins_pass()


def test_planted_doubled_ulp_is_caught(monkeypatch):
    monkeypatch.setattr(O.q1_oracle, "BF16_HALF_ULP_REL", 2.0 ** -7)
    monkeypatch.setattr(O, "BF16_HALF_ULP_REL", 2.0 ** -7)
    assert not _bound_pins_pass()


def test_planted_doubled_gate_term_is_caught(monkeypatch):
    _patch(monkeypatch, "h_perturbation_bound", lambda g, u, dg, du: _orig_hpb(g, u, 2 * np.asarray(dg), du))
    assert not _bound_pins_pass()


def test_planted_y_without_propagation_is_caught(monkeypatch):
    _patch(monkeypatch, "ffn_y_bound", lambda ref, down, weights_bf16=False: O.tolerance(ref["Ad"]))
    assert not _bound_pins_pass()


def test_planted_y_with_signed_down_matrix_is_caught(monkeypatch):
    def yb(ref, down, weights_bf16=False):
        hb = O.bf16_to_f32(ref["hb"]).astype(np.float64)
        dh = _orig_hb(ref) + np.abs(ref["h64"] - hb)
        wd = O.dequant_f32(down["packed"], down["scales"], down["biases"], down["meta"], down["symmetric"],
                           down["K"]).astype(np.float64)
        return O.tolerance(ref["Ad"]) + np.abs(dh @ wd.T)
    _patch(monkeypatch, "ffn_y_bound", yb)
    assert not _bound_pins_pass()
