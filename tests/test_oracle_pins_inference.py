"""Pins of the oracle's inference-side functions: the decode GEMV on the packed format and the AWQ
pre-scale hook. Each is checked against something other than itself: an independent bit-level
reader of the format, the dequant path where the two readings coincide, exact power-of-two
scaling, and the objective identity that defines the pre-scaled importance."""

import numpy as np
import pytest

from oracle import aaac_ref as ref

from tests.test_oracle_pins import _bf16_matrix


def _packed(rng, R, C, g, S, n, iters=1):
    W = _bf16_matrix(rng, R, C)
    I = rng.random(C) + 0.05
    out = ref.quantize(W, I, g, S, n, iters=iters)
    fin = out["final"]
    p = ref.pack(W, fin["codes"], fin["sel"], out["tables_bf16"], g, S)
    return W, p


def _bitlevel_decode(code_bytes, scales, bitmap, tables_u16, R, C, g, S):
    """Reads every weight with explicit bit operations, one at a time (tiny inputs only)."""
    def bf(bits):
        return float(np.array([bits << 16], dtype=np.uint32).view(np.float32)[0])
    cb = np.asarray(code_bytes, dtype=np.uint8).reshape(R, C // 2)
    sc = np.asarray(scales, dtype=np.uint16).reshape(R, C // g)
    out = np.zeros((R, C))
    for r in range(R):
        for c in range(C):
            byte = int(cb[r, c // 2])
            q = (byte >> 4) if (c & 1) else (byte & 15)
            word = int(sc[r, c // g])
            if bitmap is None:
                sig = word >> 15
            else:
                i = (r * C + c) // S
                sig = (int(bitmap[i >> 3]) >> (i & 7)) & 1
            out[r, c] = bf(word & 0x7FFF) * bf(int(tables_u16[sig][q]))
    return out


@pytest.mark.parametrize("g,S,n", [(128, 128, 16), (128, 16, 16), (16, 16, 15)])
def test_gemv_matches_bitlevel_reader(g, S, n):
    rng = np.random.default_rng(40 + g + S + n)
    R, C = 5, 256
    W, p = _packed(rng, R, C, g, S, n)
    x = ref.bf16_round(rng.standard_normal((3, C)))
    Wd = _bitlevel_decode(p["codes"], p["scales"], p["bitmap"], p["tables"], R, C, g, S)
    y, a = ref.gemv(p["codes"], p["scales"], p["bitmap"], p["tables"], R, C, g, S, x)
    want = np.array([[sum(Wd[r, c] * x[b, c] for c in range(C)) for r in range(R)]
                     for b in range(3)])
    assert np.allclose(y, want, rtol=1e-13, atol=1e-300)
    assert np.all(a >= np.abs(y))
    # the decoded weights are the packed approximation of W: within a group's quantization error
    assert np.max(np.abs(Wd - W)) <= np.max(np.abs(W))


def test_gemv_equals_dequant_product_when_no_rounding_occurs():
    # scales that are powers of two make |s| T~ bf16-exact, so dequant's rounding is the identity
    rng = np.random.default_rng(44)
    R, C, g, S, n = 4, 128, 32, 32, 16
    W, p = _packed(rng, R, C, g, S, n)
    sc = p["scales"].copy()
    pow2 = (rng.integers(120, 130, size=sc.shape).astype(np.uint16) << 7)
    sc = (sc & 0x8000) | pow2
    x = ref.bf16_round(rng.standard_normal((2, C)))
    W_hat = ref.dequant(p["codes"], sc, p["bitmap"], p["tables"], R, C, g, S)
    y, _ = ref.gemv(p["codes"], sc, p["bitmap"], p["tables"], R, C, g, S, x)
    assert np.array_equal(y, x @ W_hat.T)


def test_awq_prescale_exact_for_power_of_two_scales():
    rng = np.random.default_rng(45)
    W = _bf16_matrix(rng, 6, 64)
    a = np.ldexp(1.0, rng.integers(-6, 7, size=64)).astype(np.float32)
    I = (rng.random(64) + 0.1).astype(np.float32)
    Ws, Is = ref.awq_prescale(W, a, I)
    assert np.array_equal(Ws, W * a)
    assert np.array_equal(Is.astype(np.float64), I.astype(np.float64) / a.astype(np.float64) ** 2)
    Ws1, Is1 = ref.awq_prescale(W, np.ones(64, np.float32), I)
    assert np.array_equal(Ws1, W) and np.array_equal(Is1, I)


def test_awq_prescaled_importance_is_energy_of_scaled_inputs():
    # I / a^2 is the importance of the inputs x / a that the scaled matrix sees
    rng = np.random.default_rng(46)
    X = rng.standard_normal((50, 32)).astype(np.float32)
    a = np.ldexp(1.0, rng.integers(-3, 4, size=32)).astype(np.float32)
    I = ref.importance(X).astype(np.float32)
    _, Is = ref.awq_prescale(np.zeros((1, 32)), a, I)
    direct = ref.importance(X / a)
    assert np.allclose(Is, direct, rtol=2e-7)


def test_awq_prescaled_error_equals_original_space_error():
    # quantizing (W a, I / a^2) and mapping back by 1 / a gives the same weighted error in the
    # original space: the a^2 in the importance is what makes the two objectives agree
    rng = np.random.default_rng(47)
    R, C, g, S, n = 4, 128, 32, 32, 16
    W = _bf16_matrix(rng, R, C)
    I = rng.random(C) + 0.1
    a = np.ldexp(1.0, rng.integers(-2, 3, size=C)).astype(np.float32)   # keeps W a exact
    Ws, Is = ref.awq_prescale(W, a, I.astype(np.float32))
    Is = Is.astype(np.float64)
    out = ref.quantize(Ws, Is, g, S, n, iters=2)
    fin = out["final"]
    Tt = [np.asarray(t, dtype=np.float64) for t in out["tables_bf16"]]
    scaled = ref.total_error(Ws, Is, fin["codes"], fin["sel"], Tt[0], Tt[1], g, S)
    s = np.repeat(ref.group_scales(Ws, g), g, axis=1)
    sig = np.repeat(fin["sel"], S, axis=1)
    w_hat_scaled = s * np.stack(Tt)[sig, fin["codes"]]
    orig = np.sum(I.astype(np.float32).astype(np.float64) * (W - w_hat_scaled / a) ** 2)
    assert scaled == pytest.approx(orig, rel=1e-12)
    # a slip (importance divided by a instead of a^2) breaks the identity
    wrong = ref.total_error(Ws, Is * a, fin["codes"], fin["sel"], Tt[0], Tt[1], g, S)
    assert wrong != pytest.approx(orig, rel=1e-6)


def _bf16_of_fraction(x):
    """bf16 value (as a float) of an exact rational, ties to even, by exact rational arithmetic:
    the quantum of x's binade (8 significant bits; 2^-133 below 2^-126), the quotient rounded by
    Fraction's round-half-even, overflow past the largest finite value to infinity."""
    from fractions import Fraction
    if x == 0:
        return 0.0
    ax = abs(x)
    e = ax.numerator.bit_length() - ax.denominator.bit_length()
    if Fraction(2) ** e > ax:
        e -= 1                                     # now 2^e <= ax < 2^(e+1)
    e = max(e, -126)
    q = Fraction(2) ** (e - 7)
    r = round(ax / q) * q
    if r >= Fraction(2) ** 128:
        return float("inf") if x > 0 else float("-inf")
    return float(r) if x > 0 else -float(r)


def test_awq_prescale_matches_exact_rationals_for_any_scale():
    """Non-power-of-two scales (AAAC summary §4, reading R15): W_scaled is the bf16 rounding of the
    exact product w * a, and I_scaled the fp32 rounding of the fp64 rounding of the exact quotient
    I / a^2, both computed here with Python Fractions (float(Fraction) rounds correctly). Slips
    such as squaring a in fp32, dividing in fp32 or rounding the product to fp32 first disagree
    with this on some entries."""
    from fractions import Fraction
    rng = np.random.default_rng(48)
    R, C = 8, 512
    W = _bf16_matrix(rng, R, C)
    a = np.exp(rng.uniform(-3, 3, size=C)).astype(np.float32)
    I = (np.exp(rng.uniform(-8, 8, size=C))).astype(np.float32)
    Ws, Is = ref.awq_prescale(W, a, I)
    fa = [Fraction(float(v)) for v in a]
    want_W = np.array([[_bf16_of_fraction(Fraction(float(W[r, c])) * fa[c]) for c in range(C)]
                       for r in range(R)])
    assert np.array_equal(Ws, want_W)
    want_I = np.array([np.float32(float(Fraction(float(I[c])) / (fa[c] * fa[c])))
                       for c in range(C)], dtype=np.float32)
    assert np.array_equal(Is, want_I)
    # the pin has teeth: plausible slips each disagree somewhere
    a2_fp32 = (a * a).astype(np.float64)                      # a^2 rounded to fp32 first
    assert not np.array_equal((I.astype(np.float64) / a2_fp32).astype(np.float32), want_I)
    assert not np.array_equal(I / (a * a), want_I)            # all in fp32
    # products whose rounding to fp32 first would land on a bf16 rounding midpoint: the oracle
    # must round the exact product once (found by search, then checked against the rationals)
    w = ref.bf16_round(rng.standard_normal(1 << 20))
    av = np.exp(rng.uniform(-3, 3, size=1 << 20)).astype(np.float32)
    p64 = w * av.astype(np.float64)
    twice = ref.bf16_round(p64.astype(np.float32).astype(np.float64)) != ref.bf16_round(p64)
    idx = np.flatnonzero(twice)[:32]
    assert idx.size > 0
    Wd, _ = ref.awq_prescale(w[idx][None, :], av[idx])
    want_d = [_bf16_of_fraction(Fraction(float(w[i])) * Fraction(float(av[i]))) for i in idx]
    assert np.array_equal(Wd[0], np.array(want_d))
