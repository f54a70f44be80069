"""Pins of the oracle's SGD update against exact rational arithmetic.

Passage followed: explainer "LCT paper - Lossless Huffman coding of BF16
training tensors", paragraph on training traffic: the plain SGD update
W_{t+1} = W_t - eta * M_t, naive form = decode both tensors, update, re-encode.
Read as r = fmaf(-eta, f32(m), f32(w)) with one rounding to fp32, then
round-to-nearest-even to BF16; a NaN result is written as 0x7FC0.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth


def f32_of(u):
    return float(np.array([u], np.uint32).view(np.float32)[0])


def round_exact(q: Fraction, p: int, emin: int, emax: int):
    """Round a nonzero rational to the binary format with p significand bits,
    exponent range [emin, emax], nearest-even; returns a float (or +-inf)."""
    sign = -1 if q < 0 else 1
    a = abs(q)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    assert Fraction(2) ** E <= a < Fraction(2) ** (E + 1)
    E = max(E, emin)
    ulp = Fraction(2) ** (E - (p - 1))
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    v = fl * ulp
    if v >= Fraction(2) ** (emax + 1):
        return sign * float("inf")
    return sign * float(v)


def exact_fmaf(a: float, b: float, c: float):
    """IEEE fused multiply-add in binary32 from exact rationals (finite inputs)."""
    q = Fraction(a) * Fraction(b) + Fraction(c)
    if q == 0:
        # an exact zero is -0 only when the product and c are zeros of sign -
        prod_zero = a == 0 or b == 0
        prod_neg = bool(np.signbit(a)) != bool(np.signbit(b))
        return -0.0 if (prod_zero and c == 0 and prod_neg and np.signbit(c)) else 0.0
    return round_exact(q, 24, -126, 127)


def random_f32(g, n):
    """Finite float32 values covering normals, subnormals, zeros and the top range."""
    u = g.integers(0, 1 << 32, n, dtype=np.uint64).astype(np.uint32)
    u[g.random(n) < 0.1] &= 0x807FFFFF          # subnormals and zeros
    u[g.random(n) < 0.05] &= 0x80000000         # signed zeros
    f = u.view(np.float32)
    bad = ~np.isfinite(f)
    f[bad] = np.float32(1.5)
    return f


def test_fmaf_matches_exact_rational(orc):
    g = np.random.default_rng(17)
    n = 40000
    a, b, c = random_f32(g, n), random_f32(g, n), random_f32(g, n)
    # also the update's own operand shapes: BF16 w and m, -eta
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    wf = (w.astype(np.uint32) << 16).view(np.float32)
    mf = (m.astype(np.uint32) << 16).view(np.float32)
    eta = np.float32(-1e-3)
    cases = list(zip(a, b, c)) + [(eta, y, x) for x, y in zip(wf, mf)]
    for x, y, z in cases:
        got = orc.fmaf(float(x), float(y), float(z))
        want = exact_fmaf(float(x), float(y), float(z))
        if want == 0:
            assert got == 0 and np.signbit(got) == np.signbit(want), (x, y, z)
        else:
            assert got == want, (x, y, z)


def test_fmaf_special_values(orc):
    inf, nan = float("inf"), float("nan")
    assert orc.fmaf(inf, 0.0, 1.0) != orc.fmaf(inf, 0.0, 1.0)      # inf*0 -> NaN
    assert orc.fmaf(2.0, inf, -inf) != orc.fmaf(2.0, inf, -inf)    # inf - inf -> NaN
    assert orc.fmaf(-1e-3, 1.0, inf) == inf
    assert orc.fmaf(1.0, nan, 1.0) != orc.fmaf(1.0, nan, 1.0)
    # signed zeros under round-to-nearest
    assert np.signbit(orc.fmaf(-0.0, 1.0, -0.0)) and not np.signbit(orc.fmaf(-0.0, 1.0, 0.0))
    # overflow of a finite fma to inf
    assert orc.fmaf(3.0e38, 2.0, 0.0) == inf


def test_rne_matches_exact_rounding_and_torch(orc):
    g = np.random.default_rng(23)
    u = g.integers(0, 1 << 32, 60000, dtype=np.uint64).astype(np.uint32)
    # halfway cases and near-overflow values
    u[:2000] = (u[:2000] & 0xFFFF0000) | 0x8000
    u[2000:2100] = 0x7F7F8000 + np.arange(100, dtype=np.uint32)
    f = u.view(np.float32)
    fin = np.isfinite(f)
    got = np.array([orc.rne_bf16(float(x)) for x in f], np.uint16)
    # torch's CPU cast is round-to-nearest-even on finite values
    ref = torch.from_numpy(f[fin].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got[fin], ref)
    # exact rational rounding to 8 significand bits
    for x, gbits in zip(f[fin][:20000], got[fin][:20000]):
        if x == 0:
            assert gbits == (0x8000 if np.signbit(x) else 0)
            continue
        want = round_exact(Fraction(float(x)), 8, -126, 127)
        assert f32_of(int(gbits) << 16) == want
    # every NaN is written as the canonical quiet NaN
    assert (got[np.isnan(f)] == 0x7FC0).all()
    assert orc.rne_bf16(float("inf")) == 0x7F80 and orc.rne_bf16(float("-inf")) == 0xFF80


def test_eta_zero_keeps_compressed_w(orc):
    """With eta = 0, finite M and W free of NaN and -0, W' is W: the compressed
    bytes must come back identical."""
    g = np.random.default_rng(29)
    n = 3 * 4096 + 11
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    w[w == 0x8000] = 0
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    cw = orc.codebook_build(0, 0.02, 0.0, w)
    cm = orc.codebook_build(0, 1e-3, 0.0, m)
    for B, cap in [(4096, 25), (4096, 2)]:
        tw, tm = orc.encode(cw, w, B, cap), orc.encode(cm, m, B, cap)
        o = orc.sgd(cw, tw, cm, tm, 0.0)
        for k in ["sf", "pay", "cnt", "obase"]:
            assert np.array_equal(getattr(o, k), getattr(tw, k)), k
        assert np.array_equal(o.ovf[:o.spilled], tw.ovf[:tw.spilled])


def test_compressed_sgd_is_naive_round_trip(orc):
    """lcto_sgd (block by block) equals decode -> element update -> encode of the
    whole tensor, including spills on both inputs and the output."""
    g = np.random.default_rng(31)
    n = 5 * 2048 + 100
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1.0, n))
    m[:50] = [0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001] * 10     # specials in M
    cw = orc.codebook_build(1, 0.02, 0.0, w)
    cm = orc.codebook_build(0, 1.0, 0.0, m)
    eta = 0.05
    for cap in [25, 3, 2]:
        tw, tm = orc.encode(cw, w, 2048, cap), orc.encode(cm, m, 2048, cap)
        o = orc.sgd(cw, tw, cm, tm, eta)
        dense = orc.sgd_dense(orc.decode(cw, tw), orc.decode(cm, tm), eta)
        ref = orc.encode(cw, dense, 2048, cap)
        for k in ["sf", "pay", "cnt", "obase"]:
            assert np.array_equal(getattr(o, k), getattr(ref, k)), (cap, k)
        assert np.array_equal(o.ovf[:o.spilled], ref.ovf[:ref.spilled])
        assert np.array_equal(orc.decode(cw, o), dense)
        # element update against exact arithmetic on a sample
        for i in range(0, n, 97):
            wi, mi = f32_of(int(w[i]) << 16), f32_of(int(m[i]) << 16)
            if not (np.isfinite(wi) and np.isfinite(mi)):
                continue
            r = exact_fmaf(float(np.float32(-eta)), mi, wi)
            if r != 0 and np.isfinite(r):
                assert f32_of(int(dense[i]) << 16) == round_exact(Fraction(r), 8, -126, 127)


def test_non_finite_learning_rate_gives_the_canonical_nan_or_infinities(orc):
    """eta = NaN: every W' is the canonical quiet NaN 0x7FC0.  eta = +inf:
    W' = fmaf(-inf, m, w) is -inf where m > 0, +inf where m < 0 and NaN
    where m is zero (inf * 0); the compressed step decodes to exactly that."""
    g = np.random.default_rng(31)
    n = 2 * 4096 + 5
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    m[::7] = 0
    m[1::7] = 0x8000
    cw = orc.codebook_build(0, 0.02, 0.0, w)
    cm = orc.codebook_build(0, 1e-3, 0.0, m)
    tw, tm = orc.encode(cw, w, 4096, 25), orc.encode(cm, m, 4096, 25)
    y = orc.decode(cw, orc.sgd(cw, tw, cm, tm, float("nan")))
    assert (y == 0x7FC0).all()
    y = orc.decode(cw, orc.sgd(cw, tw, cm, tm, float("inf")))
    mf = (m.astype(np.uint32) << 16).view(np.float32)
    want = np.where(mf > 0, 0xFF80, np.where(mf < 0, 0x7F80, 0x7FC0)).astype(np.uint16)
    assert np.array_equal(y, want)
