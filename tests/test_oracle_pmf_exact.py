"""Pins of the oracle's model probabilities and integer weights against
50-digit arithmetic (mpmath), independent of the C library's erfc, exp,
lgamma and of the oracle's continued fraction.

The model ("LCT paper - Lossless Huffman coding of BF16 training tensors",
paragraph on bits: a Gaussian, Laplace or power-law distribution chosen by the
user) gives exponent field e in 1..254 the mass of |x| in [2^(e-127),
2^(e-126)), field 0 the mass below 2^-126 and field 255 none; the weights are
floor(p * 2^40 + 0.5).  Here the survival functions are written from their
definitions: Gaussian erfc(t / (sigma sqrt 2)), Laplace exp(-t / b), Student-t
the regularized incomplete beta I_{nu/(nu+u^2)}(nu/2, 1/2) with u = t / s.
"""
import mpmath as mp
import numpy as np
import pytest

mp.mp.dps = 50

MODELS = [
    (0, 0.02, 0.0), (0, 1e-3, 0.0), (0, 1.0, 0.0), (0, 3.7e-12, 0.0),
    (1, 0.01, 0.0), (1, 0.25, 0.0), (1, 1e30, 0.0),
    (2, 0.01, 1.0), (2, 0.01, 2.0), (2, 0.01, 3.0), (2, 1.0, 5.5), (2, 0.05, 5.5), (2, 2e-5, 2.0),
]


def survival(fam, scale, shape, t):
    t, s = mp.mpf(t), mp.mpf(scale)
    if fam == 0:
        return mp.erfc(t / (s * mp.sqrt(2)))
    if fam == 1:
        return mp.exp(-t / s)
    nu = mp.mpf(shape)
    u2 = (t / s) ** 2
    return mp.betainc(nu / 2, mp.mpf(1) / 2, 0, nu / (nu + u2), regularized=True)


def exact_pmf(fam, scale, shape):
    S = {k: survival(fam, scale, shape, mp.ldexp(1, k)) for k in range(-126, 129)}
    p = [1 - S[-126]]
    p += [S[e - 127] - S[e - 126] for e in range(1, 255)]
    p.append(mp.mpf(0))
    return p


@pytest.fixture(scope="module", params=MODELS, ids=lambda m: "f%d_s%g_nu%g" % m)
def case(request, orc):
    fam, scale, shape = request.param
    return request.param, exact_pmf(fam, scale, shape), orc.model_pmf(fam, scale, shape)


def test_pmf_bins_match_exact(case):
    """Every bin within 1e-12 relative, or a few units of 2^-52 absolute (a
    bin near the centre is the difference of two survivals close to 1, so
    its absolute error is what double arithmetic can keep)."""
    _, exact, got = case
    for e in range(256):
        x = exact[e]
        err = abs(mp.mpf(float(got[e])) - x)
        assert err <= mp.mpf("1e-12") * x + mp.mpf("1e-15"), (e, float(x), got[e])


def test_weights_match_exact(case, orc):
    """floor(p * 2^40 + 0.5) of the exact p, except where p * 2^40 lies
    within 1e-3 of a rounding boundary (the double p may then round either
    way: one unit apart at most)."""
    _, exact, got = case
    w = orc.weights(got)
    near = 0
    for e in range(256):
        v = exact[e] * mp.ldexp(1, 40)
        want = int(mp.floor(v + mp.mpf("0.5")))
        frac = v - mp.floor(v)
        if abs(frac - mp.mpf("0.5")) < mp.mpf("1e-3"):
            near += 1
            assert abs(int(w[e]) - want) <= 1, e
        else:
            assert int(w[e]) == want, (e, int(w[e]), want)
    assert near <= 2


def test_pmf_mass_and_closed_values(case):
    """The exact masses themselves: total one, and the Gaussian's central bin
    pair against the normal CDF written through erf (an identity the bins
    must satisfy whatever the survival's form)."""
    (fam, scale, shape), exact, _ = case
    assert abs(mp.fsum(exact) - 1) < mp.mpf("1e-40")
    if fam == 0:
        # mass of |x| in [2^-8, 2^-6): erf(2^-6/(s sqrt2)) - erf(2^-8/(s sqrt2))
        c = mp.erf(mp.ldexp(1, -6) / (scale * mp.sqrt(2))) - mp.erf(mp.ldexp(1, -8) / (scale * mp.sqrt(2)))
        assert abs(exact[119] + exact[120] - c) < mp.mpf("1e-40")


@pytest.mark.parametrize("n", [1, 17, 4095, 4096, 4097, 100003, 1 << 20])
def test_codebook_from_sample_equals_build(orc, n):
    """The bench's checker builds codebooks from the gathered sample; that
    equals the oracle's own build over the whole tensor."""
    g = np.random.default_rng(n)
    import synth
    for fam, scale, shape, x in [
        (0, 0.02, 0.0, synth.to_bf16_bits(g.normal(0, 0.02, n))),
        (1, 0.01, 0.0, synth.to_bf16_bits(g.laplace(0, 0.04, n))),
        (2, 0.01, 3.0, synth.to_bf16_bits(0.003 * g.standard_t(3.0, n))),
    ]:
        a = orc.codebook_from_sample(fam, scale, shape, x[orc.sample_positions(n)])
        b = orc.codebook_build(fam, scale, shape, x)
        assert np.array_equal(a.len, b.len) and a.esc_len == b.esc_len and a.shift == b.shift
        assert np.array_equal(a.code, b.code)
        assert np.array_equal(a.len_base, b.len_base)
