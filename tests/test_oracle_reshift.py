"""Pins of the oracle's shift re-estimation and of the updates that re-encode
with another codebook.

Passages followed: LCT abstract (adaptation to magnitude shifts); explainer
"LCT paper - Lossless Huffman coding of BF16 training tensors", paragraph on
bits (the code is fixed ahead of training; an exponent offset estimated on
at most 4096 sampled values adapts it to the tensor's magnitude; training
builds no new code)
and paragraph on the limits (a distribution that no longer fits the tensor
raises storage).  Reading: re-estimating keeps the base code and picks a new
shift from the tensor's current values, sampled at the build's positions.
"""
import numpy as np
import pytest

import synth

B, CAP = 4096, 25
TIGHT = 2     # 64 bits for a stream's 16 positions: stale codes spill


def gaussian(seed, n, sigma=0.02):
    x = synth.to_bf16_bits(np.random.default_rng(seed).normal(0.0, sigma, n))
    assert ((x & 0x7F80) != 0).all()     # no zeros or subnormals: scaling by 2^j is exact
    return x


def scale_pow2(x, j):
    """x * 2^j on BF16 bit patterns (normal values whose exponent stays normal)."""
    e = ((x >> 7) & 0xFF).astype(np.int64) + j
    assert (e > 0).all() and (e < 255).all()
    return ((x & 0x807F) | (e.astype(np.uint16) << 7)).astype(np.uint16)


def sample_bits_by_k(orc, cb, exps, ks):
    """Coded bits of the sample under every candidate shift, each counted from
    the rotated codebook's own final lengths."""
    return {k: sum(orc.codebook_from_base(cb.len_base, cb.esc_len, k).cost(int(e)) for e in exps)
            for k in ks}


@pytest.mark.parametrize("family,scale,shape,kind,args", [
    (0, 0.02, 0.0, "normal", {"sigma": 0.02}),
    (1, 0.01, 0.0, "laplace", {"b": 0.01}),
    (2, 0.01, 3.0, "student_t", {"dof": 3.0, "scale": 0.01}),
])
def test_reshift_of_a_fresh_encoding_is_the_build(orc, family, scale, shape, kind, args):
    """Same base code and the same sample positions: re-estimating from the
    compressed tensor lands on the build's own codebook."""
    x = synth.draw(synth.TensorSpec("x", (3 * B + 700,), 7100 + family, kind, args))
    cb = orc.codebook_build(family, scale, shape, x)
    t = orc.encode(cb, x, B, CAP)
    r = orc.reshift(cb, t)
    assert r.shift == cb.shift
    assert (r.len == cb.len).all() and (r.code == cb.code).all() and r.esc_len == cb.esc_len
    assert (r.len_base == cb.len_base).all()


@pytest.mark.parametrize("j,d", [(-3, 0), (-1, 0), (2, 0), (5, 0), (2, -2), (-3, 4)])
def test_reshift_follows_a_power_of_two_drift(orc, j, d):
    """Values scaled by 2^j move every exponent field by j: the new shift is the
    old one plus j, and re-encoding with it gives every field its original code
    length (escape literals carry the moved field), so the counts and spills
    are the original ones.  The stale codebook may itself carry a shift d away
    from the build's: the new shift still comes from the base code."""
    n = 5 * B + 333
    x = gaussian(7200, n)
    cb = orc.codebook_build(0, 0.02, 0.0, x)
    y = scale_pow2(x, j)
    stale = orc.codebook_from_base(cb.len_base, cb.esc_len, cb.shift + d)
    ty = orc.encode(stale, y, B, TIGHT)
    # the stale code spills (heavily beyond one octave): samples hit the overflow region
    assert ty.spilled > (n // 20 if abs(j - d) > 1 else 0)
    # the minimum is unique, so the tie rule plays no part
    e = ((x[orc.sample_positions(n)] >> 7) & 0xFF).astype(np.uint8)
    costs = sorted(orc.shift_cost(cb.len_base, cb.esc_len, e, k) for k in range(-12, 13))
    assert costs[0] < costs[1]
    r = orc.reshift(stale, ty)
    assert r.shift == cb.shift + j
    tx = orc.encode(cb, x, B, TIGHT)
    ry = orc.encode(r, y, B, TIGHT)
    assert (ry.cnt == tx.cnt).all() and (ry.obase == tx.obase).all()
    assert ry.spilled == tx.spilled < ty.spilled
    sp = tx.spilled
    assert (ry.ovf[:sp].astype(np.int64) == tx.ovf[:sp].astype(np.int64) + j).all()
    assert (orc.decode(r, ry) == y).all()


def test_reshift_minimises_the_sample_bits(orc):
    """Brute force over shifts: the sample's bits under each rotated codebook,
    counted element by element; the chosen shift is the cheapest, ties to the
    smallest |k|, then the smaller k."""
    n = 2 * B + 77
    g = np.random.default_rng(7300)
    # a mixture that no single power of two explains
    v = g.normal(0.0, 0.02, n) * np.where(g.random(n) < 0.5, 1.0, 5.3)
    x = synth.to_bf16_bits(v)
    cb = orc.codebook_build(0, 0.02, 0.0, gaussian(7301, 4096))
    t = orc.encode(cb, x, B, CAP)
    r = orc.reshift(cb, t)
    y = orc.decode(cb, t)
    assert (y == x).all()
    exps = ((y[orc.sample_positions(n)] >> 7) & 0xFF).astype(np.uint8)
    ks = range(-8, 9)
    bits = sample_bits_by_k(orc, cb, exps, ks)
    best = min(bits.values())
    want = min((k for k in ks if bits[k] == best), key=lambda k: (abs(k), k))
    assert r.shift == want
    # and every shift outside the window costs more than the best inside it
    far = orc.codebook_from_base(cb.len_base, cb.esc_len, 40)
    assert sum(far.cost(int(e)) for e in exps) > best


def test_reshift_small_and_empty(orc):
    """Fewer than 4096 elements: every element is in the sample.  No element:
    every shift costs nothing and the tie rule gives 0."""
    x = gaussian(7400, 1000)
    cb = orc.codebook_build(0, 0.02, 0.0, gaussian(7401, 4096))
    for j in (0, 3):
        y = scale_pow2(x, j)
        t = orc.encode(cb, y, B, CAP)
        r = orc.reshift(cb, t)
        assert r.shift == orc.best_shift(cb.len_base, cb.esc_len, ((y >> 7) & 0xFF).astype(np.uint8))
    e = orc.encode(cb, np.zeros(0, np.uint16), B, CAP)
    cb2 = orc.codebook_from_base(cb.len_base, cb.esc_len, 7)
    assert orc.reshift(cb2, e).shift == 0


def test_updates_reencode_with_the_output_codebooks(orc):
    """The update with an output codebook is the dense update of the decoded
    inputs, encoded with that codebook."""
    n = 3 * B + 500
    w = gaussian(7500, n)
    m = gaussian(7501, n, 1e-3)
    gr = gaussian(7502, n, 4e-4)
    cw = orc.codebook_build(0, 0.02, 0.0, w)
    cm = orc.codebook_build(0, 1e-3, 0.0, m)
    cw2 = orc.codebook_from_base(cw.len_base, cw.esc_len, cw.shift + 1)
    cm2 = orc.codebook_from_base(cm.len_base, cm.esc_len, cm.shift - 2)
    tw, tm = orc.encode(cw, w, B, TIGHT), orc.encode(cm, m, B, TIGHT)
    o = orc.sgd(cw, tw, cm, tm, 1e-3, cw_out=cw2)
    ref = orc.encode(cw2, orc.sgd_dense(w, m, 1e-3), B, TIGHT)
    for f in ("sf", "pay", "cnt", "obase"):
        assert (getattr(o, f) == getattr(ref, f)).all(), f
    assert (o.ovf[:o.spilled] == ref.ovf[:ref.spilled]).all() and o.spilled > 0
    ow, om = orc.momentum(cw, tw, cm, tm, gr, 0.9, 1e-3, cw_out=cw2, cm_out=cm2)
    wd, md = orc.momentum_dense(w, m, gr, 0.9, 1e-3)
    for got, want in ((ow, orc.encode(cw2, wd, B, TIGHT)), (om, orc.encode(cm2, md, B, TIGHT))):
        for f in ("sf", "pay", "cnt", "obase"):
            assert (getattr(got, f) == getattr(want, f)).all(), f
        assert (got.ovf[:got.spilled] == want.ovf[:want.spilled]).all() and got.spilled > 0


def test_reshift_samples_the_build_positions(orc):
    """Only the elements at floor(i * n / m) move by 2^3; every other element
    keeps its scale.  The new shift follows the sampled elements alone."""
    n = 2 * B + 77
    x = gaussian(7600, n)
    cb = orc.codebook_build(0, 0.02, 0.0, x)
    pos = orc.sample_positions(n).astype(np.int64)
    y = x.copy()
    y[pos] = scale_pow2(x[pos], 3)
    t = orc.encode(cb, y, B, TIGHT)
    assert orc.reshift(cb, t).shift == cb.shift + 3
    # the neighbours of the sampled positions alone would not move the shift
    z = x.copy()
    nb = np.setdiff1d(np.minimum(pos + 1, n - 1), pos)
    z[nb] = scale_pow2(x[nb], 3)
    assert orc.reshift(cb, orc.encode(cb, z, B, TIGHT)).shift == cb.shift
