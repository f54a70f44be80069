"""Pins of the oracle's momentum step (SGD with momentum on compressed W and M).

Passages followed: explainer "LCT paper - Lossless Huffman coding of BF16
training tensors", jargon entry "Optimizer state" (the momentum buffer of SGD
with momentum, stored compressed like the weights) and paragraph on training
traffic (decode, update, re-encode).  The pages give no update rule; read as
the plain heavy-ball form m' = rne(fmaf(mu, m, g)), w' = rne(fmaf(-eta, m', w))
with m' as stored in BF16, each NaN result written as 0x7FC0.
"""
from fractions import Fraction

import numpy as np

import synth
from test_oracle_sgd import exact_fmaf, f32_of, round_exact


def bf16_of_exact(r: float) -> int:
    """BF16 bits of the fp32 value r, rounded to nearest-even exactly."""
    if r == 0:
        return 0x8000 if np.signbit(r) else 0
    if not np.isfinite(r):
        return 0xFF80 if r < 0 else 0x7F80
    v = round_exact(Fraction(r), 8, -126, 127)
    return int(np.array([v], np.float32).view(np.uint32)[0] >> 16)


def bf16(u):
    return f32_of(int(u) << 16)


def test_momentum_elem_exact(orc):
    g = np.random.default_rng(41)
    n = 6000
    cases = []
    # operands shaped like training: weights, momentum, gradient
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 1e-2, n))
    cases += [(w[i], m[i], gr[i], 0.9, 1e-3) for i in range(n)]
    # raw bit patterns (all finite, zeros and subnormals included)
    u = g.integers(0, 1 << 16, (3, n), dtype=np.uint64).astype(np.uint16)
    fin = np.isfinite((u.astype(np.uint32) << 16).view(np.float32)).all(axis=0)
    u = u[:, fin]
    cases += [(u[0, i], u[1, i], u[2, i], 0.5, 0.25) for i in range(u.shape[1])]
    for wi, mi, gi, mu, eta in cases:
        wo, mo = orc.momentum_elem(int(wi), int(mi), int(gi), mu, eta)
        m2 = exact_fmaf(float(np.float32(mu)), bf16(mi), bf16(gi))
        assert mo == (0x7FC0 if m2 != m2 else bf16_of_exact(m2)), (wi, mi, gi)
        if mo == 0x7FC0:
            assert wo == 0x7FC0
            continue
        mf = bf16(mo)
        if not np.isfinite(mf):
            continue
        w2 = exact_fmaf(float(np.float32(-eta)), mf, bf16(wi))
        assert wo == (0x7FC0 if w2 != w2 else bf16_of_exact(w2)), (wi, mi, gi)


def test_momentum_special_cases(orc):
    g = np.random.default_rng(43)
    n = 4000
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    w[w == 0x8000] = 0
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 1e-2, n))
    gr[(gr & 0x7FFF) == 0] = 0x3C00          # no zero gradients (sign of 0 + 0)
    for i in range(n):
        # mu = 0: the new momentum is the gradient, bit for bit
        wo, mo = orc.momentum_elem(int(w[i]), int(m[i]), int(gr[i]), 0.0, 1e-3)
        assert mo == gr[i]
        # eta = 0: the weight is kept
        wo, mo = orc.momentum_elem(int(w[i]), int(m[i]), int(gr[i]), 0.9, 0.0)
        assert wo == w[i]
    nan, inf, ninf = 0x7FC1, 0x7F80, 0xFF80
    assert orc.momentum_elem(0x3F80, nan, 0x3F80, 0.9, 1e-3) == (0x7FC0, 0x7FC0)
    assert orc.momentum_elem(0x3F80, 0x3F80, nan, 0.9, 1e-3) == (0x7FC0, 0x7FC0)
    # inf - inf in the momentum: NaN in both outputs
    assert orc.momentum_elem(0x3F80, ninf, inf, 1.0, 1e-3) == (0x7FC0, 0x7FC0)
    # an infinite momentum drives the weight to the opposite infinity
    assert orc.momentum_elem(0x3F80, inf, 0x3F80, 1.0, 1e-3) == (ninf, inf)
    # NaN weight, finite momentum: only W' is NaN
    wo, mo = orc.momentum_elem(0xFFC3, 0x3F80, 0x3F80, 0.5, 1e-3)
    assert wo == 0x7FC0 and mo == 0x3FC0


def test_compressed_momentum_is_naive_round_trip(orc):
    """lcto_momentum (block by block) equals decode -> element step -> encode of
    both outputs, with spills on the inputs and the outputs."""
    g = np.random.default_rng(47)
    n = 5 * 2048 + 77
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1.0, n))
    gr = synth.to_bf16_bits(g.normal(0, 0.5, n))
    m[:20] = [0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001] * 4
    gr[30:40] = [0x7F80, 0x0001, 0x8000, 0xFFC0, 0x3F80] * 2
    cw = orc.codebook_build(1, 0.02, 0.0, w)
    cm = orc.codebook_build(0, 1.0, 0.0, m)
    mu, eta = 0.9, 0.05
    for cap in [25, 3, 1]:
        tw, tm = orc.encode(cw, w, 2048, cap), orc.encode(cm, m, 2048, cap)
        ow, om = orc.momentum(cw, tw, cm, tm, gr, mu, eta)
        dw, dm = orc.momentum_dense(orc.decode(cw, tw), orc.decode(cm, tm), gr, mu, eta)
        rw, rm = orc.encode(cw, dw, 2048, cap), orc.encode(cm, dm, 2048, cap)
        for got, ref in ((ow, rw), (om, rm)):
            for k in ["sf", "pay", "cnt", "obase"]:
                assert np.array_equal(getattr(got, k), getattr(ref, k)), (cap, k)
            assert np.array_equal(got.ovf[:got.spilled], ref.ovf[:ref.spilled])
        assert np.array_equal(orc.decode(cw, ow), dw)
        assert np.array_equal(orc.decode(cm, om), dm)
        if cap == 1:
            assert tw.spilled > 0 and tm.spilled > 0 and ow.spilled > 0 and om.spilled > 0
