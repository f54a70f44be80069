"""Pins of the oracle's codebook construction against things other than itself:
brute-force optimal codes, textbook Huffman, Kraft equality, closed forms of the
model CDFs, Monte Carlo histograms, and the canonical-code example of RFC 1951.

Passages followed: explainer "LCT paper - Lossless Huffman coding of BF16
training tensors", paragraph on bits (8-bit cap, one escape prefix with an
8-bit literal, precomputed codebook from a Gaussian / Laplace / power-law model
plus a shift sampled from up to 4096 elements).
"""
import heapq
import itertools
import json
import math
import os

import numpy as np
import pytest

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ helpers

def brute_min_cost(w, L):
    """Least sum(w*len) over all length vectors in 1..L with Kraft sum <= 1."""
    n = len(w)
    lens = np.array(list(itertools.product(range(1, L + 1), repeat=n)), dtype=np.int64)
    kraft = (2 ** (L - lens)).sum(axis=1)
    ok = kraft <= 2 ** L
    cost = (lens[ok] * np.asarray(w, np.int64)).sum(axis=1)
    return int(cost.min())


def textbook_huffman_lengths(w):
    """Unlimited-length Huffman by the classic heap merge (independent of package-merge)."""
    heap = [(int(x), i, [i]) for i, x in enumerate(w)]
    heapq.heapify(heap)
    lens = [0] * len(w)
    uid = len(w)
    while len(heap) > 1:
        a = heapq.heappop(heap)
        b = heapq.heappop(heap)
        for i in a[2] + b[2]:
            lens[i] += 1
        heapq.heappush(heap, (a[0] + b[0], uid, a[2] + b[2]))
        uid += 1
    return lens


def kraft_units(lens, L):
    return sum(2 ** (L - int(x)) for x in lens if x)


# ------------------------------------------------------------------ package-merge

@pytest.mark.parametrize("n,L", [(4, 3), (5, 3), (6, 4), (7, 4), (8, 4), (8, 3), (5, 8), (4, 8)])
def test_package_merge_matches_brute_force(orc, n, L):
    g = np.random.default_rng(100 * n + L)
    for trial in range(12):
        if trial % 3 == 0:
            w = g.integers(1, 10, n)            # many ties
        elif trial % 3 == 1:
            w = g.integers(1, 1 << 20, n)
        else:
            w = np.sort(2 ** g.integers(0, 16, n))  # skewed: the cap binds
        lens = orc.package_merge(w, L)
        assert lens.max() <= L and lens.min() >= 1
        assert kraft_units(lens, L) == 2 ** L          # complete code
        assert int((lens.astype(np.int64) * w).sum()) == brute_min_cost(w, L)


def test_package_merge_equals_textbook_huffman_when_cap_not_binding(orc):
    g = np.random.default_rng(7)
    checked = 0
    for trial in range(600):
        n = int(g.integers(2, 120))
        w = g.integers(1, 1 << 30, n)
        hl = textbook_huffman_lengths(w)
        if max(hl) > 8:
            continue
        lens = orc.package_merge(w, 8)
        cost = int((lens.astype(np.int64) * w).sum())
        assert cost == sum(int(a) * b for a, b in zip(w, hl))
        p = w / w.sum()
        H = float(-(p * np.log2(p)).sum())
        avg = cost / float(w.sum())
        assert H - 1e-9 <= avg < H + 1
        checked += 1
    assert checked > 150


def test_package_merge_closed_forms(orc):
    # dyadic weights: length = -log2(p)
    assert list(orc.package_merge([8, 4, 2, 1, 1], 8)) == [1, 2, 3, 4, 4]
    assert list(orc.package_merge([1, 1, 2, 4, 8], 8)) == [4, 4, 3, 2, 1]
    # 2^m equal weights: all lengths m
    for m in range(1, 9):
        assert set(orc.package_merge([5] * (1 << m), 8)) == {m}
    # 2^L leaves at limit L: every length is L even for skewed weights
    assert set(orc.package_merge(2 ** np.arange(16) + 1, 4)) == {4}
    # a binding cap: Fibonacci weights want depth n-1 unlimited
    fib = [1, 1, 2, 3, 5, 8, 13, 21, 34, 55]
    assert max(textbook_huffman_lengths(fib)) == 9
    lens = orc.package_merge(fib, 5)
    assert lens.max() == 5 and kraft_units(lens, 5) == 32
    with pytest.raises(ValueError):
        orc.package_merge([1] * 17, 4)   # more leaves than 2^L


# ------------------------------------------------------------------ escape set

def brute_escape_cost(w, L, lit):
    """Least cost over every kept set K (1 <= |K| <= min(n-1, 2^L-1)) and every
    length vector for K plus one escape leaf."""
    n = len(w)
    best = None
    for r in range(1, min(n - 1, 2 ** L - 1) + 1):
        for K in itertools.combinations(range(n), r):
            rest = sum(int(w[i]) for i in range(n) if i not in K)
            for lens in itertools.product(range(1, L + 1), repeat=r + 1):
                if sum(2 ** (L - x) for x in lens) > 2 ** L:
                    continue
                c = sum(int(w[i]) * x for i, x in zip(K, lens)) + rest * (lens[-1] + lit)
                if best is None or c < best:
                    best = c
    return best


@pytest.mark.parametrize("n,L,lit", [(4, 2, 2), (5, 2, 3), (5, 3, 2), (6, 3, 3), (6, 2, 4)])
def test_escape_choice_matches_brute_force(orc, n, L, lit):
    g = np.random.default_rng(1000 + 10 * n + L)
    for trial in range(6):
        w = g.integers(0, 50, n) ** 2   # skewed, some zeros
        w[0] = max(int(w[0]), 1)
        lens, esc, k, cost = orc.build_escape(w, L, lit)
        assert cost == brute_escape_cost(w, L, lit)
        # the reported cost is what the lengths cost
        rest = sum(int(w[i]) for i in range(n) if lens[i] == 0)
        assert cost == sum(int(w[i]) * int(lens[i]) for i in range(n)) + rest * (esc + lit)
        # kept set is the k heaviest (ties by smaller id)
        rank = sorted(range(n), key=lambda i: (-int(w[i]), i))
        assert {i for i in range(n) if lens[i]} == set(rank[:k])
        assert kraft_units(list(lens) + [esc], L) == 2 ** L


def test_base_code_over_exponent_fields(orc):
    for fam, scale, shape in [(0, 0.02, 0), (0, 1e-3, 0), (1, 0.01, 0), (2, 0.01, 3.0),
                              (0, 1.0, 0), (1, 0.25, 0), (2, 1.0, 1.0)]:
        w = orc.weights(orc.model_pmf(fam, scale, shape))
        lens, esc, k, cost = orc.build_base(w)
        assert lens.max() <= 8 and 1 <= esc <= 8
        assert kraft_units(list(lens) + [esc], 8) == 256
        assert lens[255] == 0                      # inf/NaN field has no mass: escaped
        assert (lens > 0).sum() == k
        # escaping costs at least 9 bits, so every kept symbol is at least as
        # likely as every escaped one
        kept = w[lens > 0]
        esc_w = w[lens == 0]
        assert kept.min() >= esc_w.max()


def test_uniform_weights_keep_255(orc):
    lens, esc, k, _ = orc.build_base(np.full(256, 1000, np.uint64))
    # every kept symbol and ESC at 8 bits; one symbol escaped (the last id)
    assert k == 255 and esc == 8 and set(lens[:255]) == {8} and lens[255] == 0


# ------------------------------------------------------------------ model pmf

def test_model_pmf_sums_to_one(orc):
    for fam, scale, shape in [(0, 0.02, 0), (1, 0.01, 0), (2, 0.01, 3.0), (2, 0.3, 1.5)]:
        p = orc.model_pmf(fam, scale, shape)
        assert abs(p.sum() - 1.0) < 1e-9 and (p >= 0).all() and p[255] == 0


def test_student_t_survival_closed_forms(orc):
    # nu = 1 (Cauchy): P(|T| > u) = 1 - (2/pi) atan(u) = (2/pi) atan(1/u)
    # nu = 3: P(|T| > u) = 1 - (2/pi) [ v/(1+v^2) + atan(v) ],  v = u / sqrt(3)
    for u in [1e-6, 1e-3, 0.1, 0.5, 1.0, 2.0, 10.0, 1e3, 1e6]:
        s1 = orc.survival(2, 1.0, 1.0, u)
        assert s1 == pytest.approx(2 / math.pi * math.atan(1 / u), rel=1e-12)
        v = u / math.sqrt(3)
        f3 = 2 / math.pi * (v / (1 + v * v) + math.atan(v))
        s3 = orc.survival(2, 1.0, 3.0, u)
        assert s3 == pytest.approx(1 - f3, rel=1e-9 if u < 100 else 1e-6)
        # scale: T*s
        assert orc.survival(2, 0.01, 3.0, 0.01 * u) == pytest.approx(s3, rel=1e-12)


def _exponent_field_of(x):
    """IEEE binary32 exponent field of |x| for the values' own magnitudes
    (frexp: x = f * 2^k with 0.5 <= |f| < 1  ->  field = k + 126)."""
    _, k = np.frexp(np.abs(x))
    e = k + 126
    e[np.abs(x) < 2.0 ** -126] = 0
    return e


@pytest.mark.parametrize("fam,scale,shape,draw", [
    (0, 0.02, 0.0, lambda g, n: g.normal(0, 0.02, n)),
    (1, 0.01, 0.0, lambda g, n: g.laplace(0, 0.01, n)),
    (2, 0.01, 3.0, lambda g, n: 0.01 * g.standard_t(3.0, n)),
])
def test_model_pmf_matches_monte_carlo(orc, fam, scale, shape, draw):
    n = 1 << 21
    x = draw(np.random.default_rng(5), n)
    hist = np.bincount(_exponent_field_of(x), minlength=256)[:256] / n
    p = orc.model_pmf(fam, scale, shape)
    tol = 6 * np.sqrt(p * (1 - p) / n) + 3.0 / n
    assert (np.abs(hist - p) <= tol).all()


def test_weights_quantisation(orc):
    p = orc.model_pmf(0, 0.02, 0)
    w = orc.weights(p).astype(np.float64)
    assert np.all(np.abs(w - p * 2.0 ** 40) <= 0.5)


def test_model_entropy_in_pages_range(orc):
    """Soft pin: ideal exponent cost about 2.5 to 3.1 bits for matched models
    (explainer, paragraph on bits)."""
    fig = json.load(open(os.path.join(GOLD, "pages_figures.json")))["ideal_exponent_bits"]
    for fam, scale, shape in [(0, 0.02, 0), (1, 0.01, 0), (2, 0.01, 3.0)]:
        p = orc.model_pmf(fam, scale, shape)
        q = p[p > 0]
        H = float(-(q * np.log2(q)).sum())
        assert fig["lo"] <= H <= fig["hi"], (fam, H)


# ------------------------------------------------------------------ canonical codes

def test_canonical_rfc1951_example(orc):
    ex = json.load(open(os.path.join(GOLD, "rfc1951_canonical.json")))
    lens = np.zeros(257, np.uint8)
    lens[:8] = ex["lengths"]
    code = orc.canonical(lens)
    got = [format(int(code[i]), "0%db" % ex["lengths"][i]) for i in range(8)]
    assert got == ex["codes"]


def test_canonical_is_prefix_free(orc):
    g = np.random.default_rng(3)
    for _ in range(20):
        w = orc.weights(orc.model_pmf(int(g.integers(0, 3)), float(10 ** g.uniform(-4, 1)),
                                      float(g.uniform(1, 6))))
        lens, esc, k, _ = orc.build_base(w)
        l257 = np.append(lens, esc).astype(np.uint8)
        code = orc.canonical(l257)
        words = [format(int(code[i]), "0%db" % l257[i]) for i in range(257) if l257[i]]
        assert len(set(words)) == len(words)
        for a in words:
            for b in words:
                assert a == b or not b.startswith(a)


# ------------------------------------------------------------------ shift

def test_shift_matched_sample_is_zero_and_equivariant(orc):
    import synth
    x = synth.draw(synth.TensorSpec("w", (1 << 16,), 11, "normal", {"sigma": 0.02}))
    cb0 = orc.codebook_build(0, 0.02, 0.0, x)
    assert cb0.shift == 0
    e = (x >> 7) & 0xFF
    assert e.min() > 40 and e.max() < 200    # no field clipping in the range tested
    for j in list(range(-20, 21)):
        # exact scaling by 2^j of every normal BF16 value
        xj = synth.to_bf16_bits(synth_float(x) * 2.0 ** j)
        assert ((((xj >> 7) & 0xFF).astype(int) - e.astype(int)) == j)[e > 0].all()
        cbj = orc.codebook_build(0, 0.02, 0.0, xj)
        assert cbj.shift == j
        assert np.array_equal(np.roll(cb0.len, j), cbj.len)


def synth_float(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_shift_tie_rule(orc):
    lb = np.zeros(256, np.uint8)
    lb[100] = 1
    # samples 99 and 101: k = -1 and k = +1 cost the same; the smaller k wins
    assert orc.best_shift(lb, 1, [99, 101]) == -1
    assert orc.shift_cost(lb, 1, [99, 101], -1) == orc.shift_cost(lb, 1, [99, 101], 1) == 10
    # no sample: zero
    assert orc.best_shift(lb, 1, np.zeros(0, np.uint8)) == 0


def test_shift_is_exhaustive_minimum(orc):
    g = np.random.default_rng(9)
    w = orc.weights(orc.model_pmf(1, 0.01, 0))
    lens, esc, _, _ = orc.build_base(w)
    for _ in range(5):
        smp = g.integers(60, 200, 300).astype(np.uint8)
        k = orc.best_shift(lens, esc, smp)
        costs = {kk: orc.shift_cost(lens, esc, smp, kk) for kk in range(-255, 256)}
        assert costs[k] == min(costs.values())
        # shift cost equals the independent per-sample sum
        def c(x):
            return int(lens[x]) if 0 <= x <= 255 and lens[x] else esc + 8
        assert costs[k] == sum(c(int(s) - k) for s in smp)


def test_codebook_sample_positions(orc):
    """The shift is estimated from x[floor(i*n/m)], m = min(n, 4096)."""
    import synth
    n = 10007
    x = synth.draw(synth.TensorSpec("w", (n,), 12, "laplace", {"b": 0.01}))
    cb = orc.codebook_build(1, 0.01, 0.0, x)
    w = orc.weights(orc.model_pmf(1, 0.01, 0))
    lens, esc, _, _ = orc.build_base(w)
    m = 4096
    idx = (np.arange(m, dtype=np.uint64) * n) // m
    smp = ((x[idx] >> 7) & 0xFF).astype(np.uint8)
    assert cb.shift == orc.best_shift(lens, esc, smp)
    # the final lengths are the base lengths moved by the shift
    ref = orc.codebook_from_base(lens, esc, cb.shift)
    assert np.array_equal(ref.len, cb.len) and np.array_equal(ref.code, cb.code)
