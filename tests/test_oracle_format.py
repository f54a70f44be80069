"""Pins of the oracle's block format: the byte split against IEEE semantics, two
blocks encoded by hand, round trips, capacity and marker invariants, and the
ratios printed on the pages.

Passages followed: explainer "LCT paper - Lossless Huffman coding of BF16
training tensors", paragraph on bits (sign-fraction byte kept raw, exponent
coded, escape + 8-bit literal), paragraph on blocks and streams (65,536 /
32,768-element blocks, 256 round-robin streams of fixed length, overflow with a
marker), and the idealized-arithmetic paragraph (1.4382x CLEAN bound, 16/11).
"""
import json
import os

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def as_f32(bits):
    return (np.asarray(bits, np.uint32) << 16).view(np.float32)


# ------------------------------------------------------------------ byte split

def test_split_matches_ieee_semantics_on_all_patterns(orc):
    v = np.arange(1 << 16, dtype=np.uint16)
    e = np.array([orc.exponent(int(a)) for a in v])
    sf = np.array([orc.signfrac(int(a)) for a in v])
    with np.errstate(invalid="ignore"):
        f = as_f32(v).astype(np.float64)
    # sign bit of the value is bit 7 of the sign-fraction byte
    assert np.array_equal((sf >> 7).astype(bool), np.signbit(f))
    fin = np.isfinite(f)
    assert (e[~fin] == 255).all() and (e[fin] < 255).all()
    a = np.abs(f)
    frac = (sf & 0x7F).astype(np.float64)
    normal = fin & (a >= 2.0 ** -126)
    # |x| = (1 + frac/128) * 2^(e-127) for normals, (frac/128) * 2^-126 otherwise
    assert np.array_equal(a[normal], (1 + frac[normal] / 128) * np.ldexp(1.0, e[normal] - 127))
    sub = fin & ~normal
    assert (e[sub] == 0).all()
    assert np.array_equal(a[sub], frac[sub] / 128 * 2.0 ** -126)
    # NaN vs inf: fraction nonzero iff NaN
    assert np.array_equal(np.isnan(f), (~fin) & (frac > 0))
    # the join is the inverse of the split
    back = np.array([orc.join(int(s), int(x)) for s, x in zip(sf, e)], np.uint16)
    assert np.array_equal(back, v)


# ------------------------------------------------------------------ hand-encoded blocks

def hand_codebook(orc):
    """Base lengths: field 127 -> 1 bit, 126 -> 2, 128 -> 3, ESC -> 3 (Kraft sum 1).
    Canonical codes (by length, then id; ESC has id 256):
        127 -> 0,  126 -> 10,  128 -> 110,  ESC -> 111."""
    lb = np.zeros(256, np.uint8)
    lb[127], lb[126], lb[128] = 1, 2, 3
    cb = orc.codebook_from_base(lb, 3, 0)
    assert [format(int(cb.code[i]), "0%db" % n) for i, n in
            [(127, 1), (126, 2), (128, 3), (256, 3)]] == ["0", "10", "110", "111"]
    return cb


ONE, HALF, M2, ONE5, BIG, ZERO, NZERO, QNAN = (0x3F80, 0x3F00, 0xC000, 0x3FC0, 0x7F00,
                                               0x0000, 0x8000, 0x7FC0)


def test_hand_encoded_block(orc):
    """Two rows (block of 512), one word per stream.  Stream bits are written
    from bit 0 of the word up; a code's first (most significant) bit first; an
    escaped field follows ESC least significant bit first."""
    cb = hand_codebook(orc)
    x = np.full(512, ONE, np.uint16)
    # element r = 256*j + s is position j of stream s
    x[0], x[256] = ONE, HALF          # stream 0: "0", "10"          -> bits 0,1,0
    x[1], x[257] = M2, ONE5           # stream 1: "110", "0"         -> bits 1,1,0,0
    x[2], x[258] = BIG, ONE           # stream 2: "111"+254 lsb-first, "0"
    x[3], x[259] = ZERO, QNAN         # stream 3: "111"+0, "111"+255
    sf, pay, cnt, spill = orc.encode_block(cb, x, 1)
    assert pay[0] == 0b010
    assert pay[1] == 0b0011
    # bits 0..10 = 1,1,1, 0,1,1,1,1,1,1,1 (254 = 0b11111110, lsb first), bit 11 = 0
    assert pay[2] == 0b111_1111_0111
    # bits 0..10 = 1,1,1,0*8 ; bits 11..21 = 1,1,1, 1*8
    assert pay[3] == 0b111_1111_1111_0000_0000_111
    assert (pay[4:] == 0).all()       # every other stream is "0","0"
    assert (cnt == 2).all() and spill.size == 0
    assert sf[1] == 0x80 and sf[257] == 0x40 and sf[259] == 0x40 and sf[0] == 0
    assert np.array_equal(orc.decode_block(cb, sf, pay, cnt, spill, 1), x)


def test_hand_encoded_spill(orc):
    """Three rows (block of 768), one 32-bit word per stream: three escaped
    fields need 33 bits, so the third spills.  Spilled fields go to the
    overflow in (stream, position) order; cnt holds the coded prefix length."""
    cb = hand_codebook(orc)
    x = np.full(768, ONE, np.uint16)
    x[0], x[256], x[512] = ZERO, ZERO, ZERO          # 11 + 11 bits fit, third spills
    x[5], x[261], x[517] = QNAN, NZERO, BIG          # 11 + 11 bits fit, 254 spills
    x[9], x[265], x[521] = HALF, HALF, HALF          # 6 bits, fits
    sf, pay, cnt, spill = orc.encode_block(cb, x, 1)
    assert cnt[0] == 2 and cnt[5] == 2 and cnt[9] == 3 and (np.delete(cnt, [0, 5]) == 3).all()
    assert list(spill) == [0, 254]
    # bits 0..2 ESC, 3..10 literal 0, 11..13 ESC, 14..21 literal 0
    assert pay[0] == 0b00000000_111_00000000_111
    # bits 0..2 ESC, 3..10 literal 255, 11..13 ESC, 14..21 literal 0
    assert pay[5] == 0b00000000_111_11111111_111
    assert pay[9] == 0b01_01_01
    t = orc.encode(cb, np.concatenate([x, x]), 768, 1)
    assert list(t.obase) == [0, 2, 4] and list(t.ovf[:4]) == [0, 254, 0, 254]
    assert np.array_equal(orc.decode(cb, t), np.concatenate([x, x]))


# ------------------------------------------------------------------ invariants

def check_invariants(orc, cb, x, t):
    """Per stream: coded bits fit; the first spilled field (if any) would not
    have fitted; unused payload bits are zero; markers add up."""
    B, cw = t.block_elems, t.cap_words
    cost = np.array([cb.cost(e) for e in range(256)], np.int64)
    e = ((x >> 7) & 0xFF).astype(np.int64)
    total = 0
    for b in range(t.nblk):
        xb = e[b * B:(b + 1) * B]
        nb = xb.size
        spills = 0
        for s in range(256):
            es = xb[s::256]
            c = int(t.cnt[b * 256 + s])
            used = int(cost[es[:c]].sum())
            assert c <= es.size and used <= 32 * cw
            if c < es.size:
                assert used + cost[es[c]] > 32 * cw
            spills += es.size - c
            words = t.pay[(b * cw) * 256 + s::256][:cw]
            bits = np.unpackbits(words.astype("<u4").view(np.uint8), bitorder="little")
            assert not bits[used:].any()
        assert t.obase[b + 1] - t.obase[b] == spills
        total += spills
        assert nb == min(B, x.size - b * B)
    assert t.obase[0] == 0 and t.obase[-1] == total


@pytest.mark.parametrize("n", [1, 255, 256, 257, 2047, 2048, 65535, 65537])
def test_round_trip_odd_sizes(orc, n):
    x = synth.draw(synth.TensorSpec("w", (n,), 100 + n % 97, "normal", {"sigma": 0.02}))
    cb = orc.codebook_build(0, 0.02, 0.0, x)
    for B, cw in [(65536, 25), (32768, 12), (2048, 3)]:
        t = orc.encode(cb, x, B, cw)
        assert t.status == 0
        assert np.array_equal(orc.decode(cb, t), x)
        check_invariants(orc, cb, x, t)


@pytest.mark.parametrize("B,cw", [(4096, 1), (4096, 2), (16384, 3), (32768, 5), (65536, 8),
                                  (32768, 11)])
def test_forced_overflow_round_trip(orc, B, cw):
    x = synth.draw(synth.TensorSpec("w", (3 * B + 77,), 200 + cw, "laplace", {"b": 0.01}))
    cb = orc.codebook_build(1, 0.01, 0.0, x)
    t = orc.encode(cb, x, B, cw)
    assert t.spilled > 0
    check_invariants(orc, cb, x, t)
    assert np.array_equal(orc.decode(cb, t), x)


def test_uniform_bits_and_specials_round_trip(orc):
    x = synth.draw(synth.TensorSpec("u", (5 * 2048 + 3,), 7, "uniform_bits"))
    allpat = np.arange(1 << 16, dtype=np.uint16)
    for data in [x, allpat, np.full(3000, QNAN, np.uint16), np.full(3000, 0x0001, np.uint16)]:
        for model in [(0, 1.0, 0.0), (0, 0.02, 0.0)]:
            cb = orc.codebook_build(*model, data)
            t = orc.encode(cb, data, 2048, 25)
            check_invariants(orc, cb, data, t)
            assert np.array_equal(orc.decode(cb, t), data)


def test_ovf_capacity_reporting(orc):
    x = synth.draw(synth.TensorSpec("u", (8192,), 8, "uniform_bits"))
    cb = orc.codebook_build(0, 1.0, 0.0, x)
    full = orc.encode(cb, x, 2048, 2)
    need = full.spilled
    assert need > 100
    small = orc.encode(cb, x, 2048, 2, ovf_cap=need - 1)
    assert small.status == 1 and small.spilled == need     # markers stay complete
    assert np.array_equal(small.ovf[:need - 1], full.ovf[:need - 1])
    exact = orc.encode(cb, x, 2048, 2, ovf_cap=need)
    assert exact.status == 0


# ------------------------------------------------------------------ pages' figures

def test_clean_and_medium_bounds_match_pages(orc):
    fig = json.load(open(os.path.join(GOLD, "pages_figures.json")))
    x = synth.draw(synth.config1()[0][0])
    cb = orc.codebook_build(0, 0.02, 0.0, x)
    B, cw = synth.mode_layout(synth.CLEAN)
    t = orc.encode(cb, x, B, cw)
    assert t.spilled == 0
    bits = 8.0 * (t.sf.nbytes + t.pay.nbytes) / t.n
    assert round(16.0 / bits, 4) == fig["clean_ratio_bound"]["value"]
    assert round(bits, 1) == fig["clean_bits_per_value"]["value"]
    # allocated exponent bits in CLEAN (soft range on the pages)
    alloc = 32.0 * cw / 256
    a = fig["allocated_exponent_bits_clean"]
    assert a["lo"] <= alloc <= a["hi"]
    # with markers the whole-tensor ratio stays just below the payload bound
    assert 1.43 < t.ratio() < 16.0 / bits
    # MEDIUM: 8 + 3 bits per value, the best printed ratio 16/11
    Bm, cwm = synth.mode_layout(synth.MEDIUM)
    tm = orc.encode(cb, x, Bm, cwm)
    bm = 8.0 * (tm.sf.nbytes + tm.pay.nbytes) / tm.n
    assert round(16.0 / bm, 3) == fig["best_ratio"]["value"]
    assert fig["block_elems"]["clean"] == B and fig["block_elems"]["medium"] == Bm


def test_gaussian_mean_code_length(orc):
    """Coded exponent bits on config 1 lie between the sample entropy and the
    allocation (the pages' 'about 3 bits', soft)."""
    x = synth.draw(synth.config1()[0][0])
    cb = orc.codebook_build(0, 0.02, 0.0, x)
    e = (x >> 7) & 0xFF
    cost = np.array([cb.cost(i) for i in range(256)])
    mean = cost[e].mean()
    h = np.bincount(e, minlength=256) / e.size
    q = h[h > 0]
    H = float(-(q * np.log2(q)).sum())
    assert H <= mean < min(H + 1, 3.125)
