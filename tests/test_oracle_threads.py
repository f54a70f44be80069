"""The oracle's block-range driver (encode, update and decode over ranges of
whole blocks on several host threads, overflow offsets stitched by a serial
scan) gives the serial oracle's bytes exactly: blocks are coded
independently and only the offsets chain ("LCT paper - Lossless Huffman
coding of BF16 training tensors", paragraph on blocks and streams)."""
import numpy as np
import pytest

import synth


def same(a, b):
    for k in ("sf", "pay", "cnt", "obase"):
        assert np.array_equal(getattr(a, k), getattr(b, k)), k
    assert a.spilled == b.spilled and a.status == b.status
    n = min(a.spilled, a.ovf.size)
    assert np.array_equal(a.ovf[:n], b.ovf[:n])


@pytest.mark.parametrize("B,cw,n", [(4096, 2, 37 * 4096 + 1001), (8192, 3, 11 * 8192), (65536, 25, 5 * 65536 + 7),
                                    (32768, 11, 9 * 32768 + 300)])
@pytest.mark.parametrize("threads,pieces", [(1, 1), (4, 7), (8, 64)])
def test_threaded_equals_serial(orc, B, cw, n, threads, pieces):
    g = np.random.default_rng(B + n)
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1.0, n))
    w[5:40] = 0x7FC0                                    # NaNs and escapes along the way
    cbw = orc.codebook_build(1, 0.02, 0.0, w)
    cbm = orc.codebook_build(0, 1.0, 0.0, m)
    rw, rm = orc.encode(cbw, w, B, cw), orc.encode(cbm, m, B, cw)
    tw = orc.encode_threads(cbw, w, B, cw, threads, pieces=pieces)
    same(tw, rw)
    if cw <= 3:
        assert rw.spilled > 0
    ro = orc.sgd(cbw, rw, cbm, rm, 0.05)
    to = orc.sgd_threads(cbw, tw, cbm, orc.encode_threads(cbm, m, B, cw, threads, pieces=pieces), 0.05,
                         threads, pieces=pieces)
    same(to, ro)
    assert np.array_equal(orc.decode_threads(cbw, to, threads, pieces=pieces), orc.decode(cbw, ro))


def test_threaded_small_region(orc):
    """A too-small overflow region: complete offsets, the status set, and the
    region's bytes equal to the serial run's as far as they go."""
    g = np.random.default_rng(3)
    n = 20 * 4096
    x = g.integers(0, 1 << 16, n, dtype=np.uint64).astype(np.uint16)
    cb = orc.codebook_build(0, 1.0, 0.0, x)
    full = orc.encode(cb, x, 4096, 1)
    cap = full.spilled // 3
    a = orc.encode(cb, x, 4096, 1, ovf_cap=cap)
    b = orc.encode_threads(cb, x, 4096, 1, 4, ovf_cap=cap, pieces=9)
    assert a.status == b.status == 1
    assert np.array_equal(a.obase, b.obase) and np.array_equal(a.ovf[:cap], b.ovf[:cap])
