"""Pins of the oracle's tensor groups: tensors laid side by side with one
shared overflow region (explainer "LCT paper - Lossless Huffman coding of BF16
training tensors", paragraph on the idealized arithmetic, which counts a
shared overflow buffer).  Reading: each tensor is encoded on its own; the
group places its blocks after the previous tensor's, its sign-fraction bytes
at a multiple of 256, and its spilled bytes after the previous tensors' in one
region, shifting its block offsets by their total."""
import numpy as np

import synth

B, CAP = 4096, 2


def tensors(seed, ns):
    g = np.random.default_rng(seed)
    return [synth.to_bf16_bits(g.laplace(0, 0.02 * (1 + k), n)) for k, n in enumerate(ns)]


def test_one_tensor_is_the_plain_encoding(orc):
    x = tensors(9300, [5 * B + 256])[0]
    cb = orc.codebook_build(1, 0.02, 0.0, x)
    t = orc.encode(cb, x, B, CAP)
    g = orc.encode_group([cb], [x], B, CAP)
    for f in ("sf", "pay", "cnt", "obase"):
        assert np.array_equal(getattr(g, f), getattr(t, f)), f
    assert np.array_equal(g.ovf[:g.spilled], t.ovf[:t.spilled]) and g.spilled == t.spilled > 0


def test_members_decode_and_offsets_chain(orc):
    ns = [3 * B + 5, 0, 1, 255, 4097, B, 2 * B + 300]
    xs = tensors(9301, ns)
    cbs = [orc.codebook_build(1, 0.02 * (1 + k), 0.0, x) for k, x in enumerate(xs)]
    ts = [orc.encode(cb, x, B, CAP) for cb, x in zip(cbs, xs)]
    g = orc.encode_group(cbs, xs, B, CAP)
    assert g.spilled == sum(t.spilled for t in ts) > 0
    assert g.n == sum(-(-n // 256) * 256 for n in ns)
    assert len(g.obase) == sum(-(-n // B) for n in ns) + 1
    base, e0 = 0, 0
    for k, (cb, x, t) in enumerate(zip(cbs, xs, ts)):
        m = orc.group_member(g, ns, k)
        assert int(m.obase[0]) == base                     # after the earlier tensors' spills
        assert np.array_equal(m.obase - np.uint64(base), t.obase)
        assert np.array_equal(g.ovf[base:base + t.spilled], t.ovf[:t.spilled])
        assert np.array_equal(orc.decode(cb, m), x)
        pad = -(-ns[k] // 256) * 256
        assert not g.sf[e0 + ns[k]:e0 + pad].any()          # zero padding
        base += t.spilled
        e0 += pad


def test_shared_region_too_small(orc):
    ns = [2 * B + 7, B + 1]
    xs = tensors(9302, ns)
    cbs = [orc.codebook_build(1, 0.02, 0.0, x) for x in xs]
    full = orc.encode_group(cbs, xs, B, CAP)
    small = orc.encode_group(cbs, xs, B, CAP, ovf_cap=full.spilled - 1)
    assert small.status == 1 and full.status == 0
    assert np.array_equal(small.obase, full.obase)          # offsets complete even then
