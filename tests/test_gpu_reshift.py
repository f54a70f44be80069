"""GPU parity of shift re-estimation (the sample taken from a compressed
tensor, the new codebook, the adapt policy) and of the updates that re-encode
with output codebooks, against the oracle, through the C ABI.

Bar: the sample's BF16 values identical to the oracle's decoded tensor at the
sample positions; the new codebook identical to the oracle's (shift, lengths,
codes, base code); update outputs identical byte for byte.
"""
import numpy as np
import pytest
import torch

import synth
from test_gpu_group import storage_equal
from test_gpu_parity import assert_same, check_codebook, dev, host_parts

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bf16_tensor_split_amd as L
    return L


def gaussian(seed, n, sigma=0.02):
    return synth.to_bf16_bits(np.random.default_rng(seed).normal(0.0, sigma, n))


def scale_pow2(x, j):
    """x * 2^j for normal values whose exponent stays normal (others kept)."""
    e = ((x >> 7) & 0xFF).astype(np.int64)
    ok = (e > 0) & (e < 255) & (e + j > 0) & (e + j < 255)
    y = x.copy()
    y[ok] = (x[ok] & 0x807F) | ((e[ok] + j).astype(np.uint16) << 7)
    return y


def lib_codebook(L, ocb):
    return L.lct_codebook_from_lengths(list(ocb.len_base), ocb.esc_len, ocb.shift)


def same_codebook(cb, ocb):
    assert cb.shift == ocb.shift and cb.esc_len == ocb.esc_len
    assert np.array_equal(np.frombuffer(bytes(cb.len), np.uint8), ocb.len)
    assert np.array_equal(np.frombuffer(bytes(cb.len_base), np.uint8), ocb.len_base)
    assert np.array_equal(np.frombuffer(bytes(cb.code), np.uint32), ocb.code)


def reshift_case(L, orc, x, ocb, B, cw, what=""):
    """Encode x with ocb on both sides, then sample and re-estimate on both."""
    cb = lib_codebook(L, ocb)
    same_codebook(cb, ocb)
    t = L.encode(cb, dev(x), L.layout(B, cw))
    ref = orc.encode(ocb, x, B, cw)
    assert_same(host_parts(t), ref, what + " encode")
    smp = L.lct_tensor_sample(cb, t)
    pos = orc.sample_positions(x.size).astype(np.int64)
    assert np.array_equal(smp, orc.decode(ocb, ref)[pos]), what + " sample"
    new = L.lct_codebook_reshift(cb, t)
    onew = orc.reshift(ocb, ref)
    same_codebook(new, onew)
    return new, onew, t, ref


@pytest.mark.parametrize("j", [-2, 0, 3, 6])
@pytest.mark.parametrize("B,cw", [(65536, 25), (4096, 1), (32768, 12), (32768, 11)])
def test_reshift_after_a_drift(L, orc, B, cw, j):
    """Values scaled by 2^j, encoded with the stale codebook (spilled fields
    fall in the sample), re-estimated from the compressed form."""
    n = 5 * B + 777
    x = gaussian(8000 + cw, n)
    ocb = orc.codebook_build(0, 0.02, 0.0, x)
    y = scale_pow2(x, j)
    _, onew, _, ref = reshift_case(L, orc, y, ocb, B, cw, what="B=%d cw=%d j=%d" % (B, cw, j))
    if abs(j) >= 3:
        assert ref.spilled > 0 and onew.shift == ocb.shift + j


@pytest.mark.parametrize("n", [1, 100, 4095, 4096, 4097, 65537, 300001])
def test_reshift_sizes_and_partial_blocks(L, orc, n):
    """A stale codebook carrying its own shift, tensors of every size class."""
    base = orc.codebook_build(0, 0.02, 0.0, gaussian(8100, 4096))
    ocb = orc.codebook_from_base(base.len_base, base.esc_len, -2)
    x = scale_pow2(gaussian(8101 + n % 97, n), 4)
    for B, cw in [(65536, 25), (4096, 2), (4096, 1)]:
        reshift_case(L, orc, x, ocb, B, cw, what="n=%d B=%d cw=%d" % (n, B, cw))


def test_reshift_uniform_bits_and_specials(L, orc):
    """Every pattern, escapes everywhere: a flat sample histogram whose best
    shift depends on every sampled value."""
    ub = synth.draw(synth.TensorSpec("u", (200003,), 8200, "uniform_bits"))
    allpat = np.tile(np.arange(1 << 16, dtype=np.uint16), 2)
    ocb = orc.codebook_build(0, 1.0, 0.0, ub)
    for x in (ub, allpat):
        for B, cw in [(65536, 25), (32768, 11), (4096, 1)]:
            reshift_case(L, orc, x, ocb, B, cw, what="uniform B=%d" % B)


def test_adapt_moves_a_drifted_tensor_back(L, orc):
    """A tensor whose scale drifted by 2^3 spills; adapt re-estimates the
    shift only past the limit, and encoding with the new codebook spills as
    little as the original did."""
    B, cw = 65536, 25
    n = 8 * B + 5
    x = gaussian(8300, n)
    ocb = orc.codebook_build(0, 0.02, 0.0, x)
    cb = lib_codebook(L, ocb)
    lay = L.layout(B, cw)
    t0 = L.encode(cb, dev(x), lay)
    new, changed = L.lct_codebook_adapt(cb, t0, 0.001)
    assert not changed and new.shift == cb.shift
    y = scale_pow2(x, 3)
    t1 = L.encode(cb, dev(y), lay)
    assert t1.spilled() > 0.001 * n
    kept, changed = L.lct_codebook_adapt(cb, t1, 1.0)       # limit not reached
    assert not changed and kept.shift == cb.shift
    new, changed = L.lct_codebook_adapt(cb, t1, 0.001)
    assert changed and new.shift == cb.shift + 3
    same_codebook(new, orc.reshift(ocb, orc.encode(ocb, y, B, cw)))
    t2 = L.encode(new, dev(y), lay)
    assert t2.spilled() == t0.spilled()


# ------------------------------------------------------------------ updates with output codebooks

@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(65536, 25), (4096, 2), (32768, 11)])
def test_sgd_step_recode(L, orc, B, cw, inplace):
    """W decoded with its codebook, W' encoded with a re-estimated one; the
    CLEAN case has no spilled input field (the full-block path)."""
    g = np.random.default_rng(8400 + cw)
    n = 6 * B + (0 if B == 65536 else 999)
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    cbw, ocw = check_codebook(L, orc, synth.Model(0, 0.02), w)
    cbm, ocm = check_codebook(L, orc, synth.Model(0, 1e-3), m)
    ocw2 = orc.codebook_from_base(ocw.len_base, ocw.esc_len, ocw.shift + 1)
    cbw2 = lib_codebook(L, ocw2)
    lay = L.layout(B, cw)
    tw, tm = L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)
    rw, rm = orc.encode(ocw, w, B, cw), orc.encode(ocm, m, B, cw)
    if B == 65536:
        assert rw.spilled == 0 and rm.spilled == 0
    ref = orc.sgd(ocw, rw, ocm, rm, 1e-3, cw_out=ocw2)
    out = L.alloc_tensor(n, lay)
    if inplace:
        out.sf, out.pay, out.cnt, out.obase = tw.sf, tw.pay, tw.cnt, tw.obase
    L.lct_sgd_step_recode(cbw, tw, cbm, tm, 1e-3, cbw2, out)
    gp = host_parts(out)
    assert_same(gp, ref, "sgd recode B=%d inplace=%s" % (B, inplace))
    assert gp["status"] == ref.status
    y = L.decode(cbw2, out)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), orc.sgd_dense(w, m, 1e-3))


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(8192, 3), (32768, 11)])
def test_momentum_step_recode(L, orc, B, cw, inplace):
    g = np.random.default_rng(8500 + cw)
    n = 5 * B + 77
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 4e-3, n))
    cbw, ocw = check_codebook(L, orc, synth.Model(0, 0.02), w)
    cbm, ocm = check_codebook(L, orc, synth.Model(0, 1e-3), m)
    ocw2 = orc.codebook_from_base(ocw.len_base, ocw.esc_len, ocw.shift - 1)
    ocm2 = orc.codebook_from_base(ocm.len_base, ocm.esc_len, ocm.shift + 2)
    lay = L.layout(B, cw)
    tw, tm = L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)
    rw, rm = orc.encode(ocw, w, B, cw), orc.encode(ocm, m, B, cw)
    ref_w, ref_m = orc.momentum(ocw, rw, ocm, rm, gr, 0.9, 1e-3, cw_out=ocw2, cm_out=ocm2)
    ow, om = L.alloc_tensor(n, lay), L.alloc_tensor(n, lay)
    if inplace:
        ow.sf, ow.pay, ow.cnt, ow.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        om.sf, om.pay, om.cnt, om.obase = tm.sf, tm.pay, tm.cnt, tm.obase
    L.lct_momentum_step_recode(cbw, tw, cbm, tm, dev(gr), 0.9, 1e-3, lib_codebook(L, ocw2),
                               lib_codebook(L, ocm2), ow, om)
    for out, ref, name in ((ow, ref_w, "W'"), (om, ref_m, "M'")):
        gp = host_parts(out)
        assert_same(gp, ref, "momentum recode %s inplace=%s" % (name, inplace))
        assert gp["status"] == ref.status
    assert ref_w.spilled > 0 and ref_m.spilled > 0


# ------------------------------------------------------------------ fit on the device

@pytest.mark.parametrize("case", ["gauss", "gauss_x64", "laplace_small", "uniform_bits", "one", "mixture"])
def test_device_fit_matches_the_host(L, orc, case):
    """lct_group_fit chooses the shift and builds the tables on the device:
    the same shift, encode table and peek table as the host's
    lct_codebook_reshift_dense, and an encode equal to the oracle's."""
    g = np.random.default_rng(8600)
    if case == "gauss":
        x = synth.to_bf16_bits(g.normal(0, 0.02, 300001))
    elif case == "gauss_x64":
        x = synth.to_bf16_bits(g.normal(0, 0.02 * 64, 70000))
    elif case == "laplace_small":
        x = synth.to_bf16_bits(g.laplace(0, 3.0, 1000))
    elif case == "uniform_bits":
        x = g.integers(0, 1 << 16, 131072, dtype=np.uint64).astype(np.uint16)
    elif case == "one":
        x = np.array([0x3F80], np.uint16)
    else:
        n = 90000
        x = synth.to_bf16_bits(g.normal(0, 1.0, n) * np.where(g.random(n) < 0.5, 1.0, 2.0 ** -9))
    base = L.lct_codebook_build(L.Model(0, 0.02, 0.0), None)
    xd = dev(x).view(torch.bfloat16)
    shift = torch.full((4,), -999, dtype=torch.int32, device="cuda")
    lay = L.layout(65536, 25)
    grp = L.LctGroup([x.size], lay, [base], [xd], fit=True, shift=shift)
    host = L.lct_codebook_reshift_dense(base, xd)
    torch.cuda.synchronize()
    assert int(shift[0].item()) == host.shift
    tab = grp.table.cpu().numpy()
    enc0, dec0 = 256, 1536                       # the table's parts for one tensor
    assert np.array_equal(tab[enc0:enc0 + 1024].view(np.uint32), np.frombuffer(bytes(host.enc_bits), np.uint32))
    assert np.array_equal(tab[enc0 + 1024:enc0 + 1280], np.frombuffer(bytes(host.enc_len), np.uint8))
    assert np.array_equal(tab[dec0:dec0 + 512].view(np.uint16), np.frombuffer(bytes(host.dec), np.uint16))
    assert int(tab[dec0 + 512:dec0 + 516].view(np.uint32)[0]) == host.esc_len
    ent = tab[0:32].view(np.uint64)
    assert int(ent[0]) == xd.data_ptr() and int(ent[1]) == x.size and int(ent[2]) == 0
    # the encode with the device tables is the oracle's with the same shift
    ob = orc.codebook_build(0, 0.02, 0.0, x)
    assert ob.shift == host.shift
    all_ = grp.alloc_storage(x.size)
    L.lct_encode_group(grp, all_)
    ref = orc.group([orc.encode(ob, x, 65536, 25)], x.size)
    storage_equal(L, grp, all_, ref, [x.size], "fit " + case)
    y = torch.empty(x.size, dtype=torch.bfloat16, device="cuda")
    L.lct_decode(host, grp.tensor(all_, 0), y)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x)
