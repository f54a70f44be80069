"""GPU parity: the HIP path (through the C ABI) against the oracle, byte for
byte on every compressed buffer and bit for bit on decoded and updated values.

The bar: sf, pay, cnt, obase and the used part of ovf identical; decoded
tensors identical to the input; the SGD output identical to the oracle's naive
decode -> fmaf -> RNE -> encode round trip (0 ULP).
"""
import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bf16_tensor_split_amd as L
    return L


def dev(x16: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda()


def host_parts(t):
    """Compressed buffers of a device tensor, trimmed to their sizes."""
    sz = t.sizes
    torch.cuda.synchronize()
    spilled = int(t.obase[-1].item())
    return {
        "sf": t.sf[:sz.sf].cpu().numpy(),
        "pay": t.pay[:sz.pay // 4].cpu().numpy().view(np.uint32),
        "cnt": t.cnt[:sz.cnt // 2].cpu().numpy().view(np.uint16),
        "obase": t.obase.cpu().numpy().view(np.uint64),
        "ovf": t.ovf[:min(spilled, t.ovf_cap)].cpu().numpy(),
        "status": int(t.status[0].item()),
    }


def assert_same(gpu, ref, what=""):
    for k in ["sf", "pay", "cnt", "obase"]:
        a, b = gpu[k], getattr(ref, k)
        if not np.array_equal(a, b):
            bad = np.nonzero(a != b)[0]
            raise AssertionError("%s %s differs at %d places, first %d: gpu %s oracle %s" %
                                 (what, k, bad.size, bad[0], a[bad[0]], b[bad[0]]))
    n = min(ref.spilled, len(ref.ovf))
    assert np.array_equal(gpu["ovf"][:n], ref.ovf[:n]), what + " ovf"


def check_codebook(L, orc, model, x):
    """Library build on the device vs oracle build on the host: same lengths,
    escape length, shift and codes."""
    cb = L.lct_codebook_build(L.Model(model.family, model.scale, model.shape), dev(x))
    ocb = orc.codebook_build(model.family, model.scale, model.shape, x)
    assert np.array_equal(np.frombuffer(bytes(cb.len), np.uint8), ocb.len)
    assert cb.esc_len == ocb.esc_len and cb.shift == ocb.shift
    assert np.array_equal(np.frombuffer(bytes(cb.code), np.uint32), ocb.code)
    return cb, ocb


def roundtrip_case(L, orc, x, model, block_elems, cap_words, ovf_cap=None, what=""):
    cb, ocb = check_codebook(L, orc, model, x)
    lay = L.layout(block_elems, cap_words)
    xd = dev(x)
    t = L.encode(cb, xd, lay, ovf_cap)
    ref = orc.encode(ocb, x, block_elems, cap_words, ovf_cap)
    g = host_parts(t)
    assert_same(g, ref, what)
    assert g["status"] == ref.status
    y = L.decode(cb, t)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), x), what + " decode"
    return cb, ocb, t, ref


# ------------------------------------------------------------------ encode / decode

def test_config1_gaussian_clean(L, orc):
    spec, model = synth.config1()[0]
    x = synth.draw(spec)
    B, cw = synth.mode_layout(synth.CLEAN)
    _, _, t, ref = roundtrip_case(L, orc, x, model, B, cw, what="config1")
    assert ref.spilled == 0 and abs(t.ratio() - ref.ratio()) < 1e-12


@pytest.mark.parametrize("n", [0, 1, 255, 256, 257, 2047, 2048, 2049, 65535, 65537, 300001])
def test_odd_sizes(L, orc, n):
    x = synth.draw(synth.TensorSpec("w", (n,), 500 + n % 89, "normal", {"sigma": 0.02}))
    for B, cw in [(65536, 25), (4096, 2), (4096, 1)]:
        roundtrip_case(L, orc, x, synth.Model(0, 0.02), B, cw, what="n=%d B=%d cw=%d" % (n, B, cw))


@pytest.mark.parametrize("B,cw", [(4096, 1), (8192, 3), (4096, 2), (16384, 4), (32768, 11),
                                  (65536, 8), (65536, 64)])
def test_forced_overflow_many_blocks(L, orc, B, cw):
    x = synth.draw(synth.TensorSpec("w", (97 * B + 1234,), 600 + cw, "laplace", {"b": 0.01}))
    _, _, _, ref = roundtrip_case(L, orc, x, synth.Model(1, 0.01), B, cw, what="B=%d cw=%d" % (B, cw))
    if 32.0 * cw * 256 / B < 3.5:      # capacity below the Laplace code's ~3 bits: must spill
        assert ref.spilled > 0


def test_specials_and_uniform_bits(L, orc):
    allpat = np.tile(np.arange(1 << 16, dtype=np.uint16), 3)
    ub = synth.draw(synth.TensorSpec("u", (200003,), 4002, "uniform_bits"))
    for x in [allpat, ub, np.full(70000, 0x7FC0, np.uint16), np.full(4097, 0x0001, np.uint16)]:
        for B, cw in [(65536, 25), (32768, 12), (4096, 1)]:
            roundtrip_case(L, orc, x, synth.Model(0, 1.0), B, cw, what="specials B=%d" % B)


def test_repeatable_lookback(L, orc):
    """Many small blocks with spills everywhere, encoded 20 times: identical
    bytes every time (the cross-block offset scan has a single answer)."""
    x = synth.draw(synth.TensorSpec("u", (4096 * 1500 + 17,), 77, "uniform_bits"))
    cb, ocb = check_codebook(L, orc, synth.Model(0, 1.0), x)
    ref = orc.encode(ocb, x, 4096, 2)
    lay = L.layout(4096, 2)
    xd = dev(x)
    t = L.alloc_tensor(x.size, lay)
    for _ in range(20):
        t.obase.fill_(-1)
        L.lct_encode(cb, xd, t)
        assert_same(host_parts(t), ref, "repeat")


def test_ovf_capacity_status_and_guards(L, orc):
    x = synth.draw(synth.TensorSpec("u", (40000,), 78, "uniform_bits"))
    cb, ocb = check_codebook(L, orc, synth.Model(0, 1.0), x)
    full = orc.encode(ocb, x, 4096, 2)
    need = full.spilled
    lay = L.layout(4096, 2)
    for cap in [0, 1, need // 2, need - 1, need]:
        t = L.alloc_tensor(x.size, lay, ovf_cap=cap)
        # the ovf buffer holds 4096 guard bytes past ovf_cap
        t.ovf = torch.full((cap + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
        L.lct_encode(cb, dev(x), t)
        g = host_parts(t)
        assert int(g["obase"][-1]) == need
        assert g["status"] == (0 if cap >= need else L.ST_OVF_FULL)
        ovf = t.ovf.cpu().numpy()
        # nothing is written past ovf_cap; below it the content is only
        # specified when everything fits
        assert (ovf[cap:] == 0xA5).all()
        if cap >= need:
            assert np.array_equal(ovf[:need], full.ovf[:need])
        assert np.array_equal(g["pay"], full.pay) and np.array_equal(g["cnt"], full.cnt)


# ------------------------------------------------------------------ larger workloads

@pytest.mark.parametrize("idx", [0, 1, 2])
@pytest.mark.parametrize("mode", [synth.MEDIUM, synth.HIGH])
def test_config2_overflow_stress(L, orc, idx, mode):
    spec, model = synth.config2()[idx]
    x = synth.draw(spec)
    B, cw = synth.mode_layout(mode)
    _, _, _, ref = roundtrip_case(L, orc, x, model, B, cw, what="config2 %s mode %d" % (spec.name, mode))
    if mode == synth.HIGH:
        assert ref.spilled > 0


@pytest.mark.parametrize("idx", [0, 1, 2])
def test_config4_activations(L, orc, idx):
    spec, model = synth.config4()[idx]
    x = synth.draw(spec)
    for mode in (synth.CLEAN, synth.MEDIUM):
        B, cw = synth.mode_layout(mode)
        roundtrip_case(L, orc, x, model, B, cw, what="config4 %s" % spec.name)


# ------------------------------------------------------------------ fused SGD

def sgd_case(L, orc, w, m, mw, mm, eta, B, cw, inplace, what=""):
    cbw, ocw = check_codebook(L, orc, mw, w)
    cbm, ocm = check_codebook(L, orc, mm, m)
    lay = L.layout(B, cw)
    tw = L.encode(cbw, dev(w), lay)
    tm = L.encode(cbm, dev(m), lay)
    rw = orc.encode(ocw, w, B, cw)
    rm = orc.encode(ocm, m, B, cw)
    assert_same(host_parts(tw), rw, what + " W")
    assert_same(host_parts(tm), rm, what + " M")
    ref = orc.sgd(ocw, rw, ocm, rm, eta)
    if inplace:
        out = L.alloc_tensor(w.size, lay)
        out.sf, out.pay, out.cnt, out.obase = tw.sf, tw.pay, tw.cnt, tw.obase
    else:
        out = L.alloc_tensor(w.size, lay)
    L.lct_sgd_step(cbw, tw, cbm, tm, eta, out)
    g = host_parts(out)
    assert_same(g, ref, what + " W'")
    assert g["status"] == ref.status
    y = L.decode(cbw, out)
    torch.cuda.synchronize()
    assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), orc.decode(ocw, ref))
    return ref


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(65536, 25), (4096, 2), (8192, 3), (32768, 12), (32768, 11)])
def test_sgd_small_with_spills(L, orc, B, cw, inplace):
    g = np.random.default_rng(B + cw)
    n = 7 * B + 333
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1.0, n))
    m[:64] = [0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F] * 8
    w[100:164] = [0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F] * 8
    sgd_case(L, orc, w, m, synth.Model(1, 0.02), synth.Model(0, 1.0), 0.05, B, cw, inplace,
             what="B=%d cw=%d inplace=%s" % (B, cw, inplace))


@pytest.mark.parametrize("inplace", [False, True])
def test_sgd_full_blocks_escapes_and_nans(L, orc, inplace):
    """Full blocks with no spilled input field (the update's full-block path):
    runs of escaped exponents that overrun a four-field window, and NaNs in
    either operand at several places of a slab, send single halves through
    the path's re-decode with the integer rounding."""
    g = np.random.default_rng(77)
    B = 65536
    n = 4 * B
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    tiny = synth.to_bf16_bits(np.array([1e-30, -3e-33, 2e-35, -1e-36]))
    for blk, s, j in [(0, 5, 40), (1, 130, 0), (2, 255, 252), (3, 64, 17), (0, 200, 128)]:
        for t in range(4):                    # four escapes in one window of stream s
            w[blk * B + (j + t) * 256 + s] = tiny[t]
    for blk, s, j in [(1, 7, 30), (2, 100, 161), (3, 250, 9)]:
        for t in range(2):                    # two escapes in one window of M
            m[blk * B + (j + t) * 256 + s] = tiny[t]
    w[1 * B + 100 * 256 + 3] = 0x7FC0          # NaN in W, second half of a slab
    m[2 * B + 201 * 256 + 66] = 0xFFC1          # NaN in M (negative, payload)
    w[3 * B + 255 * 256 + 255] = 0x7F81         # signalling-pattern NaN, last element
    mw, mm = synth.Model(0, 0.02), synth.Model(0, 1e-3)
    lay_b, lay_c = B, 25
    ocw = orc.codebook_build(0, 0.02, 0.0, w)
    ocm = orc.codebook_build(0, 1e-3, 0.0, m)
    assert orc.encode(ocw, w, lay_b, lay_c).spilled == 0
    assert orc.encode(ocm, m, lay_b, lay_c).spilled == 0
    sgd_case(L, orc, w, m, mw, mm, 1e-3, lay_b, lay_c, inplace, what="escapes/nans inplace=%s" % inplace)


def narrow_values(orc, g, sigma, n, extra=0.01):
    """BF16 values whose exponent fields are the two with the shortest codes
    of the Gaussian(sigma) codebook (a share `extra` takes the third
    shortest), with random signs and fractions: about two bits a field, so
    even HIGH's 2.75 bits a field hold every stream without a spill."""
    base = orc.codebook_build(0, sigma, 0.0, synth.to_bf16_bits(g.normal(0, sigma, 65536)))
    order = np.argsort(np.where(base.len == 0, 99, base.len), kind="stable")
    e = np.where(g.random(n) < extra, order[2], order[g.integers(0, 2, n)]).astype(np.uint16)
    return ((g.integers(0, 2, n).astype(np.uint16) << 15) | (e << 7)
            | g.integers(0, 128, n).astype(np.uint16)).astype(np.uint16)


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(65536, 25), (32768, 12), (32768, 11)])
def test_full_block_path_in_every_mode(L, orc, B, cw, inplace):
    """Full blocks whose inputs spill nothing in CLEAN, MEDIUM and HIGH: every
    unit of the update takes the full-block path (its own counter says so),
    and W' equals the oracle's round trip; the fused momentum step likewise
    (both outputs' counters)."""
    g = np.random.default_rng(B + 7 * cw)
    nblk = 6
    n = nblk * B
    w = narrow_values(orc, g, 0.02, n)
    m = narrow_values(orc, g, 1e-3, n)
    mw, mm = synth.Model(0, 0.02), synth.Model(0, 1e-3)
    ocw, ocm = orc.codebook_build(0, 0.02, 0.0, w), orc.codebook_build(0, 1e-3, 0.0, m)
    rw, rm = orc.encode(ocw, w, B, cw), orc.encode(ocm, m, B, cw)
    assert rw.spilled == 0 and rm.spilled == 0
    sgd_case(L, orc, w, m, mw, mm, 1e-3, B, cw, inplace, what="full path B=%d cw=%d" % (B, cw))
    # sgd_case's output: run again to read its counter
    cbw = L.lct_codebook_build(L.Model(0, 0.02, 0.0), dev(w))
    cbm = L.lct_codebook_build(L.Model(0, 1e-3, 0.0), dev(m))
    lay = L.layout(B, cw)
    tw, tm = L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)
    out = L.alloc_tensor(n, lay)
    L.lct_sgd_step(cbw, tw, cbm, tm, 1e-3, out)
    assert out.full_path_units() == 4 * nblk
    # momentum: M' = 0.9 M + g keeps M's fields within its short codes
    gr = synth.to_bf16_bits(g.normal(0, 1e-6, n))
    ref_w, ref_m = momentum_case(L, orc, w, m, gr, mw, mm, 0.9, 1e-3, B, cw, inplace,
                                 what="full path momentum B=%d cw=%d" % (B, cw))
    assert ref_m.spilled == 0
    ow, om = L.alloc_tensor(n, lay), L.alloc_tensor(n, lay)
    L.lct_momentum_step(cbw, L.encode(cbw, dev(w), lay), cbm, L.encode(cbm, dev(m), lay), dev(gr), 0.9, 1e-3,
                        ow, om)
    assert om.full_path_units() == 4 * nblk and ow.full_path_units() == 4 * nblk


@pytest.mark.parametrize("inplace", [False, True])
def test_sgd_readers_far_apart(L, orc, inplace):
    """Full CLEAN blocks where some of M's streams open (or, in other blocks,
    go on at mid-stream) with a run of escaped fields while their neighbours
    keep two-bit codes: a wave's readers of M end up hundreds of bits apart,
    farther than the rows the update holds of M at once, so the far readers'
    windows come from memory.  No input field spills, so every unit takes the
    full-block path; W' equals the oracle's round trip."""
    g = np.random.default_rng(4242)
    B, cw, nblk = 65536, 25, 4
    n = nblk * B
    w = narrow_values(orc, g, 0.02, n)
    m = narrow_values(orc, g, 1e-3, n, extra=0.0)
    tiny = synth.to_bf16_bits(np.array([1e-30, -3e-33, 2e-35, -1e-36]))
    runs = [(0, 0), (1, 100), (2, 230), (3, 40)]      # (block, first position of the runs)
    for blk, j0 in runs:
        for s in range(0, 256, 4):                     # every fourth stream of every unit
            for t in range(20):
                m[blk * B + (j0 + t) * 256 + s] = tiny[(s + t) % 4]
    mw, mm = synth.Model(0, 0.02), synth.Model(0, 1e-3)
    ocw = orc.codebook_build(0, 0.02, 0.0, w)
    ocm = orc.codebook_build(0, 1e-3, 0.0, m)
    assert orc.encode(ocw, w, B, cw).spilled == 0
    assert orc.encode(ocm, m, B, cw).spilled == 0
    # the readers' spread, from the code lengths: at some position of every
    # block two streams of one unit are more than eight rows apart
    esc = int(ocm.esc_len) + 8
    lens = np.where(ocm.len[(m >> 7) & 0xFF] == 0, esc, ocm.len[(m >> 7) & 0xFF]).astype(np.int64)
    bits = np.cumsum(lens.reshape(nblk, 256, 256), axis=1)        # [block, position, stream]
    spread = (bits.reshape(nblk, 256, 4, 64).max(axis=3) - bits.reshape(nblk, 256, 4, 64).min(axis=3)).max(axis=(1, 2))
    assert (spread > 8 * 32).all(), spread
    sgd_case(L, orc, w, m, mw, mm, 1e-3, B, cw, inplace, what="far readers inplace=%s" % inplace)
    cbw = L.lct_codebook_build(L.Model(0, 0.02, 0.0), dev(w))
    cbm = L.lct_codebook_build(L.Model(0, 1e-3, 0.0), dev(m))
    lay = L.layout(B, cw)
    tw, tm = L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)
    out = L.alloc_tensor(n, lay)
    L.lct_sgd_step(cbw, tw, cbm, tm, 1e-3, out)
    assert out.full_path_units() == 4 * nblk


@pytest.mark.parametrize("B,cw,n", [(65536, 25, 16), (65536, 25, 65536 + 4096), (65536, 25, 2 * 65536 + 256 * 7),
                                    (65536, 25, 3 * 65536 + 4096 * 5 + 16 * 7), (65536, 25, 65536 + 65520),
                                    (32768, 12, 32768 + 16 * 999), (32768, 11, 2 * 32768 + 48)])
def test_partial_last_block(L, orc, B, cw, n):
    """Tensors whose last block is partial (streams of equal or of two
    lengths) and whose inputs spill nothing: the whole blocks take the
    full-block path and the partial one the general kernel (the counters say
    so); the update and the momentum step equal the oracle's, in place and
    not."""
    g = np.random.default_rng(n + cw)
    nfull = n // B
    w = narrow_values(orc, g, 0.02, n)
    m = narrow_values(orc, g, 1e-3, n)
    gr = synth.to_bf16_bits(g.normal(0, 1e-6, n))
    mw, mm = synth.Model(0, 0.02), synth.Model(0, 1e-3)
    ocw, ocm = orc.codebook_build(0, 0.02, 0.0, w), orc.codebook_build(0, 1e-3, 0.0, m)
    assert orc.encode(ocw, w, B, cw).spilled == 0 and orc.encode(ocm, m, B, cw).spilled == 0
    for inplace in (False, True):
        what = "partial n=%d B=%d cw=%d inplace=%s" % (n, B, cw, inplace)
        sgd_case(L, orc, w, m, mw, mm, 1e-3, B, cw, inplace, what=what)
        momentum_case(L, orc, w, m, gr, mw, mm, 0.9, 1e-3, B, cw, inplace, what=what)
    cbw = L.lct_codebook_build(L.Model(0, 0.02, 0.0), dev(w))
    cbm = L.lct_codebook_build(L.Model(0, 1e-3, 0.0), dev(m))
    lay = L.layout(B, cw)
    out = L.alloc_tensor(n, lay)
    L.lct_sgd_step(cbw, L.encode(cbw, dev(w), lay), cbm, L.encode(cbm, dev(m), lay), 1e-3, out)
    assert out.full_path_units() == 4 * nfull
    ow, om = L.alloc_tensor(n, lay), L.alloc_tensor(n, lay)
    L.lct_momentum_step(cbw, L.encode(cbw, dev(w), lay), cbm, L.encode(cbm, dev(m), lay), dev(gr), 0.9, 1e-3,
                        ow, om)
    assert ow.full_path_units() == 4 * nfull and om.full_path_units() == 4 * nfull


@pytest.mark.parametrize("B", [4096, 16384, 32768])
def test_ring_kernel_short_streams(L, orc, B):
    """The 25-word capacity with blocks smaller than CLEAN's: the ring kernel
    runs streams of 16 to 128 positions (the ring's first rows hold most or
    all of a stream, and the refills reach rows past the stream's end, which
    read as zero); whole blocks take it, a partial last block the general
    kernel; the update and the momentum step equal the oracle's, in place and
    not."""
    g = np.random.default_rng(B + 25)
    n = 5 * B + 4000
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 4e-4, n))
    mw, mm = synth.Model(0, 0.02), synth.Model(0, 1e-3)
    for inplace in (False, True):
        what = "ring B=%d inplace=%s" % (B, inplace)
        sgd_case(L, orc, w, m, mw, mm, 1e-3, B, 25, inplace, what=what)
        momentum_case(L, orc, w, m, gr, mw, mm, 0.9, 1e-3, B, 25, inplace, what=what)
    cbw = L.lct_codebook_build(L.Model(0, 0.02, 0.0), dev(w))
    cbm = L.lct_codebook_build(L.Model(0, 1e-3, 0.0), dev(m))
    lay = L.layout(B, 25)
    out = L.alloc_tensor(n, lay)
    L.lct_sgd_step(cbw, L.encode(cbw, dev(w), lay), cbm, L.encode(cbm, dev(m), lay), 1e-3, out)
    assert out.full_path_units() == 4 * (n // B)


def test_sgd_eta_zero_identity(L, orc):
    g = np.random.default_rng(3)
    n = 5 * 65536 + 7
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    w[w == 0x8000] = 0
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    ref = sgd_case(L, orc, w, m, synth.Model(0, 0.02), synth.Model(0, 1e-3), 0.0, 65536, 25, False)
    assert np.array_equal(orc.decode(orc.codebook_build(0, 0.02, 0.0, w), ref), w)


def test_config3_gpt162m_flat(L, orc):
    """One fused step over the flat 162M-parameter set, checked in full."""
    ws, ms, mw, mm, eta = synth.config3()
    w = np.concatenate([synth.draw(s) for s in ws])
    m = np.concatenate([synth.draw(s) for s in ms])
    B, cw = synth.mode_layout(synth.CLEAN)
    ref = sgd_case(L, orc, w, m, mw, mm, eta, B, cw, True, what="config3")
    assert ref.spilled == 0


# ------------------------------------------------------------------ momentum step

def momentum_case(L, orc, w, m, gr, mw, mm, mu, eta, B, cw, inplace, what="", outs=None):
    cbw, ocw = check_codebook(L, orc, mw, w)
    cbm, ocm = check_codebook(L, orc, mm, m)
    lay = L.layout(B, cw)
    tw = L.encode(cbw, dev(w), lay)
    tm = L.encode(cbm, dev(m), lay)
    rw = orc.encode(ocw, w, B, cw)
    rm = orc.encode(ocm, m, B, cw)
    assert_same(host_parts(tw), rw, what + " W")
    assert_same(host_parts(tm), rm, what + " M")
    ref_w, ref_m = orc.momentum(ocw, rw, ocm, rm, gr, mu, eta)
    ow = L.alloc_tensor(w.size, lay)
    om = L.alloc_tensor(w.size, lay)
    if inplace:
        ow.sf, ow.pay, ow.cnt, ow.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        om.sf, om.pay, om.cnt, om.obase = tm.sf, tm.pay, tm.cnt, tm.obase
    L.lct_momentum_step(cbw, tw, cbm, tm, dev(gr), mu, eta, ow, om)
    if outs is not None:
        outs.extend([ow, om])
    for out, ref, cb, ocb, name in ((ow, ref_w, cbw, ocw, " W'"), (om, ref_m, cbm, ocm, " M'")):
        g = host_parts(out)
        assert_same(g, ref, what + name)
        assert g["status"] == ref.status
        y = L.decode(cb, out)
        torch.cuda.synchronize()
        assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), orc.decode(ocb, ref))
    return ref_w, ref_m


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(65536, 25), (4096, 1), (8192, 3), (32768, 12), (32768, 11)])
def test_momentum_small_with_spills(L, orc, B, cw, inplace):
    g = np.random.default_rng(B + 3 * cw)
    n = 5 * B + 531
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-2, n))
    gr = synth.to_bf16_bits(g.normal(0, 0.1, n))
    specials = [0x7FC0, 0x7F80, 0xFF80, 0x8000, 0x0001, 0x8001, 0x7F7F, 0xFF7F]
    m[:64] = specials * 8
    w[100:164] = specials * 8
    gr[300:364] = specials * 8
    ref_w, ref_m = momentum_case(L, orc, w, m, gr, synth.Model(1, 0.02), synth.Model(0, 1e-2), 0.9, 0.05,
                                 B, cw, inplace, what="B=%d cw=%d inplace=%s" % (B, cw, inplace))
    if cw == 1:
        assert ref_w.spilled > 0 and ref_m.spilled > 0


@pytest.mark.parametrize("inplace", [False, True])
def test_momentum_full_blocks_escapes_and_nans(L, orc, inplace):
    """The fused momentum kernel's full-block path (no spilled input field):
    runs of escapes that overrun a four-field window in W and in M, and NaNs
    in W, M and the gradient, send single stages through the re-decode and
    the integer rounding.  Every unit must take the full-block path."""
    g = np.random.default_rng(78)
    B, nblk = 65536, 4
    n = nblk * B
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 1e-4, n))
    tiny = synth.to_bf16_bits(np.array([1e-30, -3e-33, 2e-35, -1e-36]))
    for blk, s, j in [(0, 5, 40), (1, 130, 0), (2, 255, 252), (3, 64, 17), (0, 200, 128)]:
        for t in range(4):
            w[blk * B + (j + t) * 256 + s] = tiny[t]
    for blk, s, j in [(1, 7, 30), (2, 100, 161), (3, 250, 9), (0, 63, 200)]:
        for t in range(4):
            m[blk * B + (j + t) * 256 + s] = tiny[t]
    w[1 * B + 100 * 256 + 3] = 0x7FC0          # NaN in W
    m[2 * B + 201 * 256 + 66] = 0xFFC1          # NaN in M (negative, payload)
    gr[3 * B + 17 * 256 + 129] = 0x7F81         # NaN in g
    gr[0 * B + 255 * 256 + 255] = 0xFF80        # -inf in g: M' and W' infinite
    w[3 * B + 255 * 256 + 255] = 0x7F80         # +inf in W, last element
    ocw = orc.codebook_build(0, 0.02, 0.0, w)
    ocm = orc.codebook_build(0, 1e-3, 0.0, m)
    assert orc.encode(ocw, w, B, 25).spilled == 0
    assert orc.encode(ocm, m, B, 25).spilled == 0
    outs = []
    momentum_case(L, orc, w, m, gr, synth.Model(0, 0.02), synth.Model(0, 1e-3), 0.9, 1e-3, B, 25, inplace,
                  what="momentum escapes/nans inplace=%s" % inplace, outs=outs)
    assert outs[0].full_path_units() == 4 * nblk and outs[1].full_path_units() == 4 * nblk


@pytest.mark.parametrize("B,cw", [(65536, 25), (32768, 11)])
def test_momentum_full_blocks_outputs_spill(L, orc, B, cw):
    """Spill-free inputs on the full-block path whose outputs overflow: a
    gradient far wider than M's codebook makes most of M''s fields escape and
    W' = W - eta M' leave W's codebook too, so both writers run out of room
    mid-stream and spill (the path's checked coding and overflow staging)."""
    g = np.random.default_rng(B + cw + 1)
    nblk = 3
    n = nblk * B
    w = narrow_values(orc, g, 0.02, n)
    m = narrow_values(orc, g, 1e-3, n)
    gr = synth.to_bf16_bits(g.normal(0, 0.5, n))
    ocw, ocm = orc.codebook_build(0, 0.02, 0.0, w), orc.codebook_build(0, 1e-3, 0.0, m)
    assert orc.encode(ocw, w, B, cw).spilled == 0 and orc.encode(ocm, m, B, cw).spilled == 0
    outs = []
    ref_w, ref_m = momentum_case(L, orc, w, m, gr, synth.Model(0, 0.02), synth.Model(0, 1e-3), 0.9, 0.5, B, cw,
                                 False, what="momentum output spills B=%d cw=%d" % (B, cw), outs=outs)
    assert ref_m.spilled > n // 4 and ref_w.spilled > 0
    assert outs[0].full_path_units() == 4 * nblk and outs[1].full_path_units() == 4 * nblk


def test_momentum_zero_rates(L, orc):
    """mu = 0 makes M' the gradient; eta = 0 keeps W (no -0 in W, no zero in g)."""
    g = np.random.default_rng(5)
    n = 3 * 65536 + 17
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    w[w == 0x8000] = 0
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr[(gr & 0x7FFF) == 0] = 0x3A83
    ref_w, ref_m = momentum_case(L, orc, w, m, gr, synth.Model(0, 0.02), synth.Model(0, 1e-3), 0.0, 0.0,
                                 65536, 25, True, what="zero rates")
    assert np.array_equal(orc.decode(orc.codebook_build(0, 1e-3, 0.0, m), ref_m), gr)
    assert np.array_equal(orc.decode(orc.codebook_build(0, 0.02, 0.0, w), ref_w), w)


@pytest.mark.parametrize("inplace", [False, True])
def test_momentum_m_overflow_leaves_w_valid(L, orc, inplace):
    """M' spills past m_out's overflow region: m_out's status says so and its
    fixed side and offsets are complete; W' is computed from M' as rounded
    (one pass), so W' is complete, w_out's status is clean and W' equals the
    oracle's (which computes W' from M' as rounded too)."""
    g = np.random.default_rng(41)
    B, cw = 4096, 1
    n = 6 * B + 77
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-2, n))
    gr = synth.to_bf16_bits(g.normal(0, 0.1, n))
    mw, mm = synth.Model(0, 0.02), synth.Model(0, 1e-2)
    cbw, ocw = check_codebook(L, orc, mw, w)
    cbm, ocm = check_codebook(L, orc, mm, m)
    lay = L.layout(B, cw)
    tw, tm = L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)
    rw, rm = orc.encode(ocw, w, B, cw), orc.encode(ocm, m, B, cw)
    ref_w, ref_m = orc.momentum(ocw, rw, ocm, rm, gr, 0.9, 0.05)
    assert ref_m.spilled > 16 and ref_w.spilled > 0
    ow = L.alloc_tensor(n, lay)                      # W' has room for every spill
    om = L.alloc_tensor(n, lay, ovf_cap=ref_m.spilled // 2)
    if inplace:
        ow.sf, ow.pay, ow.cnt, ow.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        om.sf, om.pay, om.cnt, om.obase = tm.sf, tm.pay, tm.cnt, tm.obase
    L.lct_momentum_step(cbw, tw, cbm, tm, dev(gr), 0.9, 0.05, ow, om)
    gm_ = host_parts(om)
    assert gm_["status"] == L.ST_OVF_FULL
    for k in ["sf", "pay", "cnt", "obase"]:
        assert np.array_equal(gm_[k], getattr(ref_m, k)), "M' " + k
    gw_ = host_parts(ow)
    assert gw_["status"] == 0
    assert_same(gw_, ref_w, "W' beside an overflowing M'")


def test_momentum_gpt162m_flat(L, orc):
    """One momentum step over the flat 162M-parameter set, checked in full."""
    ws, ms, mw, mm, eta = synth.config3()
    w = np.concatenate([synth.draw(s) for s in ws])
    m = np.concatenate([synth.draw(s) for s in ms])
    gr = synth.draw(synth.TensorSpec("g.flat", (w.size,), 3100, "normal", {"sigma": 1e-3}))
    B, cw = synth.mode_layout(synth.CLEAN)
    momentum_case(L, orc, w, m, gr, mw, mm, 0.9, eta, B, cw, True, what="momentum config3")


@pytest.mark.parametrize("n", [1, 255, 4096, 65535, 65536, 65537, 3 * 65536 + 4097])
def test_updates_at_odd_sizes(L, orc, n):
    """The update and the momentum step on tensors of every size class (a
    single element, a partial stream, exactly one block, one element past a
    block), out of place and in place."""
    g = np.random.default_rng(9800 + n % 1000)
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 4e-4, n))
    for inplace in (False, True):
        sgd_case(L, orc, w, m, synth.Model(0, 0.02), synth.Model(0, 1e-3), 1e-3, 65536, 25, inplace,
                 what="n=%d inplace=%s" % (n, inplace))
        momentum_case(L, orc, w, m, gr, synth.Model(0, 0.02), synth.Model(0, 1e-3), 0.9, 1e-3, 65536, 25,
                      inplace, what="n=%d inplace=%s" % (n, inplace))


@pytest.mark.parametrize("eta", [float("inf"), float("-inf"), float("nan")])
@pytest.mark.parametrize("B,cw", [(65536, 25), (32768, 12)])
def test_sgd_with_a_non_finite_learning_rate(L, orc, eta, B, cw):
    """eta = +-inf or NaN: every result is an infinity or NaN (inf * 0 where
    M is zero), each element through the rounding with the NaN check, and
    most exponent fields spill; the bytes are the oracle's."""
    n = 2 * B + 777
    g = np.random.default_rng(9800)
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    m[::97] = 0
    ref = sgd_case(L, orc, w, m, synth.Model(0, 0.02), synth.Model(0, 1e-3), eta, B, cw, False,
                   what="eta=%g" % eta)
    assert ref.spilled > n // 2


def test_momentum_with_non_finite_coefficients(L, orc):
    """mu = NaN makes M' NaN everywhere and W' NaN through it; mu = inf makes
    M' infinite (NaN where M is zero), and then W' = fmaf(-0, M', W) is NaN;
    eta = NaN leaves M' finite and makes W' NaN.  The bytes are the
    oracle's."""
    n = 65536 + 3001
    g = np.random.default_rng(9810)
    w = synth.to_bf16_bits(g.normal(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    gr = synth.to_bf16_bits(g.normal(0, 1e-3, n))
    for mu, eta in [(float("nan"), 1e-3), (float("inf"), 0.0), (0.9, float("nan"))]:
        momentum_case(L, orc, w, m, gr, synth.Model(0, 0.02), synth.Model(0, 1e-3), mu, eta, 65536, 25, False,
                      what="mu=%g eta=%g" % (mu, eta))
