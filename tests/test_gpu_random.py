"""GPU parity on seeded random cases: the HIP path (through the C ABI) against
the oracle, bit for bit, over layouts, sizes, value distributions, codebooks
that fit the data or not, special values, learning rates, in-place outputs and
overflow regions too small for the spill.

Each case draws its whole configuration from its own seed and names it in the
failure message, so a failing case is reproducible from its id alone.
"""
import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import L, assert_same, check_codebook, dev, host_parts  # noqa: F401

pytestmark = pytest.mark.gpu

LAYOUTS = [(65536, 25), (32768, 12), (32768, 11), (4096, 1), (8192, 3), (4096, 2), (16384, 6), (8192, 4)]
SPECIALS = np.array([0x7FC0, 0xFFC1, 0x7F80, 0xFF80, 0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x7F7F,
                     0xFF7F, 0x0080, 0x7F81], np.uint16)
NCASES = 200
NLARGE = 24
NUS = (1.0, 2.5, 3.0, 7.0, 30.0)   # Student-t degrees of freedom


def draw_values(g, n):
    """BF16 bits from a random family, scale (and Student-t shape), with the model the codebook
    is built from (sometimes off by a power of two, so that fields shift or
    spill), and sometimes a sprinkle of special values."""
    fam = int(g.integers(0, 3))
    scale = float(10.0 ** g.uniform(-4, 0.5))
    if fam == 0:
        x = g.normal(0, scale, n)
    elif fam == 1:
        x = g.laplace(0, scale, n)
    else:
        nu = float(NUS[int(g.integers(0, len(NUS)))])
        x = g.standard_t(nu, n) * scale
    bits = synth.to_bf16_bits(x)
    if g.random() < 0.3 and n > 0:
        k = int(g.integers(1, max(2, n // 50)))
        bits[g.integers(0, n, k)] = SPECIALS[g.integers(0, SPECIALS.size, k)]
    model_scale = scale * float(2.0 ** int(g.integers(-3, 4))) if g.random() < 0.4 else scale
    shape = nu if fam == 2 else 0.0
    return bits, synth.Model(fam, model_scale, shape)


def draw_case(idx):
    g = np.random.default_rng(90210 + idx)
    B, cw = LAYOUTS[int(g.integers(0, len(LAYOUTS)))]
    kind = int(g.integers(0, 5))
    if kind == 0:
        n = int(g.integers(1, 257))
    elif kind == 1:
        n = int(g.integers(1, 3 * B))
    elif kind == 2:
        n = B * int(g.integers(1, 5))
    else:
        n = B * int(g.integers(1, 5)) + int(g.integers(-300, 301))
    n = max(1, min(n, 400000))
    op = ["roundtrip", "sgd", "momentum"][int(g.integers(0, 3))]
    return g, B, cw, n, op


def out_cap(g, spilled):
    """None (room for every spill) or, sometimes, half the spill."""
    return max(0, spilled // 2) if (spilled > 1 and g.random() < 0.25) else None


def same(gp, ref, what):
    """Every buffer equal; with the overflow region too small (status set) the
    region's content is unspecified, so only the fixed side and the offsets
    (complete either way) are compared."""
    assert gp["status"] == ref.status, what + " status"
    if ref.status == 0:
        assert_same(gp, ref, what)
        return
    for k in ["sf", "pay", "cnt", "obase"]:
        assert np.array_equal(gp[k], getattr(ref, k)), what + " " + k


@pytest.mark.parametrize("idx", range(NCASES))
def test_random_case(L, orc, idx):  # noqa: F811
    run_case(L, orc, idx, *draw_case(idx))


def draw_large_case(idx):
    """A case of 8 to 48 blocks (ragged by up to 300 elements either way), in
    any layout: many blocks at once in the update's full-block and general
    kernels, with spills where the layout is small."""
    g = np.random.default_rng(777000 + idx)
    B, cw = LAYOUTS[int(g.integers(0, len(LAYOUTS)))]
    n = B * int(g.integers(8, 49)) + int(g.integers(-300, 301))
    n = max(1, min(n, 3_200_000))
    op = ["roundtrip", "sgd", "momentum"][int(g.integers(0, 3))]
    return g, B, cw, n, op


@pytest.mark.parametrize("idx", range(NLARGE))
def test_random_large_case(L, orc, idx):  # noqa: F811
    run_case(L, orc, idx, *draw_large_case(idx))


def run_case(L, orc, idx, g, B, cw, n, op):
    what = "case %d: %s n=%d layout=(%d,%d)" % (idx, op, n, B, cw)
    lay = L.layout(B, cw)
    w, mw = draw_values(g, n)
    cbw, ocw = check_codebook(L, orc, mw, w)
    rw = orc.encode(ocw, w, B, cw)
    if op == "roundtrip":
        cap = out_cap(g, rw.spilled)
        if cap is not None:
            rw = orc.encode(ocw, w, B, cw, cap)
        t = L.encode(cbw, dev(w), lay, cap)
        same(host_parts(t), rw, what)
        if rw.status == 0:
            y = L.decode(cbw, t)
            torch.cuda.synchronize()
            assert np.array_equal(y.view(torch.int16).cpu().numpy().view(np.uint16), w), what + " decode"
        return
    m, mm = draw_values(g, n)
    cbm, ocm = check_codebook(L, orc, mm, m)
    rm = orc.encode(ocm, m, B, cw)
    tw, tm = L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)
    assert_same(host_parts(tw), rw, what + " W")
    assert_same(host_parts(tm), rm, what + " M")
    inplace = bool(g.random() < 0.5)
    eta = float([1e-3, 0.5, 0.0, -1e-2, 3.0][int(g.integers(0, 5))])
    if op == "sgd":
        ref = orc.sgd(ocw, rw, ocm, rm, eta)
        cap = out_cap(g, ref.spilled)
        if cap is not None:
            ref = orc.sgd(ocw, rw, ocm, rm, eta, cap)
        out = L.alloc_tensor(n, lay, cap)
        if inplace:
            out.sf, out.pay, out.cnt, out.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        L.lct_sgd_step(cbw, tw, cbm, tm, eta, out)
        same(host_parts(out), ref, what + " W' eta=%g inplace=%s" % (eta, inplace))
        return
    gr, _ = draw_values(g, n)
    mu = float([0.9, 0.0, 1.5, 0.99][int(g.integers(0, 4))])
    ref_w, ref_m = orc.momentum(ocw, rw, ocm, rm, gr, mu, eta)
    cap = out_cap(g, max(ref_w.spilled, ref_m.spilled))
    if cap is not None:
        ref_w, ref_m = orc.momentum(ocw, rw, ocm, rm, gr, mu, eta, cap)
    ow, om = L.alloc_tensor(n, lay, cap), L.alloc_tensor(n, lay, cap)
    if inplace:
        ow.sf, ow.pay, ow.cnt, ow.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        om.sf, om.pay, om.cnt, om.obase = tm.sf, tm.pay, tm.cnt, tm.obase
    L.lct_momentum_step(cbw, tw, cbm, tm, dev(gr), mu, eta, ow, om)
    for out, ref, name in ((ow, ref_w, " W'"), (om, ref_m, " M'")):
        same(host_parts(out), ref, what + name + " mu=%g eta=%g inplace=%s" % (mu, eta, inplace))


# ------------------------------------------------------------------ groups

NGROUPS = 40


def lib_cb(L, c):
    return L.lct_codebook_from_lengths(list(c.len_base), c.esc_len, c.shift)


def todev(x):
    return (dev(x).view(torch.bfloat16) if len(x)
            else torch.empty(8, dtype=torch.bfloat16, device="cuda"))


@pytest.mark.parametrize("idx", range(NGROUPS))
def test_random_group(L, orc, idx):  # noqa: F811
    """Random groups (1 to 9 tensors of random sizes, empty ones included,
    each with its own values and codebook) through the group encode, decode,
    update and momentum calls, against the oracle's groups."""
    from test_gpu_group import storage_equal
    g = np.random.default_rng(77000 + idx)
    B, cw = LAYOUTS[int(g.integers(0, len(LAYOUTS)))]
    count = int(g.integers(1, 10))
    ns = []
    for _ in range(count):
        kind = int(g.integers(0, 4))
        ns.append([0, int(g.integers(1, 300)), int(g.integers(1, 2 * B)),
                   B * int(g.integers(1, 3)) + int(g.integers(-200, 201))][kind])
    ns = [max(0, min(n, 200000)) for n in ns]
    op = ["encode", "sgd", "momentum"][int(g.integers(0, 3))]
    what = "group case %d: %s ns=%s layout=(%d,%d)" % (idx, op, ns, B, cw)
    lay = L.layout(B, cw)

    def tensors():
        xs, ocs = [], []
        for n in ns:
            x, model = draw_values(g, n)
            xs.append(x)
            ocs.append(orc.codebook_build(model.family, model.scale, model.shape, x))
        return xs, ocs

    ws, ocw = tensors()
    gw = L.LctGroup(ns, lay, [lib_cb(L, c) for c in ocw], [todev(x) for x in ws])
    rw = [orc.encode(c, x, B, cw) for c, x in zip(ocw, ws)]
    full = sum(r.spilled for r in rw)
    if op == "encode":
        cap = out_cap(g, full)
        cap = full + 64 if cap is None else cap
        all_ = gw.alloc_storage(max(cap, 1))
        L.lct_encode_group(gw, all_)
        ref = orc.group(rw, max(cap, 1))
        storage_equal(L, gw, all_, ref, ns, what)
        if ref.status == 0:
            for d in gw.dense:
                d.zero_()
            L.lct_decode_group(gw, all_)
            for k, (x, d) in enumerate(zip(ws, gw.dense)):
                torch.cuda.synchronize()
                assert np.array_equal(d.view(torch.int16).cpu().numpy().view(np.uint16)[:len(x)], x), what + " %d" % k
        return
    ms, ocm = tensors()
    gm = L.LctGroup(ns, lay, [lib_cb(L, c) for c in ocm], [todev(x) for x in ms])
    rm = [orc.encode(c, x, B, cw) for c, x in zip(ocm, ms)]
    big = sum(ns) + 64
    w_all, m_all = gw.alloc_storage(big), gm.alloc_storage(big)
    L.lct_encode_group(gw, w_all)
    L.lct_encode_group(gm, m_all)
    storage_equal(L, gw, w_all, orc.group(rw, big), ns, what + " W")
    storage_equal(L, gm, m_all, orc.group(rm, big), ns, what + " M")
    inplace = bool(g.random() < 0.5)
    eta = float([1e-3, 0.5, 0.0, -1e-2][int(g.integers(0, 4))])
    if op == "sgd":
        outs = [orc.sgd(ocw[k], rw[k], ocm[k], rm[k], eta) for k in range(count)]
        cap = out_cap(g, sum(o.spilled for o in outs))
        cap = big if cap is None else max(cap, 1)
        out = gw.alloc_storage(cap)
        if inplace:
            out.sf, out.pay, out.cnt, out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase
        L.lct_sgd_step_group(gw, w_all, gm, m_all, eta, out)
        storage_equal(L, gw, out, orc.group(outs, cap), ns, what + " W' eta=%g inplace=%s" % (eta, inplace))
        return
    gs = [draw_values(g, n)[0] for n in ns]
    gg = L.LctGroup(ns, lay, [lib_cb(L, c) for c in ocm], [todev(x) for x in gs])
    mu = float([0.9, 0.0, 1.5][int(g.integers(0, 3))])
    refs = [orc.momentum(ocw[k], rw[k], ocm[k], rm[k], gs[k], mu, eta) for k in range(count)]
    cap = out_cap(g, max(sum(r[0].spilled for r in refs), sum(r[1].spilled for r in refs)))
    cap = big if cap is None else max(cap, 1)
    w_out, m_out = gw.alloc_storage(cap), gm.alloc_storage(cap)
    if inplace:
        w_out.sf, w_out.pay, w_out.cnt, w_out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase
        m_out.sf, m_out.pay, m_out.cnt, m_out.obase = m_all.sf, m_all.pay, m_all.cnt, m_all.obase
    L.lct_momentum_step_group(gw, w_all, gm, m_all, gg, mu, eta, w_out, m_out)
    tag = " mu=%g eta=%g inplace=%s" % (mu, eta, inplace)
    storage_equal(L, gw, w_out, orc.group([r[0] for r in refs], cap), ns, what + " W'" + tag)
    storage_equal(L, gm, m_out, orc.group([r[1] for r in refs], cap), ns, what + " M'" + tag)
