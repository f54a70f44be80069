"""GPU parity of tensor groups (many tensors per launch, one shared overflow
region) against the oracle's groups, through the C ABI: the storage arrays
byte for byte (zero padding between members included), the shared region, members read
back with the single-tensor calls, and the group update."""
import numpy as np
import pytest
import torch

import synth
from test_gpu_parity import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bf16_tensor_split_amd as L
    return L


def bits(t):
    torch.cuda.synchronize()
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def storage_equal(L, g, all_, ref, ns, what):
    torch.cuda.synchronize()
    sz = g.sizes(all_.ovf_cap)
    pay = all_.pay[:sz.pay // 4].cpu().numpy().view(np.uint32)
    cnt = all_.cnt[:sz.cnt // 2].cpu().numpy().view(np.uint16)
    ob = all_.obase.cpu().numpy().view(np.uint64)
    sf = all_.sf[:sz.sf].cpu().numpy()
    assert np.array_equal(pay, ref.pay), what + " pay"
    assert np.array_equal(cnt, ref.cnt), what + " cnt"
    assert np.array_equal(ob, ref.obase), what + " obase"
    # every byte, the padding between members included (storage starts zeroed
    # and no call writes the padding)
    assert np.array_equal(sf, ref.sf), what + " sf"
    assert int(all_.status[0].item()) == ref.status
    if ref.status == 0:          # a region that was too small holds unspecified bytes
        sp = ref.spilled
        assert np.array_equal(all_.ovf[:sp].cpu().numpy(), ref.ovf[:sp]), what + " ovf"


def make_group(L, orc, ns, B, cw, seed, scale0=0.02):
    g = np.random.default_rng(seed)
    xs = [synth.to_bf16_bits(g.laplace(0, scale0 * (1 + k % 3), n)) for k, n in enumerate(ns)]
    ocbs = [orc.codebook_build(1, scale0 * (1 + k % 3), 0.0, x) for k, x in enumerate(xs)]
    cbs = [L.lct_codebook_from_lengths(list(c.len_base), c.esc_len, c.shift) for c in ocbs]
    dense = [dev(x).view(torch.bfloat16) if len(x) else torch.empty(8, dtype=torch.bfloat16, device="cuda")
             for x in xs]
    grp = L.LctGroup(ns, L.layout(B, cw), cbs, dense)
    return xs, ocbs, cbs, dense, grp


SIZES = [3 * 65536 + 5, 0, 1, 255, 4097, 65536, 2 * 65536 + 300, 70000, 256, 9000]


@pytest.mark.parametrize("B,cw", [(4096, 2), (65536, 25), (32768, 12), (32768, 11), (8192, 3)])
def test_group_encode_decode(L, orc, B, cw):
    xs, ocbs, cbs, dense, grp = make_group(L, orc, SIZES, B, cw, 9400 + cw)
    ref = orc.encode_group(ocbs, xs, B, cw)
    all_ = grp.alloc_storage(max(ref.spilled, 1) + 100)
    L.lct_encode_group(grp, all_)
    storage_equal(L, grp, all_, ref, SIZES, "B=%d cw=%d" % (B, cw))
    if cw <= 3:
        assert ref.spilled > 0
    # members read back with the single-tensor decode
    for k, (x, cb) in enumerate(zip(xs, cbs)):
        if not len(x):
            continue
        y = torch.empty(len(x), dtype=torch.bfloat16, device="cuda")
        L.lct_decode(cb, grp.tensor(all_, k), y)
        assert np.array_equal(bits(y), x), k
    # the group decode writes every dense buffer back
    for d in dense:
        d.zero_()
    L.lct_decode_group(grp, all_)
    for x, d in zip(xs, dense):
        assert np.array_equal(bits(d)[:len(x)], x)


def test_group_shared_region_too_small(L, orc):
    B, cw = 4096, 1
    xs, ocbs, cbs, dense, grp = make_group(L, orc, SIZES, B, cw, 9500)
    full = orc.encode_group(ocbs, xs, B, cw)
    cap = full.spilled // 2
    ref = orc.encode_group(ocbs, xs, B, cw, ovf_cap=cap)
    all_ = grp.alloc_storage(cap)
    guard = torch.full((cap + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    all_.ovf = guard
    L.lct_encode_group(grp, all_)
    storage_equal(L, grp, all_, ref, SIZES, "small region")
    assert (guard[cap:].cpu().numpy() == 0xA5).all()


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(65536, 25), (4096, 2), (32768, 12), (32768, 11)])
def test_group_sgd(L, orc, B, cw, inplace):
    """W and M groups with per-tensor codebooks: full blocks without spills
    take the update's pipelined path, the rest its general path."""
    ns = [2 * 65536, 65536 + 17, 5, 0, 3 * 65536, 40000]
    g = np.random.default_rng(9600 + cw)
    ws = [synth.to_bf16_bits(g.normal(0, 0.02 * (k + 1), n)) for k, n in enumerate(ns)]
    ms = [synth.to_bf16_bits(g.normal(0, 1e-3 * (k + 1), n)) for k, n in enumerate(ns)]
    ocw = [orc.codebook_build(0, 0.02 * (k + 1), 0.0, w) for k, w in enumerate(ws)]
    ocm = [orc.codebook_build(0, 1e-3 * (k + 1), 0.0, m) for k, m in enumerate(ms)]
    lib_cb = lambda c: L.lct_codebook_from_lengths(list(c.len_base), c.esc_len, c.shift)
    lay = L.layout(B, cw)
    wd = [dev(w).view(torch.bfloat16) if len(w) else torch.empty(8, dtype=torch.bfloat16, device="cuda")
          for w in ws]
    md = [dev(m).view(torch.bfloat16) if len(m) else torch.empty(8, dtype=torch.bfloat16, device="cuda")
          for m in ms]
    gw = L.LctGroup(ns, lay, [lib_cb(c) for c in ocw], wd)
    gm = L.LctGroup(ns, lay, [lib_cb(c) for c in ocm], md)
    rw = [orc.encode(c, w, B, cw) for c, w in zip(ocw, ws)]
    rm = [orc.encode(c, m, B, cw) for c, m in zip(ocm, ms)]
    cap = sum(len(w) for w in ws)
    w_all, m_all = gw.alloc_storage(cap), gm.alloc_storage(cap)
    L.lct_encode_group(gw, w_all)
    L.lct_encode_group(gm, m_all)
    storage_equal(L, gw, w_all, orc.group(rw, cap), ns, "W")
    storage_equal(L, gm, m_all, orc.group(rm, cap), ns, "M")
    ref = orc.group([orc.sgd(ocw[k], rw[k], ocm[k], rm[k], 1e-3) for k in range(len(ns))], cap)
    out = gw.alloc_storage(cap)
    if inplace:
        out.sf, out.pay, out.cnt, out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase
    L.lct_sgd_step_group(gw, w_all, gm, m_all, 1e-3, out)
    storage_equal(L, gw, out, ref, ns, "W' inplace=%s" % inplace)
    if B == 65536:
        assert ref.spilled == 0
    # groups of other sizes are refused
    other = L.LctGroup(ns[:-1] + [ns[-1] + 1], lay, [lib_cb(c) for c in ocm], None)
    with pytest.raises(L.LctError):
        L.lct_sgd_step_group(gw, w_all, other, other.alloc_storage(cap), 1e-3, out)


@pytest.mark.parametrize("ns", [[0], [0, 0, 0]])
def test_group_all_empty(L, orc, ns):
    """A group whose members are all empty has no blocks: every group call
    writes nothing, and the storage as allocated already holds the empty
    encoding (obase = [0], status 0)."""
    B, cw = 65536, 25
    xs, ocbs, cbs, dense, grp = make_group(L, orc, ns, B, cw, 9700 + len(ns))
    ref = orc.encode_group(ocbs, xs, B, cw)
    assert ref.obase.tolist() == [0] and ref.status == 0
    all_ = grp.alloc_storage(16)
    L.lct_encode_group(grp, all_)
    storage_equal(L, grp, all_, ref, ns, "encode")
    gm = L.LctGroup(ns, L.layout(B, cw), cbs, dense)
    m_all = gm.alloc_storage(16)
    L.lct_encode_group(gm, m_all)
    out = grp.alloc_storage(16)
    L.lct_sgd_step_group(grp, all_, gm, m_all, 1e-3, out)
    storage_equal(L, grp, out, ref, ns, "update")
    L.lct_decode_group(grp, out)
    torch.cuda.synchronize()


@pytest.mark.parametrize("inplace", [False, True])
def test_group_sgd_readers_far_apart(L, orc, inplace):
    """The group update at the CLEAN capacity with M tensors whose streams
    drift hundreds of bits apart (every fourth stream of a unit opens, or goes
    on at mid-stream, with 20 escaped fields while its neighbours keep
    two-bit codes), so that the far readers' windows come from memory rather
    than the rows held of M; a second pair of tensors is ordinary.  W' equals
    the oracle's, in place and not."""
    from test_gpu_parity import narrow_values
    B, cw = 65536, 25
    ns = [3 * 65536, 2 * 65536]
    g = np.random.default_rng(9650)
    ws = [narrow_values(orc, g, 0.02, n) for n in ns]
    ms = [narrow_values(orc, g, 1e-3, ns[0], extra=0.0), synth.to_bf16_bits(g.normal(0, 1e-3, ns[1]))]
    tiny = synth.to_bf16_bits(np.array([1e-30, -3e-33, 2e-35, -1e-36]))
    for blk, j0 in [(0, 0), (1, 100), (2, 230)]:
        for s_ in range(0, 256, 4):
            for t in range(20):
                ms[0][blk * B + (j0 + t) * 256 + s_] = tiny[(s_ + t) % 4]
    ocw = [orc.codebook_build(0, 0.02, 0.0, w) for w in ws]
    ocm = [orc.codebook_build(0, 1e-3, 0.0, m) for m in ms]
    rw = [orc.encode(c, w, B, cw) for c, w in zip(ocw, ws)]
    rm = [orc.encode(c, m, B, cw) for c, m in zip(ocm, ms)]
    assert rm[0].spilled == 0 and rw[0].spilled == 0
    lib_cb = lambda c: L.lct_codebook_from_lengths(list(c.len_base), c.esc_len, c.shift)
    lay = L.layout(B, cw)
    gw = L.LctGroup(ns, lay, [lib_cb(c) for c in ocw], [dev(w).view(torch.bfloat16) for w in ws])
    gm = L.LctGroup(ns, lay, [lib_cb(c) for c in ocm], [dev(m).view(torch.bfloat16) for m in ms])
    cap = sum(ns)
    w_all, m_all = gw.alloc_storage(cap), gm.alloc_storage(cap)
    L.lct_encode_group(gw, w_all)
    L.lct_encode_group(gm, m_all)
    storage_equal(L, gm, m_all, orc.group(rm, cap), ns, "M")
    ref = orc.group([orc.sgd(ocw[k], rw[k], ocm[k], rm[k], 1e-3) for k in range(len(ns))], cap)
    out = gw.alloc_storage(cap)
    if inplace:
        out.sf, out.pay, out.cnt, out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase
    L.lct_sgd_step_group(gw, w_all, gm, m_all, 1e-3, out)
    storage_equal(L, gw, out, ref, ns, "W' far readers inplace=%s" % inplace)


@pytest.mark.parametrize("inplace", [False, True])
@pytest.mark.parametrize("B,cw", [(65536, 25), (8192, 3), (32768, 12), (32768, 11)])
def test_group_momentum(L, orc, B, cw, inplace):
    """Momentum step on groups: W and M with per-tensor codebooks, the
    gradients bound as a third group's dense buffers."""
    ns = [65536 + 300, 2 * 65536, 7, 0, 100000]
    g = np.random.default_rng(9700 + cw)
    ws = [synth.to_bf16_bits(g.normal(0, 0.02 * (k + 1), n)) for k, n in enumerate(ns)]
    ms = [synth.to_bf16_bits(g.normal(0, 1e-3 * (k + 1), n)) for k, n in enumerate(ns)]
    gs = [synth.to_bf16_bits(g.normal(0, 4e-4 * (k + 1), n)) for k, n in enumerate(ns)]
    ocw = [orc.codebook_build(0, 0.02 * (k + 1), 0.0, w) for k, w in enumerate(ws)]
    ocm = [orc.codebook_build(0, 1e-3 * (k + 1), 0.0, m) for k, m in enumerate(ms)]
    lib_cb = lambda c: L.lct_codebook_from_lengths(list(c.len_base), c.esc_len, c.shift)
    lay = L.layout(B, cw)
    todev = lambda x: (dev(x).view(torch.bfloat16) if len(x)
                       else torch.empty(8, dtype=torch.bfloat16, device="cuda"))
    wd, md, gd = [todev(x) for x in ws], [todev(x) for x in ms], [todev(x) for x in gs]
    gw = L.LctGroup(ns, lay, [lib_cb(c) for c in ocw], wd)
    gm = L.LctGroup(ns, lay, [lib_cb(c) for c in ocm], md)
    gg = L.LctGroup(ns, lay, [lib_cb(c) for c in ocm], gd)
    cap = sum(ns)
    w_all, m_all = gw.alloc_storage(cap), gm.alloc_storage(cap)
    L.lct_encode_group(gw, w_all)
    L.lct_encode_group(gm, m_all)
    rw = [orc.encode(c, x, B, cw) for c, x in zip(ocw, ws)]
    rm = [orc.encode(c, x, B, cw) for c, x in zip(ocm, ms)]
    refs = [orc.momentum(ocw[k], rw[k], ocm[k], rm[k], gs[k], 0.9, 1e-3) for k in range(len(ns))]
    w_out, m_out = gw.alloc_storage(cap), gm.alloc_storage(cap)
    if inplace:
        w_out.sf, w_out.pay, w_out.cnt, w_out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase
        m_out.sf, m_out.pay, m_out.cnt, m_out.obase = m_all.sf, m_all.pay, m_all.cnt, m_all.obase
    L.lct_momentum_step_group(gw, w_all, gm, m_all, gg, 0.9, 1e-3, w_out, m_out)
    storage_equal(L, gw, w_out, orc.group([r[0] for r in refs], cap), ns, "W' inplace=%s" % inplace)
    storage_equal(L, gm, m_out, orc.group([r[1] for r in refs], cap), ns, "M' inplace=%s" % inplace)
    if cw == 3:
        assert sum(r[1].spilled for r in refs) > 0


@pytest.mark.parametrize("inplace", [False, True])
def test_group_sgd_shared_tables(L, orc, inplace):
    """Tensors that share code tables (same model and shift) share one table
    index in the group's device table, and the update, which stages tables
    only when the index pair changes, still matches the oracle when the
    tensors' tables alternate."""
    B, cw = 65536, 25
    ns = [2 * B] * 6 + [B + 999]
    g = np.random.default_rng(9800)
    wsig = [0.02, 0.08, 0.02, 0.02, 0.08, 0.02, 0.02]       # two W codebooks (shifts 0 and 2)
    msig = [1e-3, 1e-3, 4e-3, 1e-3, 4e-3, 4e-3, 1e-3]       # two M codebooks
    ws = [synth.to_bf16_bits(g.normal(0, s, n)) for s, n in zip(wsig, ns)]
    ms = [synth.to_bf16_bits(g.normal(0, s, n)) for s, n in zip(msig, ns)]
    ocw = [orc.codebook_build(0, 0.02, 0.0, w) for w in ws]
    ocm = [orc.codebook_build(0, 1e-3, 0.0, m) for m in ms]
    assert len({int(c.shift) for c in ocw}) == 2 and len({int(c.shift) for c in ocm}) == 2
    lib_cb = lambda c: L.lct_codebook_from_lengths(list(c.len_base), c.esc_len, c.shift)
    lay = L.layout(B, cw)
    gw = L.LctGroup(ns, lay, [lib_cb(c) for c in ocw], [dev(w).view(torch.bfloat16) for w in ws])
    gm = L.LctGroup(ns, lay, [lib_cb(c) for c in ocm], [dev(m).view(torch.bfloat16) for m in ms])
    # the table index of every block: the first tensor with the same tables
    for grp, ocs in ((gw, ocw), (gm, ocm)):
        nblk = int(grp.g.nblk)
        tab = grp.table.cpu().numpy()
        owner_at = len(tab) - 4 * nblk                      # blk_tab is the last part (256-aligned)
        owner_at -= owner_at % 256
        blk_tab = tab[owner_at:owner_at + 4 * nblk].view(np.uint32)
        want = []
        for k, c in enumerate(ocs):
            first = next(j for j in range(k + 1) if ocs[j].shift == c.shift)
            want += [first] * (-(-ns[k] // B))
        assert blk_tab.tolist() == want
    rw = [orc.encode(c, w, B, cw) for c, w in zip(ocw, ws)]
    rm = [orc.encode(c, m, B, cw) for c, m in zip(ocm, ms)]
    cap = sum(ns)
    w_all, m_all = gw.alloc_storage(cap), gm.alloc_storage(cap)
    L.lct_encode_group(gw, w_all)
    L.lct_encode_group(gm, m_all)
    storage_equal(L, gw, w_all, orc.group(rw, cap), ns, "W")
    ref = orc.group([orc.sgd(ocw[k], rw[k], ocm[k], rm[k], 1e-3) for k in range(len(ns))], cap)
    out = gw.alloc_storage(cap)
    if inplace:
        out.sf, out.pay, out.cnt, out.obase = w_all.sf, w_all.pay, w_all.cnt, w_all.obase
    L.lct_sgd_step_group(gw, w_all, gm, m_all, 1e-3, out)
    storage_equal(L, gw, out, ref, ns, "W' shared tables inplace=%s" % inplace)
