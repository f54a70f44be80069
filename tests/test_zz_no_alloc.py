"""The allocation-free update (lct_sgd_step_noalloc) against lct_sgd_step:
the same bytes on every output buffer, on two calls in a row, the second with
a smaller input (the static working memory keeps the first call's contents),
a tensor too large for the static working memory refused before any
launch, and the call captured in a HIP graph and replayed, every replay
giving the eager step's bytes with eager work between the replays."""
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


def dev(x16):
    return torch.from_numpy(np.ascontiguousarray(x16).view(np.int16)).cuda()


def parts(t):
    torch.cuda.synchronize()
    sz = t.sizes
    spilled = int(t.obase[-1].item())
    return {"sf": t.sf[:sz.sf].cpu().numpy(), "pay": t.pay[:sz.pay // 4].cpu().numpy(),
            "cnt": t.cnt[:sz.cnt // 2].cpu().numpy(), "obase": t.obase.cpu().numpy(),
            "ovf": t.ovf[:min(spilled, t.ovf_cap)].cpu().numpy(), "status": t.status_word()}


def one_case(L, n, B, cw, seed, inplace):
    g = np.random.default_rng(seed)
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1.0, n))
    lay = L.layout(B, cw)
    cbw = L.lct_codebook_build(L.Model(1, 0.02, 0.0), dev(w))
    cbm = L.lct_codebook_build(L.Model(0, 1.0, 0.0), dev(m))
    outs = []
    for fn in (L.lct_sgd_step, L.lct_sgd_step_noalloc):
        tw = L.encode(cbw, dev(w), lay)
        tm = L.encode(cbm, dev(m), lay)
        out = L.alloc_tensor(n, lay)
        if inplace:
            out.sf, out.pay, out.cnt, out.obase = tw.sf, tw.pay, tw.cnt, tw.obase
        if fn is L.lct_sgd_step_noalloc:
            out.scratch = torch.full((16,), 0xEE, dtype=torch.uint8, device="cuda")   # never used
        fn(cbw, tw, cbm, tm, 0.05, out)
        outs.append(parts(out))
    ref, got = outs
    for k in ["sf", "pay", "cnt", "obase", "ovf"]:
        assert np.array_equal(ref[k], got[k]), "%s differs (n=%d cw=%d)" % (k, n, cw)
    assert ref["status"] == got["status"] == 0
    return ref


@pytest.mark.parametrize("inplace", [False, True])
def test_noalloc_matches_the_update_twice(L, inplace):
    # first call: many blocks with spills (fills the static memory's staging
    # areas), then a smaller one
    first = one_case(L, 9 * 8192 + 4001, 8192, 3, 11, inplace)
    assert int(first["obase"][-1]) > 0
    second = one_case(L, 2 * 8192 + 17, 8192, 3, 12, inplace)
    assert int(second["obase"][-1]) > 0
    one_case(L, 3 * 65536 + 5, 65536, 25, 13, inplace)


def test_noalloc_refuses_what_does_not_fit(L):
    n = 1 << 24
    lay = L.layout(65536, 25)
    assert L.lct_sizes(n, lay, n).scratch > L.NOALLOC_SCRATCH_BYTES
    cb = L.lct_codebook_from_lengths([0] * 256, 1, 0)
    t = L.alloc_tensor(n, lay, ovf_cap=0)
    out = L.alloc_tensor(n, lay, ovf_cap=n)
    with pytest.raises(L.LctError, match=r"\[-6\]"):
        L.lct_sgd_step_noalloc(cb, t, cb, t, 0.0, out)


def inputs(L, n, B, cw, seed):
    g = np.random.default_rng(seed)
    w = synth.to_bf16_bits(g.laplace(0, 0.02, n))
    m = synth.to_bf16_bits(g.normal(0, 1.0, n))
    lay = L.layout(B, cw)
    cbw = L.lct_codebook_build(L.Model(1, 0.02, 0.0), dev(w))
    cbm = L.lct_codebook_build(L.Model(0, 1.0, 0.0), dev(m))
    return lay, cbw, cbm, L.encode(cbw, dev(w), lay), L.encode(cbm, dev(m), lay)


@pytest.mark.parametrize("n,B,cw", [(3 * 65536 + 4097, 65536, 25), (5 * 32768 + 300, 32768, 12),
                                    (6 * 8192 + 1000, 8192, 3)])
def test_noalloc_replayed_from_a_graph(L, n, B, cw):
    lay, cbw, cbm, tw, tm = inputs(L, n, B, cw, 21 + cw)
    ref = L.alloc_tensor(n, lay)
    L.lct_sgd_step(cbw, tw, cbm, tm, 0.05, ref)
    want = parts(ref)
    assert want["status"] == 0
    # another tensor's allocation-free step, run eagerly between replays
    olay, ocbw, ocbm, otw, otm = inputs(L, 9 * 8192 + 4001, 8192, 3, 31)
    other = L.alloc_tensor(otw.n, olay)
    other.scratch = None

    out = L.alloc_tensor(n, lay)
    out.scratch = None
    # one eager call first: the static memory's address and the kernels'
    # launch attributes are looked up once, outside the capture
    L.lct_sgd_step_noalloc(cbw, tw, cbm, tm, 0.05, out)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        L.lct_sgd_step_noalloc(cbw, tw, cbm, tm, 0.05, out)
    torch.cuda.synchronize()
    for rep in range(4):
        out.sf.fill_(0x5A)
        out.pay.fill_(-1)
        out.cnt.fill_(-1)
        out.obase.fill_(-1)
        out.ovf.fill_(0x77)
        out.status.fill_(7)
        if rep % 2:
            L.lct_sgd_step_noalloc(ocbw, otw, ocbm, otm, 0.05, other)
            assert int(parts(other)["obase"][-1]) > 0
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = parts(out)
        for k in ["sf", "pay", "cnt", "obase", "ovf"]:
            assert np.array_equal(want[k], got[k]), "replay %d: %s differs" % (rep, k)
        assert got["status"] == 0, rep
