"""The binding's own checks of the buffers it hands to the library, which
cannot see their sizes: each case raises before any call reaches the device."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import lossless_bf16_tensor_split_amd as L
    return L


def test_buffers_too_small_or_not_on_the_device_are_refused(L):
    n = 3 * 65536 + 17
    lay = L.layout(65536, 25)
    cb = L.lct_codebook_build(L.Model(0, 0.02, 0.0), None)
    x = (torch.randn(n, device="cuda") * 0.02).to(torch.bfloat16)
    w, m = L.encode(cb, x, lay), L.encode(cb, x, lay)
    torch.cuda.synchronize()
    sz = L.lct_sizes(n, lay, L.full_ovf_cap(n, lay))
    need = {"sf": sz.sf, "pay": sz.pay, "cnt": sz.cnt, "obase": sz.obase, "status": 4, "scratch": sz.scratch}
    for name in ("sf", "pay", "cnt", "obase", "status", "scratch"):
        out = L.alloc_tensor(n, lay)
        buf = getattr(out, name)
        # one element short of what the tensor needs
        setattr(out, name, buf[: need[name] // buf.element_size() - 1])
        with pytest.raises(ValueError, match=name):
            L.lct_sgd_step(cb, w, cb, m, 1e-3, out)
        setattr(out, name, buf.cpu())
        with pytest.raises(ValueError, match=name):
            L.lct_sgd_step(cb, w, cb, m, 1e-3, out)
    out = L.alloc_tensor(n, lay)
    out.ovf = out.ovf[:16]
    with pytest.raises(ValueError, match="ovf"):
        L.lct_encode(cb, x, out)
    # a strided view handed as a buffer
    out = L.alloc_tensor(n, lay)
    out.pay = torch.empty(2 * out.pay.numel(), dtype=torch.int32, device="cuda")[::2]
    with pytest.raises(ValueError, match="pay"):
        L.lct_decode(cb, out, torch.empty(n, dtype=torch.bfloat16, device="cuda"))
    # the allocation-free call does not use the scratch buffer
    out = L.alloc_tensor(n, lay)
    out.scratch = torch.empty(16, dtype=torch.uint8, device="cuda")
    L.lct_sgd_step_noalloc(cb, w, cb, m, 1e-3, out)
    torch.cuda.synchronize()
    assert out.status_word() == 0


def test_dense_inputs_are_checked(L):
    n = 70000
    lay = L.layout(65536, 25)
    cb = L.lct_codebook_build(L.Model(0, 0.02, 0.0), None)
    x = (torch.randn(n, device="cuda") * 0.02).to(torch.bfloat16)
    w, m = L.encode(cb, x, lay), L.encode(cb, x, lay)
    wo, mo = L.alloc_tensor(n, lay), L.alloc_tensor(n, lay)
    with pytest.raises(ValueError, match="g has"):
        L.lct_momentum_step(cb, w, cb, m, x[:-1], 0.9, 1e-3, wo, mo)
    with pytest.raises(ValueError, match="GPU"):
        L.lct_momentum_step(cb, w, cb, m, x.cpu(), 0.9, 1e-3, wo, mo)
    with pytest.raises(TypeError):
        L.lct_momentum_step(cb, w, cb, m, x.float(), 0.9, 1e-3, wo, mo)
    with pytest.raises(ValueError, match="GPU"):
        L.lct_codebook_build(L.Model(0, 0.02, 0.0), x.cpu())
    with pytest.raises(TypeError):
        L.lct_codebook_reshift_dense(cb, x.float())
    with pytest.raises(ValueError, match="dense tensor"):
        L.LctGroup([n, 5], lay, [cb, cb], [x[:100], x[:5]])
    # the checked calls still run
    L.lct_momentum_step(cb, w, cb, m, x, 0.9, 1e-3, wo, mo)
    y = L.decode(cb, wo)
    torch.cuda.synchronize()
    assert wo.status_word() == 0 and mo.status_word() == 0 and y.numel() == n
    assert np.isfinite(y.float().cpu().numpy()).all()


def test_calls_on_a_side_stream_match_the_default_stream(L):
    """Encode, update, momentum step and decode enqueued on a side stream
    (default priority) give the same bytes as on the default stream: every
    launch goes to the caller's stream and waits for nothing else."""
    n = 5 * 65536 + 999
    lay = L.layout(65536, 25)
    torch.manual_seed(9400)
    w = (torch.randn(n, device="cuda") * 0.02).to(torch.bfloat16)
    m = (torch.randn(n, device="cuda") * 1e-3).to(torch.bfloat16)
    g = (torch.randn(n, device="cuda") * 1e-3).to(torch.bfloat16)
    cbw = L.lct_codebook_build(L.Model(0, 0.02, 0.0), w)
    cbm = L.lct_codebook_build(L.Model(0, 1e-3, 0.0), m)

    def run():
        tw, tm = L.encode(cbw, w, lay), L.encode(cbm, m, lay)
        out = L.alloc_tensor(n, lay)
        L.lct_sgd_step(cbw, tw, cbm, tm, 1e-3, out)
        wo, mo = L.alloc_tensor(n, lay), L.alloc_tensor(n, lay)
        L.lct_momentum_step(cbw, out, cbm, tm, g, 0.9, 1e-3, wo, mo)
        return out, wo, mo, L.decode(cbw, wo)

    ref = run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run()
    side.synchronize()
    for a, b in zip(ref[:3], got[:3]):
        sz = a.sizes
        assert torch.equal(a.sf[:sz.sf], b.sf[:sz.sf]) and torch.equal(a.pay[:sz.pay // 4], b.pay[:sz.pay // 4])
        assert torch.equal(a.cnt[:sz.cnt // 2], b.cnt[:sz.cnt // 2]) and torch.equal(a.obase, b.obase)
        assert a.status_word() == b.status_word() == 0
    assert torch.equal(ref[3].view(torch.int16), got[3].view(torch.int16))
