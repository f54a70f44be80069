"""Host-side checks of compressed activation saving: tensors that are not on
the GPU pass through the hooks untouched, so CPU autograd is unchanged."""
import torch


def test_cpu_tensors_pass_through():
    from lossless_bf16_tensor_split_amd.activations import compressed_activations
    torch.manual_seed(0)
    x = torch.randn(64, 96, dtype=torch.bfloat16, requires_grad=True)
    w = torch.randn(128, 96, dtype=torch.bfloat16, requires_grad=True)

    def loss():
        h = torch.nn.functional.linear(x, w)
        return (torch.nn.functional.silu(h) * h).float().square().mean()

    loss().backward()
    gx, gw = x.grad.clone(), w.grad.clone()
    x.grad = w.grad = None
    with compressed_activations(min_elems=1) as codec:
        out = loss()
    out.backward()
    assert codec.saved == 0 and codec.passed > 0
    assert torch.equal(x.grad, gx) and torch.equal(w.grad, gw)


def test_default_model_suits_gated_products(orc):
    """The codec's default code (Student-t, 3 degrees of freedom) against a
    Gaussian code on a gated MLP's activations, through the oracle's encoder:
    on the heavy-tailed product silu(g) * u it spills far fewer fields, and
    on the near-Gaussian input of the gate it stores the same size."""
    import numpy as np
    from lossless_bf16_tensor_split_amd import GAUSSIAN, POWERLAW
    from lossless_bf16_tensor_split_amd.activations import ActivationCodec
    m = ActivationCodec().model
    assert (m.family, m.scale, m.shape) == (POWERLAW, 1.0, 3.0)
    f = torch.nn.functional
    g = torch.Generator().manual_seed(9000)
    x = torch.randn(64, 2560, generator=g).to(torch.bfloat16)
    w = [(torch.randn(4096, 2560, generator=g) * 0.02).to(torch.bfloat16) for _ in range(2)]
    gate = f.linear(x, w[0])
    prod = f.silu(gate) * f.linear(x, w[1])

    def stored(t, fam, shape):
        bits = t.contiguous().view(torch.int16).numpy().view(np.uint16).ravel()
        c = orc.encode(orc.codebook_build(fam, 1.0, shape, bits), bits, 65536, 25)
        return c.spilled, len(bits) + c.pay.nbytes + c.cnt.nbytes + c.obase.nbytes + c.spilled

    sp_g, size_g = stored(prod, GAUSSIAN, 0.0)
    sp_t, size_t = stored(prod, POWERLAW, 3.0)
    assert sp_t < 0.6 * sp_g and size_t < size_g
    assert stored(gate, POWERLAW, 3.0)[1] <= stored(gate, GAUSSIAN, 0.0)[1]


def test_codec_reused_across_steps():
    """One codec entered once per step: the hooks are installed only inside,
    a second enter while inside is refused, and the counts add up."""
    from lossless_bf16_tensor_split_amd.activations import ActivationCodec
    import pytest
    codec = ActivationCodec(min_elems=1)
    x = torch.randn(32, 48, dtype=torch.bfloat16, requires_grad=True)
    for step in range(3):
        with codec:
            with pytest.raises(RuntimeError):
                codec.__enter__()
            y = (torch.nn.functional.silu(x) * x).float().sum()
        y.backward()
        assert codec.passed > 0 and codec.saved == 0       # CPU tensors pass through
    passed = codec.passed
    (torch.nn.functional.silu(x) * x).float().sum().backward()  # outside: no hooks
    assert codec.passed == passed
