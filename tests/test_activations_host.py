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
