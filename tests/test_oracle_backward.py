"""Pins of the oracle's MLP backward (CPU only): torch autograd through a
forward written with torch's own tanh-GELU in fp64 (independent of the oracle's
code), central finite differences of the GELU derivative, and the additivity of
the weight-gradient contributions over token sets."""
import torch
import torch.nn.functional as F

from oracle import tsp_oracle as O

F64 = torch.float64


def test_gelu_grad_matches_finite_differences():
    u = torch.linspace(-8, 8, 1601, dtype=F64)
    hstep = 1e-5
    fd = (O.gelu_tanh(u + hstep) - O.gelu_tanh(u - hstep)) / (2 * hstep)
    assert torch.allclose(O.gelu_tanh_grad(u), fd, rtol=1e-8, atol=1e-9)


def test_gelu_grad_matches_autograd():
    u = torch.linspace(-10, 10, 2001, dtype=F64, requires_grad=True)
    (g,) = torch.autograd.grad(O.gelu_tanh(u).sum(), u)
    assert torch.allclose(O.gelu_tanh_grad(u.detach()), g, rtol=1e-13, atol=1e-14)


def _problem(n, h, F, D, seed):
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, h, generator=g, dtype=F64)
    w1 = [torch.randn(F // D, h, generator=g, dtype=F64) * 0.05 for _ in range(D)]
    w2 = [torch.randn(h, F // D, generator=g, dtype=F64) * 0.05 for _ in range(D)]
    dy = torch.randn(n, h, generator=g, dtype=F64)
    return x, w1, w2, dy


def test_mlp_backward_matches_autograd():
    for residual in (False, True):
        x, w1, w2, dy = _problem(13, 16, 48, 3, 1)
        xa = x.clone().requires_grad_(True)
        w1a = [w.clone().requires_grad_(True) for w in w1]
        w2a = [w.clone().requires_grad_(True) for w in w2]
        y = sum(F.gelu(xa @ w1a[d].t(), approximate="tanh") @ w2a[d].t() for d in range(3))
        y = y + (xa if residual else 0)
        grads = torch.autograd.grad((y * dy).sum(), [xa, *w1a, *w2a])
        dx, dw1, dw2 = O.mlp_backward(x, w1, w2, dy, residual=residual)
        assert torch.allclose(dx, grads[0], rtol=1e-12, atol=1e-12)
        for d in range(3):
            assert torch.allclose(dw1[d], grads[1 + d], rtol=1e-12, atol=1e-12)
            assert torch.allclose(dw2[d], grads[4 + d], rtol=1e-12, atol=1e-12)


def test_mlp_backward_weight_gradients_add_over_token_sets():
    # the contributions of two ranks' token sets add up to the gradient over their union
    x, w1, w2, dy = _problem(20, 16, 32, 2, 2)
    _, a1, a2 = O.mlp_backward(x[:8], w1, w2, dy[:8])
    _, b1, b2 = O.mlp_backward(x[8:], w1, w2, dy[8:])
    _, c1, c2 = O.mlp_backward(x, w1, w2, dy)
    for d in range(2):
        assert torch.allclose(a1[d] + b1[d], c1[d], rtol=1e-12, atol=1e-12)
        assert torch.allclose(a2[d] + b2[d], c2[d], rtol=1e-12, atol=1e-12)
