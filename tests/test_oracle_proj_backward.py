"""Pins of the oracle's projection backwards (CPU only): torch autograd through
forwards written here with torch's own linear map in fp64 (independent of the
oracle's code), the shard identity (the shards' weight gradients stacked are
the whole matrix's gradient), and additivity over token sets."""
import torch
import torch.nn.functional as F

from oracle import tsp_oracle as O

F64 = torch.float64


def _g(seed):
    return torch.Generator().manual_seed(seed)


def test_attn_out_backward_matches_autograd():
    g = _g(1)
    n, h, D = 11, 24, 3
    hs = h // D
    attn = torch.randn(n, h, generator=g, dtype=F64)
    wo = [torch.randn(h, hs, generator=g, dtype=F64) for _ in range(D)]
    dout = torch.randn(n, h, generator=g, dtype=F64)
    a = attn.clone().requires_grad_(True)
    ws = [w.clone().requires_grad_(True) for w in wo]
    out = sum(F.linear(a[:, d * hs:(d + 1) * hs], ws[d]) for d in range(D))
    grads = torch.autograd.grad(out, [a] + ws, grad_outputs=dout)
    d_attn, dwo = O.attn_out_backward(attn, wo, dout)
    assert torch.allclose(d_attn, grads[0], rtol=1e-13, atol=1e-13)
    for d in range(D):
        assert torch.allclose(dwo[d], grads[1 + d], rtol=1e-13, atol=1e-13)
    # whole-matrix identity: W_o = [W_o_0 | W_o_1 | ...] columns; dW_o = d_out^T attn
    assert torch.allclose(torch.cat(dwo, dim=1), dout.t() @ attn, rtol=1e-13, atol=1e-13)


def test_qkv_projection_backward_matches_autograd():
    g = _g(2)
    n, H, hd, D = 9, 4, 8, 2
    h, Hs = H * hd, H // D
    hs = Hs * hd
    x = torch.randn(n, h, generator=g, dtype=F64)
    w = [torch.randn(3 * hs, h, generator=g, dtype=F64) for _ in range(D)]
    dq, dk, dv, dy = (torch.randn(n, h, generator=g, dtype=F64) for _ in range(4))
    xa = x.clone().requires_grad_(True)
    wa = [t.clone().requires_grad_(True) for t in w]
    q = torch.cat([F.linear(xa, wa[d][:hs]) for d in range(D)], dim=1)
    k = torch.cat([F.linear(xa, wa[d][hs:2 * hs]) for d in range(D)], dim=1)
    v = torch.cat([F.linear(xa, wa[d][2 * hs:]) for d in range(D)], dim=1)
    loss = (q * dq).sum() + (k * dk).sum() + (v * dv).sum() + (xa * dy).sum()
    grads = torch.autograd.grad(loss, [xa] + wa)
    dx, dw = O.qkv_projection_backward(x, w, dq, dk, dv, hd, dy=dy)
    assert torch.allclose(dx, grads[0], rtol=1e-12, atol=1e-12)
    for d in range(D):
        assert torch.allclose(dw[d], grads[1 + d], rtol=1e-12, atol=1e-12)
    dx0, _ = O.qkv_projection_backward(x, w, dq, dk, dv, hd)
    assert torch.allclose(dx, dx0 + dy, rtol=1e-13, atol=1e-13)
    # the oracle's own forward, checked to be the map differentiated above
    qo, ko, vo = O.qkv_projection(x, w, hd)
    assert torch.allclose(qo, q.detach(), rtol=1e-13) and torch.allclose(vo, v.detach(), rtol=1e-13)


def test_weight_gradients_add_over_token_sets():
    g = _g(3)
    n, H, hd, D = 10, 2, 8, 2
    h, hs = H * hd, (H // D) * hd
    x = torch.randn(n, h, generator=g, dtype=F64)
    w = [torch.randn(3 * hs, h, generator=g, dtype=F64) for _ in range(D)]
    dq, dk, dv = (torch.randn(n, h, generator=g, dtype=F64) for _ in range(3))
    _, whole = O.qkv_projection_backward(x, w, dq, dk, dv, hd)
    _, a = O.qkv_projection_backward(x[:4], w, dq[:4], dk[:4], dv[:4], hd)
    _, b = O.qkv_projection_backward(x[4:], w, dq[4:], dk[4:], dv[4:], hd)
    for d in range(D):
        assert torch.allclose(whole[d], a[d] + b[d], rtol=1e-13, atol=1e-13)
