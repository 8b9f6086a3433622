"""Pins of the oracle's attention backward and softmax normaliser (CPU only).

Each is checked against something other than its own code:
  * torch autograd through torch's scaled-dot-product attention (a library
    forward, fp64) with an explicit causal mask at zigzag positions;
  * central finite differences of the oracle's own forward (a different
    function from the backward);
  * the zigzag identity: summing every rank's dk/dv contributions, and
    placing every rank's dq rows, gives the gradients of the full-sequence
    causal attention (library autograd with is_causal);
  * invariants: the key gradients of one head sum to zero over the keys (the
    softmax is shift-invariant), the value gradients sum to the sum of the
    output gradients, constant values give zero query and key gradients, keys
    past every local query get nothing;
  * the normaliser against torch.logsumexp, the forward's probabilities
    against exp(s - lse), and the one-key closed form.
"""
import math

import pytest
import torch
import torch.nn.functional as F

from oracle import tsp_oracle as O

F64 = torch.float64


def _inputs(m, S, H, hd, seed, positions=None):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(m, H * hd, generator=g, dtype=F64)
    k = torch.randn(S, H * hd, generator=g, dtype=F64)
    v = torch.randn(S, H * hd, generator=g, dtype=F64)
    do = torch.randn(m, H * hd, generator=g, dtype=F64)
    if positions is None:
        positions = torch.sort(torch.randperm(S, generator=g)[:m]).values
    return q, k, v, do, positions


def _heads(t, H, hd):
    return t.reshape(t.shape[0], H, hd).transpose(0, 1)  # [H, rows, hd]


def _flat(t):
    return t.transpose(0, 1).reshape(t.shape[1], -1)


def _library_grads(q, k, v, do, positions, H, hd):
    """autograd of torch's SDPA with an explicit boolean mask (True = attend)."""
    S = k.shape[0]
    mask = torch.arange(S)[None, :] <= positions[:, None]
    qa, ka, va = (_heads(t, H, hd).clone().requires_grad_(True) for t in (q, k, v))
    o = F.scaled_dot_product_attention(qa[None], ka[None], va[None], attn_mask=mask[None, None])[0]
    gq, gk, gv = torch.autograd.grad(o, (qa, ka, va), grad_outputs=_heads(do, H, hd))
    return _flat(gq), _flat(gk), _flat(gv)


@pytest.mark.parametrize("m,S,H,hd", [(7, 20, 2, 8), (16, 16, 1, 4), (25, 64, 3, 16)])
def test_backward_matches_library_autograd(m, S, H, hd):
    q, k, v, do, pos = _inputs(m, S, H, hd, 1 + m)
    dq, dk, dv = O.causal_attention_backward(q, pos, k, v, do, H, hd)
    lq, lk, lv = _library_grads(q, k, v, do, pos, H, hd)
    for got, ref in ((dq, lq), (dk, lk), (dv, lv)):
        assert torch.allclose(got, ref, rtol=1e-11, atol=1e-12)


def test_backward_matches_finite_differences():
    H, hd, m, S = 2, 4, 5, 9
    q, k, v, do, pos = _inputs(m, S, H, hd, 7)
    dq, dk, dv = O.causal_attention_backward(q, pos, k, v, do, H, hd)

    def loss(qq, kk, vv):
        return (O.causal_attention(qq, pos, kk, vv, H, hd) * do).sum().item()

    eps = 1e-6
    g = torch.Generator().manual_seed(8)
    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(6):
            base = [q, k, v][which]
            i = int(torch.randint(0, base.shape[0], (1,), generator=g))
            j = int(torch.randint(0, base.shape[1], (1,), generator=g))
            args_p = [q.clone(), k.clone(), v.clone()]
            args_m = [q.clone(), k.clone(), v.clone()]
            args_p[which][i, j] += eps
            args_m[which][i, j] -= eps
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - grad[i, j].item()) <= 1e-7 + 1e-6 * abs(fd)


@pytest.mark.parametrize("S,D", [(32, 2), (48, 3), (64, 4)])
def test_zigzag_contributions_sum_to_full_sequence_gradients(S, D):
    H, hd = 2, 8
    q, k, v, do, _ = _inputs(S, S, H, hd, 11 + S, positions=torch.arange(S))
    qa, ka, va = (_heads(t, H, hd).clone().requires_grad_(True) for t in (q, k, v))
    o = F.scaled_dot_product_attention(qa[None], ka[None], va[None], is_causal=True)[0]
    fq, fk, fv = (_flat(t) for t in torch.autograd.grad(o, (qa, ka, va), grad_outputs=_heads(do, H, hd)))
    dk_sum, dv_sum = torch.zeros_like(k), torch.zeros_like(v)
    for r in range(D):
        pos = O.zigzag_plan(S, D, r).local_to_global
        dq, dk, dv = O.causal_attention_backward(q[pos], pos, k, v, do[pos], H, hd)
        assert torch.allclose(dq, fq[pos], rtol=1e-11, atol=1e-12)
        dk_sum += dk
        dv_sum += dv
    assert torch.allclose(dk_sum, fk, rtol=1e-11, atol=1e-12)
    assert torch.allclose(dv_sum, fv, rtol=1e-11, atol=1e-12)


def test_backward_invariants():
    H, hd, m, S = 3, 8, 12, 40
    q, k, v, do, pos = _inputs(m, S, H, hd, 21)
    pos[-1] = 30  # keys 31.. are seen by no query
    pos = torch.sort(pos).values
    dq, dk, dv = O.causal_attention_backward(q, pos, k, v, do, H, hd)
    for a in range(H):
        cols = slice(a * hd, (a + 1) * hd)
        assert torch.allclose(dk[:, cols].sum(0), torch.zeros(hd, dtype=F64), atol=1e-11)
        assert torch.allclose(dv[:, cols].sum(0), do[:, cols].sum(0), rtol=1e-12, atol=1e-12)
    assert torch.equal(dk[31:], torch.zeros_like(dk[31:]))
    assert torch.equal(dv[31:], torch.zeros_like(dv[31:]))
    # every value row equal: the output no longer depends on q or k
    vc = v[:1].expand(S, -1).clone()
    dq0, dk0, _ = O.causal_attention_backward(q, pos, k, vc, do, H, hd)
    assert dq0.abs().max().item() < 1e-12 and dk0.abs().max().item() < 1e-12


def test_lse_matches_library_and_normalises_forward():
    H, hd, m, S = 2, 16, 9, 30
    q, k, _, _, pos = _inputs(m, S, H, hd, 31)
    lse = O.attention_lse(q, pos, k, H, hd)
    future = torch.arange(S)[None, :] > pos[:, None]
    for a in range(H):
        cols = slice(a * hd, (a + 1) * hd)
        s = (q[:, cols] @ k[:, cols].t() / math.sqrt(hd)).masked_fill(future, float("-inf"))
        assert torch.allclose(lse[a], torch.logsumexp(s, dim=1), rtol=1e-13, atol=1e-13)
        p = O.softmax_rows(q, pos, k, a, hd)
        assert torch.allclose(torch.exp(s - lse[a][:, None]), p, rtol=1e-12, atol=1e-15)


def test_lse_one_key_closed_form():
    q = torch.tensor([[1.0, 2.0, 0.5, -1.0]], dtype=F64)
    k = torch.tensor([[0.5, -1.0, 2.0, 3.0], [9.0, 9.0, 9.0, 9.0]], dtype=F64)
    lse = O.attention_lse(q, torch.tensor([0]), k, 1, 4)
    assert lse.shape == (1, 1)
    assert abs(lse.item() - (0.5 - 2.0 + 1.0 - 3.0) / 2.0) < 1e-15
