"""Pins of the oracle's layer variants (CPU only): RMSNorm, rotary position
embedding, grouped-query attention.

Each is checked against something other than its own code: a library routine
the case reduces to (torch's rms_norm, torch's scaled-dot-product attention
with grouped K/V heads), the closed form evaluated with Python's math module,
the complex-number form of the rotation, and invariants (norm preservation,
relative-position invariance, composition, scale invariance).
"""
import math

import pytest
import torch
import torch.nn.functional as F

from oracle import tsp_oracle as O

F64 = torch.float64


# ------------------------------------------------------------------ RMSNorm
def test_rms_norm_matches_library():
    g = torch.Generator().manual_seed(1)
    x = torch.randn(37, 96, generator=g, dtype=F64) * 3.0
    w = torch.randn(96, generator=g, dtype=F64)
    for eps in (0.0, 1e-6, 1e-2):
        ref = F.rms_norm(x, (96,), weight=w, eps=eps)
        assert torch.allclose(O.rms_norm(x, w, eps), ref, rtol=1e-13, atol=1e-14)


def test_rms_norm_hand_case():
    y = O.rms_norm(torch.tensor([[3.0, 4.0]], dtype=F64), torch.ones(2, dtype=F64), 0.0)
    r = math.sqrt((9.0 + 16.0) / 2.0)
    assert torch.allclose(y, torch.tensor([[3.0 / r, 4.0 / r]], dtype=F64), rtol=1e-15, atol=0)


def test_rms_norm_invariants():
    g = torch.Generator().manual_seed(2)
    x = torch.randn(10, 64, generator=g, dtype=F64)
    one = torch.ones(64, dtype=F64)
    y = O.rms_norm(x, one, 0.0)
    assert torch.allclose((y * y).mean(dim=1), torch.ones(10, dtype=F64), rtol=1e-13)
    assert torch.allclose(O.rms_norm(7.5 * x, one, 0.0), y, rtol=1e-13, atol=1e-14)  # scale invariance
    z = O.rms_norm(torch.zeros(1, 64, dtype=F64), one, 1e-6)
    assert torch.equal(z, torch.zeros(1, 64, dtype=F64))


# --------------------------------------------------------------------- RoPE
def test_rope_closed_form_hand_case():
    # head_dim 4, theta 10000: inverse frequencies 1 and 10000^(-1/2) = 0.01
    x = torch.tensor([[1.0, 2.0, 3.0, 4.0]], dtype=F64)
    y = O.rope(x, torch.tensor([2]), 1, 4, 10000.0)
    a0, a1 = 2.0, 0.02
    ref = [1 * math.cos(a0) - 2 * math.sin(a0), 1 * math.sin(a0) + 2 * math.cos(a0),
           3 * math.cos(a1) - 4 * math.sin(a1), 3 * math.sin(a1) + 4 * math.cos(a1)]
    assert torch.allclose(y, torch.tensor([ref], dtype=F64), rtol=1e-14, atol=1e-15)


def test_rope_complex_form():
    g = torch.Generator().manual_seed(3)
    H, hd, m = 3, 16, 11
    x = torch.randn(m, H * hd, generator=g, dtype=F64)
    pos = torch.randint(0, 200000, (m,), generator=g)
    y = O.rope(x, pos, H, hd, 500000.0)
    z = torch.view_as_complex(x.reshape(m, H, hd // 2, 2).contiguous())
    i = torch.arange(hd // 2, dtype=F64)
    ang = pos.to(F64)[:, None, None] * (500000.0 ** (-2.0 * i / hd))[None, None, :]
    ref = torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)).reshape(m, H * hd)
    assert torch.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_rope_invariants():
    g = torch.Generator().manual_seed(4)
    H, hd = 2, 8
    x = torch.randn(6, H * hd, generator=g, dtype=F64)
    k = torch.randn(6, H * hd, generator=g, dtype=F64)
    p = torch.tensor([0, 1, 5, 100, 4096, 131071])
    y = O.rope(x, p, H, hd, 10000.0)
    pairs = lambda t: t.reshape(t.shape[0], -1, 2).norm(dim=-1)
    assert torch.allclose(pairs(y), pairs(x), rtol=1e-13)              # rotations keep pair norms
    assert torch.equal(O.rope(x[:1], torch.tensor([0]), H, hd, 10000.0), x[:1])  # position 0
    # composition: rotating by p then by s is rotating by p + s
    s = torch.full_like(p, 77)
    assert torch.allclose(O.rope(y, s, H, hd, 10000.0), O.rope(x, p + s, H, hd, 10000.0), rtol=1e-11, atol=1e-11)
    # relative position: per head, <rope(q, m), rope(k, n)> depends only on m - n
    for shift in (1, 1000):
        a = (O.rope(x, p, H, hd, 10000.0) * O.rope(k, p + 3, H, hd, 10000.0)).reshape(6, H, hd).sum(-1)
        b = (O.rope(x, p + shift, H, hd, 10000.0) * O.rope(k, p + 3 + shift, H, hd, 10000.0)).reshape(6, H, hd).sum(-1)
        assert torch.allclose(a, b, rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------- GQA
def _qkv(S, H, Hkv, hd, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(S, H * hd, generator=g, dtype=F64), torch.randn(S, Hkv * hd, generator=g, dtype=F64),
            torch.randn(S, Hkv * hd, generator=g, dtype=F64))


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (8, 2), (6, 3)])
def test_gqa_matches_library(H, Hkv):
    S, hd = 40, 16
    q, k, v = _qkv(S, H, Hkv, hd, 5)
    got = O.causal_attention_gqa(q, torch.arange(S), k, v, H, Hkv, hd)
    tq = q.reshape(S, H, hd).transpose(0, 1)[None]
    tk = k.reshape(S, Hkv, hd).transpose(0, 1)[None]
    tv = v.reshape(S, Hkv, hd).transpose(0, 1)[None]
    ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    assert torch.allclose(got, ref[0].transpose(0, 1).reshape(S, H * hd), rtol=1e-12, atol=1e-13)


def test_gqa_reduces_to_mha():
    S, H, hd = 30, 4, 8
    q, k, v = _qkv(S, H, H, hd, 6)
    pos = torch.arange(S)
    assert torch.allclose(O.causal_attention_gqa(q, pos, k, v, H, H, hd), O.causal_attention(q, pos, k, v, H, hd),
                          rtol=1e-13, atol=1e-14)
    # and to MHA over K/V heads repeated for each query head of the group
    q, k, v = _qkv(S, H, 2, hd, 7)
    kr = k.reshape(S, 2, hd).repeat_interleave(2, dim=1).reshape(S, H * hd)
    vr = v.reshape(S, 2, hd).repeat_interleave(2, dim=1).reshape(S, H * hd)
    sub = torch.tensor([3, 11, 29])
    assert torch.allclose(O.causal_attention_gqa(q[sub], sub, k, v, H, 2, hd),
                          O.causal_attention(q[sub], sub, kr, vr, H, hd), rtol=1e-13, atol=1e-14)


def test_gqa_projection_reduces_to_mha_projection():
    g = torch.Generator().manual_seed(8)
    D, Hs, hd, h = 2, 2, 8, 32
    x = torch.randn(5, h, generator=g, dtype=F64)
    w = [torch.randn(3 * Hs * hd, h, generator=g, dtype=F64) for _ in range(D)]
    a = O.qkv_projection_gqa(x, w, hd, Hs, Hs)
    b = O.qkv_projection(x, w, hd)
    for u, v in zip(a, b):
        assert torch.allclose(u, v, rtol=1e-14, atol=1e-14)
    # with one K/V head per shard: K/V columns are rows Hs*hd .. of each shard, by matmul
    w1 = [torch.randn((Hs + 2) * hd, h, generator=g, dtype=F64) for _ in range(D)]
    q, k, v = O.qkv_projection_gqa(x, w1, hd, Hs, 1)
    assert torch.allclose(k[:, hd:2 * hd], x @ w1[1][Hs * hd:(Hs + 1) * hd].t(), rtol=1e-13)
    assert torch.allclose(v[:, :hd], x @ w1[0][(Hs + 1) * hd:].t(), rtol=1e-13)
    assert torch.allclose(q[:, Hs * hd:], x @ w1[1][:Hs * hd].t(), rtol=1e-13)


# ------------------------------------------------------------- backwards
def test_rms_norm_backward_matches_autograd():
    g = torch.Generator().manual_seed(41)
    x = torch.randn(9, 48, generator=g, dtype=F64) * 2.0
    w = torch.randn(48, generator=g, dtype=F64)
    dy = torch.randn(9, 48, generator=g, dtype=F64)
    for eps in (0.0, 1e-6, 1e-2):
        xa, wa = x.clone().requires_grad_(True), w.clone().requires_grad_(True)
        gx, gw = torch.autograd.grad(F.rms_norm(xa, (48,), weight=wa, eps=eps), (xa, wa), grad_outputs=dy)
        dx, dgain = O.rms_norm_backward(x, w, eps, dy)
        assert torch.allclose(dx, gx, rtol=1e-12, atol=1e-12)
        assert torch.allclose(dgain, gw, rtol=1e-12, atol=1e-12)


def test_rope_backward_is_the_inverse_rotation():
    g = torch.Generator().manual_seed(42)
    H, hd, m = 2, 16, 7
    x = torch.randn(m, H * hd, generator=g, dtype=F64)
    dy = torch.randn(m, H * hd, generator=g, dtype=F64)
    pos = torch.randint(0, 131072, (m,), generator=g)
    xa = x.clone().requires_grad_(True)
    # autograd through the complex-number form of the rotation (not the oracle's code)
    z = torch.view_as_complex(xa.reshape(m, H, hd // 2, 2))
    i = torch.arange(hd // 2, dtype=F64)
    ang = pos.to(F64)[:, None, None] * (10000.0 ** (-2.0 * i / hd))[None, None, :]
    y = torch.view_as_real(z * torch.polar(torch.ones_like(ang), ang)).reshape(m, H * hd)
    (gx,) = torch.autograd.grad(y, xa, grad_outputs=dy)
    assert torch.allclose(O.rope_backward(dy, pos, H, hd, 10000.0), gx, rtol=1e-12, atol=1e-12)
    # and undoes the forward exactly (orthogonal rotation)
    assert torch.allclose(O.rope_backward(O.rope(x, pos, H, hd, 10000.0), pos, H, hd, 10000.0), x, rtol=1e-11, atol=1e-11)


@pytest.mark.parametrize("H,Hkv", [(4, 1), (4, 2), (6, 3), (4, 4)])
def test_gqa_backward_matches_library_autograd(H, Hkv):
    S, hd, m = 24, 8, 10
    q, k, v = _qkv(S, H, Hkv, hd, 43)
    g = torch.Generator().manual_seed(44)
    pos = torch.sort(torch.randperm(S, generator=g)[:m]).values
    qm = q[pos]
    do = torch.randn(m, H * hd, generator=g, dtype=F64)
    mask = torch.arange(S)[None, :] <= pos[:, None]
    qa = qm.reshape(m, H, hd).transpose(0, 1).clone().requires_grad_(True)
    ka = k.reshape(S, Hkv, hd).transpose(0, 1).clone().requires_grad_(True)
    va = v.reshape(S, Hkv, hd).transpose(0, 1).clone().requires_grad_(True)
    o = F.scaled_dot_product_attention(qa[None], ka[None], va[None], attn_mask=mask[None, None], enable_gqa=True)[0]
    gq, gk, gv = torch.autograd.grad(o, (qa, ka, va), grad_outputs=do.reshape(m, H, hd).transpose(0, 1))
    dq, dk, dv = O.causal_attention_gqa_backward(qm, pos, k, v, do, H, Hkv, hd)
    flat = lambda t: t.transpose(0, 1).reshape(t.shape[1], -1)
    assert torch.allclose(dq, flat(gq), rtol=1e-11, atol=1e-12)
    assert torch.allclose(dk, flat(gk), rtol=1e-11, atol=1e-12)
    assert torch.allclose(dv, flat(gv), rtol=1e-11, atol=1e-12)
