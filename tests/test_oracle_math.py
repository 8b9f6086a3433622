"""Pins of the oracle's GELU and causal attention (CPU only).

Each pin checks the oracle against something other than itself: a library
routine that the special case reduces to (torch's tanh-GELU, torch's causal
scaled-dot-product attention, torch.softmax), values worked by hand
(tests/golden/attention_closed_form.txt), identities and invariants.
"""
import math

import pytest
import torch
import torch.nn.functional as F

from oracle import tsp_oracle as O

F64 = torch.float64


# ------------------------------------------------------------------- GELU
def test_gelu_matches_library_tanh_form():
    u = torch.linspace(-12, 12, 20001, dtype=F64)
    ref = F.gelu(u, approximate="tanh")
    assert torch.allclose(O.gelu_tanh(u), ref, rtol=1e-13, atol=1e-15)


def test_gelu_is_not_the_erf_form():
    # the erf form differs by up to ~5e-4 near |u| ~ 2: the oracle must be the tanh form
    u = torch.linspace(-4, 4, 801, dtype=F64)
    d = (O.gelu_tanh(u) - F.gelu(u)).abs().max().item()
    assert 1e-5 < d < 1e-3


def test_gelu_identities():
    u = torch.linspace(-30, 30, 6001, dtype=F64)
    g = O.gelu_tanh(u)
    assert O.gelu_tanh(torch.zeros(1, dtype=F64)).item() == 0.0
    # tanh is odd, so GELU(u) - GELU(-u) = u exactly in real arithmetic
    assert torch.allclose(g - O.gelu_tanh(-u), u, rtol=0, atol=1e-13)
    assert abs(O.gelu_tanh(torch.tensor([25.0], dtype=F64)).item() - 25.0) < 1e-12
    assert abs(O.gelu_tanh(torch.tensor([-25.0], dtype=F64)).item()) < 1e-12


# -------------------------------------------------------------- attention
def test_attention_closed_form(golden):
    rows = [(int(p), float(v)) for p, v in golden("attention_closed_form.txt")]
    hd = 4
    c = [0.0, math.log(3.0), math.log(2.0)]
    vals = [1.0, 5.0, 9.0]
    S = 3
    q = torch.zeros(S, hd, dtype=F64)
    q[:, 0] = 1.0
    k = torch.zeros(S, hd, dtype=F64)
    k[:, 0] = torch.tensor([2 * x for x in c], dtype=F64)
    v = torch.tensor(vals, dtype=F64)[:, None].repeat(1, hd)
    out = O.causal_attention(q, torch.arange(S), k, v, 1, hd)
    for p, expect in rows:
        assert torch.allclose(out[p], torch.full((hd,), expect, dtype=F64), rtol=0, atol=1e-14)


def _rand(shape, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=F64)


@pytest.mark.parametrize("H,hd,S", [(1, 8, 1), (2, 16, 37), (4, 64, 130)])
def test_attention_matches_library_causal_sdpa(H, hd, S):
    q, k, v = _rand((S, H * hd), 1), _rand((S, H * hd), 2), _rand((S, H * hd), 3)
    out = O.causal_attention(q, torch.arange(S), k, v, H, hd)
    qh = q.view(S, H, hd).transpose(0, 1)
    kh = k.view(S, H, hd).transpose(0, 1)
    vh = v.view(S, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True)
    assert torch.allclose(out, ref.transpose(0, 1).reshape(S, H * hd), rtol=1e-12, atol=1e-12)


def test_attention_subset_of_positions_matches_library():
    # queries at scattered global positions (as the zigzag chunks give them)
    S, H, hd = 96, 2, 16
    q, k, v = _rand((S, H * hd), 4), _rand((S, H * hd), 5), _rand((S, H * hd), 6)
    pos = torch.tensor([3, 4, 50, 95])
    out = O.causal_attention(q[pos], pos, k, v, H, hd)
    qh = q.view(S, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(qh, k.view(S, H, hd).transpose(0, 1), v.view(S, H, hd).transpose(0, 1),
                                         is_causal=True).transpose(0, 1).reshape(S, H * hd)
    assert torch.allclose(out, ref[pos], rtol=1e-12, atol=1e-12)


def test_softmax_rows_sum_to_one_and_v_ones():
    S, H, hd = 77, 2, 8
    q, k = _rand((S, H * hd), 7) * 3, _rand((S, H * hd), 8) * 3
    pos = torch.arange(S)
    for a in range(H):
        p = O.softmax_rows(q, pos, k, a, hd)
        assert torch.allclose(p.sum(1), torch.ones(S, dtype=F64), rtol=0, atol=1e-12)
        assert bool((p[torch.arange(S)[:, None] < torch.arange(S)[None, :]] == 0).all())
    out = O.causal_attention(q, pos, k, torch.ones(S, H * hd, dtype=F64), H, hd)
    assert torch.allclose(out, torch.ones_like(out), rtol=0, atol=1e-12)


def test_one_hot_values_give_probability_rows():
    # S <= hd: v_j = e_j, so o_p[j] is the probability of key j for query p
    S, hd = 12, 16
    q, k = _rand((S, hd), 9), _rand((S, hd), 10)
    v = torch.zeros(S, hd, dtype=F64)
    v[torch.arange(S), torch.arange(S)] = 1.0
    out = O.causal_attention(q, torch.arange(S), k, v, 1, hd)
    for p in range(S):
        s = torch.stack([q[p] @ k[j] / math.sqrt(hd) for j in range(p + 1)])
        prob = torch.softmax(s, 0)
        assert torch.allclose(out[p, :p + 1], prob, rtol=0, atol=1e-14)
        assert bool((out[p, p + 1:] == 0).all())


def test_causality_bit_identical():
    S, H, hd = 64, 2, 8
    q, k, v = _rand((S, H * hd), 11), _rand((S, H * hd), 12), _rand((S, H * hd), 13)
    pos = torch.arange(S)
    base = O.causal_attention(q, pos, k, v, H, hd)
    cut = 40
    k2, v2 = k.clone(), v.clone()
    k2[cut + 1:] += 5.0
    v2[cut + 1:] *= -3.0
    pert = O.causal_attention(q, pos, k2, v2, H, hd)
    assert torch.equal(base[:cut + 1], pert[:cut + 1])
    assert not torch.equal(base[cut + 1:], pert[cut + 1:])


def test_attention_large_scores_match_library():
    # scores of several hundred: exp without the running maximum would overflow
    S, H, hd = 40, 2, 16
    q, k, v = _rand((S, H * hd), 14) * 40, _rand((S, H * hd), 15) * 40, _rand((S, H * hd), 16)
    out = O.causal_attention(q, torch.arange(S), k, v, H, hd)
    heads = lambda t: t.view(S, H, hd).transpose(0, 1)
    ref = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
    assert torch.isfinite(out).all()
    assert torch.allclose(out, ref.transpose(0, 1).reshape(S, H * hd), rtol=1e-10, atol=1e-10)
