"""Pins of the oracle's projections, MLP and whole layer (CPU only).

* D = 1 reduces the rank-share layer to a plain decoder layer, which is written
  here with torch library routines (``F.linear``, causal
  ``F.scaled_dot_product_attention``, tanh ``F.gelu``) on the same weights.
* The method's identities (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU
  axis", para. 1-2): the MLP summed over shards in ring order equals the
  unsharded MLP for every ring start; D shards equal the whole weights; the D
  rank outputs, emulated one after another with the gathered K/V, reassemble
  the unsharded layer over the whole sequence.
* Special cases: zero weights make the layer the identity (both residuals).
"""
import pytest
import torch
import torch.nn.functional as F

from oracle import tsp_oracle as O

F64 = torch.float64


def _bf(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g) * std).to(torch.bfloat16)


def _weights(h, H, hd, Fd, D, seed):
    Hs, Fs = H // D, Fd // D
    wqkv = [_bf((3 * Hs * hd, h), seed + d, 0.05) for d in range(D)]
    wo = [_bf((h, Hs * hd), seed + 100 + d, 0.05) for d in range(D)]
    w1 = [_bf((Fs, h), seed + 200 + d, 0.05) for d in range(D)]
    w2 = [_bf((h, Fs), seed + 300 + d, 0.05) for d in range(D)]
    return wqkv, wo, w1, w2


def _library_layer(x, wq, wk, wv, wo, w1, w2, H, hd, proj_round=False):
    """A plain decoder layer from torch library calls (fp64); with proj_round the
    queries, keys and values pass through torch's bf16 conversion first."""
    S, h = x.shape
    q, k, v = F.linear(x, wq), F.linear(x, wk), F.linear(x, wv)
    if proj_round:
        q, k, v = (t.to(torch.bfloat16).double() for t in (q, k, v))
    heads = lambda t: t.view(S, H, hd).transpose(0, 1)
    a = F.scaled_dot_product_attention(heads(q), heads(k), heads(v), is_causal=True)
    h1 = x + F.linear(a.transpose(0, 1).reshape(S, h), wo)
    return h1 + F.linear(F.gelu(F.linear(h1, w1), approximate="tanh"), w2)


@pytest.mark.parametrize("h,H,hd,Fd,S", [(32, 2, 16, 64, 24), (64, 4, 16, 128, 40)])
def test_d1_layer_matches_library_layer(h, H, hd, Fd, S):
    wqkv, wo, w1, w2 = _weights(h, H, hd, Fd, 1, 10)
    x = _bf((S, h), 1)
    plan = O.zigzag_plan(S, 1, 0)
    out, _, _ = O.layer_forward(plan, x, wqkv, wo, w1, w2, H, hd, proj_bf16=False)
    W = O.f64(wqkv[0])
    ref = _library_layer(O.f64(x), W[:h], W[h:2 * h], W[2 * h:], O.f64(wo[0]), O.f64(w1[0]), O.f64(w2[0]), H, hd)
    assert torch.allclose(out, ref, rtol=1e-11, atol=1e-11)
    # with Q, K and V held in bf16: the library layer with them rounded to bf16
    out16, _, _ = O.layer_forward(plan, x, wqkv, wo, w1, w2, H, hd)
    ref16 = _library_layer(O.f64(x), W[:h], W[h:2 * h], W[2 * h:], O.f64(wo[0]), O.f64(w1[0]), O.f64(w2[0]), H,
                           hd, proj_round=True)
    assert torch.allclose(out16, ref16, rtol=1e-11, atol=1e-11)
    assert not torch.allclose(out16, out, rtol=1e-6, atol=1e-6)


def test_zero_weights_make_identity():
    h, H, hd, Fd, D, S = 32, 4, 8, 64, 2, 32
    wqkv, wo, w1, w2 = _weights(h, H, hd, Fd, D, 20)
    x = _bf((S // D, h), 2)
    plan = O.zigzag_plan(S, D, 1)
    kf, vf = _bf((S, h), 3), _bf((S, h), 4)
    zero = lambda ws: [torch.zeros_like(w) for w in ws]
    out, _, _ = O.layer_forward(plan, x, wqkv, zero(wo), w1, zero(w2), H, hd, kf, vf)
    assert torch.equal(out, O.f64(x))
    # GELU(0) = 0: zero W1 also removes the MLP, leaving x + attention
    h1, _, _, _ = O.attn_forward(plan, x, wqkv, wo, H, hd, kf, vf)
    out2, _, _ = O.layer_forward(plan, x, wqkv, wo, zero(w1), w2, H, hd, kf, vf)
    assert torch.allclose(out2, h1, rtol=0, atol=0)


@pytest.mark.parametrize("D", [2, 4, 8])
def test_mlp_sum_over_shards_every_ring_start(D):
    h, Fd, n = 32, 128, 20
    _, _, w1, w2 = _weights(h, D, 4, Fd, D, 30)
    x = _bf((n, h), 5)
    whole = O.mlp_forward(x, w1, w2, residual=False)
    for r in range(D):
        ring = O.zigzag_plan(2 * D, D, r).ring
        assert torch.allclose(O.mlp_sharded(x, w1, w2, ring), whole, rtol=1e-12, atol=1e-13)


def test_shards_equal_whole_weights():
    h, H, hd, Fd, S, D = 64, 4, 16, 128, 64, 4
    wqkv, wo, w1, w2 = _weights(h, H, hd, Fd, D, 40)
    W = O.assemble(wqkv, wo, w1, w2)
    # the same matrices handed over as a single shard (D = 1)
    one = ([torch.cat([W.wq, W.wk, W.wv], 0).to(torch.bfloat16)], [W.wo.to(torch.bfloat16)],
           [W.w1.to(torch.bfloat16)], [W.w2.to(torch.bfloat16)])
    x = _bf((S, h), 6)
    plan1 = O.zigzag_plan(S, 1, 0)
    a, _, _ = O.layer_forward(plan1, x, wqkv, wo, w1, w2, H, hd)
    b, _, _ = O.layer_forward(plan1, x, *one, H, hd)
    assert torch.allclose(a, b, rtol=1e-12, atol=1e-12)
    # and the head -> shard map: shard d's Q rows are heads d*H_s.. of the whole W_q
    Hs = H // D
    for d in range(D):
        assert torch.equal(O.f64(wqkv[d])[:Hs * hd], W.wq[d * Hs * hd:(d + 1) * Hs * hd])
        assert torch.equal(O.f64(wqkv[d])[2 * Hs * hd:], W.wv[d * Hs * hd:(d + 1) * Hs * hd])


@pytest.mark.parametrize("proj_bf16", [False, True])
@pytest.mark.parametrize("D,S", [(2, 32), (4, 64)])
def test_rank_emulation_reassembles_unsharded_layer(D, S, proj_bf16):
    """All D ranks, each with its zigzag rows and the gathered K/V, give the
    unsharded layer over the whole sequence."""
    h, H, hd, Fd = 32, 4, 8, 64
    wqkv, wo, w1, w2 = _weights(h, H, hd, Fd, D, 50)
    x_all = _bf((S, h), 7)
    full, _, _ = O.layer_forward(O.zigzag_plan(S, 1, 0), x_all, wqkv, wo, w1, w2, H, hd, proj_bf16=proj_bf16)
    # phase 1: every rank projects its own K/V rows into the gathered buffers
    kf = torch.full((S, h), float("nan"), dtype=F64)
    vf = torch.full((S, h), float("nan"), dtype=F64)
    for r in range(D):
        p = O.zigzag_plan(S, D, r)
        _, k_own, v_own = O.qkv_projection(x_all[p.local_to_global], wqkv, hd)
        kf[p.local_to_global], vf[p.local_to_global] = k_own, v_own
    assert not torch.isnan(kf).any()
    # phase 2: every rank runs its layer against the gathered K/V
    got = torch.empty_like(full)
    for r in range(D):
        p = O.zigzag_plan(S, D, r)
        out, _, _ = O.layer_forward(p, x_all[p.local_to_global], wqkv, wo, w1, w2, H, hd, kf, vf, proj_bf16=proj_bf16)
        got[p.local_to_global] = out
    assert torch.allclose(got, full, rtol=1e-12, atol=1e-12)


def test_own_rows_replace_supplied_rows():
    h, H, hd, Fd, S, D = 32, 4, 8, 64, 32, 2
    wqkv, wo, _, _ = _weights(h, H, hd, Fd, D, 60)
    p = O.zigzag_plan(S, D, 0)
    x = _bf((S // D, h), 8)
    kf, vf = _bf((S, h), 9), _bf((S, h), 10)
    a, _, k_own, v_own = O.attn_forward(p, x, wqkv, wo, H, hd, kf, vf)
    # garbage at the own positions of the supplied buffers must not matter
    kf2, vf2 = kf.clone(), vf.clone()
    kf2[p.local_to_global] = 1000.0
    vf2[p.local_to_global] = -1000.0
    b, _, _, _ = O.attn_forward(p, x, wqkv, wo, H, hd, kf2, vf2)
    assert torch.equal(a, b)
    k, v = O.gathered_kv(p, k_own, v_own, kf, vf)
    others = torch.ones(S, dtype=torch.bool)
    others[p.local_to_global] = False
    assert torch.equal(k[others], O.f64(kf)[others])
    assert torch.equal(v[p.local_to_global], v_own.to(torch.bfloat16).double())


def test_row_subset_equals_full_rows():
    h, H, hd, Fd, S, D = 32, 4, 8, 64, 64, 4
    wqkv, wo, w1, w2 = _weights(h, H, hd, Fd, D, 70)
    p = O.zigzag_plan(S, D, 2)
    x = _bf((S // D, h), 11)
    kf, vf = _bf((S, h), 12), _bf((S, h), 13)
    full, _, _ = O.layer_forward(p, x, wqkv, wo, w1, w2, H, hd, kf, vf)
    rows = [0, 3, 7, 8, 15]
    sub, _, _ = O.layer_forward(p, x, wqkv, wo, w1, w2, H, hd, kf, vf, rows=rows)
    assert torch.allclose(sub, full[rows], rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("D", [2, 4])
def test_attention_is_sum_over_head_shards(D):
    """Each attention weight shard applied on its own (its heads' Q/K/V rows of
    wqkv[d], then its W_o block wo[d]) and summed over shards gives the
    attention half of the layer; written per shard with library routines."""
    h, H, hd, Fd, S = 32, 4, 8, 64, 24
    wqkv, wo, _, _ = _weights(h, H, hd, Fd, D, 80)
    x = _bf((S, h), 14)
    got, _, _, _ = O.attn_forward(O.zigzag_plan(S, 1, 0), x, wqkv, wo, H, hd, residual=False, proj_bf16=False)
    xx = O.f64(x)
    Hs = H // D
    ref = torch.zeros(S, h, dtype=F64)
    for d in range(D):
        W = O.f64(wqkv[d])
        q, k, v = (F.linear(xx, W[i * Hs * hd:(i + 1) * Hs * hd]).view(S, Hs, hd).transpose(0, 1) for i in range(3))
        a = F.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1).reshape(S, Hs * hd)
        ref += F.linear(a, O.f64(wo[d]))
    assert torch.allclose(got, ref, rtol=1e-12, atol=1e-12)
