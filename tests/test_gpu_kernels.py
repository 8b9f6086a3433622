"""GPU parity of each step of the rank-share layer against the fp64 oracle, on
shapes the oracle finishes in seconds that still span several tiles and have
ragged tails (chunk lengths and token counts that are not tile multiples).

Steps: QKV projection with the K/V scatter (tsp_attn_project), causal
attention over the two zigzag chunks (tsp_attn_core), the O projection split-K
(tsp_attn_out) and the ring MLP (tsp_mlp_forward).  Special cases of the
attention kernel: V = 1 (softmax normalisation), one-hot V (the probability
rows themselves), causality (bit-identical rows under future perturbation),
and determinism."""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, gpu, require_gpu, say

pytestmark = gpu

DEV = "cuda"


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_000_000 + seed, std, "cpu")


def _weights(h, H, hd, F, D, seed):
    Hs, Fs = H // D, F // D
    wqkv = [_rnd((3 * Hs * hd, h), seed + d, 0.02) for d in range(D)]
    wo = [_rnd((h, Hs * hd), seed + 100 + d, 0.02) for d in range(D)]
    w1 = [_rnd((Fs, h), seed + 200 + d, 0.02) for d in range(D)]
    w2 = [_rnd((h, Fs), seed + 300 + d, 0.02) for d in range(D)]
    return wqkv, wo, w1, w2


def _dev(ts):
    return [t.to(DEV) for t in ts]


# (h, H, hd, D, S, rank): S/(2D) = C is the chunk length
PROJECT_CASES = [
    (256, 4, 64, 4, 2048, 1),     # tiny-layer shape
    (256, 4, 64, 2, 800, 1),      # C = 200: ragged token tiles
    (512, 4, 128, 2, 1288, 0),    # hd = 128, C = 322
    (256, 4, 64, 1, 300, 0),      # D = 1
    (512, 8, 64, 8, 48000, 3),    # 192-wide shards, 6000 tokens (ragged): 256 x 192 tiles
]


@pytest.mark.parametrize("h,H,hd,D,S,r", PROJECT_CASES)
def test_attn_project(h, H, hd, D, S, r):
    require_gpu()
    say(f"attn_project h={h} H={H} hd={hd} D={D} S={S} r={r}")
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    x = _rnd((n, h), 1)
    wqkv, _, _, _ = _weights(h, H, hd, 4 * h, D, 10)
    kf0, vf0 = _rnd((S, h), 2), _rnd((S, h), 3)
    kf, vf = kf0.to(DEV), vf0.to(DEV)
    q = bf16_nan((n, h), DEV)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    tsp.attn_project(plan, dims, x.to(DEV), _dev(wqkv), kf, vf, q)
    torch.cuda.synchronize()
    q_ref, k_ref, v_ref = O.qkv_projection(x, wqkv, hd)
    check(q, q_ref, "q")
    check(kf[l2g.to(DEV)], k_ref, "k own rows")
    check(vf[l2g.to(DEV)], v_ref, "v own rows")
    others = torch.ones(S, dtype=torch.bool)
    others[l2g] = False
    assert torch.equal(kf.cpu()[others], kf0[others]), "rows of other ranks must be untouched"
    assert torch.equal(vf.cpu()[others], vf0[others])


# (h, H, hd, D, n)
OUT_CASES = [(256, 4, 64, 4, 512), (256, 4, 64, 2, 300), (512, 4, 128, 4, 390), (256, 4, 64, 1, 129)]


@pytest.mark.parametrize("h,H,hd,D,n", OUT_CASES)
@pytest.mark.parametrize("with_residual", [False, True])
def test_attn_out(h, H, hd, D, n, with_residual):
    require_gpu()
    _, wo, _, _ = _weights(h, H, hd, 4 * h, D, 20)
    a = _rnd((n, h), 4)
    x = _rnd((n, h), 5)
    W = O.assemble(wo=wo)
    ref = O.linear(O.f64(a), W.wo) + (O.f64(x) if with_residual else 0)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    for start in range(D):
        say(f"attn_out h={h} hd={hd} D={D} n={n} start={start} residual={with_residual}")
        out = bf16_nan((n, h), DEV)
        tsp.attn_out(dims, D, start, a.to(DEV), _dev(wo), x.to(DEV) if with_residual else None, out)
        torch.cuda.synchronize()
        check(out, ref, f"attn_out start={start}")


# (h, F, D, n)
MLP_CASES = [(256, 1024, 4, 512), (256, 1024, 4, 300), (512, 2048, 8, 257), (256, 512, 1, 100), (384, 768, 2, 64)]


@pytest.mark.parametrize("h,F,D,n", MLP_CASES)
@pytest.mark.parametrize("with_residual", [False, True])
def test_mlp(h, F, D, n, with_residual):
    require_gpu()
    _, _, w1, w2 = _weights(h, 4, 64, F, D, 30)
    x = _rnd((n, h), 6)
    ref = O.mlp_forward(x, w1, w2, residual=with_residual)
    dims = tsp.make_dims(h, h // 64, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP)
    xd = x.to(DEV)
    for start in sorted({0, D - 1, D // 2}):
        say(f"mlp h={h} F={F} D={D} n={n} start={start} residual={with_residual}")
        y = bf16_nan((n, h), DEV)
        tsp.mlp_forward(dims, D, start, xd, _dev(w1), _dev(w2), xd if with_residual else None, y, ws)
        torch.cuda.synchronize()
        check(y, ref, f"mlp start={start}")


def test_mlp_in_place_residual():
    require_gpu()
    h, F, D, n = 256, 1024, 4, 200
    _, _, w1, w2 = _weights(h, 4, 64, F, D, 40)
    x = _rnd((n, h), 7)
    ref = O.mlp_forward(x, w1, w2, residual=True)
    dims = tsp.make_dims(h, 4, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP)
    xd = x.to(DEV)
    say("mlp in place (y = residual = x)")
    tsp.mlp_forward(dims, D, 1, xd, _dev(w1), _dev(w2), xd, xd, ws)
    torch.cuda.synchronize()
    check(xd, ref, "mlp in place")


def test_mlp_ring_start_independent():
    require_gpu()
    h, F, D, n = 256, 1024, 8, 256
    _, _, w1, w2 = _weights(h, 8, 32, F, D, 50)
    x = _rnd((n, h), 8).to(DEV)
    dims = tsp.make_dims(h, 4, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP)
    outs = []
    for start in range(D):
        say(f"mlp ring start {start}")
        y = bf16_nan((n, h), DEV)
        tsp.mlp_forward(dims, D, start, x, _dev(w1), _dev(w2), None, y, ws)
        outs.append(y)
    torch.cuda.synchronize()
    for start in range(1, D):
        check(outs[start], outs[0].double(), f"ring start {start} vs 0")


# ------------------------------------------------------------------ attention
# (H, hd, D, S, rank)
CORE_CASES = [
    (4, 64, 4, 2048, 1),    # tiny-layer shape
    (2, 64, 2, 800, 0),     # C = 200: ragged query tiles, rank 0 (first and last chunk)
    (2, 64, 2, 800, 1),
    (2, 128, 2, 1288, 1),   # hd = 128, C = 322
    (4, 128, 4, 4096, 2),
    (2, 64, 1, 130, 0),     # D = 1: plain causal attention, C = 65
    (1, 128, 8, 16, 5),     # C = 1: a single query per chunk
    # The cases above have small grids (fewer than 512 workgroups), where the
    # kernel splits the late chunk's keys in two and merges the halves; with
    # C = 1 the first half is empty.  The next case splits over several query
    # tiles with a ragged tail; the last has a 512-workgroup grid (64 heads x
    # 2 chunks x 4 tiles), which runs unsplit.
    (4, 128, 2, 8200, 1),   # C = 2050
    (64, 64, 1, 2048, 0),
]


def _attn_inputs(S, n, h, seed):
    return _rnd((n, h), seed), _rnd((S, h), seed + 1), _rnd((S, h), seed + 2)


@pytest.mark.parametrize("H,hd,D,S,r", CORE_CASES)
def test_attn_core(H, hd, D, S, r):
    require_gpu()
    say(f"attn_core H={H} hd={hd} D={D} S={S} r={r}")
    h = H * hd
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    q, k, v = _attn_inputs(S, n, h, 60)
    out = bf16_nan((n, h), DEV)
    tsp.attn_core(plan, tsp.make_dims(h, H, hd, 4 * h), q.to(DEV), k.to(DEV), v.to(DEV), out)
    torch.cuda.synchronize()
    ref = O.causal_attention(O.f64(q), l2g, O.f64(k), O.f64(v), H, hd)
    check(out, ref, "attention")


@pytest.mark.parametrize("hd", [64, 128])
def test_attn_core_v_ones(hd):
    """V = 1 everywhere: every output is a sum of probabilities, which must be 1."""
    require_gpu()
    H, D, S, r = 2, 4, 2048, 3
    h = H * hd
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    q = _rnd((plan.n_local, h), 70) * 3
    k = _rnd((S, h), 71)
    v = torch.ones(S, h, dtype=torch.bfloat16)
    out = bf16_nan((plan.n_local, h), DEV)
    say(f"attn_core V=1 hd={hd}")
    tsp.attn_core(plan, tsp.make_dims(h, H, hd, 4 * h), q.to(DEV), k.to(DEV), v.to(DEV), out)
    torch.cuda.synchronize()
    check(out, torch.ones(plan.n_local, h, dtype=torch.float64), "V=1")


@pytest.mark.parametrize("hd,D,S", [(64, 1, 64), (128, 2, 128)])
def test_attn_core_one_hot_values(hd, D, S):
    """S <= hd and v_j = e_j: output row p holds the softmax probabilities of
    keys 0..p (then zeros), checked against the oracle's probability rows."""
    require_gpu()
    H = 2
    h = H * hd
    for r in range(D):
        plan, l2g, _ = tsp.zigzag_plan(S, D, r)
        q = _rnd((plan.n_local, h), 80) * 2
        k = _rnd((S, h), 81)
        v = torch.zeros(S, h, dtype=torch.bfloat16)
        for a in range(H):
            v[torch.arange(S), a * hd + torch.arange(S)] = 1.0
        out = bf16_nan((plan.n_local, h), DEV)
        say(f"attn_core one-hot hd={hd} D={D} r={r}")
        tsp.attn_core(plan, tsp.make_dims(h, H, hd, 4 * h), q.to(DEV), k.to(DEV), v.to(DEV), out)
        torch.cuda.synchronize()
        for a in range(H):
            prob = O.softmax_rows(O.f64(q), l2g, O.f64(k), a, hd)  # [n, S]
            got = out.cpu()[:, a * hd:a * hd + S]
            check(got, prob, f"probability rows head {a}")
            assert bool((out.cpu()[:, a * hd + S:(a + 1) * hd] == 0).all())


def test_attn_core_causality_bit_identical():
    """Perturbing keys/values after position P leaves every query at a position
    <= P bit-identical (masked scores never reach the max or the sum)."""
    require_gpu()
    H, hd, D, S = 2, 128, 2, 1024
    h = H * hd
    for r in range(D):
        plan, l2g, _ = tsp.zigzag_plan(S, D, r)
        q, k, v = _attn_inputs(S, plan.n_local, h, 90)
        P = 700
        k2, v2 = k.clone(), v.clone()
        k2[P + 1:] = _rnd((S - P - 1, h), 93)
        v2[P + 1:] = _rnd((S - P - 1, h), 94) * 4
        dims = tsp.make_dims(h, H, hd, 4 * h)
        o1, o2 = bf16_nan((plan.n_local, h), DEV), bf16_nan((plan.n_local, h), DEV)
        say(f"attn_core causality r={r}")
        tsp.attn_core(plan, dims, q.to(DEV), k.to(DEV), v.to(DEV), o1)
        tsp.attn_core(plan, dims, q.to(DEV), k2.to(DEV), v2.to(DEV), o2)
        torch.cuda.synchronize()
        early = l2g <= P
        assert int(early.sum()) > 0
        assert torch.equal(o1.cpu()[early], o2.cpu()[early])
        if bool((~early).any()):
            assert not torch.equal(o1.cpu()[~early], o2.cpu()[~early])


def test_determinism():
    require_gpu()
    H, hd, D, S = 4, 128, 4, 4096
    h = H * hd
    plan, _, _ = tsp.zigzag_plan(S, D, 1)
    q, k, v = (t.to(DEV) for t in _attn_inputs(S, plan.n_local, h, 100))
    dims = tsp.make_dims(h, H, hd, 4 * h)
    _, wo, w1, w2 = _weights(h, H, hd, 4 * h, D, 110)
    ws = tsp.alloc_workspace(plan.n_local, dims, D, tsp.WS_MLP)
    res = []
    for _ in range(2):
        say("determinism pass")
        a = bf16_nan((plan.n_local, h), DEV)
        tsp.attn_core(plan, dims, q, k, v, a)
        o = bf16_nan((plan.n_local, h), DEV)
        tsp.attn_out(dims, D, 1, a, _dev(wo), q, o)
        y = bf16_nan((plan.n_local, h), DEV)
        tsp.mlp_forward(dims, D, 1, o, _dev(w1), _dev(w2), o, y, ws)
        res.append((a, o, y))
    torch.cuda.synchronize()
    for t1, t2 in zip(*res):
        assert torch.equal(t1, t2)


# (h, H, hd, F, D, n)
POST_CASES = [(256, 4, 64, 1024, 4, 512), (512, 4, 128, 2048, 2, 300), (384, 6, 64, 768, 2, 65)]


@pytest.mark.parametrize("h,H,hd,F,D,n", POST_CASES)
def test_layer_post(h, H, hd, F, D, n):
    """O projection + residual + ring MLP + residual (the part of the layer after
    the attention core) against the oracle's h1 = x + a W_o^T, out = h1 + MLP(h1),
    for every ring start."""
    require_gpu()
    _, wo, w1, w2 = _weights(h, H, hd, F, D, 120)
    a = _rnd((n, h), 9) * 0.3
    x = _rnd((n, h), 10)
    W = O.assemble(wo=wo)
    h1 = O.f64(x) + O.linear(O.f64(a), W.wo)
    ref = O.mlp_forward(h1, w1, w2, residual=True)
    dims = tsp.make_dims(h, H, hd, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_POST)
    for start in range(D):
        say(f"layer_post h={h} hd={hd} F={F} D={D} n={n} start={start}")
        out = bf16_nan((n, h), DEV)
        tsp.layer_post(dims, D, start, a.to(DEV), x.to(DEV), _dev(wo), _dev(w1), _dev(w2), out, ws)
        torch.cuda.synchronize()
        check(out, ref, f"layer_post start={start}")


def test_mlp_row_scaling_wide_range():
    """Rows whose magnitudes span 2^-20 .. 2^20 (the fp16 operands are scaled per
    row by a power of two, so every row keeps its relative precision)."""
    require_gpu()
    h, F, D, n = 256, 1024, 4, 96
    _, _, w1, w2 = _weights(h, 4, 64, F, D, 130)
    x = _rnd((n, h), 11).float()
    x *= torch.pow(2.0, torch.linspace(-20, 20, n)).unsqueeze(1)
    x = x.to(torch.bfloat16)
    ref = O.mlp_forward(x, w1, w2, residual=False)
    dims = tsp.make_dims(h, 4, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP)
    y = bf16_nan((n, h), DEV)
    say("mlp rows spanning 2^-20 .. 2^20")
    tsp.mlp_forward(dims, D, 0, x.to(DEV), _dev(w1), _dev(w2), None, y, ws)
    torch.cuda.synchronize()
    g = y.cpu().double()
    for i in range(n):  # per row: relative error against that row's own scale
        rr = ((g[i] - ref[i]).norm() / ref[i].norm()).item()
        assert rr <= 5e-3, f"row {i}: relative RMS {rr:.3e}"


def test_attn_core_low_part():
    """attn_lo is the rounding residual of attn_out (at most half a bf16 ulp of
    it, i.e. |lo| <= 2^-8 |hi|) and the pair is closer to the oracle than the
    bf16 output alone, on a case whose outputs are O(1) (early queries see few
    keys)."""
    require_gpu()
    H, hd, D, S, r = 2, 128, 2, 512, 0
    h = H * hd
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    q, k, v = _attn_inputs(S, plan.n_local, h, 140)
    hi, lo = bf16_nan((plan.n_local, h), DEV), bf16_nan((plan.n_local, h), DEV)
    say("attn_core with low part")
    tsp.attn_core(plan, tsp.make_dims(h, H, hd, 4 * h), q.to(DEV), k.to(DEV), v.to(DEV), hi, lo)
    torch.cuda.synchronize()
    ref = O.causal_attention(O.f64(q), l2g, O.f64(k), O.f64(v), H, hd)
    check(hi, ref, "attention hi part")
    hd_, ld_ = hi.cpu().double(), lo.cpu().double()
    assert bool((ld_.abs() <= 2.0 ** -8 * hd_.abs()).all()), "low part larger than half an ulp of the high part"
    rr_hi = ((hd_ - ref).norm() / ref.norm()).item()
    rr_pair = ((hd_ + ld_ - ref).norm() / ref.norm()).item()
    assert rr_pair < 0.8 * rr_hi, (rr_pair, rr_hi)


@pytest.mark.parametrize("D", [1, 4])
def test_attn_out_with_low_part(D):
    require_gpu()
    h, H, hd, n = 256, 4, 64, 333
    _, wo, _, _ = _weights(h, H, hd, 4 * h, D, 150)
    a32 = torch.randn(n, h, generator=torch.Generator().manual_seed(151), dtype=torch.float64)
    hi = a32.to(torch.bfloat16)
    lo = (a32 - hi.double()).to(torch.bfloat16)
    x = _rnd((n, h), 12)
    ref = O.linear(hi.double() + lo.double(), O.assemble(wo=wo).wo) + O.f64(x)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    out = bf16_nan((n, h), DEV)
    say(f"attn_out with low part D={D}")
    tsp.attn_out(dims, D, D - 1, hi.to(DEV), _dev(wo), x.to(DEV), out, attn_lo=lo.to(DEV))
    torch.cuda.synchronize()
    check(out, ref, "attn_out hi + lo")
