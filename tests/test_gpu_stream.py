"""GPU parity of the shard-streaming entry points (one ring step per call):
tsp_attn_project_shard, tsp_attn_out_shard and tsp_mlp_shard.

  * the QKV projection of each shard alone is bit-identical to the all-shard
    call's columns of that shard;
  * the O projection and the MLP, driven step by step in ring order, match the
    fp64 oracle to the same tolerance as the all-shard calls, for every ring
    start, with and without the residual, with ragged token counts, D = 1, and
    more tokens than one GELU block;
  * with the weight shards "arriving" one after another (copied on a side
    stream, each copy followed by an event that the compute stream waits for,
    the side stream first held back by unrelated work), the result is
    bit-identical to the same calls on resident weights;
  * the MLP ring at the 7B shape (16384 tokens, D = 8, ring from shard 3)
    against the oracle on sampled rows.
"""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_500_000 + seed, std, "cpu")


def _dev(ts):
    return [t.to(DEV) for t in ts]


@pytest.mark.parametrize("h,H,hd,D,S,r", [(256, 4, 64, 4, 2048, 1), (512, 4, 128, 2, 1288, 0), (256, 4, 64, 1, 300, 0)])
def test_project_shard_bit_identical(h, H, hd, D, S, r):
    require_gpu()
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    Hs = H // D
    x = _rnd((n, h), 1).to(DEV)
    wqkv = _dev([_rnd((3 * Hs * hd, h), 10 + d, 0.02) for d in range(D)])
    kf0, vf0 = _rnd((S, h), 2).to(DEV), _rnd((S, h), 3).to(DEV)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    say(f"project all shards h={h} hd={hd} D={D} S={S} r={r}")
    q_all, k_all, v_all = bf16_nan((n, h), DEV), kf0.clone(), vf0.clone()
    tsp.attn_project(plan, dims, x, wqkv, k_all, v_all, q_all)
    q_s, k_s, v_s = bf16_nan((n, h), DEV), kf0.clone(), vf0.clone()
    for d in reversed(range(D)):  # any order: the shards write disjoint columns
        say(f"project shard {d}")
        tsp.attn_project_shard(plan, dims, d, x, wqkv[d], k_s, v_s, q_s)
    torch.cuda.synchronize()
    assert torch.equal(q_s, q_all)
    assert torch.equal(k_s, k_all)
    assert torch.equal(v_s, v_all)


@pytest.mark.parametrize("h,H,hd,D,n", [(256, 4, 64, 4, 512), (512, 4, 128, 4, 390), (256, 4, 64, 1, 129)])
@pytest.mark.parametrize("with_residual", [False, True])
@pytest.mark.parametrize("with_lo", [False, True])
def test_attn_out_ring_steps(h, H, hd, D, n, with_residual, with_lo):
    require_gpu()
    Hs = H // D
    wo = [_rnd((h, Hs * hd), 20 + d, 0.02) for d in range(D)]
    a = _rnd((n, h), 4)
    lo = (_rnd((n, h), 8) * 2 ** -9).to(torch.bfloat16)
    x = _rnd((n, h), 5)
    W = O.assemble(wo=wo)
    a_tot = O.f64(a) + (O.f64(lo) if with_lo else 0)
    ref = O.linear(a_tot, W.wo) + (O.f64(x) if with_residual else 0)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_SHARD)
    wod, ad, lod, xd = _dev(wo), a.to(DEV), lo.to(DEV), x.to(DEV)
    for start in sorted({0, D - 1}):
        say(f"attn_out ring steps h={h} hd={hd} D={D} n={n} start={start} res={with_residual} lo={with_lo}")
        out = bf16_nan((n, h), DEV)
        for pos in range(D):
            d = (start + pos) % D
            tsp.attn_out_shard(dims, D, pos, d, ad, wod[d], xd if with_residual else None, out, ws,
                               attn_lo=lod if with_lo else None)
        torch.cuda.synchronize()
        check(out, ref, f"attn_out ring steps start={start}")


@pytest.mark.parametrize("h,F,D,n", [(256, 1024, 4, 512), (256, 1024, 4, 300), (512, 2048, 8, 257),
                                     (256, 512, 1, 100), (256, 1024, 2, 16500)])
@pytest.mark.parametrize("with_residual", [False, True])
def test_mlp_ring_steps(h, F, D, n, with_residual):
    require_gpu()
    Fs = F // D
    w1 = [_rnd((Fs, h), 30 + d, 0.02) for d in range(D)]
    w2 = [_rnd((h, Fs), 40 + d, 0.02) for d in range(D)]
    x = _rnd((n, h), 6)
    ref = O.mlp_forward(x, w1, w2, residual=with_residual)
    dims = tsp.make_dims(h, h // 64, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_SHARD)
    w1d, w2d, xd = _dev(w1), _dev(w2), x.to(DEV)
    for start in sorted({0, D - 1}):
        say(f"mlp ring steps h={h} F={F} D={D} n={n} start={start} res={with_residual}")
        y = bf16_nan((n, h), DEV)
        for pos in range(D):
            d = (start + pos) % D
            tsp.mlp_shard(dims, D, pos, xd, w1d[d], w2d[d], xd if with_residual else None, y, ws)
        torch.cuda.synchronize()
        check(y, ref, f"mlp ring steps start={start}")


def test_mlp_ring_steps_y_aliases_residual():
    require_gpu()
    h, F, D, n = 256, 1024, 4, 200
    Fs = F // D
    w1 = [_rnd((Fs, h), 50 + d, 0.02) for d in range(D)]
    w2 = [_rnd((h, Fs), 60 + d, 0.02) for d in range(D)]
    x = _rnd((n, h), 7)
    res = _rnd((n, h), 9)
    ref = O.mlp_forward(x, w1, w2, residual=False) + O.f64(res)
    dims = tsp.make_dims(h, 4, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_SHARD)
    xd, rd = x.to(DEV), res.to(DEV)
    w1d, w2d = _dev(w1), _dev(w2)
    say("mlp ring steps, y = residual")
    for pos in range(D):
        tsp.mlp_shard(dims, D, pos, xd, w1d[pos], w2d[pos], rd, rd, ws)
    torch.cuda.synchronize()
    check(rd, ref, "mlp ring steps in place")


def test_mlp_shards_arriving_on_a_side_stream():
    """Shards copied one by one on a side stream (held back first by unrelated
    work); each ring step waits for its shard's copy event.  The arrival
    buffers start as NaN, so a step that ran before its copy would show."""
    require_gpu()
    h, F, D, n = 512, 2048, 4, 1024
    Fs = F // D
    start = 2
    w1 = _dev([_rnd((Fs, h), 70 + d, 0.02) for d in range(D)])
    w2 = _dev([_rnd((h, Fs), 80 + d, 0.02) for d in range(D)])
    x = _rnd((n, h), 11).to(DEV)
    dims = tsp.make_dims(h, h // 64, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_SHARD)
    compute = torch.cuda.current_stream()

    say("arrival: resident reference")
    y_ref = bf16_nan((n, h), DEV)
    for pos in range(D):
        d = (start + pos) % D
        tsp.mlp_shard(dims, D, pos, x, w1[d], w2[d], x, y_ref, ws, stream=compute)
    torch.cuda.synchronize()

    say("arrival: streamed shards")
    arr1 = [torch.full_like(t, float("nan")) for t in w1]
    arr2 = [torch.full_like(t, float("nan")) for t in w2]
    busy = torch.randn(4096, 4096, device=DEV)
    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    events = []
    with torch.cuda.stream(side):
        for _ in range(8):  # unrelated work ahead of the copies
            busy = busy @ busy * 1e-3
        for pos in range(D):
            d = (start + pos) % D
            arr1[d].copy_(w1[d], non_blocking=True)
            arr2[d].copy_(w2[d], non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(side)
            events.append(ev)
    y = bf16_nan((n, h), DEV)
    for pos in range(D):
        d = (start + pos) % D
        compute.wait_event(events[pos])
        tsp.mlp_shard(dims, D, pos, x, arr1[d], arr2[d], x, y, ws, stream=compute)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref), "streamed result differs from the resident one"
    ref = O.mlp_forward(x.cpu(), [t.cpu() for t in w1], [t.cpu() for t in w2], residual=True)
    check(y, ref, "streamed mlp vs oracle")


def test_mlp_ring_steps_7b_sampled_rows():
    require_gpu()
    W = synth.WORKLOADS["mlp_7b"]
    d, D, n = W.dims, W.D, W.n_local
    say(f"{W.name}: inputs")
    x = synth.activations(W.wid, n, d.hidden, device=DEV)
    lw = synth.layer_weights(W.wid, d, D, device=DEV, parts=("w1", "w2"))
    dims = tsp.make_dims(d.hidden, d.n_heads, d.head_dim, d.ffn)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_SHARD)
    y = bf16_nan((n, d.hidden), DEV)
    for pos in range(D):
        s = (W.start_shard + pos) % D
        say(f"{W.name}: mlp ring step {pos} (shard {s})")
        tsp.mlp_shard(dims, D, pos, x, lw.w1[s], lw.w2[s], None, y, ws)
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(2)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, n // 2 - 1, n // 2, n - 1]),
                                   torch.randint(0, n, (40,), generator=g)]))
    ref = O.mlp_forward(x.cpu(), [t.cpu() for t in lw.w1], [t.cpu() for t in lw.w2], residual=False, rows=rows)
    check(y.cpu()[rows], ref, "7B MLP ring steps, sampled rows")
