"""HIP-graph capture of the library's calls (they launch kernels only: no
allocation, no memset, no synchronisation), replayed several times with eager
work between the replays; every replay must reproduce the eager results bit
for bit, starting from outputs filled with NaN.

  * a whole layer (tsp_layer_forward) at S = 2048, D = 4;
  * the backward of attention (with its forward keeping the normaliser), of
    the O and QKV projections and of the MLP, captured together;
  * the QKV, O and MLP calls that wait for their shards on a device counter
    (every shard arrived), captured together.
"""
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from parity import bf16_nan, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"
REPLAYS = 3


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_880_000 + seed, std, DEV)


def _nan_fill(ts):
    for t in ts:
        t.fill_(float("nan"))


def _replay_and_compare(graph, outs, refs, name):
    side = torch.randn(1024, 1024, device=DEV)
    for r in range(REPLAYS):
        _nan_fill(outs)
        torch.cuda.synchronize()
        side = side @ side * 1e-3  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        for o, ref in zip(outs, refs):
            assert torch.equal(o, ref), f"{name}: replay {r} differs from the eager result"
        say(f"{name}: replay {r} matches")


def test_layer_forward_graph():
    require_gpu()
    S, D, r, h, H, hd, F = 2048, 4, 1, 256, 4, 64, 1024
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    Hs, Fs = H // D, F // D
    dims = tsp.make_dims(h, H, hd, F)
    x = _rnd((n, h), 1)
    wqkv = [_rnd((3 * Hs * hd, h), 10 + d, 0.05) for d in range(D)]
    wo = [_rnd((h, Hs * hd), 20 + d, 0.05) for d in range(D)]
    w1 = [_rnd((Fs, h), 30 + d, 0.05) for d in range(D)]
    w2 = [_rnd((h, Fs), 40 + d, 0.05) for d in range(D)]
    kf, vf = _rnd((S, h), 2), _rnd((S, h), 3)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_LAYER)
    say("graph: eager layer")
    ref = bf16_nan((n, h), DEV)
    tsp.layer_forward(plan, dims, x, wqkv, wo, w1, w2, kf, vf, ref, ws)
    torch.cuda.synchronize()
    out = bf16_nan((n, h), DEV)
    g = torch.cuda.CUDAGraph()
    say("graph: capture layer")
    with torch.cuda.graph(g):
        tsp.layer_forward(plan, dims, x, wqkv, wo, w1, w2, kf, vf, out, ws)
    _replay_and_compare(g, [out], [ref], "layer_forward")


def test_backward_graph():
    require_gpu()
    S, D, r, h, H, hd, F = 2048, 4, 2, 256, 4, 64, 1024
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    Hs, Fs, hs = H // D, F // D, (H // D) * hd
    dims = tsp.make_dims(h, H, hd, F)
    q, k, v, do = _rnd((n, h), 50), _rnd((S, h), 51), _rnd((S, h), 52), _rnd((n, h), 53)
    x = _rnd((n, h), 54)
    wqkv = [_rnd((3 * hs, h), 60 + d, 0.05) for d in range(D)]
    wo = [_rnd((h, hs), 70 + d, 0.05) for d in range(D)]
    w1 = [_rnd((Fs, h), 80 + d, 0.05) for d in range(D)]
    w2 = [_rnd((h, Fs), 90 + d, 0.05) for d in range(D)]
    ws_a = tsp.alloc_workspace(n, dims, D, tsp.WS_ATTN_BWD)
    ws_o = tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_BWD)
    ws_p = tsp.alloc_workspace(n, dims, D, tsp.WS_PROJ_BWD)
    ws_m = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_BWD)
    ws_c = tsp.alloc_workspace(n, dims, D, tsp.WS_CORE)
    f32 = lambda shape: torch.empty(shape, dtype=torch.float32, device=DEV)
    bf = lambda shape: torch.empty(shape, dtype=torch.bfloat16, device=DEV)

    def buffers():
        return dict(attn=bf((n, h)), lse=f32((H, n)), dq=f32((n, h)), dk=f32((S, h)), dv=f32((S, h)),
                    d_attn=bf((n, h)), dwo=[f32((h, hs)) for _ in range(D)], dx=bf((n, h)),
                    dwqkv=[f32((3 * hs, h)) for _ in range(D)], dxm=bf((n, h)),
                    dw1=[f32((Fs, h)) for _ in range(D)], dw2=[f32((h, Fs)) for _ in range(D)])

    def run(b):
        tsp.attn_core_lse(plan, dims, q, k, v, b["attn"], b["lse"], workspace=ws_c)
        tsp.attn_core_backward(plan, dims, q, k, v, b["attn"], b["lse"], do, b["dq"], b["dk"], b["dv"],
                               workspace=ws_a)
        tsp.attn_out_backward(dims, D, r, b["attn"], wo, do, b["d_attn"], b["dwo"], ws_o)
        tsp.attn_project_backward(dims, D, r, x, wqkv, b["dq"], b["dq"], b["dq"], do, b["dx"], b["dwqkv"], ws_p)
        tsp.mlp_backward(dims, D, r, True, x, w1, w2, do, b["dxm"], b["dw1"], b["dw2"], ws_m)

    def flat(b):
        out = []
        for key in sorted(b):
            out += b[key] if isinstance(b[key], list) else [b[key]]
        return out

    say("graph: eager backward")
    eager = buffers()
    run(eager)
    torch.cuda.synchronize()
    cap = buffers()
    g = torch.cuda.CUDAGraph()
    say("graph: capture backward")
    with torch.cuda.graph(g):
        run(cap)
    _replay_and_compare(g, flat(cap), flat(eager), "backward")


def test_arrival_calls_graph():
    """The calls that wait for their shards on a device counter, captured with
    the counter showing every shard arrived: each replay equals the eager
    all-shard calls."""
    require_gpu()
    S, D, r, h, H, hd, F = 2048, 4, 1, 256, 4, 64, 1024
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    Hs, Fs = H // D, F // D
    dims = tsp.make_dims(h, H, hd, F)
    x, a = _rnd((n, h), 51), _rnd((n, h), 52)
    lo = (_rnd((n, h), 53) * 2 ** -9).to(torch.bfloat16)
    wqkv = [_rnd((3 * Hs * hd, h), 60 + d, 0.05) for d in range(D)]
    wo = [_rnd((h, Hs * hd), 70 + d, 0.05) for d in range(D)]
    w1 = [_rnd((Fs, h), 80 + d, 0.05) for d in range(D)]
    w2 = [_rnd((h, Fs), 90 + d, 0.05) for d in range(D)]
    kf0, vf0 = _rnd((S, h), 54), _rnd((S, h), 55)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP)
    counter = torch.full((4,), D, dtype=torch.int32, device=DEV)
    status = torch.zeros(4, dtype=torch.int32, device=DEV)
    arr = tsp.make_arrival(counter, 0, status)

    def eager_refs():
        q, k, v = bf16_nan((n, h), DEV), kf0.clone(), vf0.clone()
        tsp.attn_project(plan, dims, x, wqkv, k, v, q)
        o, y = bf16_nan((n, h), DEV), bf16_nan((n, h), DEV)
        tsp.attn_out(dims, D, r, a, wo, x, o, attn_lo=lo)
        tsp.mlp_forward(dims, D, r, x, w1, w2, x, y, ws)
        return [q, k, v, o, y]

    say("graph: eager all-shard calls")
    refs = eager_refs()
    torch.cuda.synchronize()
    q, k, v = bf16_nan((n, h), DEV), kf0.clone(), vf0.clone()
    o, y = bf16_nan((n, h), DEV), bf16_nan((n, h), DEV)
    g = torch.cuda.CUDAGraph()
    say("graph: capture arrival calls")
    with torch.cuda.graph(g):
        tsp.attn_project_arrival(plan, dims, r, x, wqkv, k, v, q, arr)
        tsp.attn_out_arrival(dims, D, r, a, wo, x, o, arr, attn_lo=lo)
        tsp.mlp_forward_arrival(dims, D, r, x, w1, w2, x, y, ws, arr)
    # k and v keep their other rows between replays: refill only q, o, y
    _replay_and_compare(g, [q, o, y], [refs[0], refs[3], refs[4]], "arrival calls")
    assert torch.equal(k, refs[1]) and torch.equal(v, refs[2])
    assert int(status[0]) == 0
