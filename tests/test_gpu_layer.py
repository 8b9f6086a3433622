"""GPU parity of the whole rank-share layer (tsp_attn_forward, tsp_layer_forward)
against the fp64 oracle on the tiny TSP layer (h=256, 4 heads x 64, FFN 1024,
D=4, S=2048 in 8 zigzag chunks of 256, rank 1), including the D-rank
emulation that stands in for the collectives on one GPU:

  phase 1: every rank r projects its own K/V rows into one shared k_full/v_full
           (the K/V all-gather of the method),
  phase 2: every rank runs its layer against the gathered K/V,

and the reassembled outputs of all D ranks must equal the oracle's unsharded
layer over all S tokens."""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, check_rms, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"
W = synth.WORKLOADS["tiny_layer"]


def _tiny_inputs(D=None):
    D = D or W.D
    d = W.dims
    x_all = synth.activations(W.wid, W.seq_len, d.hidden, tensor_id=synth.TID_X_ALL)
    lw = synth.layer_weights(W.wid, d, D)
    return d, x_all, lw


def _gather_phase(plan_by_rank, dims, x_all_dev, lw_dev, S, h):
    """Every rank writes its own K/V rows into the shared buffers (the all-gather)."""
    kf = bf16_nan((S, h), DEV)
    vf = bf16_nan((S, h), DEV)
    for r, (plan, l2g) in enumerate(plan_by_rank):
        q = torch.empty(plan.n_local, h, dtype=torch.bfloat16, device=DEV)
        tsp.attn_project(plan, dims, x_all_dev[l2g.to(DEV)].contiguous(), lw_dev.wqkv, kf, vf, q)
    return kf, vf


@pytest.mark.parametrize("D", [4, 2, 1])
def test_rank_emulation_reassembles_unsharded_layer(D):
    require_gpu()
    d, x_all, lw = _tiny_inputs(D)
    S, h = W.seq_len, d.hidden
    dims = tsp.make_dims(d.hidden, d.n_heads, d.head_dim, d.ffn)
    lw_dev = lw.to(DEV)
    x_dev = x_all.to(DEV)
    plans = [tsp.zigzag_plan(S, D, r)[:2] for r in range(D)]
    say(f"tiny layer D={D}: gather phase")
    kf, vf = _gather_phase(plans, dims, x_dev, lw_dev, S, h)
    torch.cuda.synchronize()
    assert not torch.isnan(kf.float()).any() and not torch.isnan(vf.float()).any(), "K/V rows left unwritten"
    out_all = bf16_nan((S, h), DEV)
    for r, (plan, l2g) in enumerate(plans):
        say(f"tiny layer D={D}: rank {r}")
        ws = tsp.alloc_workspace(plan.n_local, dims, D, tsp.WS_LAYER)
        out = bf16_nan((plan.n_local, h), DEV)
        tsp.layer_forward(plan, dims, x_dev[l2g.to(DEV)].contiguous(), lw_dev.wqkv, lw_dev.wo, lw_dev.w1,
                          lw_dev.w2, kf, vf, out, ws)
        out_all[l2g.to(DEV)] = out
    torch.cuda.synchronize()
    ref, _, _ = O.layer_forward(O.zigzag_plan(S, 1, 0), x_all, lw.wqkv, lw.wo, lw.w1, lw.w2, d.n_heads, d.head_dim)
    check(out_all, ref, f"reassembled layer D={D}")
    ref_x, _, _ = O.layer_forward(O.zigzag_plan(S, 1, 0), x_all, lw.wqkv, lw.wo, lw.w1, lw.w2, d.n_heads, d.head_dim,
                                  proj_bf16=False)
    check_rms(out_all, ref_x, f"reassembled layer D={D}, unrounded Q/K/V")


def test_tiny_layer_rank1_against_oracle_rank_view():
    """Rank 1 of the tiny layer: the oracle takes rank 1's rows and the K/V of all
    ranks computed from the same x (its own fp64 projections)."""
    require_gpu()
    d, x_all, lw = _tiny_inputs()
    S, h, D, r = W.seq_len, d.hidden, W.D, W.rank
    dims = tsp.make_dims(d.hidden, d.n_heads, d.head_dim, d.ffn)
    lw_dev = lw.to(DEV)
    x_dev = x_all.to(DEV)
    plans = [tsp.zigzag_plan(S, D, rr)[:2] for rr in range(D)]
    say("tiny layer rank 1: gather phase")
    kf, vf = _gather_phase(plans, dims, x_dev, lw_dev, S, h)
    plan, l2g = plans[r]
    ws = tsp.alloc_workspace(plan.n_local, dims, D, tsp.WS_LAYER)
    out = bf16_nan((plan.n_local, h), DEV)
    say("tiny layer rank 1: layer")
    tsp.layer_forward(plan, dims, x_dev[l2g.to(DEV)].contiguous(), lw_dev.wqkv, lw_dev.wo, lw_dev.w1, lw_dev.w2,
                      kf, vf, out, ws)
    # attention half alone, with the residual, through tsp_attn_forward
    wsa = tsp.alloc_workspace(plan.n_local, dims, D, tsp.WS_ATTN)
    h1 = bf16_nan((plan.n_local, h), DEV)
    xl = x_dev[l2g.to(DEV)].contiguous()
    tsp.attn_forward(plan, dims, xl, lw_dev.wqkv, lw_dev.wo, kf, vf, xl, h1, wsa)
    torch.cuda.synchronize()
    oplan = O.zigzag_plan(S, D, r)
    _, k_all, v_all = O.qkv_projection(x_all, lw.wqkv, d.head_dim)
    ref, _, _ = O.layer_forward(oplan, x_all[oplan.local_to_global], lw.wqkv, lw.wo, lw.w1, lw.w2, d.n_heads,
                                d.head_dim, k_all, v_all)
    check(out, ref, "tiny layer rank 1")
    ref_h1, _, _, _ = O.attn_forward(oplan, x_all[oplan.local_to_global], lw.wqkv, lw.wo, d.n_heads, d.head_dim,
                                     k_all, v_all, residual=True)
    check(h1, ref_h1, "tiny attention half rank 1")
    # the same against the oracle that keeps Q, K and V unrounded
    ref_x, _, _ = O.layer_forward(oplan, x_all[oplan.local_to_global], lw.wqkv, lw.wo, lw.w1, lw.w2, d.n_heads,
                                  d.head_dim, k_all, v_all, proj_bf16=False)
    check_rms(out, ref_x, "tiny layer rank 1, unrounded Q/K/V")
    ref_h1x, _, _, _ = O.attn_forward(oplan, x_all[oplan.local_to_global], lw.wqkv, lw.wo, d.n_heads, d.head_dim,
                                      k_all, v_all, residual=True, proj_bf16=False)
    check_rms(h1, ref_h1x, "tiny attention half rank 1, unrounded Q/K/V")


def test_layer_zero_weights_is_identity():
    """W_o = 0 and W2 = 0 make the layer the identity: out must equal x exactly."""
    require_gpu()
    d, x_all, lw = _tiny_inputs()
    S, h, D, r = W.seq_len, d.hidden, W.D, 2
    dims = tsp.make_dims(d.hidden, d.n_heads, d.head_dim, d.ffn)
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    kf, vf = synth.gathered_kv(W.wid, S, h)
    lw_dev = lw.to(DEV)
    zeros = lambda ts: [torch.zeros_like(t) for t in ts]
    xl = x_all[l2g].contiguous().to(DEV)
    ws = tsp.alloc_workspace(plan.n_local, dims, D, tsp.WS_LAYER)
    out = bf16_nan((plan.n_local, h), DEV)
    say("layer with zero W_o and W2")
    tsp.layer_forward(plan, dims, xl, lw_dev.wqkv, zeros(lw_dev.wo), lw_dev.w1, zeros(lw_dev.w2), kf.to(DEV),
                      vf.to(DEV), out, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, xl)
