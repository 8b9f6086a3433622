"""GPU parity of the projection backwards (tsp_attn_out_backward,
tsp_attn_project_backward) against the fp64 oracle.

  * O projection: d_attn and every shard's dW_o for ring starts 0 and D-1,
    ragged token counts, D = 1, head_dim 64 and 128;
  * QKV projection: dx (with and without the residual's gradient dy) and every
    shard's dW_qkv, same shapes;
  * the 7B shape the benchmark times (16384 tokens, h = 4096, D = 8): d_attn
    on sampled rows and dW_o whole; dx on sampled rows and dW_qkv on sampled
    rows of every shard (each row of dW_qkv_d is one column of dq/dk/dv
    against x: the oracle's function on that one-column sub-problem).

Tolerances.  The bf16 inputs enter the products exactly and accumulate in
fp32; the fp32 gradients dq, dk, dv of the QKV backward are rounded to bf16
first, which bounds the error of each product by 2^-9 sum |a||b|: the oracle's
own function on the absolute values gives that sum, and each element is
checked against 2^-8 of it (margin 2) plus the bf16 rounding of a bf16 output
(2^-8 |ref|) plus 1e-6 of the largest magnitude, or against the forward's
bound 1e-2 + 2e-2 |ref| when that is larger (the elements that only the
derived bound admits are tallied); the whole against relative RMS <= 5e-3.
"""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, check_within, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"
F64 = torch.float64


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_900_000 + seed, std, "cpu")


def _f32(shape, seed, std=1.0):
    g = torch.Generator().manual_seed(9_950_000 + seed)
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def _check_bound(got, ref, bound, name, out_bf16=False):
    """Per element |err| <= max(1e-2 + 2e-2 |ref|, derived), derived = 2^-8 bound
    (+ 2^-8 |ref| for a bf16 output) + 1e-6 max|ref|; relative RMS <= 5e-3.
    The elements only the derived bound admits are tallied."""
    lim = 2.0 ** -8 * bound + (2.0 ** -8 * ref.abs() if out_bf16 else 0) + 1e-6 * ref.abs().max().item() + 1e-12
    check_within(got, ref, lim, name)


def _f32_nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


SHAPES = [(256, 4, 64, 4, 512), (512, 4, 128, 2, 300), (256, 4, 64, 1, 129), (1024, 8, 128, 8, 2048)]


@pytest.mark.parametrize("h,H,hd,D,n", SHAPES)
def test_attn_out_backward(h, H, hd, D, n):
    require_gpu()
    hs = (H // D) * hd
    attn = _rnd((n, h), 1)
    wo = [_rnd((h, hs), 10 + d, 0.02) for d in range(D)]
    dout = _rnd((n, h), 2)
    r_attn, r_dwo = O.attn_out_backward(attn, wo, dout)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_BWD)
    for start in sorted({0, D - 1}):
        say(f"attn_out_backward h={h} hd={hd} D={D} n={n} start={start}")
        d_attn = bf16_nan((n, h), DEV)
        dwo = [_f32_nan((h, hs)) for _ in range(D)]
        tsp.attn_out_backward(dims, D, start, attn.to(DEV), [w.to(DEV) for w in wo], dout.to(DEV), d_attn, dwo, ws)
        torch.cuda.synchronize()
        check(d_attn, r_attn, "d_attn")
        for d in range(D):
            check(dwo[d], r_dwo[d], f"dW_o[{d}]")


@pytest.mark.parametrize("h,H,hd,D,n", SHAPES)
@pytest.mark.parametrize("with_dy", [False, True])
def test_attn_project_backward(h, H, hd, D, n, with_dy):
    require_gpu()
    hs = (H // D) * hd
    x = _rnd((n, h), 3)
    w = [_rnd((3 * hs, h), 20 + d, 0.02) for d in range(D)]
    dq, dk, dv = _f32((n, h), 4), _f32((n, h), 5), _f32((n, h), 6)
    dy = _rnd((n, h), 7) if with_dy else None
    r_dx, r_dw = O.qkv_projection_backward(x, w, dq, dk, dv, hd, dy=dy)
    b_dx, b_dw = O.qkv_projection_backward(O.f64(x).abs(), [O.f64(t).abs() for t in w], dq.abs(), dk.abs(),
                                           dv.abs(), hd)
    dims = tsp.make_dims(h, H, hd, 4 * h)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_PROJ_BWD)
    for start in sorted({0, D - 1}):
        say(f"attn_project_backward h={h} hd={hd} D={D} n={n} start={start} dy={with_dy}")
        dx = bf16_nan((n, h), DEV)
        dw = [_f32_nan((3 * hs, h)) for _ in range(D)]
        tsp.attn_project_backward(dims, D, start, x.to(DEV), [t.to(DEV) for t in w], dq.to(DEV), dk.to(DEV),
                                  dv.to(DEV), dy.to(DEV) if with_dy else None, dx, dw, ws)
        torch.cuda.synchronize()
        _check_bound(dx, r_dx, b_dx, "dx", out_bf16=True)
        for d in range(D):
            _check_bound(dw[d], r_dw[d], b_dw[d], f"dW_qkv[{d}]")


def test_projection_backwards_7b_sampled():
    require_gpu()
    W = synth.WORKLOADS["attn_7b"]
    d, D = W.dims, W.D
    n, h, H, hd = 16384, d.hidden, d.n_heads, d.head_dim
    hs = (H // D) * hd
    dims = tsp.make_dims(h, H, hd, d.ffn)
    say("7B projection backwards: inputs")
    lw = synth.layer_weights(W.wid, d, D, device=DEV, parts=("wqkv", "wo"))
    x = synth.activations(W.wid, n, h, device=DEV)
    attn = synth.randn_bf16((n, h), 9_960_001, 1.0, DEV)
    dout = synth.randn_bf16((n, h), 9_960_002, 1.0, DEV)
    dq, dk, dv = (synth.randn_bf16((n, h), 9_960_003 + i, 1.0, DEV).float() for i in range(3))
    say("7B attn_out_backward")
    d_attn = bf16_nan((n, h), DEV)
    dwo = [_f32_nan((h, hs)) for _ in range(D)]
    tsp.attn_out_backward(dims, D, W.rank, attn, lw.wo, dout, d_attn, dwo,
                          tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_BWD))
    say("7B attn_project_backward")
    dx = bf16_nan((n, h), DEV)
    dw = [_f32_nan((3 * hs, h)) for _ in range(D)]
    tsp.attn_project_backward(dims, D, W.rank, x, lw.wqkv, dq, dk, dv, dout, dx, dw,
                              tsp.alloc_workspace(n, dims, D, tsp.WS_PROJ_BWD))
    torch.cuda.synchronize()

    g = torch.Generator().manual_seed(11)
    rows = torch.unique(torch.cat([torch.tensor([0, 1, n // 2, n - 1]), torch.randint(0, n, (12,), generator=g)]))
    wo_c = [t.cpu() for t in lw.wo]
    wq_c = [t.cpu() for t in lw.wqkv]
    say("7B oracle: O projection")
    r_attn, _ = O.attn_out_backward(attn.cpu()[rows], wo_c, dout.cpu()[rows])
    check(d_attn.cpu()[rows], r_attn, "7B d_attn sampled rows")
    _, r_dwo = O.attn_out_backward(attn.cpu(), wo_c, dout.cpu())
    for s in range(D):
        check(dwo[s], r_dwo[s], f"7B dW_o[{s}]")
    say("7B oracle: QKV projection, sampled dx rows")
    xc, dqc, dkc, dvc, dyc = x.cpu(), dq.cpu(), dk.cpu(), dv.cpu(), dout.cpu()
    r_dx, _ = O.qkv_projection_backward(xc[rows], wq_c, dqc[rows], dkc[rows], dvc[rows], hd, dy=dyc[rows])
    b_dx, _ = O.qkv_projection_backward(O.f64(xc[rows]).abs(), [O.f64(t).abs() for t in wq_c], dqc[rows].abs(),
                                        dkc[rows].abs(), dvc[rows].abs(), hd)
    _check_bound(dx.cpu()[rows], r_dx, b_dx, "7B dx sampled rows", out_bf16=True)
    say("7B oracle: QKV projection, sampled dW rows")
    for s in range(D):
        c = s * hs + int(torch.randint(0, hs, (1,), generator=g))  # one q/k/v column of shard s
        one = [torch.zeros(3, h, dtype=torch.bfloat16)]                # a one-head-column "shard"
        sub = lambda t: t[:, c:c + 1]
        _, r = O.qkv_projection_backward(xc, one, sub(dqc), sub(dkc), sub(dvc), 1)
        _, b = O.qkv_projection_backward(O.f64(xc).abs(), one, sub(dqc).abs(), sub(dkc).abs(), sub(dvc).abs(), 1)
        j = c - s * hs
        got = torch.stack([dw[s][j], dw[s][hs + j], dw[s][2 * hs + j]])
        _check_bound(got, r[0], b[0], f"7B dW_qkv[{s}] rows of column {c}")
