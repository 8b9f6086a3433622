"""Edge cases of the backward calls on the GPU:
  * no tokens: the weight gradients of the MLP, O-projection and QKV-projection
    backwards are zero (the sum over an empty token set), dgain of the RMSNorm
    backward is zero, and nothing else is written;
  * the largest shard count (D = 16): the MLP and projection backwards against
    the oracle.
"""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, gpu, require_gpu, say
from test_gpu_backward import check_rounded_product
from test_gpu_proj_backward import _check_bound

pytestmark = gpu
DEV = "cuda"


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_970_000 + seed, std, "cpu")


def _nan32(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


def test_no_tokens_gives_zero_weight_gradients():
    require_gpu()
    h, H, hd, D, F = 256, 4, 64, 4, 1024
    hs, fs = (H // D) * hd, F // D
    dims = tsp.make_dims(h, H, hd, F)
    # zero-row tensors (their data pointers are null: the calls must not need them)
    empty = bf16_nan((1, h), DEV)[:0]
    dx_buf = bf16_nan((1, h), DEV)
    w1 = [_rnd((fs, h), d).to(DEV) for d in range(D)]
    w2 = [_rnd((h, fs), 10 + d).to(DEV) for d in range(D)]
    dw1, dw2 = [_nan32((fs, h)) for _ in range(D)], [_nan32((h, fs)) for _ in range(D)]
    say("no tokens: mlp_backward")
    tsp.mlp_backward(dims, D, 1, True, empty, w1, w2, empty, dx_buf[:0], dw1, dw2,
                     torch.empty(256 + tsp.workspace_size(0, dims, D, tsp.WS_MLP_BWD), dtype=torch.uint8, device=DEV))
    wo = [_rnd((h, hs), 20 + d).to(DEV) for d in range(D)]
    dwo = [_nan32((h, hs)) for _ in range(D)]
    say("no tokens: attn_out_backward")
    tsp.attn_out_backward(dims, D, 0, empty, wo, empty, dx_buf[:0], dwo, torch.empty(256 + tsp.workspace_size(
        0, dims, D, tsp.WS_OUT_BWD), dtype=torch.uint8, device=DEV))
    wq = [_rnd((3 * hs, h), 30 + d).to(DEV) for d in range(D)]
    dwq = [_nan32((3 * hs, h)) for _ in range(D)]
    g32 = _nan32((1, h))[:0]
    say("no tokens: attn_project_backward")
    tsp.attn_project_backward(dims, D, 2, empty, wq, g32, g32, g32, None, dx_buf[:0], dwq, torch.empty(
        256 + tsp.workspace_size(0, dims, D, tsp.WS_PROJ_BWD), dtype=torch.uint8, device=DEV))
    say("no tokens: rms_norm_backward")
    dgain = _nan32((h,))
    tsp.rms_norm_backward(empty, _rnd((h,), 40).to(DEV), 1e-6, empty, dx_buf[:0], dgain,
                          workspace=torch.empty(256, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    for t in dw1 + dw2 + dwo + dwq + [dgain]:
        assert torch.count_nonzero(t).item() == 0 and not torch.isnan(t).any()
    assert torch.isnan(dx_buf.float()).all(), "nothing else is written"


def test_sixteen_shards():
    require_gpu()
    h, H, hd, D, F, n = 1024, 16, 64, 16, 2048, 300
    hs, fs = (H // D) * hd, F // D
    dims = tsp.make_dims(h, H, hd, F)
    x, dy = _rnd((n, h), 50), _rnd((n, h), 51)
    w1 = [_rnd((fs, h), 60 + d, 0.02) for d in range(D)]
    w2 = [_rnd((h, fs), 80 + d, 0.02) for d in range(D)]
    say("D=16: mlp_backward")
    dx = bf16_nan((n, h), DEV)
    dw1, dw2 = [_nan32((fs, h)) for _ in range(D)], [_nan32((h, fs)) for _ in range(D)]
    tsp.mlp_backward(dims, D, 5, True, x.to(DEV), [t.to(DEV) for t in w1], [t.to(DEV) for t in w2], dy.to(DEV), dx,
                     dw1, dw2, tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_BWD))
    torch.cuda.synchronize()
    rdx, rdw1, rdw2 = O.mlp_backward(x, w1, w2, dy, residual=True)
    check(dx, rdx, "D=16 dx")
    xa, dya = O.f64(x).abs(), O.f64(dy).abs()
    for d in range(D):
        U = O.linear(O.f64(x), O.f64(w1[d]))
        dU = torch.matmul(O.f64(dy), O.f64(w2[d])) * O.gelu_tanh_grad(U)
        check_rounded_product(dw1[d], rdw1[d], dU.abs().t(), xa, f"D=16 dW1[{d}]")
        check_rounded_product(dw2[d], rdw2[d], dya.t(), O.gelu_tanh(U).abs(), f"D=16 dW2[{d}]")
    say("D=16: projection backwards")
    wq = [_rnd((3 * hs, h), 100 + d, 0.02) for d in range(D)]
    g = torch.Generator().manual_seed(7)
    dq, dk, dv = (torch.randn(n, h, generator=g) for _ in range(3))
    dxp = bf16_nan((n, h), DEV)
    dwq = [_nan32((3 * hs, h)) for _ in range(D)]
    tsp.attn_project_backward(dims, D, 15, x.to(DEV), [t.to(DEV) for t in wq], dq.to(DEV), dk.to(DEV), dv.to(DEV),
                              dy.to(DEV), dxp, dwq, tsp.alloc_workspace(n, dims, D, tsp.WS_PROJ_BWD))
    wo = [_rnd((h, hs), 120 + d, 0.02) for d in range(D)]
    d_attn = bf16_nan((n, h), DEV)
    dwo = [_nan32((h, hs)) for _ in range(D)]
    tsp.attn_out_backward(dims, D, 9, x.to(DEV), [t.to(DEV) for t in wo], dy.to(DEV), d_attn, dwo,
                          tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_BWD))
    torch.cuda.synchronize()
    r_dx, r_dw = O.qkv_projection_backward(x, wq, dq, dk, dv, hd, dy=dy)
    b_dx, b_dw = O.qkv_projection_backward(O.f64(x).abs(), [O.f64(t).abs() for t in wq], dq.abs(), dk.abs(),
                                           dv.abs(), hd)
    _check_bound(dxp, r_dx, b_dx, "D=16 QKV dx", out_bf16=True)
    for d in range(D):
        _check_bound(dwq[d], r_dw[d], b_dw[d], f"D=16 dW_qkv[{d}]")
    r_attn, r_dwo = O.attn_out_backward(x, wo, dy)
    check(d_attn, r_attn, "D=16 d_attn")
    for d in range(D):
        check(dwo[d], r_dwo[d], f"D=16 dW_o[{d}]")
