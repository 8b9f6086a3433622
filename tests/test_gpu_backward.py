"""GPU parity of the MLP ring's backward pass (tsp_mlp_backward) against the
fp64 oracle: dx, and each shard's weight-gradient contributions dW1_d, dW2_d,
for every ring start tested, with and without the forward's residual, ragged
token counts (the token contractions run over zero-padded transposes), D = 1,
and a mid-size shape (2048 tokens, h = 1024, F = 4096).

Tolerances.  dx meets the forward's bound (|err| <= 1e-2 + 2e-2 |o|).  The
weight gradients sum over all tokens products one of whose factors (dU_d or
GELU(U_d)) the GPU holds in bf16: one rounding of one operand of a dot product
bounds its error by 2^-9 sum_k |a_k| |b_k| (the fp32 accumulation adds far
less).  Each element is checked against the larger of the forward's bound and
2^-8 (|a|^T |b|) (a margin of 2), with the oracle's fp64 operands; the number
of elements that only the second admits is tallied.  The whole is checked
against relative RMS <= 5e-3."""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, check_within, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_900_000 + seed, std, "cpu")


def check_rounded_product(got, ref, a_abs, b_abs, name):
    """|got - ref| <= max(1e-2 + 2e-2 |ref|, 2^-8 (|a|^T |b|)) per element (the
    second: one bf16 rounding of one operand, margin 2), and relative RMS <=
    REL_RMS; the elements only the derived bound admits are tallied."""
    bound = 2.0 ** -8 * (a_abs @ b_abs) + 1e-9
    check_within(got, ref, bound, name)


@pytest.mark.parametrize("h,F,D,n", [(256, 1024, 4, 512), (256, 1024, 4, 300), (512, 2048, 8, 257),
                                     (256, 512, 1, 100), (1024, 4096, 4, 2048)])
@pytest.mark.parametrize("residual", [False, True])
def test_mlp_backward(h, F, D, n, residual):
    _mlp_backward_case(h, F, D, n, residual, 1.0)


@pytest.mark.parametrize("k", [2, 6, 12])
def test_mlp_backward_scaled(k):
    """x at 2.5^k times unit scale (layer k of a chained stack without a norm):
    U = x W1 far out on both tails of GELU and GELU', U up to about 10^5 at
    k = 12 (beyond fp16's range before the per-row scaling)."""
    _mlp_backward_case(512, 2048, 8, 257, True, 2.5 ** k)


def _mlp_backward_case(h, F, D, n, residual, x_scale):
    require_gpu()
    Fs = F // D
    w1 = [_rnd((Fs, h), 10 + d, 0.02) for d in range(D)]
    w2 = [_rnd((h, Fs), 30 + d, 0.02) for d in range(D)]
    x = _rnd((n, h), 1, x_scale)
    dy = _rnd((n, h), 2)
    dx_ref, dw1_ref, dw2_ref = O.mlp_backward(x, w1, w2, dy, residual=residual)
    # the oracle's per-shard factors of the weight gradients, for their rounding bounds
    xa, dya = O.f64(x).abs(), O.f64(dy).abs()
    U = [O.linear(O.f64(x), O.f64(w)) for w in w1]
    H = [O.gelu_tanh(u) for u in U]
    dU = [torch.matmul(O.f64(dy), O.f64(w2[d])) * O.gelu_tanh_grad(U[d]) for d in range(D)]
    dims = tsp.make_dims(h, h // 64, 64, F)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_BWD)
    xd, dyd, w1d, w2d = x.to(DEV), dy.to(DEV), [t.to(DEV) for t in w1], [t.to(DEV) for t in w2]
    for start in sorted({0, D - 1}):
        say(f"mlp backward h={h} F={F} D={D} n={n} start={start} residual={residual} x scale={x_scale:g}")
        dx = bf16_nan((n, h), DEV)
        dw1 = [torch.full((Fs, h), float("nan"), device=DEV) for _ in range(D)]
        dw2 = [torch.full((h, Fs), float("nan"), device=DEV) for _ in range(D)]
        tsp.mlp_backward(dims, D, start, residual, xd, w1d, w2d, dyd, dx, dw1, dw2, ws)
        torch.cuda.synchronize()
        check(dx, dx_ref, f"dx start={start}")
        for d in range(D):
            check_rounded_product(dw1[d], dw1_ref[d], dU[d].abs().t(), xa, f"dW1[{d}]")
            check_rounded_product(dw2[d], dw2_ref[d], dya.t(), H[d].abs(), f"dW2[{d}]")
