"""GPU parity of the layer variants' backwards (tsp_rms_norm_backward,
tsp_rope_backward, tsp_attn_core_gqa_lse, tsp_attn_core_gqa_backward) against
the fp64 oracle.

  * RMSNorm: dx and dgain for ragged row counts (more than one 64-row block),
    widths 256 and 4096, eps 1e-6 and 1e-2;
  * RoPE: the inverse rotation of fp32 gradients of q and of the rank's own K
    rows at their global zigzag positions, up to position 131071;
  * grouped-query attention: dq and the K/V heads' dk/dv (summed over each
    head's query heads) for 1, 2 and 4 query heads per K/V head, with and
    without the forward's low part; with as many K/V heads as query heads the
    GQA calls are bit-identical to the MHA ones.
Tolerances: as the MHA attention backward's (its rounding bound, per query
head, summed over each K/V head's group); RMSNorm and RoPE run in fp32 on
exact inputs and use the standard bound.
"""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, gpu, require_gpu, say
from test_gpu_attn_backward import _bounds, _check

pytestmark = gpu
DEV = "cuda"
F64 = torch.float64


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_990_000 + seed, std, "cpu")


def _f32_nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.float32, device=DEV)


@pytest.mark.parametrize("n,h,eps", [(300, 256, 1e-6), (2048, 4096, 1e-6), (17, 512, 1e-2)])
def test_rms_norm_backward(n, h, eps):
    require_gpu()
    x, gain, dy = _rnd((n, h), 1, 3.0), _rnd((h,), 2), _rnd((n, h), 3)
    rdx, rdg = O.rms_norm_backward(x, gain, eps, dy)
    say(f"rms_norm_backward n={n} h={h} eps={eps}")
    dx = bf16_nan((n, h), DEV)
    dgain = _f32_nan((h,))
    tsp.rms_norm_backward(x.to(DEV), gain.to(DEV), eps, dy.to(DEV), dx, dgain)
    torch.cuda.synchronize()
    check(dx, rdx, "rms_norm dx")
    check(dgain, rdg, "rms_norm dgain")


@pytest.mark.parametrize("S,D,r,H,Hkv,hd,theta", [(2048, 4, 1, 4, 2, 64, 10000.0),
                                                   (131072, 8, 0, 4, 4, 128, 500000.0),
                                                   (1288, 2, 1, 4, 1, 128, 10000.0)])
def test_rope_backward(S, D, r, H, Hkv, hd, theta):
    require_gpu()
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    g = torch.Generator().manual_seed(5)
    dq = torch.randn(n, H * hd, generator=g)
    dk = torch.randn(n, Hkv * hd, generator=g)
    dqd, dkd = dq.to(DEV), dk.to(DEV)
    say(f"rope_backward S={S} D={D} r={r} H={H} Hkv={Hkv} hd={hd}")
    tsp.rope_backward(plan, H, Hkv, hd, theta, dqd, dkd)
    torch.cuda.synchronize()
    check(dqd, O.rope_backward(dq, l2g, H, hd, theta), "rope backward dq")
    check(dkd, O.rope_backward(dk, l2g, Hkv, hd, theta), "rope backward dk_own")


def _gqa_bounds(qf, kf, vf, dof, pos, H, Hkv, hd, with_lo):
    group = H // Hkv
    S, m = kf.shape[0], qf.shape[0]
    bq = torch.zeros(m, H * hd, dtype=F64)
    bk = torch.zeros(S, Hkv * hd, dtype=F64)
    bv = torch.zeros(S, Hkv * hd, dtype=F64)
    for a in range(H):
        qc = slice(a * hd, (a + 1) * hd)
        kc = slice((a // group) * hd, (a // group + 1) * hd)
        q1, k1, v1 = _bounds(qf[:, qc], kf[:, kc], vf[:, kc], dof[:, qc], pos, 1, hd, with_lo)
        bq[:, qc] = q1
        bk[:, kc] += k1
        bv[:, kc] += v1
    return bq, bk, bv


@pytest.mark.parametrize("S,D,r,H,Hkv,hd", [(2048, 4, 1, 8, 4, 64), (1288, 2, 1, 4, 2, 128), (640, 1, 0, 4, 1, 64)])
@pytest.mark.parametrize("with_lo", [False, True])
def test_gqa_backward(S, D, r, H, Hkv, hd, with_lo):
    require_gpu()
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n, h, kvw = plan.n_local, H * hd, Hkv * hd
    dims = tsp.make_dims(h, H, hd, 4 * h)
    q, k, v, do = _rnd((n, h), 10), _rnd((S, kvw), 11), _rnd((S, kvw), 12), _rnd((n, h), 13)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out = bf16_nan((n, h), DEV)
    lo = bf16_nan((n, h), DEV) if with_lo else None
    lse = _f32_nan((H, n))
    say(f"gqa backward S={S} D={D} r={r} H={H} Hkv={Hkv} hd={hd} lo={with_lo}")
    tsp.attn_core_gqa_lse(plan, dims, Hkv, qd, kd, vd, out, lse, attn_lo=lo)
    dq, dk, dv = _f32_nan((n, h)), _f32_nan((S, kvw)), _f32_nan((S, kvw))
    tsp.attn_core_gqa_backward(plan, dims, Hkv, qd, kd, vd, out, lse, dod, dq, dk, dv, attn_lo=lo)
    torch.cuda.synchronize()
    qf, kf, vf, dof = (O.f64(t) for t in (q, k, v, do))
    check(out, O.causal_attention_gqa(qf, l2g, kf, vf, H, Hkv, hd), "gqa forward with lse")
    rq, rk, rv = O.causal_attention_gqa_backward(qf, l2g, kf, vf, dof, H, Hkv, hd)
    bq, bk, bv = _gqa_bounds(qf, kf, vf, dof, l2g, H, Hkv, hd, with_lo)
    _check(dq, rq, bq, "gqa dq")
    _check(dk, rk, bk, "gqa dk")
    _check(dv, rv, bv, "gqa dv")


def test_gqa_backward_with_all_heads_is_mha():
    require_gpu()
    S, D, r, H, hd = 2048, 4, 2, 4, 64
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    n, h = plan.n_local, H * hd
    dims = tsp.make_dims(h, H, hd, 4 * h)
    q, k, v, do = (_rnd(s, 20 + i).to(DEV) for i, s in enumerate([(n, h), (S, h), (S, h), (n, h)]))
    out, lse = bf16_nan((n, h), DEV), _f32_nan((H, n))
    out2, lse2 = bf16_nan((n, h), DEV), _f32_nan((H, n))
    say("gqa = mha: forward with lse")
    tsp.attn_core_lse(plan, dims, q, k, v, out, lse)
    tsp.attn_core_gqa_lse(plan, dims, H, q, k, v, out2, lse2)
    res = []
    for fn in ("mha", "gqa"):
        say(f"gqa = mha: backward ({fn})")
        dq, dk, dv = _f32_nan((n, h)), _f32_nan((S, h)), _f32_nan((S, h))
        if fn == "mha":
            tsp.attn_core_backward(plan, dims, q, k, v, out, lse, do, dq, dk, dv)
        else:
            tsp.attn_core_gqa_backward(plan, dims, H, q, k, v, out, lse, do, dq, dk, dv)
        res.append((dq, dk, dv))
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    for a, b in zip(*res):
        assert torch.equal(a, b)
