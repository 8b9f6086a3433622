"""GPU parity of the layer variants (tsp_rms_norm, tsp_rope, tsp_attn_project_gqa,
tsp_attn_core_gqa) against the fp64 oracle.

  * RMSNorm: ragged row counts, widths 256 and 4096, in place, eps 1e-6 and 1e-2;
  * RoPE of the local queries and of the rank's own K rows at their global
    zigzag positions, up to position 131071 (the 128K sequence), with the rows
    of other ranks untouched; theta 10^4 and 5*10^5;
  * grouped-query projection and attention: the projection's Q, K and V
    columns, and attention with 1, 2 and 4 query heads per K/V head; with as
    many K/V heads as query heads the GQA calls are bit-identical to the MHA
    ones; the composed projection -> RoPE -> attention path against the oracle.
The rotated Q and K are bf16 tensors, like the projections' outputs, so the
oracle rounds them before attention (the same reading as for Q, K and V).
"""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_700_000 + seed, std, "cpu")


def _bf16(t):
    return t.to(torch.bfloat16)


@pytest.mark.parametrize("n,h,eps", [(300, 256, 1e-6), (2048, 4096, 1e-6), (17, 512, 1e-2)])
def test_rms_norm(n, h, eps):
    require_gpu()
    x = _rnd((n, h), 1, 3.0)
    gain = _rnd((h,), 2)
    ref = O.rms_norm(x, gain, eps)
    say(f"rms_norm n={n} h={h} eps={eps}")
    y = bf16_nan((n, h), DEV)
    tsp.rms_norm(x.to(DEV), gain.to(DEV), eps, y)
    torch.cuda.synchronize()
    check(y, ref, "rms_norm")
    say("rms_norm in place")
    xd = x.to(DEV)
    tsp.rms_norm(xd, gain.to(DEV), eps, xd)
    torch.cuda.synchronize()
    assert torch.equal(xd, y)


@pytest.mark.parametrize("S,D,r,H,Hkv,hd,theta", [(2048, 4, 1, 4, 2, 64, 10000.0),
                                                   (131072, 8, 0, 4, 4, 128, 500000.0),
                                                   (1288, 2, 1, 4, 1, 128, 10000.0)])
def test_rope_local_queries_and_own_keys(S, D, r, H, Hkv, hd, theta):
    require_gpu()
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    q = _rnd((n, H * hd), 3)
    k = _rnd((S, Hkv * hd), 4)
    qd, kd = q.to(DEV), k.to(DEV)
    say(f"rope S={S} D={D} r={r} H={H} Hkv={Hkv} hd={hd} theta={theta}")
    tsp.rope(plan, H, Hkv, hd, theta, qd, kd)
    torch.cuda.synchronize()
    check(qd, O.rope(q, l2g, H, hd, theta), "rope q")
    check(kd.cpu()[l2g], O.rope(k[l2g], l2g, Hkv, hd, theta), "rope own k rows")
    others = torch.ones(S, dtype=torch.bool)
    others[l2g] = False
    assert torch.equal(kd.cpu()[others], k[others]), "rows of other ranks must be untouched"


def test_gqa_with_all_heads_is_mha():
    require_gpu()
    S, D, r, H, hd = 2048, 4, 1, 4, 64
    h = H * hd
    plan, _, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    dims = tsp.make_dims(h, H, hd, 4 * h)
    x = _rnd((n, h), 5).to(DEV)
    w = [_rnd((3 * (H // D) * hd, h), 10 + d, 0.02).to(DEV) for d in range(D)]
    k0, v0 = _rnd((S, h), 6).to(DEV), _rnd((S, h), 7).to(DEV)
    say("gqa = mha: projection")
    qa, ka, va = bf16_nan((n, h), DEV), k0.clone(), v0.clone()
    tsp.attn_project(plan, dims, x, w, ka, va, qa)
    qb, kb, vb = bf16_nan((n, h), DEV), k0.clone(), v0.clone()
    tsp.attn_project_gqa(plan, dims, H, x, w, kb, vb, qb)
    torch.cuda.synchronize()
    assert torch.equal(qa, qb) and torch.equal(ka, kb) and torch.equal(va, vb)
    say("gqa = mha: attention")
    oa, ob = bf16_nan((n, h), DEV), bf16_nan((n, h), DEV)
    tsp.attn_core(plan, dims, qa, ka, va, oa)
    tsp.attn_core_gqa(plan, dims, H, qa, ka, va, ob)
    torch.cuda.synchronize()
    assert torch.equal(oa, ob)


def test_gqa_project_wide_tiles():
    """The GQA projection at a size that takes the 256 x 192 tiles: shards of
    (4 + 2*1) heads of 64 = 384 columns, 6000 local tokens (a ragged last tile
    row), against the oracle's projection (bf16 tensors)."""
    require_gpu()
    S, D, r, H, Hkv, hd = 24000, 4, 1, 16, 4, 64
    h = H * hd
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    Hs, Ks = H // D, Hkv // D
    dims = tsp.make_dims(h, H, hd, 4 * h)
    x = _rnd((n, h), 12)
    w = [_rnd(((Hs + 2 * Ks) * hd, h), 40 + d, 0.02) for d in range(D)]
    k0, v0 = _rnd((S, Hkv * hd), 13), _rnd((S, Hkv * hd), 14)
    q_ref, k_ref, v_ref = (O.proj_rows(t) for t in O.qkv_projection_gqa(x, w, hd, Hs, Ks))
    kd, vd = _bf16(k0).to(DEV), _bf16(v0).to(DEV)
    q = bf16_nan((n, h), DEV)
    say(f"gqa projection, wide tiles: S={S} D={D} H={H} Hkv={Hkv} hd={hd} n={n}")
    tsp.attn_project_gqa(plan, dims, Hkv, x.to(DEV), [t.to(DEV) for t in w], kd, vd, q)
    torch.cuda.synchronize()
    check(q, q_ref, "gqa q")
    check(kd[l2g.to(DEV)], k_ref, "gqa own k rows")
    check(vd[l2g.to(DEV)], v_ref, "gqa own v rows")
    others = torch.ones(S, dtype=torch.bool)
    others[l2g] = False
    assert torch.equal(kd.cpu()[others], _bf16(k0)[others]), "rows of other ranks must be untouched"
    assert torch.equal(vd.cpu()[others], _bf16(v0)[others])


@pytest.mark.parametrize("S,D,r,H,Hkv,hd", [(2048, 4, 1, 8, 4, 64), (2048, 2, 0, 8, 2, 64),
                                             (1288, 2, 1, 4, 2, 128), (640, 1, 0, 4, 1, 64)])
def test_gqa_project_rope_attention(S, D, r, H, Hkv, hd):
    require_gpu()
    h = H * hd
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n = plan.n_local
    Hs, Ks = H // D, Hkv // D
    dims = tsp.make_dims(h, H, hd, 4 * h)
    x = _rnd((n, h), 8)
    w = [_rnd(((Hs + 2 * Ks) * hd, h), 20 + d, 0.02) for d in range(D)]
    k_other, v_other = _rnd((S, Hkv * hd), 9), _rnd((S, Hkv * hd), 11)
    theta = 10000.0
    # oracle: projection (bf16 tensors), RoPE (bf16 tensors), own rows into the gathered K/V, attention
    q_ref, k_ref, v_ref = (O.proj_rows(t) for t in O.qkv_projection_gqa(x, w, hd, Hs, Ks))
    k_all, v_all = O.f64(k_other).clone(), O.f64(v_other).clone()
    k_all[l2g], v_all[l2g] = k_ref, v_ref
    q_rot = O.proj_rows(O.rope(_bf16(q_ref), l2g, H, hd, theta))
    k_rot = k_all.clone()
    k_rot[l2g] = O.proj_rows(O.rope(_bf16(k_ref), l2g, Hkv, hd, theta))
    ref = O.causal_attention_gqa(q_rot, l2g, k_rot, v_all, H, Hkv, hd)

    kd, vd = _bf16(k_other).to(DEV), _bf16(v_other).to(DEV)
    q = bf16_nan((n, h), DEV)
    say(f"gqa projection S={S} D={D} H={H} Hkv={Hkv} hd={hd}")
    tsp.attn_project_gqa(plan, dims, Hkv, x.to(DEV), [t.to(DEV) for t in w], kd, vd, q)
    torch.cuda.synchronize()
    check(q, q_ref, "gqa q")
    check(kd.cpu()[l2g], k_ref, "gqa own k rows")
    check(vd.cpu()[l2g], v_ref, "gqa own v rows")
    say("gqa rope + attention")
    tsp.rope(plan, H, Hkv, hd, theta, q, kd)
    o = bf16_nan((n, h), DEV)
    tsp.attn_core_gqa(plan, dims, Hkv, q, kd, vd, o)
    torch.cuda.synchronize()
    check(o, ref, "gqa attention")
