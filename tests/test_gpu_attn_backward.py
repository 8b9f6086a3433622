"""GPU parity of the attention backward (tsp_attn_core_lse, tsp_attn_core_backward)
against the fp64 oracle.

  * the softmax normaliser from tsp_attn_core_lse against oracle.attention_lse,
    and its output bit-identical to tsp_attn_core's;
  * dq, and this rank's dk/dv contributions for every key row, against
    oracle.causal_attention_backward: head_dim 64 and 128, both zigzag
    chunks, ragged chunks (not a multiple of 64 queries), D = 1, with and
    without the forward's low output part;
  * keys past every local query get exact zeros.

Tolerances.  The kernels feed P and dS to the MFMAs as bf16: one rounding of
one operand of a dot product bounds its error by 2^-9 sum |a||b|, with the
fp64 factors (P and |dS| <= P (|dP| + |delta|)).  delta = rowsum(dO * o) is
taken from the forward's output, which carries the forward's rounding of P
(2^-9 P|v| per element) and, without its low part, the bf16 rounding of o
(at most as much again): e_t = 2^-9 (1 or 2) sum_d |dO| (P|v|), which reaches
dq through P|k| e and dk through P^T (e |q|).  Each element is checked against
twice the sum of these (margin 2), plus 1e-5 of the output's largest magnitude
for the fp32 accumulation.  An element passes within the larger of that and
the forward's bound 1e-2 + 2e-2 |o| (the elements that only the derived bound
admits are tallied); the whole must meet relative RMS <= 5e-3.
"""
import math

import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check_within, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"
F64 = torch.float64


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_800_000 + seed, std, "cpu")


def _bounds(q, k, v, do, pos, H, hd, with_lo):
    """Per-element rounding bounds of dq, dk, dv (fp64, [rows, H*hd]), in units
    of 2^-9 (one bf16 rounding)."""
    S, m = k.shape[0], q.shape[0]
    bq, bk, bv = (torch.zeros(m, H * hd, dtype=F64), torch.zeros(S, H * hd, dtype=F64),
                  torch.zeros(S, H * hd, dtype=F64))
    for a in range(H):
        cols = slice(a * hd, (a + 1) * hd)
        p = O.softmax_rows(q, pos, k, a, hd)
        dp = do[:, cols] @ v[:, cols].t()
        delta = (p * dp).sum(1, keepdim=True)
        ds_abs = p * (dp.abs() + delta.abs())
        e = (1.0 if with_lo else 2.0) * (do[:, cols].abs() * (p @ v[:, cols].abs())).sum(1, keepdim=True)
        bv[:, cols] = p.t() @ do[:, cols].abs()
        bk[:, cols] = (ds_abs.t() @ q[:, cols].abs() + p.t() @ (e * q[:, cols].abs())) / math.sqrt(hd)
        bq[:, cols] = (ds_abs @ k[:, cols].abs() + (p @ k[:, cols].abs()) * e) / math.sqrt(hd)
    return bq, bk, bv


def _check(got, ref, bound, name):
    """Per element |err| <= max(1e-2 + 2e-2 |ref|, 2^-8 bound + 1e-5 max|ref|),
    relative RMS <= 5e-3; elements only the derived bound admits are tallied."""
    lim = 2.0 ** -8 * bound + 1e-5 * ref.abs().max().item() + 1e-12
    st = check_within(got, ref, lim, name)
    say(f"{name}: max err {st['max_abs']:.3e}, rel rms {st['rel_rms']:.2e}, "
        f"{st['derived_only']}/{st['n']} admitted by the derived bound only")


def _run(S, D, r, H, hd, with_lo, seed, qk_scale=1.0):
    plan, l2g, _ = tsp.zigzag_plan(S, D, r)
    n, h = plan.n_local, H * hd
    dims = tsp.make_dims(h, H, hd, 4 * h)
    q, k, v = _rnd((n, h), seed, qk_scale), _rnd((S, h), seed + 1, qk_scale), _rnd((S, h), seed + 2)
    do = _rnd((n, h), seed + 3)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    out = bf16_nan((n, h), DEV)
    lo = bf16_nan((n, h), DEV) if with_lo else None
    lse = torch.full((H, n), float("nan"), dtype=torch.float32, device=DEV)
    say(f"attn backward S={S} D={D} r={r} H={H} hd={hd} lo={with_lo}: forward with lse")
    tsp.attn_core_lse(plan, dims, qd, kd, vd, out, lse, attn_lo=lo)
    dq = torch.full((n, h), float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full((S, h), float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full((S, h), float("nan"), dtype=torch.float32, device=DEV)
    say("backward")
    tsp.attn_core_backward(plan, dims, qd, kd, vd, out, lse, dod, dq, dk, dv, attn_lo=lo)
    torch.cuda.synchronize()
    return plan, l2g, (q, k, v, do), (out, lse, dq, dk, dv)


@pytest.mark.parametrize("S,D,r,H,hd", [(2048, 4, 1, 4, 64), (1288, 2, 1, 2, 128), (640, 1, 0, 2, 64)])
def test_lse_and_same_output(S, D, r, H, hd):
    require_gpu()
    plan, l2g, (q, k, v, _), (out, lse, _, _, _) = _run(S, D, r, H, hd, False, 10)
    ref = O.attention_lse(O.f64(q), l2g, O.f64(k), H, hd)
    err = (lse.cpu().to(F64) - ref).abs()
    assert float(err.max()) <= 1e-4 + 1e-5 * float(ref.abs().max()), f"lse max err {float(err.max()):.3e}"
    h = H * hd
    dims = tsp.make_dims(h, H, hd, 4 * h)
    out2 = bf16_nan((plan.n_local, h), DEV)
    tsp.attn_core(plan, dims, q.to(DEV), k.to(DEV), v.to(DEV), out2)
    torch.cuda.synchronize()
    assert torch.equal(out, out2)


@pytest.mark.parametrize("S,D,r,H,hd", [(2048, 4, 1, 4, 64), (2048, 2, 0, 2, 128), (1288, 2, 1, 2, 128),
                                         (640, 1, 0, 2, 64), (4096, 4, 3, 2, 128)])
@pytest.mark.parametrize("with_lo", [False, True])
def test_attn_backward(S, D, r, H, hd, with_lo):
    require_gpu()
    plan, l2g, (q, k, v, do), (_, _, dq, dk, dv) = _run(S, D, r, H, hd, with_lo, 20)
    qf, kf, vf, dof = (O.f64(t) for t in (q, k, v, do))
    rq, rk, rv = O.causal_attention_backward(qf, l2g, kf, vf, dof, H, hd)
    bq, bk, bv = _bounds(qf, kf, vf, dof, l2g, H, hd, with_lo)
    _check(dq, rq, bq, "dq")
    _check(dk, rk, bk, "dk")
    _check(dv, rv, bv, "dv")
    last = int(l2g.max()) + 1
    if last < S:
        assert torch.count_nonzero(dk[last:]).item() == 0 and torch.count_nonzero(dv[last:]).item() == 0


@pytest.mark.parametrize("k", [2, 4])
@pytest.mark.parametrize("S,D,r,H,hd", [(2048, 4, 1, 4, 64), (2048, 2, 0, 2, 128)])
def test_attn_backward_scaled(S, D, r, H, hd, k):
    """q and K at 2.5^k times unit scale, as a chained stack without a norm
    gives them at layer k: scores 2.5^(2k) times the unit ones (39x at k = 2,
    1526x at k = 4), softmax rows near one-hot.  P is recomputed against the
    forward's fp32 normaliser (natural log), which carries about 2^-24 of the
    row's largest score as an error in the exponent: below a bf16 rounding of
    P up to k = 4; at k = 6 (scores near 10^5) it reaches about 1 % of P."""
    require_gpu()
    s = 2.5 ** k
    plan, l2g, (q, kk, v, do), (_, _, dq, dk, dv) = _run(S, D, r, H, hd, True, 40, qk_scale=s)
    qf, kf, vf, dof = (O.f64(t) for t in (q, kk, v, do))
    rq, rk, rv = O.causal_attention_backward(qf, l2g, kf, vf, dof, H, hd)
    bq, bk, bv = _bounds(qf, kf, vf, dof, l2g, H, hd, True)
    _check(dq, rq, bq, f"dq (q, K x 2.5^{k})")
    _check(dk, rk, bk, f"dk (q, K x 2.5^{k})")
    _check(dv, rv, bv, f"dv (q, K x 2.5^{k})")


def test_attn_backward_7b_sampled():
    """The 7B shape the benchmark times (S = 131072, D = 8, 32 heads x 128, rank 3),
    generated q, K/V and dO: dq on sampled rows (each row depends only on its
    own query); dk/dv of the rank's last 8 keys, which only its last 8 queries
    see (so the oracle on those rows gives them whole); and at every key, the
    column sums fixed by the softmax: sum_j dv[j] = sum_t dO[t] within the bf16
    rounding of P (each probability row then sums to 1 within 2^-9), and
    sum_j dk[j] = 0 within the rounding of dS (sum_j |dS_tj| <= 2 |dO_t| max_j |v_j|
    by Cauchy-Schwarz) and of delta."""
    require_gpu()
    W = synth.WORKLOADS["attn_7b"]
    d, D, S = W.dims, W.D, W.seq_len
    plan, l2g, _ = tsp.zigzag_plan(S, D, W.rank)
    n, h, H, hd = plan.n_local, d.hidden, d.n_heads, d.head_dim
    dims = tsp.make_dims(h, H, hd, d.ffn)
    say(f"{W.name}: inputs")
    q = synth.activations(W.wid, n, h, device=DEV)
    kd, vd = synth.gathered_kv(W.wid, S, h, device=DEV)
    do = synth.randn_bf16((n, h), 9_800_777, 1.0, DEV)
    out, lo = bf16_nan((n, h), DEV), bf16_nan((n, h), DEV)
    lse = torch.full((H, n), float("nan"), dtype=torch.float32, device=DEV)
    say(f"{W.name}: forward with lse")
    tsp.attn_core_lse(plan, dims, q, kd, vd, out, lse, attn_lo=lo)
    dq = torch.full((n, h), float("nan"), dtype=torch.float32, device=DEV)
    dk = torch.full((S, h), float("nan"), dtype=torch.float32, device=DEV)
    dv = torch.full((S, h), float("nan"), dtype=torch.float32, device=DEV)
    say(f"{W.name}: backward")
    tsp.attn_core_backward(plan, dims, q, kd, vd, out, lse, do, dq, dk, dv, attn_lo=lo)
    torch.cuda.synchronize()

    say(f"{W.name}: column sums")
    last = int(l2g.max()) + 1
    assert torch.count_nonzero(dk[last:]).item() == 0 and torch.count_nonzero(dv[last:]).item() == 0
    dk64, dv64 = dk[:last].to(F64), dv[:last].to(F64)
    do64, q64 = do.to(F64), q.to(F64)
    sum_dv, sum_do = dv64.sum(0), do64.sum(0)
    lim_v = 2 * (2.0 ** -9 * do64.abs().sum(0)) + 1e-6 * dv64.abs().sum(0)
    assert bool(((sum_dv - sum_do).abs() <= lim_v).all()), "sum_j dv[j] != sum_t dO[t]"
    vmax = vd.to(F64).reshape(S, H, hd)
    vnorm_max = vmax.norm(dim=2).max(dim=0).values           # [H]: max_j |v_j| per head
    vabs_max = vmax.abs().max(dim=0).values                   # [H, hd]: max_j |v_jd|
    do_h = do64.reshape(n, H, hd)
    per_t = 2.0 ** -9 * 2 * do_h.norm(dim=2) * vnorm_max + 2.0 ** -8 * (do_h.abs() * vabs_max).sum(2)  # [n, H]
    lim_k = 2 * (q64.reshape(n, H, hd).abs() * per_t[:, :, None]).sum(0).reshape(h) / math.sqrt(hd)
    lim_k += 1e-6 * dk64.abs().sum(0)
    assert bool((dk64.sum(0).abs() <= lim_k).all()), "sum_j dk[j] != 0"
    del dk64, dv64

    say(f"{W.name}: oracle on sampled rows")
    g = torch.Generator().manual_seed(5)
    C = plan.chunk_len
    rows = torch.unique(torch.cat([torch.tensor([0, 1, C - 1, C, C + 1, n - 1]), torch.randint(0, n, (14,), generator=g)]))
    kc, vc = O.f64(kd), O.f64(vd)
    qc, dc = O.f64(q), O.f64(do)
    rq, _, _ = O.causal_attention_backward(qc[rows], l2g[rows], kc, vc, dc[rows], H, hd)
    bq, _, _ = _bounds(qc[rows], kc, vc, dc[rows], l2g[rows], H, hd, True)
    _check(dq[rows.to(DEV)], rq, bq, "7B dq sampled rows")
    tail = torch.arange(n - 8, n)
    _, rk, rv = O.causal_attention_backward(qc[tail], l2g[tail], kc, vc, dc[tail], H, hd)
    _, bk, bv = _bounds(qc[tail], kc, vc, dc[tail], l2g[tail], H, hd, True)
    keys = torch.arange(last - 8, last)
    _check(dk[keys.to(DEV)], rk[keys], bk[keys], "7B dk of the last 8 keys")
    _check(dv[keys.to(DEV)], rv[keys], bv[keys], "7B dv of the last 8 keys")
