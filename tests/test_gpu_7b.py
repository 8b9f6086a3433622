"""GPU parity at the 7B rank-share shapes (h=4096, 32 heads x 128, FFN 16384,
D=8), in the launch configuration the benchmark times, against the fp64
oracle on sampled rows (the oracle computes those rows one by one; every row
of a GEMM or of attention is independent given its inputs).

  * MLP ring, 16384 local tokens, ring from shard 3, no residual;
  * attention + O projection, S=131072 in 16 zigzag chunks of 8192, rank 3,
    generated gathered K/V (the rank's own rows replaced by its projections);
  * whole layer at S=16384 (2048 local tokens, rank 0), generated K/V.

Sampled rows always include the first and last row of each zigzag chunk.

The gating oracle holds the projection outputs Q, K and V as the bf16 tensors
the model stores; the attention and layer tests also compare, by relative RMS,
with the oracle that keeps them unrounded (fp64), which charges the GPU path
with the bf16 rounding of Q, K and V as well."""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from oracle import tsp_oracle as O
from parity import bf16_nan, check, check_rms, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"


def _rows(n, C, k, seed):
    g = torch.Generator().manual_seed(seed)
    fixed = torch.tensor([0, 1, C - 1, C, C + 1, n - 1])
    extra = torch.randint(0, n, (k,), generator=g)
    return torch.unique(torch.cat([fixed, extra]))


def _dims(d):
    return tsp.make_dims(d.hidden, d.n_heads, d.head_dim, d.ffn)


def test_mlp_7b_sampled_rows():
    require_gpu()
    W = synth.WORKLOADS["mlp_7b"]
    d, D, n = W.dims, W.D, W.n_local
    say(f"{W.name}: inputs")
    x = synth.activations(W.wid, n, d.hidden, device=DEV)
    lw = synth.layer_weights(W.wid, d, D, device=DEV, parts=("w1", "w2"))
    dims = _dims(d)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP)
    y = bf16_nan((n, d.hidden), DEV)
    say(f"{W.name}: mlp_forward start {W.start_shard}")
    tsp.mlp_forward(dims, D, W.start_shard, x, lw.w1, lw.w2, None, y, ws)
    torch.cuda.synchronize()
    rows = _rows(n, n // 2, 40, 1)
    ref = O.mlp_forward(x.cpu(), [t.cpu() for t in lw.w1], [t.cpu() for t in lw.w2], residual=False, rows=rows)
    check(y.cpu()[rows], ref, "7B MLP sampled rows")


def test_attention_7b_sampled_rows():
    require_gpu()
    W = synth.WORKLOADS["attn_7b"]
    d, D, S = W.dims, W.D, W.seq_len
    plan, l2g, _ = tsp.zigzag_plan(S, D, W.rank)
    n, h = plan.n_local, d.hidden
    say(f"{W.name}: inputs")
    x = synth.activations(W.wid, n, h, device=DEV)
    lw = synth.layer_weights(W.wid, d, D, device=DEV, parts=("wqkv", "wo"))
    kf, vf = synth.gathered_kv(W.wid, S, h, device=DEV)
    kf_cpu, vf_cpu = kf.cpu(), vf.cpu()
    dims = _dims(d)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_ATTN)
    out = bf16_nan((n, h), DEV)
    say(f"{W.name}: attn_forward")
    tsp.attn_forward(plan, dims, x, lw.wqkv, lw.wo, kf, vf, None, out, ws)
    torch.cuda.synchronize()
    rows = _rows(n, plan.chunk_len, 26, 2)
    oplan = O.zigzag_plan(S, D, W.rank)
    ref, _, k_own, v_own = O.attn_forward(oplan, x.cpu(), [t.cpu() for t in lw.wqkv], [t.cpu() for t in lw.wo],
                                          d.n_heads, d.head_dim, kf_cpu, vf_cpu, residual=False, rows=rows)
    check(out.cpu()[rows], ref, "7B attention + O projection sampled rows")
    say(f"{W.name}: oracle with unrounded projections")
    ref_x, _, _, _ = O.attn_forward(oplan, x.cpu(), [t.cpu() for t in lw.wqkv], [t.cpu() for t in lw.wo], d.n_heads,
                                    d.head_dim, kf_cpu, vf_cpu, residual=False, rows=rows, k_own=k_own, v_own=v_own,
                                    proj_bf16=False)
    check_rms(out.cpu()[rows], ref_x, "7B attention + O projection sampled rows, unrounded Q/K/V")
    pos = l2g[rows]
    check(kf.cpu()[pos], k_own[rows], "7B own K rows")
    check(vf.cpu()[pos], v_own[rows], "7B own V rows")


def test_layer_16k_sampled_rows():
    require_gpu()
    W = synth.WORKLOADS["stream_7b_16k"]
    d, D, S = W.dims, W.D, W.seq_len
    plan, _, _ = tsp.zigzag_plan(S, D, W.rank)
    n, h = plan.n_local, d.hidden
    say(f"{W.name}: inputs")
    x = synth.activations(W.wid, n, h, device=DEV)
    lw = synth.layer_weights(W.wid, d, D, device=DEV)
    kf, vf = synth.gathered_kv(W.wid, S, h, device=DEV)
    kf_cpu, vf_cpu = kf.cpu(), vf.cpu()
    dims = _dims(d)
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_LAYER)
    out = bf16_nan((n, h), DEV)
    say(f"{W.name}: layer_forward")
    tsp.layer_forward(plan, dims, x, lw.wqkv, lw.wo, lw.w1, lw.w2, kf, vf, out, ws)
    torch.cuda.synchronize()
    rows = _rows(n, plan.chunk_len, 26, 3)
    lc = lw.to("cpu")
    ref, _, _ = O.layer_forward(O.zigzag_plan(S, D, W.rank), x.cpu(), lc.wqkv, lc.wo, lc.w1, lc.w2, d.n_heads,
                                d.head_dim, kf_cpu, vf_cpu, rows=rows)
    check(out.cpu()[rows], ref, "16K layer sampled rows")
    say(f"{W.name}: oracle with unrounded projections")
    ref_x, _, _ = O.layer_forward(O.zigzag_plan(S, D, W.rank), x.cpu(), lc.wqkv, lc.wo, lc.w1, lc.w2, d.n_heads,
                                  d.head_dim, kf_cpu, vf_cpu, rows=rows, proj_bf16=False)
    check_rms(out.cpu()[rows], ref_x, "16K layer sampled rows, unrounded Q/K/V")
