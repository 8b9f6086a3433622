#!/usr/bin/env python3
"""Benchmark of the TSP rank-share layer on one MI355X.

Default workload: the full rank-share forward of the 7B dense decoder at 128K
(32 layers, h=4096, 32 heads x 128, FFN 16384, bf16, D=8, S=131072, rank 0,
16384 local tokens).  One step = the whole hot path over one batch: for each of
the 32 layers, the shard-iterated QKV projection with the K/V scatter, causal
attention of the two zigzag chunks against that layer's gathered K/V, the O
projection split-K with the residual, and the ring MLP with the residual; the
output of layer l is the input of layer l+1.  All inputs (weights, generated
per-layer K/V, x) are resident in HBM before timing starts.  ``value`` is
local tokens/s per layer over the timed steps.

The step calls the three entry points that tsp_layer_forward composes
(tsp_attn_project, tsp_attn_core, tsp_layer_post), with HIP events recorded
between them on the launch stream.

Roofline.  The dominant kernel is the attention core (about 73% of the
layer's FLOPs).  Its roofline figure is taken on unit-scale inputs: after the
warmup steps and before the timed ones, the core is launched on layer 0's
inputs (x ~ N(0,1), the layer's generated K/V) twice untimed and then
``--roofline-launches`` times, each bracketed by HIP events on the launch
stream.  The layer has no norm, so in the chained steps the activations grow
about 2.5x per layer and the softmax rows of later layers are close to
one-hot, which makes the same kernel faster; that chained per-launch figure is
reported beside it (``roofline.chained``).  A ``--kernel-trace`` profile of
this command averages exactly the timed unit-scale launches by their place in
the dispatch order (profile_summary ``--first``/``--skip``).

``stream_7b_16k``: the weight-streaming regime, timed in the same run (S =
16384, 2048 local tokens, 32 distinct layers whose 402.65 MB of weights each
are read from HBM): layer time, local tokens/s, fraction of the bf16 MFMA peak,
and HBM bytes per second (algorithmic, and counted from the counter summary
of ``bench.py --workload stream_7b_16k``).  ``--workload stream_7b_16k`` makes
that regime the main workload instead.

After the timed steps, each step's entry point is also timed alone on layer
0's inputs (``rows_layer0``: QKV projection, attention, O projection, MLP),
each against the bf16 MFMA peak, and so are the shard-streaming forms of the
projections and the MLP (the D ring steps called one by one, weights
resident), the backward of every step (MLP ring, attention core, O and QKV
projections), and the layer variants (RMSNorm and RoPE
against the HBM peak, grouped-query attention with 8 K/V heads); ``--no-rows``
skips them.

``cpu_baseline``: the fp64 oracle timed on the host cores the process may run
on, on a bounded sample of layer 0 (the K/V projection of all local rows, the
attention half for 64 query rows stratified over both zigzag chunks, the MLP
for 256 rows), extrapolated to local tokens/s per layer.

Prints ONE JSON line.  ``--gpus`` above 1 is refused: this build runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import torch

from folded_tensor_sequence_tsp_amd import profile_summary, synth, tsp

ROOT = os.path.dirname(os.path.abspath(__file__))
# rocprofv3 counter summaries, per workload: (file, unit).  On the 128K
# workload the dominant unit is the attention core; on the 16K weight-streaming
# workload the whole layer is reported (its HBM traffic against the weights it
# streams).  A figure is used only while the kernels' sources are the ones
# profiled.
TRAFFIC_SUMMARY = {
    "full_7b_128k": (os.path.join(ROOT, "profiles", "tsp_attn_core_7b_128k_rank0_unit_scale.md"), "tsp_attn_core"),
    "stream_7b_16k": (os.path.join(ROOT, "profiles", "tsp_layer_forward_7b_16k_rank0_32layers.md"),
                      "tsp_layer_forward"),
}

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
METRIC = "local tokens/sec per 7B TSP layer (D=8, 128K seq) + % bf16 MFMA peak"
DTYPE = "bf16 (MLP GEMMs on fp16 operands scaled per row by a power of two)"


def layer_flops(n, S, D, C, d):
    """Algorithmic FLOPs of one rank-share layer, by step."""
    h, F, H, hd = d.hidden, d.ffn, d.n_heads, d.head_dim
    pairs = 2 * D * C * C + C  # (query, key) pairs with key <= query, per head
    return {
        "qkv": 2.0 * n * h * 3 * h,
        "attn": 4.0 * hd * H * pairs,
        "oproj": 2.0 * n * h * h,  # O projection
        "mlp": 4.0 * n * h * F,
    }


def layer_bytes(plan, d):
    """Algorithmic HBM bytes of one rank-share layer: its weights (all D
    shards, bf16), the gathered K and V rows up to the rank's last query
    position, the input rows and the output rows."""
    h, F = d.hidden, d.ffn
    kv_rows = plan.chunk_start[1] + plan.chunk_len
    return (4 * h * h + 2 * h * F) * 2 + 2 * kv_rows * h * 2 + 2 * plan.n_local * h * 2


def arrival_overlap(plan, dims, D, layer0, x0, q, a, a_lo, out, dev, reps=3):
    """Layer 0's QKV and O projections with their D weight shards delivered
    while they run, by the one-workgroup simulated producer
    (tsp_simulate_arrival) into separate buffers, one shard every `interval`
    (about the producer's own copy time per shard, 47 GB/s).

    A call's waiting workgroups would hold every CU, so the producer is
    launched first on a side stream and given a 1 ms host pause to become
    resident before the call is launched.  So that the shards still arrive
    during the call, the producer first delivers k 16-byte dummies (k = the
    interval's multiples in 1 ms), which raise the counter too: the call's
    arrival base is k.  The waits are bounded and the status word is
    reported.  Times (ms, events on the call's stream around it): the call
    with every shard arrived; delivery then call on one stream; the call with
    its shards arriving (from the call's launch)."""
    lw, kf, vf = layer0
    ring = [(plan.rank + k) % D for k in range(D)]
    counter = torch.zeros(4, dtype=torch.int32, device=dev)
    status = torch.zeros(4, dtype=torch.int32, device=dev)
    dummy_src = torch.zeros(16, dtype=torch.uint8, device=dev)
    dummy_dst = torch.zeros(64, 16, dtype=torch.uint8, device=dev)  # one 16-byte row per dummy
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ev = lambda: torch.cuda.Event(enable_timing=True)

    def measure(shards, run_call):
        src = [shards[d] for d in ring]
        dst = [torch.empty_like(t) for t in src]
        w_arr = [None] * D
        for p, d in enumerate(ring):
            w_arr[d] = dst[p]
        call = lambda base: run_call(w_arr, tsp.make_arrival(counter, base, status, spin_limit=1 << 15))
        for d_, s_ in zip(dst, src):
            d_.copy_(s_)
        counter.fill_(D)
        call(0)
        torch.cuda.synchronize()
        e0, e1 = ev(), ev()
        e0.record(main)
        for _ in range(reps):
            call(0)
        e1.record(main)
        torch.cuda.synchronize()
        call_ms = e0.elapsed_time(e1) / reps
        shard_mb = src[0].numel() * src[0].element_size() / 1e6
        interval_us = int(shard_mb / 47e3 * 1e6) + 1  # MB / (47 GB/s) in microseconds
        k = min(64 - D, -(-1000 // interval_us))
        res = {"call_all_arrived_ms": round(call_ms, 4), "shard_interval_us": interval_us,
               "shards": f"{D} shards of {shard_mb:.1f} MB"}
        for kind in ("deliver_then_call", "arriving_during_call"):
            times = []
            for _ in range(reps):
                counter.zero_()
                torch.cuda.synchronize()
                e0, e1 = ev(), ev()
                if kind == "deliver_then_call":
                    e0.record(main)
                    tsp.simulate_arrival(src, dst, counter, 0, interval_us, stream=main)
                    call(0)
                else:
                    side.wait_stream(main)
                    tsp.simulate_arrival([dummy_src] * k + src, [dummy_dst[i] for i in range(k)] + dst, counter,
                                         0, interval_us, stream=side)
                    time.sleep(0.001)
                    e0.record(main)
                    call(k)
                    main.wait_stream(side)
                e1.record(main)
                torch.cuda.synchronize()
                times.append(e0.elapsed_time(e1))
            res[kind + "_ms"] = round(sum(times) / reps, 4)
        return res

    res = {
        "qkv (N-sharded)": measure(lw.wqkv, lambda w, arr: tsp.attn_project_arrival(
            plan, dims, plan.rank, x0, w, kf, vf, q, arr)),
        "oproj (K-sharded)": measure(lw.wo, lambda w, arr: tsp.attn_out_arrival(
            dims, D, plan.rank, a, w, x0, out, arr, attn_lo=a_lo)),
    }
    res["status"] = int(status[0])
    return res


def row_timings(plan, dims, D, layer0, x0, q, a, a_lo, out, ws_core, fl, dev, reps=3):
    """Each hot-path step's entry point alone, on layer 0's inputs, after the
    timed steps: ms per call, FLOP/s and the fraction of the bf16 MFMA peak.
    The O projection's FLOPs are the algorithmic ones (it contracts the
    attention output's hi and lo parts, twice that many are executed)."""
    lw, kf, vf = layer0
    n = plan.n_local
    ws_mlp = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP, device=dev)
    ws_mlp_s = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_SHARD, device=dev)
    ws_out_s = tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_SHARD, device=dev)
    ring = [(plan.rank + k) % D for k in range(D)]

    def project_streamed():
        for s in ring:
            tsp.attn_project_shard(plan, dims, s, x0, lw.wqkv[s], kf, vf, q)

    def out_streamed():
        for pos, s in enumerate(ring):
            tsp.attn_out_shard(dims, D, pos, s, a, lw.wo[s], x0, out, ws_out_s, attn_lo=a_lo)

    def mlp_streamed():
        for pos, s in enumerate(ring):
            tsp.mlp_shard(dims, D, pos, x0, lw.w1[s], lw.w2[s], x0, out, ws_mlp_s)

    calls = [
        ("A2 qkv projection (tsp_attn_project)", "qkv",
         lambda: tsp.attn_project(plan, dims, x0, lw.wqkv, kf, vf, q)),
        ("A4 causal attention (tsp_attn_core)", "attn",
         lambda: tsp.attn_core(plan, dims, q, kf, vf, a, a_lo, workspace=ws_core)),
        ("A5 O projection, split-K + residual (tsp_attn_out)", "oproj",
         lambda: tsp.attn_out(dims, D, plan.rank, a, lw.wo, x0, out, attn_lo=a_lo)),
        ("A6+A7 MLP: W1+GELU, W2 ring split-K + residual (tsp_mlp_forward)", "mlp",
         lambda: tsp.mlp_forward(dims, D, plan.rank, x0, lw.w1, lw.w2, x0, out, ws_mlp)),
        ("A2 streamed: D x tsp_attn_project_shard", "qkv", project_streamed),
        ("A5 streamed: D x tsp_attn_out_shard", "oproj", out_streamed),
        ("A6+A7 streamed: D x tsp_mlp_shard", "mlp", mlp_streamed),
    ]
    # the other two 7B configurations at their own parameters: the MLP ring
    # from shard 3 (config 2) and the attention half at rank 3, whose chunks
    # are 3 and 12 (config 3: QKV projection, attention, O projection)
    plan3, _, _ = tsp.zigzag_plan(plan.seq_len, D, 3)
    ws_attn3 = tsp.alloc_workspace(n, dims, D, tsp.WS_ATTN, device=dev)
    fl = dict(fl, cfg3=fl["qkv"] + fl["attn"] + fl["oproj"])
    calls += [
        ("config 2: MLP ring from shard 3, 16384 tokens (tsp_mlp_forward)", "mlp",
         lambda: tsp.mlp_forward(dims, D, 3, x0, lw.w1, lw.w2, x0, out, ws_mlp)),
        ("config 3: attention half at rank 3 (tsp_attn_forward: QKV, attention, O)", "cfg3",
         lambda: tsp.attn_forward(plan3, dims, x0, lw.wqkv, lw.wo, kf, vf, x0, out, ws_attn3)),
    ]
    # the all-shard calls that wait for each shard inside the kernels, with
    # every shard already arrived (the counter preset): the cost of streaming
    # when the next shards are prefetched while the current ones compute
    counter = torch.full((4,), D, dtype=torch.int32, device=dev)
    status = torch.zeros(4, dtype=torch.int32, device=dev)
    arr = tsp.make_arrival(counter, 0, status)
    calls += [
        ("A2 shards awaited in the kernel, all arrived (tsp_attn_project_arrival)", "qkv",
         lambda: tsp.attn_project_arrival(plan, dims, plan.rank, x0, lw.wqkv, kf, vf, q, arr)),
        ("A5 shards awaited in the kernel, all arrived (tsp_attn_out_arrival)", "oproj",
         lambda: tsp.attn_out_arrival(dims, D, plan.rank, a, lw.wo, x0, out, arr, attn_lo=a_lo)),
        ("A6+A7 shards awaited in the kernel, all arrived (tsp_mlp_forward_arrival)", "mlp",
         lambda: tsp.mlp_forward_arrival(dims, D, plan.rank, x0, lw.w1, lw.w2, x0, out, ws_mlp, arr)),
    ]
    # backward of the MLP ring on layer 0's shapes: recomputes U = x W1^T, then
    # dU, dW2, dW1 and dx (five n x h x F products, 10 n h F FLOPs)
    dy = (torch.randn(n, dims.hidden, device=dev) * 0.02).to(torch.bfloat16)
    dx = torch.empty_like(dy)
    Fs = dims.ffn // D
    dw1 = [torch.empty(Fs, dims.hidden, dtype=torch.float32, device=dev) for _ in range(D)]
    dw2 = [torch.empty(dims.hidden, Fs, dtype=torch.float32, device=dev) for _ in range(D)]
    ws_bwd = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP_BWD, device=dev)
    fl = dict(fl, mlp_bwd=10.0 * n * dims.hidden * dims.ffn)
    calls.append(("MLP backward: dx ring + dW1, dW2 per shard (tsp_mlp_backward)", "mlp_bwd",
                  lambda: tsp.mlp_backward(dims, D, plan.rank, True, x0, lw.w1, lw.w2, dy, dx, dw1, dw2, ws_bwd)))
    # backward of the causal attention on layer 0's shapes (forward with the
    # normaliser first, outside the timing): 5 products of the forward's size,
    # 2.5x its FLOPs (the dQ kernel recomputes S and dP: 7 are executed)
    lse = torch.empty(dims.n_heads, n, dtype=torch.float32, device=dev)
    tsp.attn_core_lse(plan, dims, q, kf, vf, a, lse, attn_lo=a_lo, workspace=ws_core)
    d_attn = (torch.randn(n, dims.hidden, device=dev) * 0.02).to(torch.bfloat16)
    dq_b = torch.empty(n, dims.hidden, dtype=torch.float32, device=dev)
    dk_b = torch.empty(plan.seq_len, dims.hidden, dtype=torch.float32, device=dev)
    dv_b = torch.empty(plan.seq_len, dims.hidden, dtype=torch.float32, device=dev)
    ws_abwd = tsp.alloc_workspace(n, dims, D, tsp.WS_ATTN_BWD, device=dev)
    fl["attn_bwd"] = 2.5 * fl["attn"]
    calls.append(("attention backward: dq, dk, dv contributions (tsp_attn_core_backward)", "attn_bwd",
                  lambda: tsp.attn_core_backward(plan, dims, q, kf, vf, a, lse, d_attn, dq_b, dk_b, dv_b,
                                                 attn_lo=a_lo, workspace=ws_abwd)))
    # backward of the O and QKV projections on layer 0's shapes: twice the
    # forward products' FLOPs each (the input and the weight gradients)
    hs_ = (dims.n_heads // D) * dims.head_dim
    dwo_b = [torch.empty(dims.hidden, hs_, dtype=torch.float32, device=dev) for _ in range(D)]
    dwqkv_b = [torch.empty(3 * hs_, dims.hidden, dtype=torch.float32, device=dev) for _ in range(D)]
    d_attn_b = torch.empty(n, dims.hidden, dtype=torch.bfloat16, device=dev)
    dx_b = torch.empty(n, dims.hidden, dtype=torch.bfloat16, device=dev)
    ws_obwd = tsp.alloc_workspace(n, dims, D, tsp.WS_OUT_BWD, device=dev)
    ws_pbwd = tsp.alloc_workspace(n, dims, D, tsp.WS_PROJ_BWD, device=dev)
    fl["oproj_bwd"] = 2.0 * fl["oproj"]
    fl["qkv_bwd"] = 2.0 * fl["qkv"]
    calls += [
        ("O projection backward: d_attn, dW_o per shard (tsp_attn_out_backward)", "oproj_bwd",
         lambda: tsp.attn_out_backward(dims, D, plan.rank, a, lw.wo, d_attn, d_attn_b, dwo_b, ws_obwd)),
        ("QKV projection backward: dx, dW_qkv per shard (tsp_attn_project_backward)", "qkv_bwd",
         lambda: tsp.attn_project_backward(dims, D, plan.rank, x0, lw.wqkv, dq_b, dq_b, dq_b,
                                           d_attn, dx_b, dwqkv_b, ws_pbwd)),
    ]
    # layer variants on the same shapes: RMSNorm and RoPE (HBM-bound passes),
    # attention with 8 K/V heads (grouped-query) on generated K/V of that width
    h, H, hd = dims.hidden, dims.n_heads, dims.head_dim
    gain = torch.ones(h, dtype=torch.bfloat16, device=dev)
    kv8 = 8 * hd
    k8 = torch.randn(plan.seq_len, kv8, device=dev).to(torch.bfloat16)
    v8 = torch.randn(plan.seq_len, kv8, device=dev).to(torch.bfloat16)
    calls += [
        ("variant: RMSNorm (tsp_rms_norm)", "hbm:" + str(2 * n * h * 2 + h * 2),
         lambda: tsp.rms_norm(x0, gain, 1e-6, out)),
        ("variant: RoPE of q and own k rows (tsp_rope)", "hbm:" + str(2 * 2 * n * h * 2),
         lambda: tsp.rope(plan, H, H, hd, 10000.0, q, kf)),
        ("variant: GQA attention, 8 K/V heads (tsp_attn_core_gqa)", "attn",
         lambda: tsp.attn_core_gqa(plan, dims, 8, q, k8, v8, a, a_lo, workspace=ws_core)),
    ]
    # the variants' backwards: RMSNorm (x, dy read, dx written), RoPE of the fp32
    # gradients of q and the own K rows (read and written), GQA attention
    lse8 = torch.empty(H, n, dtype=torch.float32, device=dev)
    tsp.attn_core_gqa_lse(plan, dims, 8, q, k8, v8, a, lse8, attn_lo=a_lo, workspace=ws_core)
    dk8 = torch.empty(plan.seq_len, kv8, dtype=torch.float32, device=dev)
    dv8 = torch.empty(plan.seq_len, kv8, dtype=torch.float32, device=dev)
    dgain = torch.empty(h, dtype=torch.float32, device=dev)
    dq_rope = torch.zeros(n, h, dtype=torch.float32, device=dev)
    dk_rope = torch.zeros(n, h, dtype=torch.float32, device=dev)
    ws_rms = tsp.alloc_workspace(n, dims, 1, tsp.WS_RMS_BWD, device=dev)
    calls += [
        ("variant backward: RMSNorm dx, dgain (tsp_rms_norm_backward)", "hbm:" + str(3 * n * h * 2 + h * 2),
         lambda: tsp.rms_norm_backward(x0, gain, 1e-6, d_attn, d_attn_b, dgain, workspace=ws_rms)),
        ("variant backward: RoPE of dq and own dk rows (tsp_rope_backward)", "hbm:" + str(2 * 2 * n * h * 4),
         lambda: tsp.rope_backward(plan, H, H, hd, 10000.0, dq_rope, dk_rope)),
        ("variant backward: GQA attention, 8 K/V heads (tsp_attn_core_gqa_backward)", "attn_bwd",
         lambda: tsp.attn_core_gqa_backward(plan, dims, 8, q, k8, v8, a, lse8, d_attn, dq_b, dk8, dv8,
                                            attn_lo=a_lo, workspace=ws_abwd)),
    ]
    stream = torch.cuda.current_stream()
    rows = {}
    for name, key, f in calls:
        f()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            f()
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / reps
        if key.startswith("hbm:"):
            gbs = int(key[4:]) / (ms * 1e-3) / 1e9
            rows[name] = {"ms": round(ms, 4), "GB/s": round(gbs, 1), "frac": round(gbs / PEAK_HBM_GBS, 4)}
        else:
            tf = fl[key] / (ms * 1e-3) / 1e12
            rows[name] = {"ms": round(ms, 4), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    torch.cuda.synchronize()
    if int(status[0]) != 0:
        raise RuntimeError("an arrival wait gave up with every shard arrived")
    del ws_attn3
    del ws_mlp, ws_mlp_s, ws_out_s, k8, v8, ws_bwd, dw1, dw2, dy, dx, ws_abwd, dq_b, dk_b, dv_b, lse, d_attn
    del dwo_b, dwqkv_b, d_attn_b, dx_b, ws_obwd, ws_pbwd, lse8, dk8, dv8, dgain, dq_rope, dk_rope, ws_rms
    return rows


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="full_7b_128k", choices=["full_7b_128k", "stream_7b_16k"])
    ap.add_argument("--layers", type=int, default=None, help="layers per step (default: the workload's)")
    ap.add_argument("--roofline-launches", type=int, default=10,
                    help="timed unit-scale launches of the attention core for the roofline figure")
    ap.add_argument("--no-stream", action="store_true",
                    help="skip the weight-streaming regime's object (timed after the main workload)")
    ap.add_argument("--stream-steps", type=int, default=10, help="timed steps of the weight-streaming stack")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--arrival-overlap", action="store_true",
                    help="also time layer 0's O projection with its shards delivered during the call")
    ap.add_argument("--no-rows", action="store_true",
                    help="skip the per-entry-point timings after the timed steps (a kernel-trace profile of the "
                         "timed steps alone then averages only their launches)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB before timing, so that a counter "
                         "profile of the same command holds a reference kernel of known traffic")
    return ap.parse_args()


def build_inputs(W, n_layers, dev):
    d, D, S = W.dims, W.D, W.seq_len
    layers = []
    for l in range(n_layers):
        lw = synth.layer_weights(W.wid, d, D, layer=l, device=dev)
        kf, vf = synth.gathered_kv(W.wid, S, d.hidden, layer=l, device=dev)
        layers.append((lw, kf, vf))
    return layers


class Stack:
    """One workload's resident inputs and buffers, and its chained step:
    tsp_layer_forward's three parts per layer, optionally with HIP events
    recorded between them on the launch stream."""

    def __init__(self, W, n_layers, dev):
        self.W, self.n_layers = W, n_layers
        d, D, S = W.dims, W.D, W.seq_len
        self.plan, _, _ = tsp.zigzag_plan(S, D, W.rank)
        n, h = self.plan.n_local, d.hidden
        self.dims = tsp.make_dims(d.hidden, d.n_heads, d.head_dim, d.ffn)
        self.layers = build_inputs(W, n_layers, dev)
        self.x0 = synth.activations(W.wid, n, h, device=dev)
        self.q = torch.empty(n, h, dtype=torch.bfloat16, device=dev)
        self.a = torch.empty(n, h, dtype=torch.bfloat16, device=dev)
        self.a_lo = torch.empty(n, h, dtype=torch.bfloat16, device=dev)
        self.bufs = [torch.empty(n, h, dtype=torch.bfloat16, device=dev) for _ in range(2)]
        self.ws = tsp.alloc_workspace(n, self.dims, D, tsp.WS_POST, device=dev)
        self.ws_core = tsp.alloc_workspace(n, self.dims, D, tsp.WS_CORE, device=dev)
        self.fl = layer_flops(n, S, D, self.plan.chunk_len, d)

    def step(self, stream, events=None):
        plan, dims, D = self.plan, self.dims, self.W.D
        x = self.x0
        for l, (lw, kf, vf) in enumerate(self.layers):
            out = self.bufs[l % 2]
            ev = events[l] if events is not None else None
            if ev: ev[0].record(stream)
            tsp.attn_project(plan, dims, x, lw.wqkv, kf, vf, self.q)
            if ev: ev[1].record(stream)
            tsp.attn_core(plan, dims, self.q, kf, vf, self.a, self.a_lo, workspace=self.ws_core)
            if ev: ev[2].record(stream)
            tsp.layer_post(dims, D, plan.rank, self.a, x, lw.wo, lw.w1, lw.w2, out, self.ws, attn_lo=self.a_lo)
            if ev: ev[3].record(stream)
            x = out
        return x

    def timed(self, stream, steps, warmup):
        """(ms per step, per-stage ms per launch over all layers, per-stage ms of layer 0)."""
        for _ in range(warmup):
            self.step(stream)
        torch.cuda.synchronize()
        events = [[[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(self.n_layers)]
                  for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s in range(steps):
            self.step(stream, events[s])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        stages = ["qkv", "attn", "post"]
        stage_ms = {k: 0.0 for k in stages}
        first_ms = {k: 0.0 for k in stages}
        for s in range(steps):
            for l in range(self.n_layers):
                ev = events[s][l]
                for i, k in enumerate(stages):
                    t = ev[i].elapsed_time(ev[i + 1])
                    stage_ms[k] += t
                    if l == 0:
                        first_ms[k] += t / steps
        stage_ms = {k: v / (steps * self.n_layers) for k, v in stage_ms.items()}
        return elapsed * 1e3 / steps, stage_ms, first_ms


ROOF_UNTIMED = 2  # untimed unit-scale launches before the timed ones


def unit_scale_attention(stack, stream, launches):
    """The roofline figure's launches: tsp_attn_core on layer 0's unit-scale
    inputs (Q projected from x0, the layer's generated K/V with the rank's own
    rows), ROOF_UNTIMED untimed, then `launches` each between HIP events on the
    launch stream.  Made after the warmup steps (the chip in its sustained
    state) and before the timed steps, so in a kernel trace of the command they
    are the attention dispatches warmup*layers + ROOF_UNTIMED + 1 ..
    warmup*layers + ROOF_UNTIMED + launches.  Returns the mean ms per launch."""
    lw, kf, vf = stack.layers[0]
    tsp.attn_project(stack.plan, stack.dims, stack.x0, lw.wqkv, kf, vf, stack.q)
    call = lambda: tsp.attn_core(stack.plan, stack.dims, stack.q, kf, vf, stack.a, stack.a_lo,
                                 workspace=stack.ws_core)
    for _ in range(ROOF_UNTIMED):
        call()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(launches)]
    for e0, e1 in ev:
        e0.record(stream)
        call()
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / launches


def cpu_baseline(W, plan, x_local, layer0):
    """Time the fp64 oracle on a bounded sample of layer 0 of the same workload
    and extrapolate to local tokens/s per layer.

    The oracle computes each row from its definition, so rows are independent
    given the K/V: the fixed cost is the K/V projection of all local rows, the
    rest is a cost per row.  Call A: the attention half (attention, O
    projection, residual) for the first row, which also computes the K/V
    projection of all local rows.  Call B: the attention half for 64 query rows
    stratified over the two zigzag chunks (32 evenly spaced rows of each chunk,
    its first and last row included), with those K/V reused.  Call C: the MLP
    (with its residual) for 256 rows evenly spaced over the local rows.
    Full layer = fixed + n * (attention per row + MLP per row).  The threads
    are the host cores this process may run on (its affinity mask)."""
    from oracle import tsp_oracle as O  # test infrastructure, used only here
    cores = len(os.sched_getaffinity(0))
    prev_threads = torch.get_num_threads()
    torch.set_num_threads(cores)
    try:
        lw, kf, vf = layer0
        d = W.dims
        lc = lw.to("cpu")
        x = x_local.cpu()
        kf_c, vf_c = kf.cpu(), vf.cpu()
        oplan = O.zigzag_plan(W.seq_len, W.D, W.rank)
        n, C = plan.n_local, plan.chunk_len
        per_chunk = torch.linspace(0, C - 1, 32).round().to(torch.int64)
        rows_attn = torch.cat([per_chunk, C + per_chunk])
        rows_mlp = torch.linspace(0, n - 1, 256).round().to(torch.int64)
        t0 = time.perf_counter()
        _, _, k_own, v_own = O.attn_forward(oplan, x, lc.wqkv, lc.wo, d.n_heads, d.head_dim, kf_c, vf_c,
                                            rows=rows_attn[:1])
        t1 = time.perf_counter()
        O.attn_forward(oplan, x, lc.wqkv, lc.wo, d.n_heads, d.head_dim, kf_c, vf_c, rows=rows_attn,
                       k_own=k_own, v_own=v_own)
        t2 = time.perf_counter()
        O.mlp_forward(x, lc.w1, lc.w2, residual=True, rows=rows_mlp)
        t3 = time.perf_counter()
    finally:
        torch.set_num_threads(prev_threads)
    attn_row = (t2 - t1) / len(rows_attn)
    mlp_row = (t3 - t2) / len(rows_mlp)
    fixed = max((t1 - t0) - attn_row, 0.0)
    layer_s = fixed + n * (attn_row + mlp_row)
    return {
        "value": n / layer_s,
        "unit": "local tokens/s per layer",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"fp64 oracle on layer 0 of the same workload, {cores} threads: K/V projection of all {n} local "
                   f"rows ({fixed:.1f} s), attention half for {len(rows_attn)} query rows stratified over both "
                   f"zigzag chunks ({t2 - t1:.1f} s), MLP for {len(rows_mlp)} rows ({t3 - t2:.1f} s); per layer = "
                   f"fixed + {n} x per-row = {layer_s:.0f} s"),
        "measured_s": round(t3 - t0, 2),
    }


def stream_object(stack, stream, steps, warmup):
    """The weight-streaming regime's figures, timed in this run."""
    W, plan, d = stack.W, stack.plan, stack.W.dims
    ms_step, stage_ms, _ = stack.timed(stream, steps, warmup)
    layer_ms = ms_step / stack.n_layers
    total_flops = sum(stack.fl.values())
    tflops = total_flops / (layer_ms * 1e-3) / 1e12
    alg_bytes = layer_bytes(plan, d)
    summary, unit = TRAFFIC_SUMMARY["stream_7b_16k"]
    counted = profile_summary.read_traffic(summary, unit)
    return {
        "workload": W.name,
        "layers_per_step": stack.n_layers,
        "steps": steps,
        "layer_ms": round(layer_ms, 4),
        "local_tokens_per_s": round(plan.n_local / (layer_ms * 1e-3), 1),
        "tflops": round(tflops, 1),
        "mfma_frac": round(tflops / PEAK_BF16_TFLOPS, 4),
        "stages_ms_per_launch": {k: round(v, 4) for k, v in stage_ms.items()},
        "hbm_algorithmic_bytes_per_layer": alg_bytes,
        "hbm_algorithmic_GBs": round(alg_bytes / (layer_ms * 1e-3) / 1e9, 1),
        "hbm_counted_bytes_per_layer": counted,
        "hbm_counted_GBs": round(counted / (layer_ms * 1e-3) / 1e9, 1) if counted else None,
        "hbm_peak_GBs": PEAK_HBM_GBS,
        "hbm_counted_frac": round(counted / (layer_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if counted else None,
        "hbm_counted_over_algorithmic": round(counted / alg_bytes, 3) if counted else None,
        "traffic_source": os.path.relpath(summary, ROOT),
    }


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures the rank-share layer of ONE GPU; runs on more than one GPU "
              "(--gpus above 1) are not supported.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("no HIP device", file=sys.stderr)
        sys.exit(1)
    torch.cuda.set_device(0)
    dev = "cuda"
    tsp.lib()

    W = synth.WORKLOADS[args.workload]
    n_layers = args.layers or W.n_layers
    d, D, S = W.dims, W.D, W.seq_len
    print(f"[bench] generating inputs: {W.name}, {n_layers} layers", file=sys.stderr, flush=True)
    main_stack = Stack(W, n_layers, dev)
    plan, dims, n = main_stack.plan, main_stack.dims, main_stack.plan.n_local
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    if args.copy_probe_mib > 0:
        nb = args.copy_probe_mib << 20
        src = torch.ones(nb // 2, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy probe: {nb} bytes read, {nb} bytes written", file=sys.stderr, flush=True)
        del src, dst

    summary, unit = TRAFFIC_SUMMARY[args.workload]
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        main_stack.step(stream)
    torch.cuda.synchronize()
    unit_ms = None
    if unit == "tsp_attn_core":
        print(f"[bench] roofline: {ROOF_UNTIMED} + {args.roofline_launches} unit-scale launches of tsp_attn_core",
              file=sys.stderr, flush=True)
        unit_ms = unit_scale_attention(main_stack, stream, args.roofline_launches)

    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    ms_per_step, stage_ms, first_ms = main_stack.timed(stream, args.steps, 0)
    fl_rows = main_stack.fl
    fl = dict(fl_rows)
    fl["post"] = fl.pop("oproj") + fl.pop("mlp")
    layer_ms = ms_per_step / n_layers
    value = n / (layer_ms * 1e-3)
    total_flops = sum(fl.values())

    if unit == "tsp_attn_core":
        roof = {"kernel": "tsp_attn_core (attn_kernel<128, false>), unit-scale layer-0 inputs",
                "flops": fl["attn"], "ms": unit_ms}
    else:
        roof = {"kernel": "tsp_layer_forward (QKV, attention, O projection, MLP)", "flops": total_flops,
                "ms": sum(stage_ms.values())}
    roof_tflops = roof["flops"] / (roof["ms"] * 1e-3) / 1e12
    traffic = profile_summary.read_traffic(summary, unit)
    alg_bytes = layer_bytes(plan, d)
    layer_stream_ms = sum(stage_ms.values())
    layer_traffic = traffic if unit == "tsp_layer_forward" else None

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "local tokens/s per layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic",
        "config": {
            "workload": W.name,
            "layers_per_step": n_layers,
            "seq_len": S, "D": D, "rank": W.rank, "n_local": n,
            "hidden": d.hidden, "n_heads": d.n_heads, "head_dim": d.head_dim, "ffn": d.ffn,
        },
        "layer_ms": round(layer_ms, 4),
        "layer_tflops": round(total_flops / (layer_ms * 1e-3) / 1e12, 1),
        "layer_mfma_frac": round(total_flops / (layer_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        "stages_ms_per_launch": {k: round(v, 4) for k, v in stage_ms.items()},
        "stages_tflops": {k: round(fl[k] / (stage_ms[k] * 1e-3) / 1e12, 1) for k in stage_ms},
        "stages_ms_layer0": {k: round(v, 4) for k, v in first_ms.items()},
        "roofline": {
            "kernel": roof["kernel"],
            "bound": "mfma",
            "achieved": round(roof_tflops, 1),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(roof_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": roof["flops"],
            "ms_per_launch": round(roof["ms"], 4),
            "launches": args.roofline_launches if unit == "tsp_attn_core" else args.steps * n_layers,
            "traffic_source": os.path.relpath(summary, ROOT),
            "profile_ms_per_launch": profile_summary.read_avg_ms(summary, unit),
        },
        # the layer against the HBM roof: algorithmic bytes (weights, the K/V
        # rows read, input and output rows) and, from the counter summary when
        # it covers the whole layer, the bytes actually moved
        "hbm": {
            "algorithmic_bytes_per_layer": alg_bytes,
            "achieved_GBs": round(alg_bytes / (layer_stream_ms * 1e-3) / 1e9, 1),
            "traffic_bytes_per_layer": layer_traffic,
            "traffic_GBs": (round(layer_traffic / (layer_stream_ms * 1e-3) / 1e9, 1) if layer_traffic else None),
            "peak": PEAK_HBM_GBS,
            "frac": (round(layer_traffic / (layer_stream_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4) if layer_traffic
                     else round(alg_bytes / (layer_stream_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)),
        },
        "cpu_baseline": None,
    }
    if unit == "tsp_attn_core":
        chained_tf = fl["attn"] / (stage_ms["attn"] * 1e-3) / 1e12
        result["roofline"]["chained"] = {
            "what": "the same kernel's mean over all layers of the timed chained steps (activations grow about "
                    "2.5x per layer without a norm)",
            "ms_per_launch": round(stage_ms["attn"], 4),
            "achieved": round(chained_tf, 1),
            "frac": round(chained_tf / PEAK_BF16_TFLOPS, 4),
        }
    if not args.no_rows:
        print("[bench] per-step timing on layer 0", file=sys.stderr, flush=True)
        result["rows_layer0"] = row_timings(plan, dims, D, main_stack.layers[0], main_stack.x0, main_stack.q,
                                            main_stack.a, main_stack.a_lo, main_stack.bufs[0], main_stack.ws_core,
                                            fl_rows, dev)
    if args.arrival_overlap:
        print("[bench] arrival overlap on layer 0's O projection", file=sys.stderr, flush=True)
        result["arrival_overlap_layer0"] = arrival_overlap(plan, dims, D, main_stack.layers[0], main_stack.x0,
                                                           main_stack.q, main_stack.a, main_stack.a_lo,
                                                           main_stack.bufs[0], dev)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (fp64 oracle, bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(W, plan, main_stack.x0, main_stack.layers[0])
    if args.workload != "stream_7b_16k" and not args.no_stream:
        SW = synth.WORKLOADS["stream_7b_16k"]
        del main_stack
        torch.cuda.empty_cache()
        print(f"[bench] weight-streaming regime: {SW.name}, {SW.n_layers} layers", file=sys.stderr, flush=True)
        sstack = Stack(SW, SW.n_layers, dev)
        torch.cuda.synchronize()
        result["stream_7b_16k"] = stream_object(sstack, stream, args.stream_steps, 2)
        del sstack
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
