"""Seeded synthetic inputs for the TSP rank-share layer.

This module draws random tensors and nothing else: it holds none of the
layer's arithmetic, so both the HIP path and the fp64 oracle can take their
inputs from it without sharing any computation.

Seeding rule: every tensor has its own ``torch.Generator`` seeded with
``1000 * workload_id + tensor_id + 1_000_000 * layer``.  Values are
``randn`` in fp32 times a standard deviation, then rounded to bf16 (RNE by
torch's ``.to(torch.bfloat16)``).  Activations and generated K/V have std 1,
weights std 0.02 (``N(0, 0.02)`` is read as a standard deviation).

Weights are stored ``out x in`` row-major (the ``nn.Linear`` layout), one
tensor per shard:

* ``wqkv[d]``  ``[3 * H_s * hd, h]``  rows: Q heads, then K heads, then V heads
  of shard d's ``H_s = H / D`` heads (heads ``d*H_s .. (d+1)*H_s - 1``);
* ``wo[d]``    ``[h, H_s * hd]``      input columns = shard d's heads;
* ``w1[d]``    ``[F_s, h]``           FFN units ``d*F_s .. (d+1)*F_s - 1``;
* ``w2[d]``    ``[h, F_s]``           same FFN units as input columns.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

TID_X = 1
TID_X_ALL = 2
TID_Q = 3
TID_WQKV = 10
TID_WO = 30
TID_W1 = 50
TID_W2 = 70
TID_K = 100
TID_V = 101
LAYER_STRIDE = 1_000_000

WEIGHT_STD = 0.02
ACT_STD = 1.0


def seed_for(workload_id: int, tensor_id: int, layer: int = 0) -> int:
    return 1000 * workload_id + tensor_id + LAYER_STRIDE * layer


def randn_bf16(shape, seed: int, std: float = 1.0, device="cpu") -> torch.Tensor:
    """``randn(shape) * std`` drawn from a generator seeded with ``seed``, as bf16."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(torch.bfloat16)


@dataclass(frozen=True)
class Dims:
    """Layer shape: hidden h, heads H, head_dim hd, FFN width F."""
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int


@dataclass(frozen=True)
class Workload:
    """A rank-share workload: shapes, axis size D, rank and sequence length."""
    wid: int
    name: str
    dims: Dims
    D: int
    rank: int
    seq_len: int
    n_layers: int = 1
    start_shard: int | None = None  # MLP-only workloads: ring start
    kind: str = "layer"              # "layer" | "mlp" | "attn"

    @property
    def n_local(self) -> int:
        return self.seq_len // self.D


DIMS_TINY = Dims(hidden=256, n_heads=4, head_dim=64, ffn=1024)
DIMS_7B = Dims(hidden=4096, n_heads=32, head_dim=128, ffn=16384)

WORKLOADS = {
    # tiny layer: D=4, S=2048 in 8 chunks of 256, rank 1 (512 local tokens);
    # full K/V derived from the x of all ranks.
    "tiny_layer": Workload(1, "tiny TSP layer, S=2048, D=4, rank 1", DIMS_TINY, 4, 1, 2048),
    # 7B MLP ring only: 16384 local tokens, D=8 shard pairs, ring from shard 3.
    "mlp_7b": Workload(2, "7B MLP ring, 16384 local tokens, D=8, start shard 3", DIMS_7B, 8, 3,
                       131072, start_shard=3, kind="mlp"),
    # 7B attention only: S=131072, 16 chunks of 8192, rank 3 (16384 queries).
    "attn_7b": Workload(3, "7B attention + O projection, S=131072, D=8, rank 3", DIMS_7B, 8, 3,
                        131072, kind="attn"),
    # full 32-layer rank-share forward at 128K, rank 0.
    "full_7b_128k": Workload(4, "7B dense decoder, 32 layers, S=131072, D=8, rank 0", DIMS_7B, 8, 0,
                             131072, n_layers=32),
    # weight-streaming regime: S=16384, 2048 local tokens, rank 0.
    "stream_7b_16k": Workload(5, "7B layer, S=16384, D=8, rank 0 (2048 local tokens)", DIMS_7B, 8, 0,
                              16384, n_layers=32),
}


@dataclass
class LayerWeights:
    wqkv: list = field(default_factory=list)
    wo: list = field(default_factory=list)
    w1: list = field(default_factory=list)
    w2: list = field(default_factory=list)

    def to(self, device):
        return LayerWeights(*[[t.to(device) for t in ts] for ts in (self.wqkv, self.wo, self.w1, self.w2)])


def layer_weights(wid: int, dims: Dims, D: int, layer: int = 0, device="cpu",
                  parts=("wqkv", "wo", "w1", "w2")) -> LayerWeights:
    """The D per-shard weight tensors of one layer, seeded per (workload, tensor, shard, layer)."""
    h, H, hd, F = dims.hidden, dims.n_heads, dims.head_dim, dims.ffn
    Hs, Fs = H // D, F // D
    lw = LayerWeights()
    for d in range(D):
        if "wqkv" in parts:
            lw.wqkv.append(randn_bf16((3 * Hs * hd, h), seed_for(wid, TID_WQKV + d, layer), WEIGHT_STD, device))
        if "wo" in parts:
            lw.wo.append(randn_bf16((h, Hs * hd), seed_for(wid, TID_WO + d, layer), WEIGHT_STD, device))
        if "w1" in parts:
            lw.w1.append(randn_bf16((Fs, h), seed_for(wid, TID_W1 + d, layer), WEIGHT_STD, device))
        if "w2" in parts:
            lw.w2.append(randn_bf16((h, Fs), seed_for(wid, TID_W2 + d, layer), WEIGHT_STD, device))
    return lw


def activations(wid: int, n_tokens: int, hidden: int, device="cpu", tensor_id: int = TID_X,
                layer: int = 0) -> torch.Tensor:
    return randn_bf16((n_tokens, hidden), seed_for(wid, tensor_id, layer), ACT_STD, device)


def gathered_kv(wid: int, seq_len: int, hidden: int, layer: int = 0, device="cpu"):
    """Generated stand-ins for the gathered full-sequence K and V, ``[S, h]`` each."""
    k = randn_bf16((seq_len, hidden), seed_for(wid, TID_K + 2 * layer), ACT_STD, device)
    v = randn_bf16((seq_len, hidden), seed_for(wid, TID_V + 2 * layer), ACT_STD, device)
    return k, v
