"""fp64 CPU oracle for the TSP rank-share layer.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The product path (the HIP library and its
Python binding) never imports, links or calls it, and this module imports
nothing from the product package.

What it computes.  Tensor + Sequence Parallelism folds the tensor-parallel and
sequence-parallel axes onto one mesh axis of size D: a device holds 1/D of every
weight matrix and 1/D of the tokens (zubnet.ai, "Zyphra TSP folds TP+SP onto one
GPU axis", para. 1).  The attention weight shards are applied one after another
to the local tokens, K/V are gathered over a zigzag partition of the sequence,
and the MLP weight shard pairs travel a ring while each device sums the partial
products of its own tokens, which is what removes tensor parallelism's
all-reduce (same page, para. 2).  All of this is an exact re-partitioning of one
decoder layer, so the oracle computes the *plain, unsharded* layer for the
rank's own tokens, in fp64, directly from its definition; the shard arrays are
only reassembled into whole matrices.  Sharded forms appear in
:func:`mlp_sharded` alone, which the pins use to check the method's identity
(sum over shards = unsharded MLP) on the oracle itself.

Readings of points the pages leave open:

* zigzag partition: 2D equal chunks of C = S/(2D); rank r owns chunks r and
  2D-1-r; local rows are the owned positions in ascending order;
* ring order of shards: (r + k) mod D, k = 0..D-1;
* layer: h1 = x + Attn(x), out = h1 + MLP(h1); MHA; no bias, no norm, no
  positional encoding; GELU in its tanh form;
* attention: causal with the diagonal included, scale 1/sqrt(hd);
* O projection: row blocks of W_o by head shard (the shard's heads are the
  input columns of ``wo[d]``);
* the rank's own rows of the gathered K/V are the ones it projects itself;
  the caller-supplied rows at those positions are replaced;
* the outputs of the attention projections are bf16 tensors, like every
  tensor of the bf16 model the page describes (para. 1): each weight shard,
  applied to the local tokens, produces its heads' Q, K and V as bf16 tensors
  (round to nearest even), and the gathered K/V that the workloads hand over
  is bf16, so the rank's own K/V rows enter it rounded exactly as they would
  travel through the all-gather.  ``proj_bf16=False`` keeps Q, K and V in
  fp64, for the pins that compare with exact library routines.

Inputs are bf16 tensors (converted exactly to fp64); apart from the
projection outputs above, no intermediate is rounded.
Matrix products use ``torch.matmul`` in fp64 as a library step; everything else
(GELU, masking, softmax) is written out below.

Layer variants at the end of the module (RMSNorm, rotary position embedding,
grouped-query attention) are not on the pages: they are the published
definitions (Zhang & Sennrich 2019; Su et al. 2021, RoFormer, with the
interleaved pairs (x_{2i}, x_{2i+1}) of that paper; Ainslie et al. 2023),
for the layer variants of a real decoder.

Backward passes at the end of the module (the MLP ring and causal attention)
are the chain rule of the forward definitions above, written out per shard
and per head; the pages name training as a use of the method but give no
backward.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
(library special cases, closed forms, invariants and brute force); none is
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

F64 = torch.float64


def f64(t: torch.Tensor) -> torch.Tensor:
    """Exact widening of a bf16 (or any float) tensor to fp64 on the CPU."""
    return t.detach().to("cpu").to(F64)


# ---------------------------------------------------------------------------
# zigzag plan (para. 2: "zigzag partition" for load balancing of K/V)
# ---------------------------------------------------------------------------
@dataclass
class Plan:
    seq_len: int
    D: int
    rank: int
    chunk_len: int
    chunk_ids: list
    chunk_starts: list
    local_to_global: torch.Tensor  # int64 [S/D]
    ring: list                     # shard visit order


def zigzag_plan(seq_len: int, D: int, rank: int) -> Plan:
    """The rank's share of the sequence under the zigzag partition.

    The sequence is cut into 2D chunks of equal length; chunk c belongs to the
    rank min(c, 2D-1-c), so every rank gets one chunk from the front half and
    its mirror from the back half (equal causal work per rank).  The local rows
    are the owned positions in ascending order.  Written as an enumeration over
    all chunks (not a closed form) so it is independent of the HIP planner.
    """
    if D < 1 or not (0 <= rank < D) or seq_len <= 0 or seq_len % (2 * D) != 0:
        raise ValueError("zigzag plan needs D >= 1, 0 <= rank < D and seq_len a positive multiple of 2D")
    n_chunks = 2 * D
    C = seq_len // n_chunks
    owned = [c for c in range(n_chunks) if min(c, n_chunks - 1 - c) == rank]
    positions = []
    for c in owned:
        positions.extend(range(c * C, (c + 1) * C))
    l2g = torch.tensor(positions, dtype=torch.int64)
    ring = [(rank + k) % D for k in range(D)]
    return Plan(seq_len, D, rank, C, owned, [c * C for c in owned], l2g, ring)


# ---------------------------------------------------------------------------
# whole matrices from the shard arrays (para. 1: each device holds 1/D of each weight)
# ---------------------------------------------------------------------------
@dataclass
class Whole:
    wq: torch.Tensor  # [h, h] out x in
    wk: torch.Tensor
    wv: torch.Tensor
    wo: torch.Tensor  # [h, h]
    w1: torch.Tensor  # [F, h]
    w2: torch.Tensor  # [h, F]


def assemble(wqkv=None, wo=None, w1=None, w2=None, head_dim: int | None = None) -> Whole:
    """Concatenate the D shards of each weight back into one fp64 matrix.

    ``wqkv[d]`` holds, as output rows, shard d's Q heads, then its K heads, then
    its V heads; shard d owns the contiguous head block d*H_s .. (d+1)*H_s-1.
    ``wo[d]`` takes shard d's heads as input columns; ``w1[d]`` / ``w2[d]`` hold
    the FFN block d as output rows / input columns.
    """
    wq = wk = wv = wo_ = w1_ = w2_ = None
    if wqkv:
        qs, ks, vs = [], [], []
        for w in wqkv:
            w = f64(w)
            third = w.shape[0] // 3
            qs.append(w[:third])
            ks.append(w[third:2 * third])
            vs.append(w[2 * third:])
        wq, wk, wv = torch.cat(qs, 0), torch.cat(ks, 0), torch.cat(vs, 0)
    if wo:
        wo_ = torch.cat([f64(w) for w in wo], 1)
    if w1:
        w1_ = torch.cat([f64(w) for w in w1], 0)
    if w2:
        w2_ = torch.cat([f64(w) for w in w2], 1)
    return Whole(wq, wk, wv, wo_, w1_, w2_)


# ---------------------------------------------------------------------------
# elementwise pieces
# ---------------------------------------------------------------------------
def gelu_tanh(u: torch.Tensor) -> torch.Tensor:
    """GELU in its tanh form: 0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + torch.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u * u * u)))


def linear(x: torch.Tensor, w: torch.Tensor) -> torch.Tensor:
    """x W^T for a weight stored out x in."""
    return torch.matmul(x, w.t())


# ---------------------------------------------------------------------------
# causal attention of local queries against the full gathered K/V
# ---------------------------------------------------------------------------
def causal_attention(q: torch.Tensor, positions: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                     n_heads: int, head_dim: int) -> torch.Tensor:
    """o[t, a] = sum_{j <= p_t} softmax_j(q[t,a] . k[j,a] / sqrt(hd)) v[j,a].

    ``q`` [m, H*hd] are the query rows at global positions ``positions`` [m];
    ``k``/``v`` [S, H*hd] the full-sequence keys and values (fp64).  Keys at
    positions greater than the query's are excluded (causal; the diagonal is
    included).  The softmax is written out: subtract the row maximum,
    exponentiate, divide by the sum.
    """
    m = q.shape[0]
    S = k.shape[0]
    out = torch.empty((m, n_heads * head_dim), dtype=F64)
    key_pos = torch.arange(S, dtype=torch.int64)
    future = key_pos[None, :] > positions[:, None]          # [m, S]
    scale = 1.0 / math.sqrt(head_dim)
    for a in range(n_heads):
        cols = slice(a * head_dim, (a + 1) * head_dim)
        s = torch.matmul(q[:, cols], k[:, cols].t()) * scale  # [m, S]
        s = s.masked_fill(future, float("-inf"))
        s_max = s.max(dim=1, keepdim=True).values
        e = torch.exp(s - s_max)
        p = e / e.sum(dim=1, keepdim=True)
        out[:, cols] = torch.matmul(p, v[:, cols])
    return out


def softmax_rows(q: torch.Tensor, positions: torch.Tensor, k: torch.Tensor, head: int,
                 head_dim: int) -> torch.Tensor:
    """The causal probability rows of one head (used by the pins)."""
    S = k.shape[0]
    cols = slice(head * head_dim, (head + 1) * head_dim)
    s = torch.matmul(q[:, cols], k[:, cols].t()) / math.sqrt(head_dim)
    future = torch.arange(S)[None, :] > positions[:, None]
    s = s.masked_fill(future, float("-inf"))
    e = torch.exp(s - s.max(dim=1, keepdim=True).values)
    return e / e.sum(dim=1, keepdim=True)


# ---------------------------------------------------------------------------
# the layer's two halves for the rank's own tokens
# ---------------------------------------------------------------------------
def qkv_projection(x_local, wqkv, head_dim):
    """q, k, v of the local tokens (fp64), all heads: the attention projections
    produced by applying every attention weight shard to the local tokens (para. 2)."""
    W = assemble(wqkv=wqkv, head_dim=head_dim)
    x = f64(x_local)
    return linear(x, W.wq), linear(x, W.wk), linear(x, W.wv)


def proj_rows(t: torch.Tensor, proj_bf16: bool = True) -> torch.Tensor:
    """A projection output as the bf16 model holds it: rounded to bf16 (nearest
    even) when ``proj_bf16``, else unchanged (fp64)."""
    t = f64(t)
    return t.to(torch.bfloat16).to(F64) if proj_bf16 else t


def gathered_kv(plan: Plan, k_own, v_own, k_full=None, v_full=None, proj_bf16: bool = True):
    """Full-sequence K/V as the K/V all-gather delivers it (para. 2).

    Rows at the rank's own positions are its own projections; all other rows are
    the caller-supplied ones (``k_full``/``v_full``, the other ranks'
    contributions).  With ``k_full`` None the own rows must cover the sequence
    (D = 1).  Every row is as the bf16 gathered tensor holds it (``proj_rows``).
    """
    S = plan.seq_len
    h = k_own.shape[1]
    if k_full is None:
        k = torch.full((S, h), float("nan"), dtype=F64)
        v = torch.full((S, h), float("nan"), dtype=F64)
    else:
        k, v = proj_rows(k_full, proj_bf16).clone(), proj_rows(v_full, proj_bf16).clone()
    k[plan.local_to_global] = proj_rows(k_own, proj_bf16)
    v[plan.local_to_global] = proj_rows(v_own, proj_bf16)
    return k, v


def attn_forward(plan: Plan, x_local, wqkv, wo, n_heads, head_dim, k_full=None, v_full=None,
                 residual=True, rows=None, k_own=None, v_own=None, proj_bf16: bool = True):
    """Attention half of the layer for the rank's local rows (or the subset ``rows``).

    Returns (out [m, h], q_own [n, h], k_own [n, h], v_own [n, h]) in fp64, where
    out = [x +] concat_a(o_a) W_o^T.  ``k_own``/``v_own`` may be passed in to skip
    recomputing them.
    """
    W = assemble(wqkv=wqkv, wo=wo, head_dim=head_dim)
    x = f64(x_local)
    sel = torch.arange(x.shape[0]) if rows is None else torch.as_tensor(rows, dtype=torch.int64)
    q = proj_rows(linear(x[sel], W.wq), proj_bf16)
    if k_own is None:
        k_own = linear(x, W.wk)
        v_own = linear(x, W.wv)
    k, v = gathered_kv(plan, k_own, v_own, k_full, v_full, proj_bf16)
    o = causal_attention(q, plan.local_to_global[sel], k, v, n_heads, head_dim)
    out = linear(o, W.wo)
    if residual:
        out = out + x[sel]
    return out, q, k_own, v_own


def mlp_forward(x, w1, w2, residual=True, rows=None):
    """y = [x +] GELU(x W1^T) W2^T for the given rows (unsharded form)."""
    W = assemble(w1=w1, w2=w2)
    xx = f64(x)
    if rows is not None:
        xx = xx[torch.as_tensor(rows, dtype=torch.int64)]
    y = linear(gelu_tanh(linear(xx, W.w1)), W.w2)
    return xx + y if residual else y


def mlp_sharded(x, w1, w2, order):
    """The method's MLP: shard pairs visited in ``order``, partial products summed
    locally in place of the all-reduce (para. 2).  Used only to pin the identity
    sum over shards = unsharded MLP."""
    xx = f64(x)
    y = torch.zeros((xx.shape[0], f64(w2[0]).shape[0]), dtype=F64)
    for d in order:
        y = y + linear(gelu_tanh(linear(xx, f64(w1[d]))), f64(w2[d]))
    return y


def layer_forward(plan: Plan, x_local, wqkv, wo, w1, w2, n_heads, head_dim, k_full=None,
                  v_full=None, rows=None, proj_bf16: bool = True):
    """One decoder layer for the local rows: h1 = x + Attn(x); out = h1 + MLP(h1)."""
    h1, _, k_own, v_own = attn_forward(plan, x_local, wqkv, wo, n_heads, head_dim, k_full, v_full,
                                       residual=True, rows=rows, proj_bf16=proj_bf16)
    out = mlp_forward(h1, w1, w2, residual=True)
    return out, k_own, v_own


# ---------------------------------------------------------------------------
# layer variants of a real decoder (not on the pages: the pages' layer has no
# norm, no positional encoding and MHA).  Each is the published definition,
# written out in fp64.
# ---------------------------------------------------------------------------
def rms_norm(x: torch.Tensor, gain: torch.Tensor, eps: float) -> torch.Tensor:
    """RMSNorm (Zhang & Sennrich, 2019): y = x / sqrt(mean_j x_j^2 + eps) * gain, per row."""
    xx = f64(x)
    ms = (xx * xx).mean(dim=-1, keepdim=True)
    return xx / torch.sqrt(ms + eps) * f64(gain)


def rope_angles(positions: torch.Tensor, head_dim: int, theta: float) -> torch.Tensor:
    """Rotary angles (RoFormer, Su et al., 2021): angle[t, i] = p_t * theta^(-2i/hd),
    i = 0 .. hd/2 - 1, in fp64."""
    i = torch.arange(head_dim // 2, dtype=F64)
    inv_freq = torch.pow(torch.tensor(theta, dtype=F64), -2.0 * i / head_dim)
    return positions.to(F64)[:, None] * inv_freq[None, :]


def rope(x: torch.Tensor, positions: torch.Tensor, n_heads: int, head_dim: int, theta: float) -> torch.Tensor:
    """Rotary position embedding of rows ``x`` [m, n_heads*hd] at ``positions`` [m]:
    in every head, the pair (x_{2i}, x_{2i+1}) is rotated by angle[t, i]:
        (x_{2i} cos - x_{2i+1} sin,  x_{2i} sin + x_{2i+1} cos)."""
    xx = f64(x).reshape(x.shape[0], n_heads, head_dim // 2, 2)
    ang = rope_angles(positions, head_dim, theta)[:, None, :]
    c, s = torch.cos(ang), torch.sin(ang)
    a, b = xx[..., 0], xx[..., 1]
    out = torch.stack([a * c - b * s, a * s + b * c], dim=-1)
    return out.reshape(x.shape[0], n_heads * head_dim)


def causal_attention_gqa(q: torch.Tensor, positions: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                         n_heads: int, n_kv_heads: int, head_dim: int) -> torch.Tensor:
    """Grouped-query attention (Ainslie et al., 2023): query head a reads K/V head
    a // (n_heads / n_kv_heads); ``k``/``v`` are [S, n_kv_heads*hd].  Otherwise as
    :func:`causal_attention`, written out per head."""
    group = n_heads // n_kv_heads
    m, S = q.shape[0], k.shape[0]
    out = torch.empty((m, n_heads * head_dim), dtype=F64)
    future = torch.arange(S, dtype=torch.int64)[None, :] > positions[:, None]
    scale = 1.0 / math.sqrt(head_dim)
    for a in range(n_heads):
        qc = slice(a * head_dim, (a + 1) * head_dim)
        kvh = a // group
        kc = slice(kvh * head_dim, (kvh + 1) * head_dim)
        s = torch.matmul(q[:, qc], k[:, kc].t()) * scale
        s = s.masked_fill(future, float("-inf"))
        e = torch.exp(s - s.max(dim=1, keepdim=True).values)
        out[:, qc] = torch.matmul(e / e.sum(dim=1, keepdim=True), v[:, kc])
    return out


def qkv_projection_gqa(x_local, wqkv, head_dim: int, heads_per_shard: int, kv_heads_per_shard: int):
    """Q, K, V of the local rows for grouped-query attention: shard d's weights
    are [(H_s + 2 Hkv_s) hd x h], columns [Q heads | K heads | V heads]; query
    heads and K/V heads are numbered shard by shard.  fp64, unrounded."""
    xx = f64(x_local)
    qs, ks, vs = [], [], []
    qw, kw = heads_per_shard * head_dim, kv_heads_per_shard * head_dim
    for w in wqkv:
        ww = f64(w)
        qs.append(linear(xx, ww[:qw]))
        ks.append(linear(xx, ww[qw:qw + kw]))
        vs.append(linear(xx, ww[qw + kw:qw + 2 * kw]))
    return torch.cat(qs, dim=1), torch.cat(ks, dim=1), torch.cat(vs, dim=1)


# ---------------------------------------------------------------------------
# backward pass of the MLP ring (not on the pages, which describe the forward
# schedule; the rank's gradient contributions for its own tokens)
# ---------------------------------------------------------------------------
def gelu_tanh_grad(u: torch.Tensor) -> torch.Tensor:
    """d/du of the tanh-form GELU: with z = c (u + a u^3), c = sqrt(2/pi), a = 0.044715,
    0.5 (1 + tanh z) + 0.5 u (1 - tanh^2 z) c (1 + 3 a u^2)."""
    c, a = math.sqrt(2.0 / math.pi), 0.044715
    t = torch.tanh(c * (u + a * u * u * u))
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * c * (1.0 + 3.0 * a * u * u)


def mlp_backward(x, w1, w2, dy, residual=True):
    """Gradients of y = [x +] sum_d GELU(x W1_d^T) W2_d^T for the rank's rows x,
    given dy = dL/dy (all fp64, from the chain rule written out per shard):
        U_d = x W1_d^T,  H_d = GELU(U_d),  dH_d = dy W2_d,  dU_d = dH_d * GELU'(U_d)
        dx    = [dy +] sum_d dU_d W1_d
        dW1_d = dU_d^T x        ([F_s x h], this rank's contribution)
        dW2_d = dy^T H_d        ([h x F_s], this rank's contribution)
    Returns (dx, [dW1_d], [dW2_d])."""
    xx, g = f64(x), f64(dy)
    dx = g.clone() if residual else torch.zeros_like(g)
    dw1, dw2 = [], []
    for a_w1, a_w2 in zip(w1, w2):
        W1, W2 = f64(a_w1), f64(a_w2)
        U = linear(xx, W1)
        H = gelu_tanh(U)
        dU = torch.matmul(g, W2) * gelu_tanh_grad(U)
        dx = dx + torch.matmul(dU, W1)
        dw1.append(torch.matmul(dU.t(), xx))
        dw2.append(torch.matmul(g.t(), H))
    return dx, dw1, dw2


def attention_lse(q: torch.Tensor, positions: torch.Tensor, k: torch.Tensor, n_heads: int,
                  head_dim: int) -> torch.Tensor:
    """lse[a, t] = log sum_{j <= p_t} exp(q[t,a] . k[j,a] / sqrt(hd)): the natural
    log of the causal softmax's normaliser, per head a and query row t
    ([n_heads, m]).  Written out as the row maximum plus the log of the sum of
    the shifted exponentials."""
    m, S = q.shape[0], k.shape[0]
    future = torch.arange(S, dtype=torch.int64)[None, :] > positions[:, None]
    out = torch.empty((n_heads, m), dtype=F64)
    for a in range(n_heads):
        cols = slice(a * head_dim, (a + 1) * head_dim)
        s = torch.matmul(q[:, cols], k[:, cols].t()) / math.sqrt(head_dim)
        s = s.masked_fill(future, float("-inf"))
        s_max = s.max(dim=1).values
        out[a] = s_max + torch.log(torch.exp(s - s_max[:, None]).sum(dim=1))
    return out


def causal_attention_backward(q: torch.Tensor, positions: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                              dout: torch.Tensor, n_heads: int, head_dim: int):
    """Gradients of o = causal_attention(q, positions, k, v) given dout = dL/do,
    per head, from the chain rule through o = P V, P = softmax_rows(S),
    S = q k^T / sqrt(hd) (causal mask as in the forward):
        dV = P^T dO,   dP = dO V^T,
        dS[t, j] = P[t, j] (dP[t, j] - sum_i P[t, i] dP[t, i])   (softmax Jacobian),
        dQ = dS K / sqrt(hd),   dK = dS^T Q / sqrt(hd).
    ``q`` [m, H*hd] are this rank's query rows at ``positions``; ``k``/``v``
    [S, H*hd] the full sequence.  Returns (dq [m, H*hd], dk [S, H*hd],
    dv [S, H*hd]); dk and dv are this rank's contributions for every key row
    (the owners of the key rows would sum them over ranks), zero for keys no
    local query sees."""
    m, S = q.shape[0], k.shape[0]
    future = torch.arange(S, dtype=torch.int64)[None, :] > positions[:, None]
    scale = 1.0 / math.sqrt(head_dim)
    dq = torch.zeros((m, n_heads * head_dim), dtype=F64)
    dk = torch.zeros((S, n_heads * head_dim), dtype=F64)
    dv = torch.zeros((S, n_heads * head_dim), dtype=F64)
    for a in range(n_heads):
        cols = slice(a * head_dim, (a + 1) * head_dim)
        qa, ka, va, ga = q[:, cols], k[:, cols], v[:, cols], dout[:, cols]
        s = (torch.matmul(qa, ka.t()) * scale).masked_fill(future, float("-inf"))
        e = torch.exp(s - s.max(dim=1, keepdim=True).values)
        p = e / e.sum(dim=1, keepdim=True)
        dv[:, cols] = torch.matmul(p.t(), ga)
        dp = torch.matmul(ga, va.t())
        ds = p * (dp - (p * dp).sum(dim=1, keepdim=True))
        dq[:, cols] = torch.matmul(ds, ka) * scale
        dk[:, cols] = torch.matmul(ds.t(), qa) * scale
    return dq, dk, dv


def attn_out_backward(attn, wo, d_out):
    """Gradients of the O projection out = [residual +] sum_d attn[:, cols_d] W_o_d^T
    (W_o taken in row blocks by head shard: ``wo[d]`` is [h, H_s*hd], the input
    columns of shard d's heads), given d_out = dL/dout:
        d_attn[:, cols_d] = d_out W_o_d,    dW_o_d = d_out^T attn[:, cols_d].
    Returns (d_attn [n, h], [dW_o_d])."""
    a, g = f64(attn), f64(d_out)
    d_attn = torch.empty_like(a)
    dwo = []
    c0 = 0
    for w in wo:
        W = f64(w)
        cols = slice(c0, c0 + W.shape[1])
        d_attn[:, cols] = torch.matmul(g, W)
        dwo.append(torch.matmul(g.t(), a[:, cols]))
        c0 += W.shape[1]
    return d_attn, dwo


def qkv_projection_backward(x, wqkv, dq, dk, dv, head_dim, dy=None):
    """Gradients of the shard-iterated projections [q_d | k_d | v_d] = x W_qkv_d^T
    (``wqkv[d]`` rows: shard d's Q heads, then its K heads, then its V heads;
    its heads are the columns c_d of q, k, v), given dq, dk, dv for the same
    rows (dk and dv: the rows' own K and V gradients, i.e. after every rank's
    contribution to them has been summed):
        dx = [dy +] sum_d (dq[:, c_d] Wq_d + dk[:, c_d] Wk_d + dv[:, c_d] Wv_d)
        dW_qkv_d = [dq[:, c_d]^T x ; dk[:, c_d]^T x ; dv[:, c_d]^T x].
    ``dy`` is the gradient arriving through the layer's residual.  Returns
    (dx [n, h], [dW_qkv_d])."""
    xx = f64(x)
    gq, gk, gv = f64(dq), f64(dk), f64(dv)
    dx = f64(dy).clone() if dy is not None else torch.zeros_like(xx)
    dw = []
    c0 = 0
    for w in wqkv:
        W = f64(w)
        hs = W.shape[0] // 3
        cols = slice(c0, c0 + hs)
        parts = (gq[:, cols], gk[:, cols], gv[:, cols])
        for i, gp in enumerate(parts):
            dx = dx + torch.matmul(gp, W[i * hs:(i + 1) * hs])
        dw.append(torch.cat([torch.matmul(gp.t(), xx) for gp in parts], dim=0))
        c0 += hs
    return dx, dw


def rms_norm_backward(x, gain, eps: float, dy):
    """Gradients of y = x / r * gain with r = sqrt(mean_j x_j^2 + eps), per row:
        dx = (gain * dy) / r - x * sum_j(gain_j dy_j x_j) / (h r^3),
        dgain = sum over rows of dy * x / r.
    Returns (dx, dgain)."""
    xx, g, w = f64(x), f64(dy), f64(gain)
    h = xx.shape[1]
    r = torch.sqrt((xx * xx).mean(dim=1, keepdim=True) + eps)
    gw = g * w
    dx = gw / r - xx * (gw * xx).sum(dim=1, keepdim=True) / (h * r ** 3)
    dgain = (g * xx / r).sum(dim=0)
    return dx, dgain


def rope_backward(dy: torch.Tensor, positions: torch.Tensor, n_heads: int, head_dim: int, theta: float):
    """Gradient of the rotary embedding: each pair was rotated by an orthogonal
    2x2 matrix R(angle), so the gradient is R(angle)^T dy = R(-angle) dy."""
    g = f64(dy)
    m = g.shape[0]
    ang = rope_angles(positions, head_dim, theta)          # [m, hd/2]
    c, s = torch.cos(ang)[:, None, :], torch.sin(ang)[:, None, :]
    pairs = g.reshape(m, n_heads, head_dim // 2, 2)
    y0, y1 = pairs[..., 0], pairs[..., 1]
    out = torch.stack([y0 * c + y1 * s, -y0 * s + y1 * c], dim=-1)
    return out.reshape(m, n_heads * head_dim)


def causal_attention_gqa_backward(q, positions, k, v, dout, n_heads: int, n_kv_heads: int, head_dim: int):
    """Gradients of causal_attention_gqa: per query head a, the chain rule of
    causal_attention_backward against K/V head a / (H / H_kv); the K/V
    gradients of one K/V head sum over the query heads that read it.
    Returns (dq [m, H*hd], dk [S, H_kv*hd], dv [S, H_kv*hd])."""
    m, S = q.shape[0], k.shape[0]
    group = n_heads // n_kv_heads
    dq = torch.zeros((m, n_heads * head_dim), dtype=F64)
    dk = torch.zeros((S, n_kv_heads * head_dim), dtype=F64)
    dv = torch.zeros((S, n_kv_heads * head_dim), dtype=F64)
    for a in range(n_heads):
        qc = slice(a * head_dim, (a + 1) * head_dim)
        kc = slice((a // group) * head_dim, (a // group + 1) * head_dim)
        gq, gk, gv = causal_attention_backward(q[:, qc], positions, k[:, kc], v[:, kc], dout[:, qc], 1, head_dim)
        dq[:, qc] = gq
        dk[:, kc] += gk
        dv[:, kc] += gv
    return dq, dk, dv
