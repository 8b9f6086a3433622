"""The C-ABI library on the CPU: it loads, exports every entry point the header
declares, its zigzag planner is bit-exact with the oracle's, and every invalid
argument is rejected with its status before anything is launched (no GPU is
touched: the pointers below are never dereferenced)."""
import ctypes
import os
import re

import pytest
import torch

from folded_tensor_sequence_tsp_amd import tsp
from oracle import tsp_oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "tsp.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tsp_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return tsp.lib()


def test_exports_every_declared_symbol(L):
    declared = _header_functions()
    assert declared, "no declarations parsed from include/tsp.h"
    assert sorted(declared) == sorted(tsp.EXPORTS)
    for name in declared:
        assert hasattr(L, name), name


def test_status_strings(L):
    for s in range(8):
        assert tsp.status_string(s).startswith("TSP_")
    assert "unknown" in tsp.status_string(99)


GRID = [(2, 1), (8, 2), (24, 3), (64, 4), (2048, 4), (96, 6), (256, 8), (16384, 8), (131072, 8), (1024, 16)]


@pytest.mark.parametrize("S,D", GRID)
def test_plan_bit_exact_with_oracle(S, D):
    for r in range(D):
        plan, l2g, ring = tsp.zigzag_plan(S, D, r)
        ref = O.zigzag_plan(S, D, r)
        assert plan.seq_len == S and plan.D == D and plan.rank == r
        assert plan.chunk_len == ref.chunk_len
        assert plan.n_local == S // D
        assert list(plan.chunk_id) == ref.chunk_ids
        assert list(plan.chunk_start) == ref.chunk_starts
        assert torch.equal(l2g, ref.local_to_global)
        assert ring == ref.ring


def test_plan_golden_cases(golden):
    for S, D, r, C, c0, c1, s0, s1 in (map(int, row) for row in golden("zigzag_plans.txt")):
        plan, l2g, _ = tsp.zigzag_plan(S, D, r)
        assert (plan.chunk_len, list(plan.chunk_id), list(plan.chunk_start)) == (C, [c0, c1], [s0, s1])


@pytest.mark.parametrize("S,D,r,status", [
    (30, 4, 0, tsp.TSP_ERR_SHAPE), (0, 2, 0, tsp.TSP_ERR_SHAPE), (-8, 2, 0, tsp.TSP_ERR_SHAPE),
    (16, 2, 2, tsp.TSP_ERR_INVALID_ARG), (16, 2, -1, tsp.TSP_ERR_INVALID_ARG),
    (64, 0, 0, tsp.TSP_ERR_INVALID_ARG), (64, 17, 0, tsp.TSP_ERR_INVALID_ARG)])
def test_plan_rejects(L, S, D, r, status):
    plan = tsp.Plan()
    assert L.tsp_zigzag_plan(S, D, r, ctypes.byref(plan), None, None) == status
    assert L.tsp_zigzag_plan(64, 2, 0, None, None, None) == tsp.TSP_ERR_INVALID_ARG


# ----------------------------------------------------------------- error paths
A = 0x10000          # aligned fake device address, never dereferenced
MIS = 0x10002        # misaligned fake device address


def _arr(vals):
    arr = (ctypes.c_void_p * len(vals))()
    for i, v in enumerate(vals):
        arr[i] = v
    return arr


def _plan(S=2048, D=4, r=1):
    return tsp.zigzag_plan(S, D, r)[0]


DIMS = dict(hidden=256, n_heads=4, head_dim=64, ffn=1024)


def _dims(**kw):
    d = dict(DIMS)
    d.update(kw)
    return tsp.Dims(d["hidden"], d["n_heads"], d["head_dim"], d["ffn"])


def project(L, plan=None, dims=None, x=A, w=None, k=A, v=A, q=A):
    plan = plan or _plan()
    dims = dims or _dims()
    w = w if w is not None else _arr([A] * plan.D)
    return L.tsp_attn_project(ctypes.byref(plan) if plan is not False else None, ctypes.byref(dims), x, w, k, v, q, None)


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), tsp.TSP_ERR_INVALID_ARG),
    (dict(k=None), tsp.TSP_ERR_INVALID_ARG),
    (dict(q=MIS), tsp.TSP_ERR_ALIGNMENT),
    (dict(v=MIS), tsp.TSP_ERR_ALIGNMENT),
    (dict(w=_arr([A, A, 0, A])), tsp.TSP_ERR_INVALID_ARG),      # a lost shard
    (dict(w=_arr([A, MIS, A, A])), tsp.TSP_ERR_ALIGNMENT),
    (dict(dims=_dims(n_heads=3, hidden=192)), tsp.TSP_ERR_SHAPE),  # H % D != 0
    (dict(dims=_dims(hidden=320)), tsp.TSP_ERR_SHAPE),             # hidden != H * hd
    (dict(dims=_dims(head_dim=32, n_heads=8)), tsp.TSP_ERR_UNSUPPORTED),
    (dict(dims=_dims(head_dim=96, n_heads=4, hidden=384)), tsp.TSP_ERR_UNSUPPORTED),
])
def test_project_rejects(L, kw, status):
    assert project(L, **kw) == status


def test_tampered_plan_rejected(L):
    p = _plan()
    p.chunk_start[1] = 1537
    assert project(L, plan=p) == tsp.TSP_ERR_SHAPE
    p = _plan()
    p.n_local = 1024
    assert project(L, plan=p) == tsp.TSP_ERR_SHAPE
    p = _plan()
    p.rank = 4
    assert project(L, plan=p) == tsp.TSP_ERR_INVALID_ARG


def test_core_rejects(L):
    p, d = _plan(), _dims()
    assert L.tsp_attn_core(None, ctypes.byref(d), A, A, A, A + 64, None, A + 128, 1 << 40, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, A, A, None, A + 128, 1 << 40, None) == tsp.TSP_ERR_INVALID_ARG  # alias
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, MIS, A + 64, None, A + 128, 1 << 40, None) == tsp.TSP_ERR_ALIGNMENT
    assert L.tsp_attn_core(ctypes.byref(p), None, A, A, A, A + 64, None, A + 128, 1 << 40, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, A, A + 64, A + 64, A + 128, 1 << 40, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, A, A + 64, MIS, A + 128, 1 << 40, None) == tsp.TSP_ERR_ALIGNMENT
    need = tsp.workspace_size(p.n_local, d, p.D, tsp.WS_CORE)
    # the partials of the late chunk's two key halves (a short sequence: the
    # grid is small); nothing else
    C, H = p.chunk_len, d.n_heads
    assert need == 2 * C * 256 * 4 + 2 * H * C * 2 * 4
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, A, A + 64, None, A + 128, need - 1, None) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, A, A + 64, None, None, need, None) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_attn_core(ctypes.byref(p), ctypes.byref(d), A, A, A, A + 64, None, MIS, need, None) == tsp.TSP_ERR_ALIGNMENT


def test_noalloc_rejects(L):
    """tsp_attn_forward_noalloc: a call that needs more scratch than the fixed
    array returns TSP_ERR_SCRATCH before any HIP call; invalid plans or dims
    return tsp_attn_forward's statuses (argument checks only, no GPU)."""
    d = tsp.make_dims(4096, 32, 128, 16384)
    p, _, _ = tsp.zigzag_plan(131072, 8, 0)
    assert tsp.workspace_size(p.n_local, d, 8, tsp.WS_ATTN) > tsp.NOALLOC_SCRATCH_BYTES
    w = _arr([A] * 8)
    call = lambda plan, dims: L.tsp_attn_forward_noalloc(plan, dims, A, w, w, A + 64, A + 128, None, A + 192, None)
    assert call(ctypes.byref(p), ctypes.byref(d)) == tsp.TSP_ERR_SCRATCH
    assert call(None, ctypes.byref(d)) == tsp.TSP_ERR_INVALID_ARG
    assert call(ctypes.byref(p), None) == tsp.TSP_ERR_INVALID_ARG
    bad = tsp.make_dims(4096, 32, 96, 16384)
    assert call(ctypes.byref(p), ctypes.byref(bad)) == tsp.TSP_ERR_SHAPE
    assert "fixed array" in tsp.status_string(tsp.TSP_ERR_SCRATCH)


def test_core_workspace_none_on_large_grids(L):
    """A grid of 512 or more query tiles is not split: the attention core then
    needs no workspace, and a null one is accepted (nothing is launched here:
    argument checks only, on a shape whose launch would need a GPU)."""
    d = tsp.make_dims(4096, 32, 128, 16384)
    p, _, _ = tsp.zigzag_plan(131072, 8, 0)
    assert tsp.workspace_size(p.n_local, d, 8, tsp.WS_CORE) == 0
    p2, _, _ = tsp.zigzag_plan(16384, 8, 0)
    C = p2.chunk_len
    assert tsp.workspace_size(p2.n_local, d, 8, tsp.WS_CORE) == 2 * C * 4096 * 4 + 2 * 32 * C * 2 * 4
    # the split threshold: 2 * heads * ceil(C / 256) work items below 512
    d4 = tsp.make_dims(256, 4, 64, 1024)
    for S, D in [(2048, 4), (131072, 8)]:
        q, _, _ = tsp.zigzag_plan(S, D, 0)
        items = 2 * 4 * ((q.chunk_len + 255) // 256)
        assert (tsp.workspace_size(q.n_local, d4, D, tsp.WS_CORE) > 0) == (items < 512)


def test_out_rejects(L):
    d = _dims()
    w = _arr([A] * 4)
    assert L.tsp_attn_out(512, ctypes.byref(d), 4, 4, A, None, w, None, A + 64, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_out(512, ctypes.byref(d), 4, -1, A, None, w, None, A + 64, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_out(-1, ctypes.byref(d), 4, 0, A, None, w, None, A + 64, None) == tsp.TSP_ERR_SHAPE
    assert L.tsp_attn_out(512, ctypes.byref(d), 4, 0, A, None, w, MIS, A + 64, None) == tsp.TSP_ERR_ALIGNMENT
    assert L.tsp_attn_out(512, ctypes.byref(d), 4, 0, A, None, w, None, A, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_out(512, ctypes.byref(d), 4, 0, A, None, None, None, A + 64, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_attn_out(512, ctypes.byref(d), 0, 0, A, None, w, None, A + 64, None) == tsp.TSP_ERR_INVALID_ARG


def test_mlp_rejects(L):
    d = _dims()
    w = _arr([A] * 4)
    ws = tsp.workspace_size(512, d, 4, tsp.WS_MLP)
    # fp16 GELU block + fp16 copy of the W2 shards + int32 row exponents (256-byte aligned parts)
    assert ws == 512 * 1024 * 2 + 256 * 1024 * 2 + 512 * 4
    call = lambda **k: L.tsp_mlp_forward(k.get("n", 512), ctypes.byref(k.get("dims", d)), k.get("D", 4),
                                         k.get("start", 0), k.get("x", A), k.get("w1", w), k.get("w2", w),
                                         k.get("res", None), k.get("y", A + 64), k.get("ws", A + 128),
                                         k.get("nb", ws), None)
    assert call(ws=None) == tsp.TSP_ERR_WORKSPACE
    assert call(nb=ws - 1) == tsp.TSP_ERR_WORKSPACE
    assert call(ws=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert call(dims=_dims(ffn=1002)) == tsp.TSP_ERR_SHAPE          # F % D != 0
    assert call(dims=_dims(ffn=1152)) == tsp.TSP_ERR_UNSUPPORTED    # F_s = 288 not a multiple of 64
    assert call(start=4) == tsp.TSP_ERR_INVALID_ARG
    assert call(y=A) == tsp.TSP_ERR_INVALID_ARG                     # y aliases x without being the residual
    assert call(w2=_arr([A, A, A, 0])) == tsp.TSP_ERR_INVALID_ARG
    assert call(n=-5) == tsp.TSP_ERR_SHAPE


def test_layer_and_forward_reject(L):
    p, d = _plan(), _dims()
    w = _arr([A] * 4)
    need = tsp.workspace_size(p.n_local, d, 4, tsp.WS_LAYER)
    assert need > 0
    args = lambda ws, nb, out=A + 64: (ctypes.byref(p), ctypes.byref(d), A, w, w, w, w, A, A, out, ws, nb, None)
    assert L.tsp_layer_forward(*args(A + 128, need - 1)) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_layer_forward(*args(None, need)) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_layer_forward(*args(A + 128, need, out=A)) == tsp.TSP_ERR_INVALID_ARG
    need_a = tsp.workspace_size(p.n_local, d, 4, tsp.WS_ATTN)
    assert L.tsp_attn_forward(ctypes.byref(p), ctypes.byref(d), A, w, w, A, A, None, A + 64, A + 128, need_a - 16,
                              None) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_attn_forward(ctypes.byref(p), ctypes.byref(d), A, w, w, A, A, MIS, A + 64, A + 128, need_a,
                              None) == tsp.TSP_ERR_ALIGNMENT


def test_layer_post_rejects(L):
    d = _dims()
    w = _arr([A] * 4)
    need = tsp.workspace_size(512, d, 4, tsp.WS_POST)
    assert need > 0
    call = lambda **k: L.tsp_layer_post(k.get("n", 512), ctypes.byref(k.get("dims", d)), k.get("D", 4),
                                        k.get("start", 0), k.get("attn", A), k.get("lo", None), k.get("x", A + 64),
                                        k.get("wo", w), k.get("w1", w), k.get("w2", w), k.get("out", A + 128),
                                        k.get("ws", A + 192), k.get("nb", need), None)
    assert call(nb=need - 1) == tsp.TSP_ERR_WORKSPACE
    assert call(ws=None) == tsp.TSP_ERR_WORKSPACE
    assert call(ws=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert call(out=A + 64) == tsp.TSP_ERR_INVALID_ARG             # out aliases x
    assert call(out=A) == tsp.TSP_ERR_INVALID_ARG                  # out aliases attn
    assert call(lo=A + 128) == tsp.TSP_ERR_INVALID_ARG             # out aliases attn_lo
    assert call(lo=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert call(start=-1) == tsp.TSP_ERR_INVALID_ARG
    assert call(w1=_arr([A, 0, A, A])) == tsp.TSP_ERR_INVALID_ARG
    assert call(x=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert call(dims=_dims(ffn=1002)) == tsp.TSP_ERR_SHAPE
    assert call(n=-1) == tsp.TSP_ERR_SHAPE


def test_workspace_sizes(L):
    d = _dims()
    n = 512
    attn = tsp.workspace_size(n, d, 4, tsp.WS_ATTN)
    mlp = tsp.workspace_size(n, d, 4, tsp.WS_MLP)
    layer = tsp.workspace_size(n, d, 4, tsp.WS_LAYER)
    assert attn >= 2 * n * 256 * 2
    assert mlp >= n * 1024 * 2 + 256 * 1024 * 2 + n * 4
    post = tsp.workspace_size(n, d, 4, tsp.WS_POST)
    # post: fp32 h1, fp16 h1, row exponents, fp16 W1 and W2, fp16 GELU block
    assert post == n * 256 * 4 + n * 256 * 2 + n * 4 + 2 * 1024 * 256 * 2 + n * 1024 * 2
    core = tsp.workspace_size(n, d, 4, tsp.WS_CORE)
    # the grid of this short sequence is small (2 chunks x 4 heads x 1 query
    # tile), so the late chunk's keys are split in two: the halves' fp32
    # outputs [2][C][h] and (max, sum) pairs [2][H][C][2]
    C = n // 2
    assert core == 2 * C * 256 * 4 + 2 * 4 * C * 2 * 4
    assert attn == 3 * n * 256 * 2 + core  # Q, the attention output as a (hi, lo) bf16 pair, the partials
    assert layer == attn + post
    assert tsp.workspace_size(n, d, 4, 99) == 0
    assert tsp.workspace_size(n, _dims(hidden=300), 4, tsp.WS_LAYER) == 0
    # a long sequence (2 x 32 heads x 32 query tiles) is not split: no workspace
    big = tsp.make_dims(4096, 32, 128, 16384)
    assert tsp.workspace_size(16384, big, 8, tsp.WS_CORE) == 0
    assert tsp.workspace_size(-1, d, 4, tsp.WS_ATTN) == 0


def test_shard_streaming_rejects(L):
    p, d = _plan(), _dims()
    n = p.n_local
    # project one shard: shard index in [0, D)
    pr = lambda shard=0, x=A, w=A + 64: L.tsp_attn_project_shard(ctypes.byref(p), ctypes.byref(d), shard, x, w,
                                                                 A + 128, A + 192, A + 256, None)
    assert pr(shard=4) == tsp.TSP_ERR_INVALID_ARG
    assert pr(shard=-1) == tsp.TSP_ERR_INVALID_ARG
    assert pr(w=None) == tsp.TSP_ERR_INVALID_ARG
    assert pr(x=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert L.tsp_attn_project_shard(None, ctypes.byref(d), 0, A, A, A, A, A, None) == tsp.TSP_ERR_INVALID_ARG
    # O projection ring step
    need_o = tsp.workspace_size(n, d, 4, tsp.WS_OUT_SHARD)
    assert need_o == n * 256 * 4  # the fp32 accumulator
    out = lambda **k: L.tsp_attn_out_shard(k.get("n", n), ctypes.byref(d), 4, k.get("pos", 0), k.get("shard", 0),
                                           k.get("attn", A), k.get("lo", None), k.get("wo", A + 64),
                                           k.get("res", None), k.get("out", A + 128), k.get("ws", A + 192),
                                           k.get("nb", need_o), None)
    assert out(pos=4) == tsp.TSP_ERR_INVALID_ARG
    assert out(pos=-1) == tsp.TSP_ERR_INVALID_ARG
    assert out(shard=4) == tsp.TSP_ERR_INVALID_ARG
    assert out(out=A) == tsp.TSP_ERR_INVALID_ARG          # out aliases attn
    assert out(wo=None) == tsp.TSP_ERR_INVALID_ARG
    assert out(nb=need_o - 1) == tsp.TSP_ERR_WORKSPACE
    assert out(ws=None) == tsp.TSP_ERR_WORKSPACE
    assert out(ws=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert out(n=-1) == tsp.TSP_ERR_SHAPE
    # MLP ring step
    need_m = tsp.workspace_size(512, d, 4, tsp.WS_MLP_SHARD)
    # fp32 accumulator, row exponents, fp16 W2_d [256 x 256], fp16 GELU block [512 x 256]
    assert need_m == 512 * 256 * 4 + 512 * 4 + 256 * 256 * 2 + 512 * 256 * 2
    mlp = lambda **k: L.tsp_mlp_shard(k.get("n", 512), ctypes.byref(k.get("dims", d)), 4, k.get("pos", 0),
                                      k.get("x", A), k.get("w1", A + 64), k.get("w2", A + 128), k.get("res", None),
                                      k.get("y", A + 192), k.get("ws", A + 256), k.get("nb", need_m), None)
    assert mlp(pos=4) == tsp.TSP_ERR_INVALID_ARG
    assert mlp(y=A) == tsp.TSP_ERR_INVALID_ARG              # y aliases x
    assert mlp(w2=None) == tsp.TSP_ERR_INVALID_ARG
    assert mlp(w1=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert mlp(nb=need_m - 1) == tsp.TSP_ERR_WORKSPACE
    assert mlp(dims=_dims(ffn=1002)) == tsp.TSP_ERR_SHAPE
    assert mlp(n=-3) == tsp.TSP_ERR_SHAPE
    assert tsp.workspace_size(512, _dims(ffn=1002), 4, tsp.WS_MLP_SHARD) == 0


def test_variants_reject(L):
    p, d = _plan(), _dims()
    # RMSNorm
    assert L.tsp_rms_norm(-1, 256, A, A + 64, ctypes.c_float(1e-6), A + 128, None) == tsp.TSP_ERR_SHAPE
    assert L.tsp_rms_norm(10, 0, A, A + 64, ctypes.c_float(1e-6), A + 128, None) == tsp.TSP_ERR_SHAPE
    assert L.tsp_rms_norm(10, 260, A, A + 64, ctypes.c_float(1e-6), A + 128, None) == tsp.TSP_ERR_UNSUPPORTED
    assert L.tsp_rms_norm(10, 256, A, A + 64, ctypes.c_float(-1.0), A + 128, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_rms_norm(10, 256, A, A + 64, ctypes.c_float(float("nan")), A + 128, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_rms_norm(10, 256, A, None, ctypes.c_float(1e-6), A + 128, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_rms_norm(10, 256, MIS, A, ctypes.c_float(1e-6), A + 128, None) == tsp.TSP_ERR_ALIGNMENT
    # RoPE
    assert L.tsp_rope(ctypes.byref(p), 4, 4, 64, ctypes.c_double(1.0), A, A, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_rope(ctypes.byref(p), 4, 4, 60, ctypes.c_double(1e4), A, A, None) == tsp.TSP_ERR_UNSUPPORTED
    assert L.tsp_rope(ctypes.byref(p), 0, 4, 64, ctypes.c_double(1e4), A, A, None) == tsp.TSP_ERR_SHAPE
    assert L.tsp_rope(ctypes.byref(p), 4, 4, 64, ctypes.c_double(1e4), MIS, A, None) == tsp.TSP_ERR_ALIGNMENT
    assert L.tsp_rope(None, 4, 4, 64, ctypes.c_double(1e4), A, A, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_rope(ctypes.byref(p), 4, 4, 64, ctypes.c_double(1e4), None, None, None) == tsp.TSP_OK  # nothing to do
    # GQA
    w = _arr([A] * 4)
    need = tsp.workspace_size(p.n_local, d, 4, tsp.WS_CORE)
    core = lambda kv, **k: L.tsp_attn_core_gqa(ctypes.byref(p), ctypes.byref(d), kv, A, A + 64, A + 128,
                                               k.get("out", A + 192), None, k.get("ws", A + 256), k.get("nb", need), None)
    assert core(3) == tsp.TSP_ERR_SHAPE          # 4 query heads do not group over 3 K/V heads
    assert core(0) == tsp.TSP_ERR_SHAPE
    assert core(8) == tsp.TSP_ERR_SHAPE          # more K/V heads than query heads
    assert core(2, out=A) == tsp.TSP_ERR_INVALID_ARG
    assert core(2, nb=need - 1) == tsp.TSP_ERR_WORKSPACE
    proj = lambda kv: L.tsp_attn_project_gqa(ctypes.byref(p), ctypes.byref(d), kv, A, w, A + 64, A + 128, A + 192, None)
    assert proj(2) == tsp.TSP_ERR_SHAPE          # 2 K/V heads do not split over D = 4 shards
    assert proj(3) == tsp.TSP_ERR_SHAPE


def test_mlp_backward_rejects(L):
    d = _dims()
    n = 300
    np_ = 320  # tokens rounded up to 64
    need = tsp.workspace_size(n, d, 4, tsp.WS_MLP_BWD)
    # x^T, dy^T, U (fp32), GELU(U)^T and dU^T (all shards), dU (all shards), W1^T (all shards), W2^T
    assert need == (2 * 256 * np_ * 2 + n * 256 * 4 + 2 * 1024 * np_ * 2 + n * 1024 * 2 + 256 * 1024 * 2
                    + 256 * 256 * 2)
    w = _arr([A] * 4)
    g = _arr([A + 512] * 4)
    call = lambda **k: L.tsp_mlp_backward(k.get("n", n), ctypes.byref(k.get("dims", d)), 4, k.get("start", 0), 1,
                                          k.get("x", A), k.get("w1", w), k.get("w2", w), k.get("dy", A + 64),
                                          k.get("dx", A + 128), k.get("dw1", g), k.get("dw2", g),
                                          k.get("ws", A + 256), k.get("nb", need), None)
    assert call(start=4) == tsp.TSP_ERR_INVALID_ARG
    assert call(dx=A) == tsp.TSP_ERR_INVALID_ARG                    # dx aliases x
    assert call(dx=A + 64) == tsp.TSP_ERR_INVALID_ARG               # dx aliases dy
    assert call(dw1=None) == tsp.TSP_ERR_INVALID_ARG
    assert call(dw2=_arr([A, A, 0, A])) == tsp.TSP_ERR_INVALID_ARG
    assert call(dw1=_arr([A, MIS, A, A])) == tsp.TSP_ERR_ALIGNMENT
    assert call(nb=need - 1) == tsp.TSP_ERR_WORKSPACE
    assert call(ws=None) == tsp.TSP_ERR_WORKSPACE
    assert call(dims=_dims(ffn=1002)) == tsp.TSP_ERR_SHAPE
    assert call(n=-1) == tsp.TSP_ERR_SHAPE


def test_attn_backward_rejects(L):
    d = _dims()
    p, _, _ = tsp.zigzag_plan(2048, 4, 1)
    n, S, C = p.n_local, 2048, p.chunk_len
    need = tsp.workspace_size(n, d, 4, tsp.WS_ATTN_BWD)
    # K^T tiles of the sequence, Q^T and dO^T tiles of both chunks, 1 KB of stats per 64-query tile
    tiles_c = -(-C // 64)
    assert need == 4 * (S // 64) * 64 * 64 * 2 + 2 * (2 * 4 * tiles_c * 64 * 64 * 2) + 2 * 4 * tiles_c * 1024
    # head_dim 128: K^T, Q^T and dO^T come from transposing LDS reads, so only the stats
    d128 = tsp.make_dims(512, 4, 128, 1024)
    assert tsp.workspace_size(n, d128, 4, tsp.WS_ATTN_BWD) == 2 * 4 * tiles_c * 1024
    lse = lambda **k: L.tsp_attn_core_lse(ctypes.byref(p), ctypes.byref(d), A, A + 64, A + 128, k.get("out", A + 192),
                                          None, k.get("lse", A + 512), A + 1024,
                                          tsp.workspace_size(n, d, 4, tsp.WS_CORE), None)
    assert lse(lse=None) == tsp.TSP_ERR_INVALID_ARG
    assert lse(lse=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert lse(out=A) == tsp.TSP_ERR_INVALID_ARG                     # output aliases q
    bwd = lambda **k: L.tsp_attn_core_backward(ctypes.byref(p), ctypes.byref(d), A, A + 64, A + 128, A + 192, None,
                                               k.get("lse", A + 256), A + 320, k.get("dq", A + 384),
                                               k.get("dk", A + 448), k.get("dv", A + 512), k.get("ws", A + 1024),
                                               k.get("nb", need), None)
    assert bwd(dk=A + 512) == tsp.TSP_ERR_INVALID_ARG                # dk = dv
    assert bwd(dq=A + 448) == tsp.TSP_ERR_INVALID_ARG                # dq = dk
    assert bwd(lse=None) == tsp.TSP_ERR_INVALID_ARG
    assert bwd(nb=need - 1) == tsp.TSP_ERR_WORKSPACE
    assert bwd(ws=None) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_attn_core_backward(None, ctypes.byref(d), A, A, A, A, None, A, A, A + 64, A + 128, A + 192, A,
                                    need, None) == tsp.TSP_ERR_INVALID_ARG


def test_projection_backward_rejects(L):
    d = _dims()
    n, np_, h, hs = 300, 320, 256, 64
    w = _arr([A] * 4)
    g = _arr([A + 512] * 4)
    need_o = tsp.workspace_size(n, d, 4, tsp.WS_OUT_BWD)
    assert need_o == h * h * 2 + h * np_ * 2 + h * np_ * 2        # W_o^T (all shards), d_out^T, attn^T
    out = lambda **k: L.tsp_attn_out_backward(k.get("n", n), ctypes.byref(d), 4, k.get("start", 0), A, w,
                                              A + 64, k.get("d_attn", A + 128), k.get("dwo", g),
                                              k.get("ws", A + 256), k.get("nb", need_o), None)
    assert out(start=4) == tsp.TSP_ERR_INVALID_ARG
    assert out(d_attn=A) == tsp.TSP_ERR_INVALID_ARG                  # d_attn aliases attn
    assert out(dwo=_arr([A, 0, A, A])) == tsp.TSP_ERR_INVALID_ARG
    assert out(nb=need_o - 1) == tsp.TSP_ERR_WORKSPACE
    assert out(n=-1) == tsp.TSP_ERR_SHAPE
    need_p = tsp.workspace_size(n, d, 4, tsp.WS_PROJ_BWD)
    # bf16 [dq | dk | dv], x^T, every shard's gradients transposed, W_qkv^T blocks
    assert need_p == n * 3 * h * 2 + h * np_ * 2 + 3 * h * np_ * 2 + 3 * h * h * 2
    prj = lambda **k: L.tsp_attn_project_backward(n, ctypes.byref(d), 4, k.get("start", 1), A, w, A + 64, A + 128,
                                                  A + 192, k.get("dy", None), k.get("dx", A + 320),
                                                  k.get("dw", g), k.get("ws", A + 1024), k.get("nb", need_p), None)
    assert prj(dx=A) == tsp.TSP_ERR_INVALID_ARG                      # dx aliases x
    assert prj(dy=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert prj(dw=None) == tsp.TSP_ERR_INVALID_ARG
    assert prj(start=-1) == tsp.TSP_ERR_INVALID_ARG
    assert prj(nb=need_p - 1) == tsp.TSP_ERR_WORKSPACE
    assert L.tsp_attn_project_backward(n, ctypes.byref(_dims(n_heads=3, hidden=192)), 4, 0, A, w, A, A, A, None,
                                       A + 64, g, A, need_p, None) == tsp.TSP_ERR_SHAPE


def test_variant_backward_rejects(L):
    p, _, _ = tsp.zigzag_plan(2048, 4, 1)
    rb = lambda **k: L.tsp_rope_backward(ctypes.byref(p), k.get("H", 4), 4, k.get("hd", 64), ctypes.c_double(1e4),
                                         k.get("dq", A), k.get("dk", A + 64), None)
    assert rb(dk=A) == tsp.TSP_ERR_INVALID_ARG                       # dq and dk_own coincide
    assert rb(hd=60) == tsp.TSP_ERR_UNSUPPORTED
    assert rb(H=0) == tsp.TSP_ERR_SHAPE
    assert rb(dq=MIS) == tsp.TSP_ERR_ALIGNMENT
    assert rb(dq=None, dk=None) == tsp.TSP_OK                        # nothing to do
    n, h = 300, 256
    need = tsp.workspace_size(n, _dims(), 1, tsp.WS_RMS_BWD)
    assert need == 10 * h * 4                                        # fp32 partial sums per 32-row block
    nb = lambda **k: L.tsp_rms_norm_backward(n, k.get("h", h), A, A + 64, ctypes.c_float(k.get("eps", 1e-6)), A + 128,
                                             k.get("dx", A + 192), k.get("dgain", A + 256), k.get("ws", A + 512),
                                             k.get("nb", need), None)
    assert nb(dx=A) == tsp.TSP_ERR_INVALID_ARG                       # dx aliases x
    assert nb(dx=A + 128) == tsp.TSP_ERR_INVALID_ARG                 # dx aliases dy
    assert nb(h=8200) == tsp.TSP_ERR_UNSUPPORTED                     # wider than the LDS partial sums allow
    assert nb(h=100) == tsp.TSP_ERR_UNSUPPORTED
    assert nb(eps=-1.0) == tsp.TSP_ERR_INVALID_ARG
    assert nb(dgain=None) == tsp.TSP_ERR_INVALID_ARG
    assert nb(nb=need - 1) == tsp.TSP_ERR_WORKSPACE
    d = _dims()
    need_b = tsp.workspace_size(p.n_local, d, 4, tsp.WS_ATTN_BWD)
    gb = lambda kv, **k: L.tsp_attn_core_gqa_backward(ctypes.byref(p), ctypes.byref(d), kv, A, A + 64, A + 128,
                                                      A + 192, None, A + 256, A + 320, A + 384, k.get("dk", A + 448),
                                                      A + 512, A + 1024, need_b, None)
    assert gb(3) == tsp.TSP_ERR_SHAPE                                 # 4 query heads do not group over 3
    assert gb(2, dk=A + 512) == tsp.TSP_ERR_INVALID_ARG               # dk = dv
    gl = lambda kv: L.tsp_attn_core_gqa_lse(ctypes.byref(p), ctypes.byref(d), kv, A, A + 64, A + 128, A + 192, None,
                                            None, A + 1024, need_b, None)
    assert gl(2) == tsp.TSP_ERR_INVALID_ARG                           # lse missing


def test_arrival_rejects(L):
    p, d = _plan(), _dims()
    w = _arr([A] * 4)
    ok = tsp.Arrival(A, 0, 0, A + 16)
    by = lambda arr: ctypes.byref(arr) if arr is not None else None

    def proj(start=0, arr=ok):
        return L.tsp_attn_project_arrival(ctypes.byref(p), ctypes.byref(d), start, A, w, A, A, A + 64, by(arr), None)

    assert proj(arr=None) == tsp.TSP_ERR_INVALID_ARG
    assert proj(arr=tsp.Arrival(None, 0, 0, A)) == tsp.TSP_ERR_INVALID_ARG      # no counter
    assert proj(arr=tsp.Arrival(A, 0, 0, None)) == tsp.TSP_ERR_INVALID_ARG      # no status word
    assert proj(arr=tsp.Arrival(A + 2, 0, 0, A)) == tsp.TSP_ERR_ALIGNMENT
    assert proj(arr=tsp.Arrival(A, 0, 0, A + 1)) == tsp.TSP_ERR_ALIGNMENT
    assert proj(start=4) == tsp.TSP_ERR_INVALID_ARG
    assert proj(start=-1) == tsp.TSP_ERR_INVALID_ARG

    def out(n=512, start=0, arr=ok, o=A + 64):
        return L.tsp_attn_out_arrival(n, ctypes.byref(d), 4, start, A, None, w, None, o, by(arr), None)

    assert out(arr=None) == tsp.TSP_ERR_INVALID_ARG
    assert out(start=4) == tsp.TSP_ERR_INVALID_ARG
    assert out(n=-1) == tsp.TSP_ERR_SHAPE
    assert out(o=A) == tsp.TSP_ERR_INVALID_ARG                                   # out aliases attn
    assert out(arr=tsp.Arrival(A + 1, 0, 0, A)) == tsp.TSP_ERR_ALIGNMENT

    need = tsp.workspace_size(512, d, 4, tsp.WS_MLP)

    def mlp(arr=ok, nb=need, start=0):
        return L.tsp_mlp_forward_arrival(512, ctypes.byref(d), 4, start, A, w, w, None, A + 64, A + 128, nb, by(arr),
                                         None)

    assert mlp(arr=None) == tsp.TSP_ERR_INVALID_ARG
    assert mlp(nb=need - 1) == tsp.TSP_ERR_WORKSPACE
    assert mlp(start=5) == tsp.TSP_ERR_INVALID_ARG
    assert mlp(arr=tsp.Arrival(A, 0, 0, A + 2)) == tsp.TSP_ERR_ALIGNMENT

    src, dst, nb = _arr([A]), _arr([A + 64]), (ctypes.c_size_t * 1)(64)
    assert L.tsp_simulate_arrival(65, src, dst, nb, A, 0, 0, None) == tsp.TSP_ERR_INVALID_ARG   # more than 64
    assert L.tsp_simulate_arrival(-1, src, dst, nb, A, 0, 0, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_simulate_arrival(1, src, dst, nb, None, 0, 0, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_simulate_arrival(1, None, dst, nb, A, 0, 0, None) == tsp.TSP_ERR_INVALID_ARG
    assert L.tsp_simulate_arrival(1, src, dst, nb, A + 2, 0, 0, None) == tsp.TSP_ERR_ALIGNMENT
    assert L.tsp_simulate_arrival(1, _arr([MIS]), dst, nb, A, 0, 0, None) == tsp.TSP_ERR_ALIGNMENT
    assert L.tsp_simulate_arrival(1, src, dst, (ctypes.c_size_t * 1)(40), A, 0, 0, None) == tsp.TSP_ERR_SHAPE
    assert L.tsp_simulate_arrival(1, src, dst, nb, A, 0, 2_000_000, None) == tsp.TSP_ERR_INVALID_ARG
