"""Thin ctypes binding of libtsp.so (C ABI in include/tsp.h).

Argument marshalling only: tensors are checked for dtype, device, contiguity
and shape (so that no kernel is handed a buffer smaller than it will touch),
then their device pointers and torch's current HIP stream are passed to the C
entry point of the same name.  Every step of the layer runs in the HIP
kernels; there is no fallback path: if ``libtsp.so`` is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_int32, c_int64, c_size_t, c_void_p

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtsp.so")

(TSP_OK, TSP_ERR_INVALID_ARG, TSP_ERR_SHAPE, TSP_ERR_ALIGNMENT, TSP_ERR_WORKSPACE, TSP_ERR_UNSUPPORTED, TSP_ERR_HIP,
 TSP_ERR_SCRATCH) = range(8)
NOALLOC_SCRATCH_BYTES = 96 * 1024 * 1024
(WS_ATTN, WS_MLP, WS_LAYER, WS_POST, WS_CORE, WS_OUT_SHARD, WS_MLP_SHARD, WS_MLP_BWD, WS_ATTN_BWD, WS_OUT_BWD,
 WS_PROJ_BWD, WS_RMS_BWD) = range(12)
MAX_D = 16

EXPORTS = ["tsp_zigzag_plan", "tsp_workspace_size", "tsp_attn_project", "tsp_attn_core", "tsp_attn_out",
           "tsp_attn_forward", "tsp_mlp_forward", "tsp_layer_post", "tsp_layer_forward", "tsp_attn_project_shard",
           "tsp_attn_out_shard", "tsp_mlp_shard", "tsp_rms_norm", "tsp_rope", "tsp_attn_project_gqa",
           "tsp_attn_core_gqa", "tsp_mlp_backward", "tsp_attn_core_lse", "tsp_attn_core_backward",
           "tsp_attn_out_backward", "tsp_attn_project_backward", "tsp_rope_backward", "tsp_rms_norm_backward",
           "tsp_attn_core_gqa_lse", "tsp_attn_core_gqa_backward", "tsp_memory_footprint", "tsp_status_string",
           "tsp_attn_forward_noalloc", "tsp_attn_project_arrival", "tsp_attn_out_arrival",
           "tsp_mlp_forward_arrival", "tsp_simulate_arrival"]
ARRIVAL_SPIN_DEFAULT = 1 << 20
MEM_TSP, MEM_TP = range(2)


class TSPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


class Plan(ctypes.Structure):
    _fields_ = [("seq_len", c_int64), ("chunk_len", c_int64), ("n_local", c_int64), ("D", c_int32),
                ("rank", c_int32), ("chunk_id", c_int32 * 2), ("chunk_start", c_int64 * 2)]


class Dims(ctypes.Structure):
    _fields_ = [("hidden", c_int32), ("n_heads", c_int32), ("head_dim", c_int32), ("ffn", c_int32)]


class Arrival(ctypes.Structure):
    """tsp_arrival: a device counter of delivered shards, its value before the
    call's first shard, the poll budget of one wait and a device status word."""
    _fields_ = [("counter", c_void_p), ("base", ctypes.c_uint32), ("spin_limit", ctypes.c_uint32),
                ("status", c_void_p)]


class Memory(ctypes.Structure):
    _fields_ = [(f, ctypes.c_uint64) for f in
                ("weights", "streamed", "kv", "activations", "train_state", "grads", "total")]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m folded_tensor_sequence_tsp_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, PP = c_void_p, POINTER(c_void_p)
        sig = {
            "tsp_zigzag_plan": [c_int64, c_int32, c_int32, POINTER(Plan), P, P],
            "tsp_workspace_size": [c_int64, POINTER(Dims), c_int32, c_int32],
            "tsp_attn_project": [POINTER(Plan), POINTER(Dims), P, PP, P, P, P, P],
            "tsp_attn_core": [POINTER(Plan), POINTER(Dims), P, P, P, P, P, P, c_size_t, P],
            "tsp_attn_out": [c_int64, POINTER(Dims), c_int32, c_int32, P, P, PP, P, P, P],
            "tsp_attn_forward": [POINTER(Plan), POINTER(Dims), P, PP, PP, P, P, P, P, P, c_size_t, P],
            "tsp_attn_forward_noalloc": [POINTER(Plan), POINTER(Dims), P, PP, PP, P, P, P, P, P],
            "tsp_mlp_forward": [c_int64, POINTER(Dims), c_int32, c_int32, P, PP, PP, P, P, P, c_size_t, P],
            "tsp_layer_post": [c_int64, POINTER(Dims), c_int32, c_int32, P, P, P, PP, PP, PP, P, P, c_size_t, P],
            "tsp_layer_forward": [POINTER(Plan), POINTER(Dims), P, PP, PP, PP, PP, P, P, P, P, c_size_t, P],
            "tsp_attn_project_shard": [POINTER(Plan), POINTER(Dims), c_int32, P, P, P, P, P, P],
            "tsp_attn_out_shard": [c_int64, POINTER(Dims), c_int32, c_int32, c_int32, P, P, P, P, P, P, c_size_t, P],
            "tsp_mlp_shard": [c_int64, POINTER(Dims), c_int32, c_int32, P, P, P, P, P, P, c_size_t, P],
            "tsp_rms_norm": [c_int64, c_int32, P, P, ctypes.c_float, P, P],
            "tsp_rope": [POINTER(Plan), c_int32, c_int32, c_int32, ctypes.c_double, P, P, P],
            "tsp_attn_project_gqa": [POINTER(Plan), POINTER(Dims), c_int32, P, PP, P, P, P, P],
            "tsp_attn_core_gqa": [POINTER(Plan), POINTER(Dims), c_int32, P, P, P, P, P, P, c_size_t, P],
            "tsp_mlp_backward": [c_int64, POINTER(Dims), c_int32, c_int32, c_int32, P, PP, PP, P, P, PP, PP, P,
                                 c_size_t, P],
            "tsp_attn_core_lse": [POINTER(Plan), POINTER(Dims), P, P, P, P, P, P, P, c_size_t, P],
            "tsp_attn_core_backward": [POINTER(Plan), POINTER(Dims), P, P, P, P, P, P, P, P, P, P, P, c_size_t, P],
            "tsp_attn_out_backward": [c_int64, POINTER(Dims), c_int32, c_int32, P, PP, P, P, PP, P, c_size_t, P],
            "tsp_attn_project_backward": [c_int64, POINTER(Dims), c_int32, c_int32, P, PP, P, P, P, P, P, PP, P,
                                          c_size_t, P],
            "tsp_rope_backward": [POINTER(Plan), c_int32, c_int32, c_int32, ctypes.c_double, P, P, P],
            "tsp_rms_norm_backward": [c_int64, c_int32, P, P, ctypes.c_float, P, P, P, P, c_size_t, P],
            "tsp_attn_core_gqa_lse": [POINTER(Plan), POINTER(Dims), c_int32, P, P, P, P, P, P, P, c_size_t, P],
            "tsp_attn_core_gqa_backward": [POINTER(Plan), POINTER(Dims), c_int32, P, P, P, P, P, P, P, P, P, P, P,
                                           c_size_t, P],
            "tsp_memory_footprint": [c_int64, POINTER(Dims), c_int32, c_int32, c_int32, c_int32, POINTER(Memory)],
            "tsp_status_string": [c_int32],
            "tsp_attn_project_arrival": [POINTER(Plan), POINTER(Dims), c_int32, P, PP, P, P, P, POINTER(Arrival), P],
            "tsp_attn_out_arrival": [c_int64, POINTER(Dims), c_int32, c_int32, P, P, PP, P, P, POINTER(Arrival), P],
            "tsp_mlp_forward_arrival": [c_int64, POINTER(Dims), c_int32, c_int32, P, PP, PP, P, P, P, c_size_t,
                                        POINTER(Arrival), P],
            "tsp_simulate_arrival": [c_int32, PP, PP, POINTER(c_size_t), P, ctypes.c_uint32, ctypes.c_uint32, P],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = c_int32
        L.tsp_workspace_size.restype = c_size_t
        L.tsp_status_string.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().tsp_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != TSP_OK:
        raise TSPError(status, where)


# ---------------------------------------------------------------- marshalling
def _dev_tensor(t: torch.Tensor, shape, name: str) -> c_void_p:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor")
    if t.dtype != torch.bfloat16:
        raise ValueError(f"{name}: expected bfloat16, got {t.dtype}")
    if t.device.type != "cuda" or t.device.index != torch.cuda.current_device():
        raise ValueError(f"{name}: expected a tensor on the current HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return c_void_p(t.data_ptr())


def _opt_tensor(t, shape, name):
    return c_void_p(None) if t is None else _dev_tensor(t, shape, name)


def _shards(ts, D: int, shape, name: str):
    if len(ts) != D:
        raise ValueError(f"{name}: expected {D} shards, got {len(ts)}")
    arr = (c_void_p * D)()
    for d, t in enumerate(ts):
        arr[d] = _dev_tensor(t, shape, f"{name}[{d}]").value
    return arr


def _workspace(ws: torch.Tensor, need: int) -> tuple:
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace: expected a contiguous tensor on the HIP device")
    nbytes = ws.numel() * ws.element_size()
    if nbytes < need:
        raise ValueError(f"workspace: {nbytes} bytes, need {need}")
    return c_void_p(ws.data_ptr()), nbytes


def _stream(stream) -> c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return c_void_p(s.cuda_stream)


# ------------------------------------------------------------------ entry points
def make_dims(hidden: int, n_heads: int, head_dim: int, ffn: int) -> Dims:
    return Dims(hidden, n_heads, head_dim, ffn)


def zigzag_plan(seq_len: int, D: int, rank: int):
    """(Plan, local_to_global int64 CPU tensor, ring order list) from the C planner."""
    plan = Plan()
    if D < 1 or D > MAX_D:
        _check(TSP_ERR_INVALID_ARG, "tsp_zigzag_plan")
    n = max(seq_len // D, 0) if seq_len > 0 else 0
    l2g = torch.empty(max(n, 1), dtype=torch.int64)
    ring = (c_int32 * D)()
    _check(lib().tsp_zigzag_plan(seq_len, D, rank, ctypes.byref(plan), c_void_p(l2g.data_ptr()),
                                 ctypes.cast(ring, c_void_p)), "tsp_zigzag_plan")
    return plan, l2g[:plan.n_local], list(ring)


def workspace_size(n_tokens: int, dims: Dims, D: int, kind: int) -> int:
    return int(lib().tsp_workspace_size(n_tokens, ctypes.byref(dims), D, kind))


def memory_footprint(seq_len: int, dims: Dims, D: int, n_layers: int, scheme: int = MEM_TSP,
                     training: bool = False) -> dict:
    """Per-rank memory accounting in bytes, by component (tsp_memory_footprint)."""
    m = Memory()
    _check(lib().tsp_memory_footprint(seq_len, ctypes.byref(dims), D, n_layers, scheme, int(training),
                                      ctypes.byref(m)), "tsp_memory_footprint")
    return {f: int(getattr(m, f)) for f, _ in Memory._fields_}


def attn_project(plan: Plan, dims: Dims, x_local, wqkv, k_full, v_full, q_out, stream=None):
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    args = (_dev_tensor(x_local, (n, h), "x_local"), _shards(wqkv, D, (3 * Hs * dims.head_dim, h), "wqkv"),
            _dev_tensor(k_full, (S, h), "k_full"), _dev_tensor(v_full, (S, h), "v_full"),
            _dev_tensor(q_out, (n, h), "q_out"))
    _check(lib().tsp_attn_project(ctypes.byref(plan), ctypes.byref(dims), *args, _stream(stream)),
           "tsp_attn_project")


def attn_core(plan: Plan, dims: Dims, q, k_full, v_full, attn_out, attn_lo=None, workspace=None, stream=None):
    """Causal attention of the plan's local queries; ``workspace`` defaults to a
    fresh allocation of tsp_workspace_size(..., WS_CORE) bytes."""
    n, h, S = plan.n_local, dims.hidden, plan.seq_len
    need = workspace_size(n, dims, plan.D, WS_CORE)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(q, (n, h), "q"), _dev_tensor(k_full, (S, h), "k_full"), _dev_tensor(v_full, (S, h), "v_full"),
            _dev_tensor(attn_out, (n, h), "attn_out"), _opt_tensor(attn_lo, (n, h), "attn_lo"))
    _check(lib().tsp_attn_core(ctypes.byref(plan), ctypes.byref(dims), *args, ws, nbytes, _stream(stream)),
           "tsp_attn_core")


def _f32_tensor(t, shape, name: str) -> c_void_p:
    if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device.type != "cuda" \
            or t.device.index != torch.cuda.current_device() or not t.is_contiguous() \
            or tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected a contiguous float32 tensor of shape {tuple(shape)} on the HIP device")
    return c_void_p(t.data_ptr())


def attn_core_lse(plan: Plan, dims: Dims, q, k_full, v_full, attn_out, lse, attn_lo=None, workspace=None,
                  stream=None):
    """attn_core that also writes lse [n_heads, n_local] (fp32): the natural log
    of each query row's softmax normaliser."""
    n, h, S = plan.n_local, dims.hidden, plan.seq_len
    need = workspace_size(n, dims, plan.D, WS_CORE)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(q, (n, h), "q"), _dev_tensor(k_full, (S, h), "k_full"), _dev_tensor(v_full, (S, h), "v_full"),
            _dev_tensor(attn_out, (n, h), "attn_out"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _f32_tensor(lse, (dims.n_heads, n), "lse"))
    _check(lib().tsp_attn_core_lse(ctypes.byref(plan), ctypes.byref(dims), *args, ws, nbytes, _stream(stream)),
           "tsp_attn_core_lse")


def attn_core_backward(plan: Plan, dims: Dims, q, k_full, v_full, attn_out, lse, d_attn, dq, dk_full, dv_full,
                       attn_lo=None, workspace=None, stream=None):
    """Gradients of attn_core: dq [n_local, hidden], and this rank's
    contributions dk_full, dv_full [seq_len, hidden] (all fp32)."""
    n, h, S = plan.n_local, dims.hidden, plan.seq_len
    need = workspace_size(n, dims, plan.D, WS_ATTN_BWD)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(q, (n, h), "q"), _dev_tensor(k_full, (S, h), "k_full"), _dev_tensor(v_full, (S, h), "v_full"),
            _dev_tensor(attn_out, (n, h), "attn_out"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _f32_tensor(lse, (dims.n_heads, n), "lse"), _dev_tensor(d_attn, (n, h), "d_attn"),
            _f32_tensor(dq, (n, h), "dq"), _f32_tensor(dk_full, (S, h), "dk_full"),
            _f32_tensor(dv_full, (S, h), "dv_full"))
    _check(lib().tsp_attn_core_backward(ctypes.byref(plan), ctypes.byref(dims), *args, ws, nbytes, _stream(stream)),
           "tsp_attn_core_backward")


def attn_out(dims: Dims, D: int, start_shard: int, attn, wo, residual, out, attn_lo=None, stream=None):
    n, h = attn.shape[0], dims.hidden
    Hs = dims.n_heads // D if D > 0 else 0
    args = (_dev_tensor(attn, (n, h), "attn"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _shards(wo, D, (h, Hs * dims.head_dim), "wo"),
            _opt_tensor(residual, (n, h), "residual"), _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_attn_out(n, ctypes.byref(dims), D, start_shard, *args, _stream(stream)), "tsp_attn_out")


def attn_forward(plan: Plan, dims: Dims, x_local, wqkv, wo, k_full, v_full, residual, out, workspace, stream=None):
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_ATTN)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(x_local, (n, h), "x_local"), _shards(wqkv, D, (3 * Hs * dims.head_dim, h), "wqkv"),
            _shards(wo, D, (h, Hs * dims.head_dim), "wo"), _dev_tensor(k_full, (S, h), "k_full"),
            _dev_tensor(v_full, (S, h), "v_full"), _opt_tensor(residual, (n, h), "residual"),
            _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_attn_forward(ctypes.byref(plan), ctypes.byref(dims), *args, ws, nbytes, _stream(stream)),
           "tsp_attn_forward")


def attn_forward_noalloc(plan: Plan, dims: Dims, x_local, wqkv, wo, k_full, v_full, residual, out, stream=None):
    """tsp_attn_forward with its scratch in the library's fixed device array
    (no workspace argument; see tsp_attn_forward_noalloc in tsp.h)."""
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    args = (_dev_tensor(x_local, (n, h), "x_local"), _shards(wqkv, D, (3 * Hs * dims.head_dim, h), "wqkv"),
            _shards(wo, D, (h, Hs * dims.head_dim), "wo"), _dev_tensor(k_full, (S, h), "k_full"),
            _dev_tensor(v_full, (S, h), "v_full"), _opt_tensor(residual, (n, h), "residual"),
            _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_attn_forward_noalloc(ctypes.byref(plan), ctypes.byref(dims), *args, _stream(stream)),
           "tsp_attn_forward_noalloc")


def mlp_forward(dims: Dims, D: int, start_shard: int, x, w1, w2, residual, y, workspace, stream=None):
    n, h = x.shape[0], dims.hidden
    Fs = dims.ffn // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_MLP)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(x, (n, h), "x"), _shards(w1, D, (Fs, h), "w1"), _shards(w2, D, (h, Fs), "w2"),
            _opt_tensor(residual, (n, h), "residual"), _dev_tensor(y, (n, h), "y"))
    _check(lib().tsp_mlp_forward(n, ctypes.byref(dims), D, start_shard, *args, ws, nbytes, _stream(stream)),
           "tsp_mlp_forward")


def layer_post(dims: Dims, D: int, start_shard: int, attn, x, wo, w1, w2, out, workspace, attn_lo=None,
               stream=None):
    n, h = attn.shape[0], dims.hidden
    Hs = dims.n_heads // D if D > 0 else 0
    Fs = dims.ffn // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_POST)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(attn, (n, h), "attn"), _opt_tensor(attn_lo, (n, h), "attn_lo"), _dev_tensor(x, (n, h), "x"),
            _shards(wo, D, (h, Hs * dims.head_dim), "wo"), _shards(w1, D, (Fs, h), "w1"),
            _shards(w2, D, (h, Fs), "w2"), _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_layer_post(n, ctypes.byref(dims), D, start_shard, *args, ws, nbytes, _stream(stream)),
           "tsp_layer_post")


def layer_forward(plan: Plan, dims: Dims, x_local, wqkv, wo, w1, w2, k_full, v_full, out, workspace, stream=None):
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    Fs = dims.ffn // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_LAYER)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(x_local, (n, h), "x_local"), _shards(wqkv, D, (3 * Hs * dims.head_dim, h), "wqkv"),
            _shards(wo, D, (h, Hs * dims.head_dim), "wo"), _shards(w1, D, (Fs, h), "w1"),
            _shards(w2, D, (h, Fs), "w2"), _dev_tensor(k_full, (S, h), "k_full"),
            _dev_tensor(v_full, (S, h), "v_full"), _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_layer_forward(ctypes.byref(plan), ctypes.byref(dims), *args, ws, nbytes, _stream(stream)),
           "tsp_layer_forward")


# ---- shard streaming: one ring step per call (see include/tsp.h)
def attn_project_shard(plan: Plan, dims: Dims, shard: int, x_local, wqkv_d, k_full, v_full, q_out, stream=None):
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    args = (_dev_tensor(x_local, (n, h), "x_local"), _dev_tensor(wqkv_d, (3 * Hs * dims.head_dim, h), "wqkv_d"),
            _dev_tensor(k_full, (S, h), "k_full"), _dev_tensor(v_full, (S, h), "v_full"),
            _dev_tensor(q_out, (n, h), "q_out"))
    _check(lib().tsp_attn_project_shard(ctypes.byref(plan), ctypes.byref(dims), shard, *args, _stream(stream)),
           "tsp_attn_project_shard")


def attn_out_shard(dims: Dims, D: int, pos: int, shard: int, attn, wo_d, residual, out, workspace, attn_lo=None,
                   stream=None):
    n, h = attn.shape[0], dims.hidden
    Hs = dims.n_heads // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_OUT_SHARD)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(attn, (n, h), "attn"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _dev_tensor(wo_d, (h, Hs * dims.head_dim), "wo_d"), _opt_tensor(residual, (n, h), "residual"),
            _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_attn_out_shard(n, ctypes.byref(dims), D, pos, shard, *args, ws, nbytes, _stream(stream)),
           "tsp_attn_out_shard")


def mlp_shard(dims: Dims, D: int, pos: int, x, w1_d, w2_d, residual, y, workspace, stream=None):
    n, h = x.shape[0], dims.hidden
    Fs = dims.ffn // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_MLP_SHARD)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(x, (n, h), "x"), _dev_tensor(w1_d, (Fs, h), "w1_d"), _dev_tensor(w2_d, (h, Fs), "w2_d"),
            _opt_tensor(residual, (n, h), "residual"), _dev_tensor(y, (n, h), "y"))
    _check(lib().tsp_mlp_shard(n, ctypes.byref(dims), D, pos, *args, ws, nbytes, _stream(stream)), "tsp_mlp_shard")


# ---- calls that wait for their shards inside the kernels (see include/tsp.h)
def _word(t, name: str) -> c_void_p:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dtype not in (torch.int32, torch.uint32) \
            or t.numel() < 1:
        raise ValueError(f"{name}: expected a 32-bit integer tensor on the HIP device")
    return c_void_p(t.data_ptr())


def make_arrival(counter, base: int, status, spin_limit: int = 0) -> Arrival:
    """An arrival descriptor over the first element of the device tensors
    ``counter`` and ``status`` (32-bit integers)."""
    return Arrival(_word(counter, "counter").value, base & 0xFFFFFFFF, spin_limit, _word(status, "status").value)


def attn_project_arrival(plan: Plan, dims: Dims, start_shard: int, x_local, wqkv, k_full, v_full, q_out,
                         arrival: Arrival, stream=None):
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    args = (_dev_tensor(x_local, (n, h), "x_local"), _shards(wqkv, D, (3 * Hs * dims.head_dim, h), "wqkv"),
            _dev_tensor(k_full, (S, h), "k_full"), _dev_tensor(v_full, (S, h), "v_full"),
            _dev_tensor(q_out, (n, h), "q_out"))
    _check(lib().tsp_attn_project_arrival(ctypes.byref(plan), ctypes.byref(dims), start_shard, *args,
                                          ctypes.byref(arrival), _stream(stream)), "tsp_attn_project_arrival")


def attn_out_arrival(dims: Dims, D: int, start_shard: int, attn, wo, residual, out, arrival: Arrival,
                     attn_lo=None, stream=None):
    n, h = attn.shape[0], dims.hidden
    Hs = dims.n_heads // D if D > 0 else 0
    args = (_dev_tensor(attn, (n, h), "attn"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _shards(wo, D, (h, Hs * dims.head_dim), "wo"),
            _opt_tensor(residual, (n, h), "residual"), _dev_tensor(out, (n, h), "out"))
    _check(lib().tsp_attn_out_arrival(n, ctypes.byref(dims), D, start_shard, *args, ctypes.byref(arrival),
                                      _stream(stream)), "tsp_attn_out_arrival")


def mlp_forward_arrival(dims: Dims, D: int, start_shard: int, x, w1, w2, residual, y, workspace,
                        arrival: Arrival, stream=None):
    n, h = x.shape[0], dims.hidden
    Fs = dims.ffn // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_MLP)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(x, (n, h), "x"), _shards(w1, D, (Fs, h), "w1"), _shards(w2, D, (h, Fs), "w2"),
            _opt_tensor(residual, (n, h), "residual"), _dev_tensor(y, (n, h), "y"))
    _check(lib().tsp_mlp_forward_arrival(n, ctypes.byref(dims), D, start_shard, *args, ws, nbytes,
                                         ctypes.byref(arrival), _stream(stream)), "tsp_mlp_forward_arrival")


def simulate_arrival(srcs, dsts, counter, base: int, delay_us: int, stream=None):
    """Copy srcs[i] -> dsts[i] (device tensors of equal byte size) one after
    another, (i + 1) * delay_us after the kernel starts, raising the counter to
    base + i + 1 after each copy (tsp_simulate_arrival)."""
    n = len(srcs)
    if len(dsts) != n:
        raise ValueError("simulate_arrival: srcs and dsts differ in length")
    src, dst, nb = (c_void_p * max(n, 1))(), (c_void_p * max(n, 1))(), (c_size_t * max(n, 1))()
    for i, (a, b) in enumerate(zip(srcs, dsts)):
        if a.device.type != "cuda" or b.device.type != "cuda" or not a.is_contiguous() or not b.is_contiguous():
            raise ValueError(f"simulate_arrival: shard {i} is not a contiguous device tensor")
        if a.numel() * a.element_size() != b.numel() * b.element_size():
            raise ValueError(f"simulate_arrival: shard {i} sizes differ")
        src[i], dst[i], nb[i] = a.data_ptr(), b.data_ptr(), a.numel() * a.element_size()
    _check(lib().tsp_simulate_arrival(n, src, dst, nb, _word(counter, "counter"), base & 0xFFFFFFFF, delay_us,
                                      _stream(stream)), "tsp_simulate_arrival")


# ---- layer variants (see include/tsp.h)
def rms_norm(x, gain, eps: float, y, stream=None):
    n, h = x.shape
    args = (_dev_tensor(x, (n, h), "x"), _dev_tensor(gain, (h,), "gain"))
    _check(lib().tsp_rms_norm(n, h, *args, float(eps), _dev_tensor(y, (n, h), "y"), _stream(stream)), "tsp_rms_norm")


def rope(plan: Plan, n_heads: int, n_kv_heads: int, head_dim: int, theta: float, q=None, k_full=None, stream=None):
    qa = _opt_tensor(q, (plan.n_local, n_heads * head_dim), "q")
    ka = _opt_tensor(k_full, (plan.seq_len, n_kv_heads * head_dim), "k_full")
    _check(lib().tsp_rope(ctypes.byref(plan), n_heads, n_kv_heads, head_dim, float(theta), qa, ka, _stream(stream)),
           "tsp_rope")


def attn_project_gqa(plan: Plan, dims: Dims, n_kv_heads: int, x_local, wqkv, k_full, v_full, q_out, stream=None):
    n, h, S, D = plan.n_local, dims.hidden, plan.seq_len, plan.D
    Hs = dims.n_heads // D if D > 0 else 0
    Ks = n_kv_heads // D if D > 0 else 0
    kvw = n_kv_heads * dims.head_dim
    args = (_dev_tensor(x_local, (n, h), "x_local"), _shards(wqkv, D, ((Hs + 2 * Ks) * dims.head_dim, h), "wqkv"),
            _dev_tensor(k_full, (S, kvw), "k_full"), _dev_tensor(v_full, (S, kvw), "v_full"),
            _dev_tensor(q_out, (n, h), "q_out"))
    _check(lib().tsp_attn_project_gqa(ctypes.byref(plan), ctypes.byref(dims), n_kv_heads, *args, _stream(stream)),
           "tsp_attn_project_gqa")


def attn_core_gqa(plan: Plan, dims: Dims, n_kv_heads: int, q, k_full, v_full, attn_out, attn_lo=None, workspace=None,
                  stream=None):
    n, h, S = plan.n_local, dims.hidden, plan.seq_len
    kvw = n_kv_heads * dims.head_dim
    need = workspace_size(n, dims, plan.D, WS_CORE)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(q, (n, h), "q"), _dev_tensor(k_full, (S, kvw), "k_full"), _dev_tensor(v_full, (S, kvw), "v_full"),
            _dev_tensor(attn_out, (n, h), "attn_out"), _opt_tensor(attn_lo, (n, h), "attn_lo"))
    _check(lib().tsp_attn_core_gqa(ctypes.byref(plan), ctypes.byref(dims), n_kv_heads, *args, ws, nbytes,
                                   _stream(stream)), "tsp_attn_core_gqa")


def rope_backward(plan: Plan, n_heads: int, n_kv_heads: int, head_dim: int, theta: float, dq=None, dk_own=None,
                  stream=None):
    """Inverse rotation of fp32 gradients in place: dq [n_local, H*hd], dk_own
    [n_local, H_kv*hd] (the rank's own K rows, local order)."""
    qa = _opt_f32(dq, (plan.n_local, n_heads * head_dim), "dq")
    ka = _opt_f32(dk_own, (plan.n_local, n_kv_heads * head_dim), "dk_own")
    _check(lib().tsp_rope_backward(ctypes.byref(plan), n_heads, n_kv_heads, head_dim, float(theta), qa, ka,
                                   _stream(stream)), "tsp_rope_backward")


def rms_norm_backward(x, gain, eps: float, dy, dx, dgain, workspace=None, stream=None):
    """dx (bf16) and dgain (fp32 [h]) of y = rms_norm(x) * gain."""
    n, h = x.shape
    need = workspace_size(n, Dims(h, 1, h, 0), 1, WS_RMS_BWD)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    ws, nbytes = _workspace(workspace, need)
    _check(lib().tsp_rms_norm_backward(n, h, _dev_tensor(x, (n, h), "x"), _dev_tensor(gain, (h,), "gain"), float(eps),
                                       _dev_tensor(dy, (n, h), "dy"), _dev_tensor(dx, (n, h), "dx"),
                                       _f32_tensor(dgain, (h,), "dgain"), ws, nbytes, _stream(stream)),
           "tsp_rms_norm_backward")


def attn_core_gqa_lse(plan: Plan, dims: Dims, n_kv_heads: int, q, k_full, v_full, attn_out, lse, attn_lo=None,
                      workspace=None, stream=None):
    n, h, S = plan.n_local, dims.hidden, plan.seq_len
    kvw = n_kv_heads * dims.head_dim
    need = workspace_size(n, dims, plan.D, WS_CORE)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(q, (n, h), "q"), _dev_tensor(k_full, (S, kvw), "k_full"), _dev_tensor(v_full, (S, kvw), "v_full"),
            _dev_tensor(attn_out, (n, h), "attn_out"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _f32_tensor(lse, (dims.n_heads, n), "lse"))
    _check(lib().tsp_attn_core_gqa_lse(ctypes.byref(plan), ctypes.byref(dims), n_kv_heads, *args, ws, nbytes,
                                       _stream(stream)), "tsp_attn_core_gqa_lse")


def attn_core_gqa_backward(plan: Plan, dims: Dims, n_kv_heads: int, q, k_full, v_full, attn_out, lse, d_attn, dq,
                           dk_full, dv_full, attn_lo=None, workspace=None, stream=None):
    n, h, S = plan.n_local, dims.hidden, plan.seq_len
    kvw = n_kv_heads * dims.head_dim
    need = workspace_size(n, dims, plan.D, WS_ATTN_BWD)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(q, (n, h), "q"), _dev_tensor(k_full, (S, kvw), "k_full"), _dev_tensor(v_full, (S, kvw), "v_full"),
            _dev_tensor(attn_out, (n, h), "attn_out"), _opt_tensor(attn_lo, (n, h), "attn_lo"),
            _f32_tensor(lse, (dims.n_heads, n), "lse"), _dev_tensor(d_attn, (n, h), "d_attn"),
            _f32_tensor(dq, (n, h), "dq"), _f32_tensor(dk_full, (S, kvw), "dk_full"),
            _f32_tensor(dv_full, (S, kvw), "dv_full"))
    _check(lib().tsp_attn_core_gqa_backward(ctypes.byref(plan), ctypes.byref(dims), n_kv_heads, *args, ws, nbytes,
                                            _stream(stream)), "tsp_attn_core_gqa_backward")


def _opt_f32(t, shape, name):
    return c_void_p(None) if t is None else _f32_tensor(t, shape, name)


def _f32_shards(ts, D: int, shape, name: str):
    if len(ts) != D:
        raise ValueError(f"{name}: expected {D} shards, got {len(ts)}")
    arr = (c_void_p * D)()
    for d, t in enumerate(ts):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device.type != "cuda" \
                or not t.is_contiguous() or tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name}[{d}]: expected a contiguous float32 HIP tensor of shape {tuple(shape)}")
        arr[d] = t.data_ptr()
    return arr


def mlp_backward(dims: Dims, D: int, start_shard: int, residual: bool, x, w1, w2, dy, dx, dw1, dw2, workspace,
                 stream=None):
    n, h = x.shape[0], dims.hidden
    Fs = dims.ffn // D if D > 0 else 0
    need = workspace_size(n, dims, D, WS_MLP_BWD)
    ws, nbytes = _workspace(workspace, need)
    args = (_dev_tensor(x, (n, h), "x"), _shards(w1, D, (Fs, h), "w1"), _shards(w2, D, (h, Fs), "w2"),
            _dev_tensor(dy, (n, h), "dy"), _dev_tensor(dx, (n, h), "dx"), _f32_shards(dw1, D, (Fs, h), "dw1"),
            _f32_shards(dw2, D, (h, Fs), "dw2"))
    _check(lib().tsp_mlp_backward(n, ctypes.byref(dims), D, start_shard, int(bool(residual)), *args, ws, nbytes,
                                  _stream(stream)), "tsp_mlp_backward")


def attn_out_backward(dims: Dims, D: int, start_shard: int, attn, wo, d_out, d_attn, dwo, workspace, stream=None):
    """Gradients of the O projection: d_attn (bf16) and this rank's dW_o_d (fp32)."""
    n, h = attn.shape[0], dims.hidden
    hs = (dims.n_heads // D) * dims.head_dim if D > 0 else 0
    ws, nbytes = _workspace(workspace, workspace_size(n, dims, D, WS_OUT_BWD))
    args = (_dev_tensor(attn, (n, h), "attn"), _shards(wo, D, (h, hs), "wo"), _dev_tensor(d_out, (n, h), "d_out"),
            _dev_tensor(d_attn, (n, h), "d_attn"), _f32_shards(dwo, D, (h, hs), "dwo"))
    _check(lib().tsp_attn_out_backward(n, ctypes.byref(dims), D, start_shard, *args, ws, nbytes, _stream(stream)),
           "tsp_attn_out_backward")


def attn_project_backward(dims: Dims, D: int, start_shard: int, x, wqkv, dq, dk, dv, dy, dx, dwqkv, workspace,
                          stream=None):
    """Gradients of the shard-iterated QKV projection: dx (bf16, plus dy when
    given) and this rank's dW_qkv_d (fp32); dq, dk, dv are fp32."""
    n, h = x.shape[0], dims.hidden
    hs = (dims.n_heads // D) * dims.head_dim if D > 0 else 0
    ws, nbytes = _workspace(workspace, workspace_size(n, dims, D, WS_PROJ_BWD))
    args = (_dev_tensor(x, (n, h), "x"), _shards(wqkv, D, (3 * hs, h), "wqkv"), _f32_tensor(dq, (n, h), "dq"),
            _f32_tensor(dk, (n, h), "dk"), _f32_tensor(dv, (n, h), "dv"), _opt_tensor(dy, (n, h), "dy"),
            _dev_tensor(dx, (n, h), "dx"), _f32_shards(dwqkv, D, (3 * hs, h), "dwqkv"))
    _check(lib().tsp_attn_project_backward(n, ctypes.byref(dims), D, start_shard, *args, ws, nbytes,
                                           _stream(stream)), "tsp_attn_project_backward")


def alloc_workspace(n_tokens: int, dims: Dims, D: int, kind: int, device=None) -> torch.Tensor:
    """A uint8 device tensor large enough for the given kind of call."""
    nbytes = workspace_size(n_tokens, dims, D, kind)
    if nbytes == 0 and n_tokens > 0 and kind != WS_CORE:  # the attention core may need none
        raise ValueError("invalid dims for a workspace")
    return torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device or torch.cuda.current_device())
