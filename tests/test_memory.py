"""Per-rank memory accounting (tsp_memory_footprint) on the CPU.

The TSP page (zubnet.ai, "Zyphra TSP folds TP+SP onto one GPU axis") states
that under TSP both parameter and activation memory fall by 1/D (para. 1) and
compares 38.8 GB per GPU for TSP with 70.0 GB for plain TP at 128K tokens on 8
GPUs (para. 2), without saying what those figures hold.  The accounting is
pinned here by what does not depend on those unknowns: the parameter count of
the page's 7B layer shape in closed form, the identity of the two schemes at
D = 1 (one device holds the whole layer either way), the forward workspace
the library itself asks for, and the 1/D relations between the schemes.
"""
import pytest

from folded_tensor_sequence_tsp_amd import tsp

FIELDS = ("weights", "streamed", "kv", "activations", "train_state", "grads", "total")
SHAPES = [  # (hidden, heads, head_dim, ffn, S)
    (256, 4, 64, 1024, 2048),
    (512, 8, 64, 2048, 4096),
    (4096, 32, 128, 16384, 131072),
]


def _round256(x):
    return (x + 255) // 256 * 256


@pytest.mark.parametrize("h,H,hd,F,S", SHAPES)
@pytest.mark.parametrize("training", [False, True])
def test_one_rank_schemes_coincide(h, H, hd, F, S, training):
    d = tsp.make_dims(h, H, hd, F)
    a = tsp.memory_footprint(S, d, 1, 3, tsp.MEM_TSP, training)
    b = tsp.memory_footprint(S, d, 1, 3, tsp.MEM_TP, training)
    assert a == b
    assert a["streamed"] == 0


@pytest.mark.parametrize("h,H,hd,F,S", SHAPES)
@pytest.mark.parametrize("D", [1, 2, 4])
def test_tsp_activations_are_the_layer_buffers(h, H, hd, F, S, D):
    # input and output rows plus exactly the workspace tsp_layer_forward asks for
    d = tsp.make_dims(h, H, hd, F)
    n = S // D
    m = tsp.memory_footprint(S, d, D, 2, tsp.MEM_TSP)
    assert m["activations"] == 2 * _round256(n * h * 2) + tsp.workspace_size(n, d, D, tsp.WS_LAYER)
    assert m["kv"] == 2 * S * h * 2
    assert m["train_state"] == 0 and m["grads"] == 0
    assert m["total"] == sum(m[f] for f in FIELDS[:-1])


def test_7b_parameter_count_closed_form():
    # FFN = 4h gives 12 h^2 parameters per layer (Q, K, V, O: 4 h^2; W1, W2: 8 h^2)
    h, L, D = 4096, 32, 8
    d = tsp.make_dims(h, 32, 128, 4 * h)
    m = tsp.memory_footprint(131072, d, D, L, tsp.MEM_TSP, True)
    assert m["weights"] == L * 12 * h * h // D * 2
    assert m["streamed"] == (D - 1) * 12 * h * h // D * 2
    # bf16 grads, fp32 master, Adam m, v: 14 bytes per own parameter, plus the
    # layer inputs of the 16384 local tokens
    assert m["train_state"] == L * 12 * h * h // D * 14 + L * (131072 // D) * h * 2
    assert m["grads"] == 12 * h * h * 4


@pytest.mark.parametrize("D", [2, 4, 8])
def test_scheme_relations(D):
    h, L, S = 4096, 32, 131072
    d = tsp.make_dims(h, 32, 128, 16384)
    a = tsp.memory_footprint(S, d, D, L, tsp.MEM_TSP, True)
    b = tsp.memory_footprint(S, d, D, L, tsp.MEM_TP, True)
    assert a["weights"] == b["weights"]  # both hold 1/D of the parameters
    assert b["streamed"] == 0
    assert a["kv"] == D * b["kv"]  # gathered K/V of all heads vs own heads
    assert a["grads"] == D * b["grads"]  # contributions to every shard vs own shard
    # the kept layer inputs: S/D tokens vs S tokens; the parameter part is equal
    assert b["train_state"] - a["train_state"] == L * (S - S // D) * h * 2
    # the page's comparison at 128K: TSP needs less than plain TP
    assert a["total"] < b["total"]
    assert a["activations"] < b["activations"]


def test_tsp_total_falls_with_D():
    d = tsp.make_dims(4096, 32, 128, 16384)
    tot = [tsp.memory_footprint(131072, d, D, 32, tsp.MEM_TSP, True)["total"] for D in (1, 2, 4, 8)]
    assert all(x > y for x, y in zip(tot, tot[1:]))


def test_zero_layers_hold_nothing():
    d = tsp.make_dims(256, 4, 64, 1024)
    for sch in (tsp.MEM_TSP, tsp.MEM_TP):
        assert tsp.memory_footprint(2048, d, 4, 0, sch, True)["total"] == 0


@pytest.mark.parametrize("args,status", [
    ((2048, 4, 2, 7, 0), tsp.TSP_ERR_INVALID_ARG),  # unknown scheme
    ((2048, 0, 2, 0, 0), tsp.TSP_ERR_INVALID_ARG),  # D out of range
    ((2048, 17, 2, 0, 0), tsp.TSP_ERR_INVALID_ARG),
    ((2048, 4, -1, 0, 0), tsp.TSP_ERR_INVALID_ARG),  # negative layer count
    ((2047, 4, 2, 0, 0), tsp.TSP_ERR_SHAPE),  # S not a multiple of 2D
    ((0, 4, 2, 0, 0), tsp.TSP_ERR_SHAPE),
    ((2048, 3, 2, 0, 0), tsp.TSP_ERR_SHAPE),  # heads not divisible by D
])
def test_rejects(args, status):
    import ctypes
    S, D, L, scheme, training = args
    d = tsp.make_dims(256, 4, 64, 1024)
    m = tsp.Memory()
    got = tsp.lib().tsp_memory_footprint(S, ctypes.byref(d), D, L, scheme, training, ctypes.byref(m))
    assert got == status
    assert tsp.lib().tsp_memory_footprint(2048, ctypes.byref(d), 4, 2, 0, 0, None) == tsp.TSP_ERR_INVALID_ARG
    assert tsp.lib().tsp_memory_footprint(2048, None, 4, 2, 0, 0, ctypes.byref(m)) == tsp.TSP_ERR_INVALID_ARG
