"""GPU tests of the calls that wait for their weight shards inside the kernels
(tsp_attn_project_arrival, tsp_attn_out_arrival, tsp_mlp_forward_arrival) and
of the simulated arrival that feeds them (tsp_simulate_arrival).

In TSP the shards of a layer reach a device one after another (zubnet.ai,
"Zyphra TSP folds TP+SP onto one GPU axis", para. 2).  These calls are the
all-shard GEMMs with a per-tile wait on an arrival counter, so the checks are
bit-identity with the all-shard calls on resident weights:

  * every shard arrived before the launch (counter preset), for ring starts 0
    and D-1, with a counter base that wraps modulo 2^32;
  * shards delivered while the call runs: the shard buffers start as NaN, and
    a one-workgroup producer on a side stream, launched just before the call,
    copies the shards in ring order, 150 us apart, raising the counter after
    each; any read before arrival would leave NaN or another value in the
    result;
  * a wait that gives up: the counter is never raised and the poll budget is
    tiny, so every wait gives up, sets the status word and the call finishes
    on the (resident) buffers;
  * the 7B shapes at S = 16384 and 131072, D = 8, rank 0 (the two benchmark
    workloads), all shards arrived.
"""
import pytest
import torch

from folded_tensor_sequence_tsp_amd import synth, tsp
from parity import bf16_nan, gpu, require_gpu, say

pytestmark = gpu
DEV = "cuda"


def _rnd(shape, seed, std=1.0):
    return synth.randn_bf16(shape, 9_700_000 + seed, std, DEV)


def _words(value=0):
    """(counter, status) as int32 device words."""
    c = torch.full((4,), value, dtype=torch.int32, device=DEV)
    return c, torch.zeros(4, dtype=torch.int32, device=DEV)


def _u32(v):
    return v & 0xFFFFFFFF


def _preset(base, D):
    counter, status = _words(0)
    counter[0] = _u32(base + D) - (1 << 32) if _u32(base + D) >= 1 << 31 else _u32(base + D)
    return counter, status


class Case:
    """A small layer: x, shard weights, QKV outputs, attention output parts."""

    def __init__(self, h, H, hd, D, S, r, seed):
        self.plan, _, _ = tsp.zigzag_plan(S, D, r)
        self.D, self.h = D, h
        n = self.plan.n_local
        Hs, F = H // D, 4 * h
        self.Fs = F // D
        self.dims = tsp.make_dims(h, H, hd, F)
        self.x = _rnd((n, h), seed)
        self.wqkv = [_rnd((3 * Hs * hd, h), seed + 10 + d, 0.02) for d in range(D)]
        self.wo = [_rnd((h, Hs * hd), seed + 30 + d, 0.02) for d in range(D)]
        # W1_d and W2_d of one pair share a buffer, so one copy delivers a pair
        self.pairs = [torch.cat([_rnd((self.Fs, h), seed + 50 + d, 0.02).flatten(),
                                 _rnd((h, self.Fs), seed + 70 + d, 0.02).flatten()]) for d in range(D)]
        self.a = _rnd((n, h), seed + 1)
        self.lo = (_rnd((n, h), seed + 2) * 2 ** -9).to(torch.bfloat16)
        self.kv0 = _rnd((S, h), seed + 3), _rnd((S, h), seed + 4)
        self.ws = tsp.alloc_workspace(n, self.dims, D, tsp.WS_MLP)

    def w1w2(self, pairs):
        n1 = self.Fs * self.h
        return ([p[:n1].view(self.Fs, self.h) for p in pairs], [p[n1:].view(self.h, self.Fs) for p in pairs])

    # reference: the all-shard calls on the resident weights
    def project_ref(self):
        n, S = self.plan.n_local, self.plan.seq_len
        q, k, v = bf16_nan((n, self.h), DEV), self.kv0[0].clone(), self.kv0[1].clone()
        tsp.attn_project(self.plan, self.dims, self.x, self.wqkv, k, v, q)
        return q, k, v

    def out_ref(self, start, lo):
        out = bf16_nan(self.x.shape, DEV)
        tsp.attn_out(self.dims, self.D, start, self.a, self.wo, self.x, out, attn_lo=self.lo if lo else None)
        return out

    def mlp_ref(self, start):
        w1, w2 = self.w1w2(self.pairs)
        y = bf16_nan(self.x.shape, DEV)
        tsp.mlp_forward(self.dims, self.D, start, self.x, w1, w2, self.x, y, self.ws)
        return y

    # the arrival calls, on the given shard buffers
    def project_arr(self, wqkv, start, arr, stream=None):
        n = self.plan.n_local
        q, k, v = bf16_nan((n, self.h), DEV), self.kv0[0].clone(), self.kv0[1].clone()
        tsp.attn_project_arrival(self.plan, self.dims, start, self.x, wqkv, k, v, q, arr, stream=stream)
        return q, k, v

    def out_arr(self, wo, start, lo, arr, stream=None):
        out = bf16_nan(self.x.shape, DEV)
        tsp.attn_out_arrival(self.dims, self.D, start, self.a, wo, self.x, out, arr,
                             attn_lo=self.lo if lo else None, stream=stream)
        return out

    def mlp_arr(self, pairs, start, arr, stream=None):
        w1, w2 = self.w1w2(pairs)
        y = bf16_nan(self.x.shape, DEV)
        tsp.mlp_forward_arrival(self.dims, self.D, start, self.x, w1, w2, self.x, y, self.ws, arr, stream=stream)
        return y


SHAPES = [(256, 4, 64, 4, 2048, 1), (512, 4, 128, 2, 1288, 0), (256, 4, 64, 1, 300, 0)]


@pytest.mark.parametrize("h,H,hd,D,S,r", SHAPES)
@pytest.mark.parametrize("base", [0, 7, 0xFFFFFFFE])
def test_arrived_before_launch_bit_identical(h, H, hd, D, S, r, base):
    require_gpu()
    c = Case(h, H, hd, D, S, r, 100)
    for start in sorted({0, D - 1}):
        counter, status = _preset(base, D)
        arr = tsp.make_arrival(counter, base, status)
        say(f"arrival preset h={h} hd={hd} D={D} S={S} r={r} base={base:#x} start={start}")
        got, want = c.project_arr(c.wqkv, start, arr), c.project_ref()
        for g_, w_ in zip(got, want):
            assert torch.equal(g_, w_)
        for lo in (False, True):
            assert torch.equal(c.out_arr(c.wo, start, lo, arr), c.out_ref(start, lo))
        assert torch.equal(c.mlp_arr(c.pairs, start, arr), c.mlp_ref(start))
        torch.cuda.synchronize()
        assert int(status[0]) == 0


def _deliver(c, kind, start, delay_us=150):
    """Deliver the shards in ring order from a side stream into NaN shard
    buffers, with the arrival call launched right after the producer; returns
    (result, status)."""
    D = c.D
    src = {"qkv": c.wqkv, "out": c.wo, "mlp": c.pairs}[kind]
    dst = [torch.full_like(t, float("nan")) for t in src]
    counter, status = _words(0)
    base = 1000
    counter[0] = base
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    side.wait_stream(main)  # the NaN fills and the counter are in place first
    arr = tsp.make_arrival(counter, base, status)
    # the producer goes first: streams may share a hardware queue (more streams
    # than queues), and a producer queued behind the waiting consumer could not
    # run until the consumer's waits gave up
    ring = [(start + p) % D for p in range(D)]
    tsp.simulate_arrival([src[d] for d in ring], [dst[d] for d in ring], counter, base, delay_us, stream=side)
    if kind == "qkv":
        res = c.project_arr(dst, start, arr)
    elif kind == "out":
        res = c.out_arr(dst, start, True, arr)
    else:
        res = c.mlp_arr(dst, start, arr)
    torch.cuda.synchronize()
    for d in range(D):
        assert torch.equal(dst[d], src[d])
    return res, status


@pytest.mark.parametrize("h,H,hd,D,S,r", SHAPES[:2])
@pytest.mark.parametrize("kind", ["qkv", "out", "mlp"])
def test_delivered_during_the_call(h, H, hd, D, S, r, kind):
    require_gpu()
    c = Case(h, H, hd, D, S, r, 200)
    start = D - 1
    say(f"arrival during the call kind={kind} h={h} hd={hd} D={D} S={S} start={start}")
    res, status = _deliver(c, kind, start)
    assert int(status[0]) == 0
    if kind == "qkv":
        for g_, w_ in zip(res, c.project_ref()):
            assert torch.equal(g_, w_)
    elif kind == "out":
        assert torch.equal(res, c.out_ref(start, True))
    else:
        assert torch.equal(res, c.mlp_ref(start))


@pytest.mark.parametrize("kind", ["qkv", "out", "mlp"])
def test_wait_gives_up(kind):
    require_gpu()
    c = Case(256, 4, 64, 4, 2048, 1, 300)
    counter, status = _words(5)
    arr = tsp.make_arrival(counter, 5, status, spin_limit=16)  # nothing ever arrives
    say(f"arrival never comes kind={kind}")
    if kind == "qkv":
        got, want = c.project_arr(c.wqkv, 0, arr), c.project_ref()
    elif kind == "out":
        got, want = (c.out_arr(c.wo, 0, True, arr),), (c.out_ref(0, True),)
    else:
        got, want = (c.mlp_arr(c.pairs, 0, arr),), (c.mlp_ref(0),)
    torch.cuda.synchronize()
    assert int(status[0]) == 1
    for g_, w_ in zip(got, want):  # the shard buffers were resident all along
        assert torch.equal(g_, w_)


@pytest.mark.parametrize("S", [16384, 131072])
def test_7b_arrived_bit_identical(S):
    require_gpu()
    d = synth.DIMS_7B
    D = 8
    plan, _, _ = tsp.zigzag_plan(S, D, 0)
    n, h = plan.n_local, d.hidden
    dims = tsp.make_dims(h, d.n_heads, d.head_dim, d.ffn)
    lw = synth.layer_weights(41, d, D, device=DEV)
    x = synth.activations(42, n, h, device=DEV)
    a = _rnd((n, h), 43)
    lo = (_rnd((n, h), 44) * 2 ** -9).to(torch.bfloat16)
    counter, status = _preset(0, D)
    arr = tsp.make_arrival(counter, 0, status)
    say(f"arrival 7B S={S} D=8 qkv")
    k0, v0 = torch.zeros(S, h, dtype=torch.bfloat16, device=DEV), torch.zeros(S, h, dtype=torch.bfloat16, device=DEV)
    q1, k1, v1 = bf16_nan((n, h), DEV), k0.clone(), v0.clone()
    q2, k2, v2 = bf16_nan((n, h), DEV), k0.clone(), v0.clone()
    tsp.attn_project(plan, dims, x, lw.wqkv, k1, v1, q1)
    tsp.attn_project_arrival(plan, dims, 0, x, lw.wqkv, k2, v2, q2, arr)
    assert torch.equal(q1, q2) and torch.equal(k1, k2) and torch.equal(v1, v2)
    say(f"arrival 7B S={S} D=8 out")
    o1, o2 = bf16_nan((n, h), DEV), bf16_nan((n, h), DEV)
    tsp.attn_out(dims, D, 0, a, lw.wo, x, o1, attn_lo=lo)
    tsp.attn_out_arrival(dims, D, 0, a, lw.wo, x, o2, arr, attn_lo=lo)
    assert torch.equal(o1, o2)
    say(f"arrival 7B S={S} D=8 mlp")
    ws = tsp.alloc_workspace(n, dims, D, tsp.WS_MLP, device=DEV)
    y1, y2 = bf16_nan((n, h), DEV), bf16_nan((n, h), DEV)
    tsp.mlp_forward(dims, D, 0, x, lw.w1, lw.w2, x, y1, ws)
    tsp.mlp_forward_arrival(dims, D, 0, x, lw.w1, lw.w2, x, y2, ws, arr)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert int(status[0]) == 0
