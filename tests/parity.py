"""Shared helpers of the GPU parity tests.

Tolerance (per element, against the fp64 oracle):
    |gpu - oracle| <= 1e-2 + 2e-2 * |oracle|
and over the compared set ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3.
The GPU path rounds its inputs' products into bf16 at the stated stage
boundaries (Q/K/V, attention output, h1, GELU output, layer output); the
per-element bound leaves room for those roundings, the relative RMS bound is the
binding check.
"""
import sys

import pytest
import torch

ATOL = 1e-2
RTOL = 2e-2
REL_RMS = 5e-3

gpu = pytest.mark.gpu


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from folded_tensor_sequence_tsp_amd import tsp
    tsp.lib()  # raises if the library is missing: there is no fallback


def say(msg):
    """Name the case on stderr (flushed) before a GPU step."""
    sys.stderr.write(f"[case] {msg}\n")
    sys.stderr.flush()


def check(got: torch.Tensor, ref: torch.Tensor, name: str, rel_rms: float = REL_RMS):
    g = got.detach().to("cpu").to(torch.float64)
    o = ref.detach().to("cpu").to(torch.float64)
    assert g.shape == o.shape, f"{name}: shape {tuple(g.shape)} vs {tuple(o.shape)}"
    assert torch.isfinite(g).all(), f"{name}: non-finite GPU values"
    err = (g - o).abs()
    bound = ATOL + RTOL * o.abs()
    bad = err > bound
    rr = ((g - o).norm() / o.norm().clamp_min(1e-300)).item()
    stats = dict(max_abs=err.max().item(), rel_rms=rr, n=g.numel())
    assert not bool(bad.any()), (f"{name}: {int(bad.sum())}/{g.numel()} elements outside "
                                 f"{ATOL} + {RTOL}|o|; worst err {err.max().item():.3e} {stats}")
    assert rr <= rel_rms, f"{name}: relative RMS {rr:.3e} > {rel_rms}"
    return stats


def bf16_nan(shape, device):
    """A bf16 tensor filled with quiet NaNs (0x7fc0) to expose unwritten elements."""
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
