"""Shared helpers of the GPU parity tests.

Tolerance (per element, against the fp64 oracle):
    |gpu - oracle| <= 1e-2 + 2e-2 * |oracle|
and over the compared set ||gpu - oracle||_2 / ||oracle||_2 <= 5e-3.
The GPU path rounds its inputs' products into bf16 at the stated stage
boundaries (Q/K/V, attention output, h1, GELU output, layer output); the
per-element bound leaves room for those roundings, the relative RMS bound is the
binding check.

Every check appends a line to ``TALLY``; the test session prints the lines in
its terminal summary (tests/conftest.py), so a run records, for each compared
set, its worst error, its relative RMS and how many elements a derived rounding
bound had to admit beyond the per-element bound above.
"""
import sys

import pytest
import torch

ATOL = 1e-2
RTOL = 2e-2
REL_RMS = 5e-3

gpu = pytest.mark.gpu

# (name, elements compared, elements beyond ATOL + RTOL|o|, max abs error, relative RMS, kind)
TALLY = []


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    from folded_tensor_sequence_tsp_amd import tsp
    tsp.lib()  # raises if the library is missing: there is no fallback


def say(msg):
    """Name the case on stderr (flushed) before a GPU step."""
    sys.stderr.write(f"[case] {msg}\n")
    sys.stderr.flush()


def _prep(got, ref, name):
    g = got.detach().to("cpu").to(torch.float64)
    o = ref.detach().to("cpu").to(torch.float64)
    assert g.shape == o.shape, f"{name}: shape {tuple(g.shape)} vs {tuple(o.shape)}"
    assert torch.isfinite(g).all(), f"{name}: non-finite GPU values"
    return g, o


def _rel_rms(g, o):
    return ((g - o).norm() / o.norm().clamp_min(1e-300)).item()


def check(got: torch.Tensor, ref: torch.Tensor, name: str, rel_rms: float = REL_RMS, scale: float = 1.0):
    """Per element |gpu - oracle| <= ATOL*scale + RTOL|oracle| and relative RMS.

    ``scale`` is the size of the output relative to its unit-scale size when
    the inputs are not unit-scale: the absolute term of the bound is stated for
    unit-scale activations, so it is taken in units of the output's scale (the
    relative term and the RMS bound do not depend on it)."""
    g, o = _prep(got, ref, name)
    err = (g - o).abs()
    bound = ATOL * scale + RTOL * o.abs()
    bad = err > bound
    rr = _rel_rms(g, o)
    stats = dict(max_abs=err.max().item(), rel_rms=rr, n=g.numel())
    TALLY.append((name, g.numel(), int(bad.sum()), stats["max_abs"], rr, "bound"))
    assert not bool(bad.any()), (f"{name}: {int(bad.sum())}/{g.numel()} elements outside "
                                 f"{ATOL * scale:g} + {RTOL}|o|; worst err {err.max().item():.3e} {stats}")
    assert rr <= rel_rms, f"{name}: relative RMS {rr:.3e} > {rel_rms}"
    return stats


def check_rms(got: torch.Tensor, ref: torch.Tensor, name: str, rel_rms: float = REL_RMS, scale: float = 1.0):
    """Relative RMS only, with the per-element figures reported, not asserted:
    used against the oracle that keeps the projection outputs unrounded, whose
    difference from the GPU path includes the bf16 rounding of Q, K and V that
    the model itself performs."""
    g, o = _prep(got, ref, name)
    err = (g - o).abs()
    beyond = int((err > ATOL * scale + RTOL * o.abs()).sum())
    rr = _rel_rms(g, o)
    TALLY.append((name, g.numel(), beyond, err.max().item(), rr, "rms"))
    say(f"{name}: max err {err.max().item():.3e}, rel rms {rr:.3e}, {beyond}/{g.numel()} beyond the element bound")
    assert rr <= rel_rms, f"{name}: relative RMS {rr:.3e} > {rel_rms}"
    return dict(max_abs=err.max().item(), rel_rms=rr, beyond=beyond, n=g.numel())


def check_within(got: torch.Tensor, ref: torch.Tensor, derived: torch.Tensor, name: str,
                 rel_rms: float = REL_RMS):
    """Per element |gpu - oracle| <= max(ATOL + RTOL|oracle|, derived), and
    relative RMS.  ``derived`` is a rounding bound worked out from the
    operands of the products (bf16 rounding of one factor of a long dot
    product); the count of elements that only it admits is recorded."""
    g, o = _prep(got, ref, name)
    err = (g - o).abs()
    ns = ATOL + RTOL * o.abs()
    lim = torch.maximum(ns, derived.to(torch.float64))
    bad = err > lim
    need = int(((err > ns) & ~bad).sum())
    rr = _rel_rms(g, o)
    TALLY.append((name, g.numel(), need, err.max().item(), rr, "derived"))
    assert not bool(bad.any()), (f"{name}: {int(bad.sum())}/{g.numel()} elements beyond max(element bound, "
                                 f"derived bound); worst excess {float((err - lim).max()):.3e}")
    assert rr <= rel_rms, f"{name}: relative RMS {rr:.3e} > {rel_rms}"
    return dict(max_abs=err.max().item(), rel_rms=rr, derived_only=need, n=g.numel())


def bf16_nan(shape, device):
    """A bf16 tensor filled with quiet NaNs (0x7fc0) to expose unwritten elements."""
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=device)
