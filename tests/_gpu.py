"""Helpers shared by the GPU parity tests: move seeded inputs to the device,
build the positives, and compare against the oracle with the stated
tolerances."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import workloads as wl

DEV = "cuda:0"
# bf16 inputs, fp32 accumulation: |err| <= 1e-2 * sum|x_i w_i| + 1e-5;
# fp32 configs: 1e-5 relative to sum|x_i w_i|.
TOL_BF16 = (1e-2, 1e-5)
TOL_F32 = (1e-5, 1e-9)
U = 2.0 ** -8   # one bf16 rounding (relative, round-to-nearest: 2^-9; kept 2x loose)
E32 = 2.0 ** -24


def dev_array(a: np.ndarray, dtype: str) -> torch.Tensor:
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


class Dev:
    """Device copies of one workload."""

    def __init__(self, inp: wl.Inputs):
        c = inp.cfg
        self.inp = inp
        self.X = dev_array(inp.X, c.dtype)
        self.Wh = dev_array(inp.Wh, c.dtype)
        self.W = dev_array(inp.W, c.dtype)
        self.idx = torch.from_numpy(inp.idx).to(DEV)
        self.row_ptr = torch.from_numpy(inp.row_ptr).to(DEV)
        self.labels = torch.from_numpy(inp.labels).to(DEV)
        self.tdtype = torch.bfloat16 if c.dtype == "bf16" else torch.float32

    def bce(self, offset, s, loss=True):
        from sparse_output_layer_amd import haste as H
        lt = torch.zeros(1, dtype=torch.float32, device=DEV) if loss else None
        return H.Bce(self.row_ptr, self.labels, label_offset=offset, grad_scale=s, loss=lt)


def check(name, got, ref, absref, dtype, nterms=None):
    """Element-wise parity: the stated tolerance, plus (bf16) a bound derived
    from the arithmetic: one bf16 rounding of each product's dz or of the
    output, plus fp32 accumulation of nterms terms."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    absref = np.asarray(absref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    err = np.abs(got - ref)
    rel, ab = TOL_BF16 if dtype == "bf16" else TOL_F32
    tol = rel * absref + ab
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{name}: {bad.sum()} / {err.size} outside tolerance; worst at {i}: "
                             f"got {got[i]!r} ref {ref[i]!r} tol {tol[i]!r}")
    if dtype == "bf16" and nterms is not None:
        derived = (U + nterms * E32) * absref + U * np.abs(ref) + 1e-7
        bad = err > derived
        if bad.any():
            i = np.unravel_index(np.argmax(err - derived), err.shape)
            raise AssertionError(f"{name}: {bad.sum()} / {err.size} outside the derived bound; "
                                 f"worst at {i}: got {got[i]!r} ref {ref[i]!r} "
                                 f"bound {derived[i]!r}")
    return float(err.max()) if err.size else 0.0


def check_loss(name, got, ref, dtype):
    rel = 1e-4 if dtype == "bf16" else 1e-5
    assert abs(got - ref) <= rel * abs(ref) + 1e-6, f"{name}: got {got} ref {ref}"
