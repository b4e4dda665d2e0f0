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


def check_topk_lists(name, got_v, got_i, ov, oi, tol, zfun, K, N, id0=0):
    """Per-row top-K against the oracle's top-(K+1) lists ov / oi (value
    descending, ties to the smaller id), with per-row logit tolerance tol[b]
    and zfun(b, id) giving the oracle logit of one label.  The kernels rank
    fp32 logits, the oracle fp64 ones, so the order is compared where the
    oracle's neighbours are further apart than twice the tolerance;
    everywhere the returned value must be the k-th largest within tolerance
    and the returned id's own logit."""
    got_v = np.asarray(got_v, dtype=np.float64)
    got_i = np.asarray(got_i, dtype=np.int64)
    n = min(K, N)
    for b in range(got_v.shape[0]):
        ids = got_i[b]
        assert np.all(ids[:n] >= 0) and np.all(ids[n:] == -1), f"{name}: row {b} ids {ids}"
        assert np.all(np.isneginf(got_v[b, n:])), f"{name}: row {b} padding {got_v[b]}"
        li = ids[:n]
        assert len(set(li.tolist())) == li.size, f"{name}: row {b} repeats an id: {li}"
        assert np.all((li >= id0) & (li < id0 + N)), f"{name}: row {b} id out of range: {li}"
        for k in range(n):
            zk = zfun(b, int(ids[k]))
            assert abs(got_v[b, k] - zk) <= tol[b], \
                f"{name}: row {b} pos {k}: value {got_v[b, k]} vs its logit {zk} (tol {tol[b]})"
            assert abs(got_v[b, k] - ov[b, k]) <= tol[b], \
                f"{name}: row {b} pos {k}: value {got_v[b, k]} vs k-th largest {ov[b, k]} (tol {tol[b]})"
            if k > 0:
                assert got_v[b, k] <= got_v[b, k - 1], f"{name}: row {b} not descending"
            sep_hi = k == 0 or ov[b, k - 1] - ov[b, k] > 2 * tol[b]
            sep_lo = k + 1 >= n or k + 1 >= ov.shape[1] or ov[b, k] - ov[b, k + 1] > 2 * tol[b]
            if sep_hi and sep_lo:
                assert ids[k] == oi[b, k], f"{name}: row {b} pos {k}: id {ids[k]} vs oracle {oi[b, k]}"


def topk_tol(zabs_rowmax, dtype):
    rel, ab = TOL_BF16 if dtype == "bf16" else TOL_F32
    return rel * np.asarray(zabs_rowmax, dtype=np.float64) + ab


def check_topk(name, got_v, got_i, z, zabs, K, dtype, id0=0):
    """check_topk_lists with the oracle's full logits z / zabs (rows x N,
    column c has id id0 + c)."""
    rows, N = z.shape
    ov, oi = oracle.topk(z, min(K + 1, N), id_offset=id0) if N > 0 else (np.zeros((rows, 0)), None)
    tol = topk_tol(zabs.max(axis=1) if N else np.zeros(rows), dtype)
    check_topk_lists(name, got_v, got_i, ov, oi, tol, lambda b, i: z[b, i - id0], K, N, id0)
