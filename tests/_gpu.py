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
    """Reading C16: relative 1e-4 with bf16 inputs, 1e-6 with fp32 ones."""
    rel = 1e-4 if dtype == "bf16" else 1e-6
    err = abs(got - ref)
    print(f"  {name}: relative error {err / max(abs(ref), 1e-30):.2e} (bound {rel:.0e})", flush=True)
    assert err <= rel * abs(ref) + 1e-6, f"{name}: got {got} ref {ref}"


def rank_tol(zabs, nterms):
    """Reading C17: the kernels' logit of a label is an fp32 sum of nterms
    products of exact bf16 inputs (fp32 inputs: each product rounded once
    more), so it lies within (nterms + 1) * 2^-24 * sum|x w| of the exact
    value; twice that separates two logits whose order both sides must
    agree on."""
    return 2.0 * (nterms + 1) * 2.0 ** -24 * np.asarray(zabs, dtype=np.float64)


def check_topk_lists(name, got_v, got_i, ov, oi, otol, zfun, K, N, id0=0, oamb=None):
    """Per-row top-K against the oracle's top-(K+1) lists ov / oi (value
    descending, ties to the smaller id) whose entries carry rank tolerances
    otol (rank_tol of each listed label; reading C17), with zfun(b, id) giving
    (oracle logit, rank tolerance) of any label.  Every returned value must be
    its own id's logit and the oracle's k-th largest within tolerance.  A row
    is tie-free when every gap between consecutive entries of its oracle
    top-(K+1) exceeds the two entries' tolerances: its K ids must equal the
    oracle's.  In other rows an id is compared where the gaps to both
    neighbours exceed their tolerances.  oamb (optional, rows x (K+1) bool):
    entries whose own id the oracle could not fix (the two-stage form's bucket
    representative, a near-tie inside its bucket); they are not compared by
    id.  Returns (tie-free rows, positions compared by id)."""
    got_v = np.asarray(got_v, dtype=np.float64)
    got_i = np.asarray(got_i, dtype=np.int64)
    n = min(K, N)
    rows_ok = positions = 0
    for b in range(got_v.shape[0]):
        ids = got_i[b]
        assert np.all(ids[:n] >= 0) and np.all(ids[n:] == -1), f"{name}: row {b} ids {ids}"
        assert np.all(np.isneginf(got_v[b, n:])), f"{name}: row {b} padding {got_v[b]}"
        li = ids[:n]
        assert len(set(li.tolist())) == li.size, f"{name}: row {b} repeats an id: {li}"
        assert np.all((li >= id0) & (li < id0 + N)), f"{name}: row {b} id out of range: {li}"
        m = min(n + 1, ov.shape[1])
        valid = oi[b, :m] >= 0
        tk = np.where(valid, otol[b, :m], 0.0)
        amb = np.zeros(m, bool) if oamb is None else np.asarray(oamb[b, :m], bool)
        gaps_ok = [bool(ov[b, k] - ov[b, k + 1] > tk[k] + tk[k + 1]) if valid[k + 1] else True
                   for k in range(m - 1)]
        tie_free = all(gaps_ok[:n]) and not amb[:n].any()
        for k in range(n):
            zk, tz = zfun(b, int(ids[k]))
            assert abs(got_v[b, k] - zk) <= tz, \
                f"{name}: row {b} pos {k}: value {got_v[b, k]} vs its logit {zk} (tol {tz})"
            assert abs(got_v[b, k] - ov[b, k]) <= tz + tk[k], \
                f"{name}: row {b} pos {k}: value {got_v[b, k]} vs k-th largest {ov[b, k]} (tol {tz + tk[k]})"
            if k > 0:
                assert got_v[b, k] <= got_v[b, k - 1], f"{name}: row {b} not descending"
            sep_hi = k == 0 or gaps_ok[k - 1]
            sep_lo = k + 1 >= m or gaps_ok[k]
            if sep_hi and sep_lo and not amb[k]:
                positions += 1
                assert ids[k] == oi[b, k], f"{name}: row {b} pos {k}: id {ids[k]} vs oracle {oi[b, k]}"
        if tie_free:
            rows_ok += 1
            assert np.array_equal(ids[:n], oi[b, :n]), f"{name}: tie-free row {b}: {ids[:n]} vs {oi[b, :n]}"
    return rows_ok, positions


def topk_tol(zabs_rowmax, dtype):
    rel, ab = TOL_BF16 if dtype == "bf16" else TOL_F32
    return rel * np.asarray(zabs_rowmax, dtype=np.float64) + ab


def check_topk(name, got_v, got_i, z, zabs, K, dtype, id0=0, nterms=None):
    """check_topk_lists with the oracle's full logits z / zabs (rows x N,
    column c has id id0 + c); nterms: products per logit (an int, or an
    array over the columns)."""
    rows, N = z.shape
    nt = np.broadcast_to(np.asarray(nterms, dtype=np.float64), (N,)) if N else np.zeros(0)
    rt = rank_tol(zabs, nt[None, :]) if N else np.zeros((rows, 0))
    if N > 0:
        ov, oi = oracle.topk(z, min(K + 1, N), id_offset=id0)
        otol = np.take_along_axis(rt, np.maximum(oi - id0, 0), axis=1)
    else:
        ov, oi, otol = np.zeros((rows, 0)), np.zeros((rows, 0), np.int64), np.zeros((rows, 0))
    res = check_topk_lists(name, got_v, got_i, ov, oi, otol,
                           lambda b, i: (z[b, i - id0], rt[b, i - id0]), K, N, id0)
    print(f"  {name}: tie-free rows {res[0]} of {rows}, positions compared by id {res[1]}", flush=True)
    return res
