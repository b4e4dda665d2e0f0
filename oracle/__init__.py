"""fp64 CPU oracle for the group-shared fixed fan-in output layer.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the
bench's CPU-baseline leg, never by the product package.  It shares no code
with the HIP library.  The arithmetic lives in ``haste_oracle.c`` (plain C,
fp64, OpenMP over independent outputs); this module builds it with gcc and
exposes it through ctypes, plus a ``step`` helper that composes the pieces
into one full training step (head + tail, sigmoid-BCE, all gradients).

Definitions follow the HASTE summary page (gist.science, "HASTE: Hardware-Aware
Dynamic Sparse Training for Large Output Spaces"), section "Method": item 1
(group-shared fan-in: one index set per group, own weights per label) and
item 2 (dense head classifier for the frequent labels).  The loss and the
gradient formulas are not printed on the pages; they are the exact sigmoid
binary cross-entropy and its exact gradients (readings listed in the design doc).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "haste_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

_d = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32 = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64 = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_vp = ctypes.c_void_p


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (host only)."""
    if force or not os.path.exists(_LIB_PATH) or \
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-std=c11", "-Wall", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or \
                os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_threads.restype = ctypes.c_int
        L.oracle_set_threads.argtypes = [ctypes.c_int]
        L.oracle_layout.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_int, _i64]
        L.oracle_tail_logits.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int, ctypes.c_int, _d, _i32, _d,
                                         _i32, ctypes.c_int, ctypes.c_int64,
                                         ctypes.c_int64, _d, _vp]
        L.oracle_head_logits.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         _d, _d, _i32, ctypes.c_int, ctypes.c_int,
                                         ctypes.c_int, _d, _vp]
        L.oracle_positive_mask.argtypes = [_i32, _i32, _i32, ctypes.c_int,
                                           ctypes.c_int64, ctypes.c_int64, _d]
        L.oracle_bce.argtypes = [ctypes.c_int64, _d, _d, ctypes.c_double, _vp, _vp]
        L.oracle_tail_dW.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                     ctypes.c_int, ctypes.c_int, _d, _i32, _d,
                                     ctypes.c_int64, ctypes.c_int64, _d, _vp]
        L.oracle_tail_dX.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_int,
                                     ctypes.c_int, _i32, _d, _d, ctypes.c_int, _d, _vp]
        L.oracle_head_dW.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                     _d, _d, _d, _vp]
        L.oracle_head_dX.argtypes = [ctypes.c_int, ctypes.c_int, _d, _d,
                                     ctypes.c_int, _d, _vp]
        L.oracle_topk.argtypes = [ctypes.c_int, ctypes.c_int64, _d, _vp,
                                  ctypes.c_int64, ctypes.c_int, _d, _i64]
        L.oracle_group_positives.restype = ctypes.c_int64
        L.oracle_group_positives.argtypes = [ctypes.c_int, _i32, _i32, ctypes.c_int64,
                                             ctypes.c_int64, ctypes.c_int, _i32, _i32]
        L.oracle_tail_step.restype = ctypes.c_double
        L.oracle_tail_step.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int, ctypes.c_int, _d, _i32, _d,
                                       _i32, _i32, ctypes.c_int64, ctypes.c_double,
                                       ctypes.c_int64, ctypes.c_int64, _vp, _vp]
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def threads() -> int:
    return lib().oracle_threads()


def set_threads(n: int) -> None:
    lib().oracle_set_threads(int(n))


# --------------------------------------------------------------- primitives
def layout(L: int, G: int, F: int) -> dict:
    out = np.zeros(4, np.int64)
    lib().oracle_layout(L, G, F, out)
    return {"n_groups": int(out[0]), "index_count": int(out[1]),
            "weight_rows": int(out[2]), "last_group_live": int(out[3])}


def n_live(L: int, G: int, g0: int, g1: int) -> int:
    return min(g1 * G, L) - g0 * G


def tail_logits(X, idx, Wt, L, G, rows=None, g0=0, g1=None, want_abs=True):
    X, idx, Wt = _c(X, np.float64), _c(idx, np.int32), _c(Wt, np.float64)
    B, D = X.shape
    F = idx.shape[1]
    ng = (L + G - 1) // G
    g1 = ng if g1 is None else g1
    rows = np.arange(B, dtype=np.int32) if rows is None else _c(rows, np.int32)
    nc = n_live(L, G, g0, g1)
    Z = np.empty((rows.size, nc))
    Za = np.empty((rows.size, nc)) if want_abs else None
    lib().oracle_tail_logits(B, D, L, G, F, X, idx, Wt, rows, rows.size, g0, g1,
                             Z, _ptr(Za))
    return Z, Za


def head_logits(X, Wh, rows=None, h0=0, h1=None, want_abs=True):
    X, Wh = _c(X, np.float64), _c(Wh, np.float64)
    B, D = X.shape
    H = Wh.shape[0]
    h1 = H if h1 is None else h1
    rows = np.arange(B, dtype=np.int32) if rows is None else _c(rows, np.int32)
    Z = np.empty((rows.size, h1 - h0))
    Za = np.empty((rows.size, h1 - h0)) if want_abs else None
    lib().oracle_head_logits(B, D, H, X, Wh, rows, rows.size, h0, h1, Z, _ptr(Za))
    return Z, Za


def positive_mask(row_ptr, labels, label_begin, n_cols, rows=None):
    row_ptr, labels = _c(row_ptr, np.int32), _c(labels, np.int32)
    B = row_ptr.size - 1
    rows = np.arange(B, dtype=np.int32) if rows is None else _c(rows, np.int32)
    Y = np.empty((rows.size, n_cols))
    lib().oracle_positive_mask(row_ptr, labels, rows, rows.size, label_begin,
                               n_cols, Y)
    return Y


def bce(z, y, s):
    z, y = _c(z, np.float64), _c(y, np.float64)
    dz = np.empty_like(z)
    lt = np.empty_like(z)
    lib().oracle_bce(z.size, z, y, float(s), _ptr(dz), _ptr(lt))
    return dz, lt


def tail_dW(X, idx, dZ, L, G, g0=0, g1=None, want_abs=True):
    X, idx, dZ = _c(X, np.float64), _c(idx, np.int32), _c(dZ, np.float64)
    B, D = X.shape
    F = idx.shape[1]
    g1 = (L + G - 1) // G if g1 is None else g1
    nc = n_live(L, G, g0, g1)
    assert dZ.shape == (B, nc)
    dW = np.empty((nc, F))
    dWa = np.empty((nc, F)) if want_abs else None
    lib().oracle_tail_dW(B, D, L, G, F, X, idx, dZ, g0, g1, dW, _ptr(dWa))
    return dW, dWa


def tail_dX(idx, Wt, dZ, D, L, G, want_abs=True):
    idx, Wt, dZ = _c(idx, np.int32), _c(Wt, np.float64), _c(dZ, np.float64)
    F = idx.shape[1]
    n_rows = dZ.shape[0]
    assert dZ.shape[1] == L
    dX = np.empty((n_rows, D))
    dXa = np.empty((n_rows, D)) if want_abs else None
    lib().oracle_tail_dX(D, L, G, F, idx, Wt, dZ, n_rows, dX, _ptr(dXa))
    return dX, dXa


def head_dW(X, dZh, want_abs=True):
    X, dZh = _c(X, np.float64), _c(dZh, np.float64)
    B, D = X.shape
    H = dZh.shape[1]
    dW = np.empty((H, D))
    dWa = np.empty((H, D)) if want_abs else None
    lib().oracle_head_dW(B, D, H, X, dZh, dW, _ptr(dWa))
    return dW, dWa


def head_dX(Wh, dZh, want_abs=True):
    Wh, dZh = _c(Wh, np.float64), _c(dZh, np.float64)
    H, D = Wh.shape
    n_rows = dZh.shape[0]
    dX = np.empty((n_rows, D))
    dXa = np.empty((n_rows, D)) if want_abs else None
    lib().oracle_head_dX(D, H, Wh, dZh, n_rows, dX, _ptr(dXa))
    return dX, dXa


def topk(z, K, ids=None, id_offset=0):
    z = _c(z, np.float64)
    n_rows, n_cols = z.shape
    ids_a = None if ids is None else _c(ids, np.int64)
    val = np.empty((n_rows, K))
    out = np.empty((n_rows, K), np.int64)
    lib().oracle_topk(n_rows, n_cols, z, _ptr(ids_a), id_offset, K, val, out)
    return val, out


# ----------------------------------------------------------------- top-K
# Two-stage top-K of the top-K page (gist.science summary of "A Faster
# Generalized Two-Stage Approximate Top-K", sections "Method" and
# "Theoretical analysis").  Buckets are runs of consecutive labels:
# seg_len = ceil(n / buckets) (the last bucket shorter).

def topk_seg_len(n, buckets):
    assert buckets >= 1
    return -(-n // min(buckets, n))


def topk_two_stage(z, K, kprime, seg_len, id_offset=0):
    """Stage 1: the top-K' of every bucket (value descending, ties to the
    smaller id); stage 2: the top-K of all the buckets' picks.  Rows with
    fewer than K picks are padded with (-inf, -1).  Returns (val, idx) with
    K + 1 columns (the extra one for separation checks)."""
    z = _c(z, np.float64)
    rows, n = z.shape
    SENT = 1 << 62                      # id of a missing pick: sorts last
    cv, ci = [], []
    for c0 in range(0, n, seg_len):
        c1 = min(c0 + seg_len, n)
        v, i = topk(z[:, c0:c1], kprime, id_offset=id_offset + c0)
        i = np.where(i < 0, SENT, i)    # a bucket shorter than K' pads
        cv.append(v)
        ci.append(i)
    V = np.concatenate(cv, axis=1)
    I = np.concatenate(ci, axis=1)
    val = np.empty((rows, K + 1))
    idx = np.empty((rows, K + 1), np.int64)
    for r in range(rows):               # merge over the row's picks (ids given)
        v, i = topk(V[r:r + 1], K + 1, ids=I[r])
        val[r], idx[r] = v[0], i[0]
    missing = idx >= SENT
    val[missing] = -np.inf
    idx[missing] = -1
    return val, idx


def topk_expected_recall(n, K, kprime, seg_len):
    """Expected recall as an exact fraction: the K largest of n items fall on
    a uniformly random K-subset of the positions, the number X that lands in a
    bucket of m items is hypergeometric, P(X = x) = C(K, x) C(n-K, m-x) / C(n, m),
    and a bucket returns min(X, K') of them; recall = sum over buckets of
    E[min(X, K')] / min(K, n)."""
    from fractions import Fraction
    from math import comb
    Kt = min(K, n)
    nseg = -(-n // seg_len)
    sizes = [seg_len] * (nseg - 1) + [n - (nseg - 1) * seg_len]
    total = Fraction(0)
    cache = {}
    for m in sizes:
        if m not in cache:
            e = Fraction(0)
            for x in range(0, min(Kt, m) + 1):
                if m - x > n - Kt:
                    continue
                e += Fraction(comb(Kt, x) * comb(n - Kt, m - x), comb(n, m)) * min(x, kprime)
            cache[m] = e
        total += cache[m]
    return total / Kt


def topk_plan(n, K, target, min_buckets=1):
    """Plain search: for every K' in 1..K the smallest bucket count in
    min_buckets..min(n, 65535) whose expected recall reaches the target; the
    pair with the fewest stage-2 candidates (buckets x K'), ties to the
    smaller K'."""
    from fractions import Fraction
    target = Fraction(target)
    best = None
    for kp in range(1, K + 1):
        for b in range(min_buckets, min(n, 65535) + 1):
            if topk_expected_recall(n, K, kp, topk_seg_len(n, b)) >= target:
                if best is None or b * kp < best[0]:
                    best = (b * kp, kp, b)
                break
    return None if best is None else (best[1], best[2])


def group_positives(row_ptr, labels, label_offset, L, G):
    row_ptr, labels = _c(row_ptr, np.int32), _c(labels, np.int32)
    B = row_ptr.size - 1
    ng = (L + G - 1) // G
    grp_ptr = np.empty(ng + 1, np.int32)
    entries = np.empty(max(1, labels.size), np.int32)
    n = lib().oracle_group_positives(B, row_ptr, labels, label_offset, L, G,
                                     grp_ptr, entries)
    return grp_ptr, entries[:n].copy()


def tail_step(X, idx, Wt, row_ptr, labels, label_offset, L, G, s,
              g0=0, g1=None, want_dW=True, want_dX=True):
    """Streaming tail training step over groups [g0, g1): (loss, dW, dX)."""
    X, idx, Wt = _c(X, np.float64), _c(idx, np.int32), _c(Wt, np.float64)
    row_ptr, labels = _c(row_ptr, np.int32), _c(labels, np.int32)
    B, D = X.shape
    F = idx.shape[1]
    g1 = (L + G - 1) // G if g1 is None else g1
    dW = np.empty((n_live(L, G, g0, g1), F)) if want_dW else None
    dX = np.zeros((B, D)) if want_dX else None
    loss = lib().oracle_tail_step(B, D, L, G, F, X, idx, Wt, row_ptr, labels,
                                  label_offset, float(s), g0, g1, _ptr(dW), _ptr(dX))
    return loss, dW, dX


# ------------------------------------------------------------- composition
@dataclass
class StepResult:
    loss: float
    Zt: np.ndarray
    Zt_abs: np.ndarray
    Zh: np.ndarray
    Zh_abs: np.ndarray
    dZt: np.ndarray
    dZh: np.ndarray
    dWt: np.ndarray
    dWt_abs: np.ndarray
    dWh: np.ndarray
    dWh_abs: np.ndarray
    dX: np.ndarray
    dX_abs: np.ndarray
    dX_tail: np.ndarray
    dX_tail_abs: np.ndarray
    dX_head: np.ndarray
    dX_head_abs: np.ndarray
    loss_head: float
    loss_tail: float


def step(X, Wh, idx, Wt, row_ptr, labels, L, G, s=None) -> StepResult:
    """Full training step, head + tail, for sizes that fit in memory:
    logits, sigmoid-BCE over every (row, label) with the row-CSR positives
    (global ids: head [0, H), tail H + t), and all gradients."""
    X = _c(X, np.float64)
    B, D = X.shape
    H = Wh.shape[0]
    s = 1.0 / B if s is None else s
    Zt, Zta = tail_logits(X, idx, Wt, L, G)
    Zh, Zha = head_logits(X, Wh)
    Yt = positive_mask(row_ptr, labels, H, L)
    Yh = positive_mask(row_ptr, labels, 0, H)
    dZt, lt = bce(Zt, Yt, s)
    dZh, lh = bce(Zh, Yh, s)
    dWt, dWta = tail_dW(X, idx, dZt, L, G)
    dWh, dWha = head_dW(X, dZh)
    dXt, dXta = tail_dX(idx, Wt, dZt, D, L, G)
    dXh, dXha = head_dX(Wh, dZh)
    return StepResult(loss=float(lt.sum() + lh.sum()), Zt=Zt, Zt_abs=Zta, Zh=Zh,
                      Zh_abs=Zha, dZt=dZt, dZh=dZh, dWt=dWt, dWt_abs=dWta,
                      dWh=dWh, dWh_abs=dWha, dX=dXt + dXh, dX_abs=dXta + dXha,
                      dX_tail=dXt, dX_tail_abs=dXta, dX_head=dXh,
                      dX_head_abs=dXha, loss_head=float(lh.sum()),
                      loss_tail=float(lt.sum()))


def sgd(W, dW, lr):
    """Plain gradient-descent update after a step, W - lr * dW (fp64).  The
    pages name no optimizer; this is the textbook step the fused update
    implements."""
    return _c(W, np.float64) - lr * _c(dW, np.float64)


# ------------------------------------------------------ dynamic rewiring
def rewire_scores(Wg, live):
    """Magnitude of each position of one group: the L1 norm of its weight
    column over the group's live labels, summed in float32 in ascending
    label order (the precision and order in which the rewiring decides which
    positions to prune; the inputs are exact in float32)."""
    Wg = np.asarray(Wg, np.float32)
    s = np.zeros(Wg.shape[1], np.float32)
    for j in range(live):
        s = (s + np.abs(Wg[j])).astype(np.float32)
    return s


def tail_rewire(idx, W, L, G, D, k, cand):
    """One prune-and-regrow step of every group's fan-in set (dynamic sparse
    training at group granularity; HASTE page title, and "Method" item 1:
    one index set per group).  The pages give no rule; the reading here:

    1. score every position f of group g by `rewire_scores`;
    2. prune the k positions that come first in (score, feature) order;
    3. regrow k features outside the kept ones: the caller's candidates
       cand[g] in list order, skipping values outside [0, D), kept features
       and repeats; if the list runs out, the smallest features left;
    4. the new set, sorted ascending, replaces idx[g]; a kept feature's
       weight column moves with it (every row of the group, padded rows
       too), a regrown feature's column is zero.

    idx: N_g x F int; W: (N_g*G) x F float32 (exact bf16 or fp32 values);
    cand: N_g x R int.  Returns (idx', W') as new arrays."""
    idx = np.asarray(idx, np.int64)
    W = np.asarray(W, np.float32)
    cand = np.asarray(cand, np.int64)
    ng, F = idx.shape
    idx_new = np.empty_like(idx)
    W_new = np.zeros_like(W)
    for g in range(ng):
        live = min(G, L - g * G)
        rows = slice(g * G, (g + 1) * G)
        score = rewire_scores(W[rows], live)
        order = sorted(range(F), key=lambda f: (float(score[f]), int(idx[g, f])))
        pruned = set(order[:k])
        src = {int(idx[g, f]): f for f in range(F) if f not in pruned}
        taken = []
        for c in cand[g]:
            if len(taken) == k:
                break
            c = int(c)
            if 0 <= c < D and c not in src and c not in taken:
                taken.append(c)
        d = 0
        while len(taken) < k:
            if d not in src and d not in taken:
                taken.append(d)
            d += 1
        new = sorted(list(src) + taken)
        idx_new[g] = new
        for p, feat in enumerate(new):
            if feat in src:
                W_new[rows, p] = W[rows, src[feat]]
    return idx_new.astype(np.int32), W_new
